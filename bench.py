"""Throughput of the block-scaled FP8 hot path on one MI355X.

One step = one pass of the whole path over the prefill-shaped linear layer:

  1. act_quant (ue8m0 scales) of bf16 activations [8192, 7168]
     (the act_quant bandwidth workload's shape, 0.1% outliers x100);
  2. weight_dequant of the E4M3 weight [18432, 7168] with its [144, 56]
     block scales to bf16 (the dequant bandwidth workload);
  3. the block-scaled GEMM of the quantized activations with that weight,
     bf16 out (the prefill GEMM, 8192 x 18432 x 7168), through
     fp8_block_gemm_ue8m0: the activation scales are act_quant's ue8m0 powers
     of two, applied inside the MX-scaled MFMA (bit-identical to
     fp8_block_gemm).

``value`` = 2*M*N*K / step time (TFLOP/s of the whole step, inputs resident
in HBM).  Per-kernel times come from HIP events recorded on the stream the
kernels run on, created without the system-scope fence a default event adds
(that fence's cache write-back would otherwise be timed with the next
kernel); the GEMM is the dominant kernel and its roofline is the dense FP8
MFMA peak.  Each step touches about 1 GB, well beyond the 256 MB Infinity
Cache, so every kernel reads its inputs from HBM.

``cpu_baseline`` times the CPU oracle (test infrastructure, never tuned) on a
bounded sample of the same workload: the first ``--cpu-rows`` activation rows
through act_quant and the GEMM, and the matching fraction of the weight through
weight_dequant.

``roofline.traffic`` is the GEMM's HBM traffic per launch measured with
rocprofv3 counters (FETCH_SIZE + WRITE_SIZE, each scaled by what the counter
reads for a copy of known size), read from profiles/block_gemm_prefill_traffic.json;
it is reported as null when the GEMM source has changed since those counters
were taken.

Usage: python bench.py [--gpus 1] [--steps 50] [--warmup 10]
       python bench.py --profile-workload NAME [--iters N]   (one kernel, for rocprofv3)
       python bench.py --calibrate-copy                      (copy of known size, for rocprofv3)
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

M, N, K = 8192, 18432, 7168
PEAK_FP8_TFLOPS = 5000.0     # MI355X dense FP8 MFMA, TFLOP/s
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E, GB/s

# algorithmic bytes per launch (what the method must move)
ACT_QUANT_BYTES = M * K * 2 + M * K + M * (K // 128) * 4                 # 177,995,776
DEQUANT_BYTES = N * K + (N // 128) * (K // 128) * 4 + N * K * 2          # 396,393,984 incl. scales
GEMM_FLOP = 2 * M * N * K                                                # 2,164,663,517,184


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--cpu-rows", type=int, default=6144,
                   help="activation rows in the CPU oracle sample (0 skips it)")
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--profile-workload", default=None,
                   choices=["act_quant", "act_quant_ue8m0", "dequant", "dequant_ragged", "weight_quant",
                            "weight_quant_ue8m0", "decode1", "decode8", "decode32", "decode64",
                            "act_quant_gemm1", "act_quant_gemm2", "prefill1", "prefill2"],
                   help="run only this workload's kernel --iters times (for rocprofv3)")
    p.add_argument("--iters", type=int, default=20)
    p.add_argument("--calibrate-copy", action="store_true",
                   help="copy 1 GiB once with torch (counter calibration under rocprofv3)")
    return p.parse_args()


GEMM_SOURCE = os.path.join(ROOT, "fp8_block_scaled_quant_amd", "csrc", "block_gemm.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "block_gemm_prefill_traffic.json")


def source_hash(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def measured_traffic():
    """HBM bytes per GEMM launch from the committed counter summary, or None
    if it is missing or was taken on a different GEMM source."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("block_gemm_hip_sha256") != source_hash(GEMM_SOURCE):
        return None
    return rec.get("bytes_per_launch")


def profile_workload(name, iters):
    """Run one workload's kernel `iters` times (inputs resident in HBM)."""
    import torch

    import fp8_block_scaled_quant_amd as fb
    from inputs import gen

    dev = torch.device("cuda:0")
    # the decode workloads cycle through eight copies of the 132 MB weight so
    # that every read comes from HBM, not the 256 MB Infinity Cache
    step = [0]

    def rotating(ws_list):
        step[0] += 1
        return ws_list[step[0] % len(ws_list)]

    if name.startswith("act_quant_gemm"):
        d = gen.decode_gemm(int(name[len("act_quant_gemm"):]))
        x = d["x"].to(dev)
        w0 = torch.from_numpy(d["w"]).to(dev)
        wl = [w0] + [w0.clone() for _ in range(7)]
        ws = torch.from_numpy(d["w_s"]).to(dev)
        run = lambda: fb.act_quant_gemm(x, rotating(wl), ws)
    elif name.startswith("act_quant"):
        x = gen.act_quant_workload()["x"].to(dev)
        fmt = "ue8m0" if name.endswith("ue8m0") else None
        run = lambda: fb.act_quant(x, 128, fmt)
    elif name.startswith("dequant"):
        d = gen.dequant_workload(n=18440 if name.endswith("ragged") else 18432)
        w = torch.from_numpy(d["w"]).to(dev)
        ws = torch.from_numpy(d["w_s"]).to(dev)
        run = lambda: fb.weight_dequant(w, ws, 128, torch.bfloat16)
    elif name.startswith("weight_quant"):
        w = gen.weight_quant_workload()["w"].to(dev)
        fmt = "ue8m0" if name.endswith("ue8m0") else None
        run = lambda: fb.weight_quant(w, 128, fmt)
    elif name.startswith("decode"):
        d = gen.decode_gemm(int(name[len("decode"):]))
        y, s = fb.act_quant(d["x"].to(dev))
        w0 = torch.from_numpy(d["w"]).to(dev)
        wl = [w0] + [w0.clone() for _ in range(7)]
        ws = torch.from_numpy(d["w_s"]).to(dev)
        run = lambda: fb.fp8_gemm(y, s, rotating(wl), ws, torch.bfloat16)
    else:
        d = gen.prefill_gemm(int(name[-1]))
        y, s = fb.act_quant(d["x"].to(dev), 128, "ue8m0")
        w = torch.from_numpy(d["w"]).to(dev)
        ws = torch.from_numpy(d["w_s"]).to(dev)
        run = lambda: fb.fp8_gemm(y, s, w, ws, torch.bfloat16, "ue8m0")
    for _ in range(iters):
        run()
    torch.cuda.synchronize()
    print(f"ran {name} x{iters}", flush=True)


def calibrate_copy():
    import torch
    dev = torch.device("cuda:0")
    a = torch.ones(1 << 30, dtype=torch.uint8, device=dev)
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    print("copied 1073741824 bytes", flush=True)


class TimingEvents:
    """HIP events for timing only, created with hipEventDisableSystemFence.

    A default event performs a system-scope fence (an L2 write-back and
    invalidate) when it is reached, and a kernel bracketed by such events is
    timed with that flush and its aftermath.  These events skip it; their
    elapsed times are read after a device synchronization.  The HIP runtime is
    the one torch and the library already loaded (soname libamdhip64.so.7).
    """
    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self, count):
        import ctypes
        self._c = ctypes
        self._hip = hip = ctypes.CDLL("libamdhip64.so.7")
        hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.events = []
        for _ in range(count):
            e = ctypes.c_void_p()
            if hip.hipEventCreateWithFlags(ctypes.byref(e), self.DISABLE_SYSTEM_FENCE) != 0:
                raise RuntimeError("hipEventCreateWithFlags failed")
            self.events.append(e)

    def record(self, i, stream):
        if self._hip.hipEventRecord(self.events[i], self._c.c_void_p(stream.cuda_stream)) != 0:
            raise RuntimeError("hipEventRecord failed")

    def elapsed_ms(self, i, j):
        ms = self._c.c_float()
        if self._hip.hipEventElapsedTime(self._c.byref(ms), self.events[i], self.events[j]) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def close(self):
        for e in self.events:
            self._hip.hipEventDestroy(e)
        self.events = []


def cpu_baseline(x_bf16, w, ws, rows):
    """Time the oracle on the first `rows` rows (and rows/M of the weight)."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas_threads = None
    x = x_bf16[:rows].float().numpy()
    wrows = max(128, (N * rows // M) // 128 * 128)
    t0 = time.perf_counter()
    a, a_s = oracle.act_quant(x, 128, "ue8m0")
    oracle.weight_dequant(w[:wrows], np.ascontiguousarray(ws[:wrows // 128]), 128, "bf16")
    oracle.fp8_gemm(a, a_s, w, ws)
    dt = time.perf_counter() - t0
    flop = 2.0 * rows * N * K
    cores = len(os.sched_getaffinity(0))
    return {
        "value": flop / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": blas_threads if blas_threads else cores,
        "kind": "oracle",
        "sample": (f"first {rows} of {M} activation rows through act_quant(ue8m0) + fp8_gemm "
                   f"(all {N} columns) and {wrows} of {N} weight rows through weight_dequant; "
                   f"{dt:.2f} s; value = 2*{rows}*N*K / time; host has {cores} usable cores"),
        "seconds": dt,
    }


def main():
    args = parse()
    if args.profile_workload:
        profile_workload(args.profile_workload, args.iters)
        return
    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(every kernel here runs on a single device with no cross-GPU work).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import fp8_block_scaled_quant_amd as fb
    from inputs import gen

    dev = torch.device("cuda:0")
    fb.load_library()

    d = gen.prefill_gemm(1)
    x_cpu, w_np, ws_np = d["x"], d["w"], d["w_s"]
    x = x_cpu.to(dev)
    w = torch.from_numpy(w_np).to(dev).view(torch.float8_e4m3fn)
    ws = torch.from_numpy(ws_np).to(dev)
    stream = torch.cuda.current_stream(dev)

    def step(i=None):
        if i is not None:
            ev.record(4 * i, stream)
        y, s = fb.act_quant(x, 128, "ue8m0")
        if i is not None:
            ev.record(4 * i + 1, stream)
        wd = fb.weight_dequant(w, ws, 128, torch.bfloat16)
        if i is not None:
            ev.record(4 * i + 2, stream)
        c = fb.fp8_gemm(y, s, w, ws, torch.bfloat16, "ue8m0")
        if i is not None:
            ev.record(4 * i + 3, stream)
        return c, wd

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region: exactly `steps` steps, synchronized on both sides
    ev = TimingEvents(4 * args.steps)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    aq_ms = float(np.mean([ev.elapsed_ms(4 * i, 4 * i + 1) for i in range(args.steps)]))
    dq_ms = float(np.mean([ev.elapsed_ms(4 * i + 1, 4 * i + 2) for i in range(args.steps)]))
    gm_ms = float(np.mean([ev.elapsed_ms(4 * i + 2, 4 * i + 3) for i in range(args.steps)]))
    ev.close()
    ms_per_step = elapsed * 1e3 / args.steps

    gemm_tflops = GEMM_FLOP / (gm_ms * 1e-3) / 1e12
    aq_gbs = ACT_QUANT_BYTES / (aq_ms * 1e-3) / 1e9
    dq_gbs = DEQUANT_BYTES / (dq_ms * 1e-3) / 1e9

    result = {
        "metric": "block-scaled FP8 GEMM TFLOP/s (% FP8 MFMA peak); act_quant/dequant HBM GB/s",
        "value": GEMM_FLOP / (ms_per_step * 1e-3) / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3",
        "data": "synthetic",
        "config": {
            "workload": ("prefill linear layer: act_quant ue8m0 of bf16 [8192,7168] + weight_dequant "
                         "[18432,7168]->bf16 + block-scaled FP8 GEMM 8192x18432x7168, bf16 out"),
            "m": M, "n": N, "k": K, "scale_fmt": "ue8m0", "out": "bf16",
        },
        "roofline": {
            "bound": "mfma",
            "achieved": gemm_tflops,
            "peak": PEAK_FP8_TFLOPS,
            "unit": "TFLOP/s",
            "frac": gemm_tflops / PEAK_FP8_TFLOPS,
            "traffic": measured_traffic(),
        },
        "kernels": {
            "act_quant": {"us": aq_ms * 1e3, "GB/s": aq_gbs, "frac_hbm": aq_gbs / PEAK_HBM_GBS,
                          "bytes": ACT_QUANT_BYTES},
            "weight_dequant": {"us": dq_ms * 1e3, "GB/s": dq_gbs, "frac_hbm": dq_gbs / PEAK_HBM_GBS,
                               "bytes": DEQUANT_BYTES},
            "block_gemm": {"us": gm_ms * 1e3, "TFLOP/s": gemm_tflops,
                           "frac_mfma": gemm_tflops / PEAK_FP8_TFLOPS, "flop": GEMM_FLOP},
        },
        "cpu_baseline": None,
    }
    if not args.no_cpu and args.cpu_rows > 0:
        result["cpu_baseline"] = cpu_baseline(x_cpu, w_np, ws_np, args.cpu_rows)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
