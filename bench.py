"""Throughput of the block-scaled FP8 hot path on one MI355X.

One step = one pass of the whole hot path over the prefill-shaped workload:

  1. act_quant (ue8m0 scales) of bf16 activations [8192, 7168]
     (0.1% outliers x100);
  2. weight_dequant of the E4M3 weight [18432, 7168] with its [144, 56] block
     scales to bf16 (the dequantizer's step of the path; the GEMM below does
     not read its output, since it applies the block scales itself);
  3. the block-scaled GEMM of the quantized activations with that weight, bf16
     out (8192 x 18432 x 7168), through fp8_block_gemm_ue8m0: the activation
     scales are act_quant's ue8m0 powers of two, applied inside the MX-scaled
     MFMA (bit-identical to fp8_block_gemm).

``value`` = 2*M*N*K / step time (TFLOP/s of the whole step, inputs resident
in HBM).  Per-kernel times come from HIP events recorded on the stream the
kernels run on, created without the system-scope fence a default event adds
(that fence's cache write-back would otherwise be timed with the next
kernel); the GEMM is the dominant kernel and its roofline is the dense FP8
MFMA peak.  Each step touches about 1 GB, well beyond the 256 MB Infinity
Cache, so every kernel reads its inputs from HBM.

``configs`` times every workload on its own, each next to the CPU oracle run
on the same inputs in this process (the whole tensor where that takes seconds,
a stated row sample for the prefill GEMMs).  Bandwidth-bound workloads cycle
through enough copies of their buffers (at least 1 GB in all) that no launch
finds its inputs in the Infinity Cache.  Each record gives the mean and the
median of 50 timed launches; short kernels, whose Python launch overhead could
otherwise leave the GPU waiting between them, are queued behind a spin kernel
so that they run back to back.

``cpu_baseline`` times the CPU oracle (test infrastructure, never tuned) on a
bounded sample of the step's workload: the first ``--cpu-rows`` activation rows
through act_quant and the GEMM, and the matching fraction of the weight through
weight_dequant.  OPENBLAS_NUM_THREADS is set to the host threads this process
may use before numpy is imported; the thread count, numpy and OpenBLAS versions
are recorded.

``roofline.traffic`` is the GEMM's HBM traffic per launch measured with
rocprofv3 counters (FETCH_SIZE + WRITE_SIZE, each scaled by what the counter
reads for a copy of known size), read from profiles/block_gemm_prefill_traffic.json;
it is reported as null when the GEMM source has changed since those counters
were taken.

Usage: python bench.py [--gpus 1] [--steps 50] [--warmup 20] [--no-configs] [--no-cpu]
       python bench.py --profile-workload NAME [--iters N]   (one kernel, for rocprofv3)
       python bench.py --calibrate-copy                      (copy of known size, for rocprofv3)
"""

import argparse
import hashlib
import json
import os
import sys
import time


def host_threads() -> int:
    """Host threads this process may use: its CPU affinity, capped by
    OMP_NUM_THREADS when that is set (the machine's share of its cores)."""
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    omp = os.environ.get("OMP_NUM_THREADS", "")
    if omp.isdigit() and int(omp) > 0:
        n = min(n, int(omp))
    return max(1, n)


if __name__ == "__main__":
    # before numpy (and its OpenBLAS) is first imported
    os.environ.setdefault("OPENBLAS_NUM_THREADS", str(host_threads()))

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

M, N, K = 8192, 18432, 7168
PEAK_FP8_TFLOPS = 5000.0     # MI355X dense FP8 MFMA, TFLOP/s
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E, GB/s
ROTATE_BYTES = 1 << 30       # bandwidth workloads cycle through at least this much

# algorithmic bytes per launch (what the method must move)
ACT_QUANT_BYTES = M * K * 2 + M * K + M * (K // 128) * 4                 # 177,995,776
DEQUANT_BYTES = N * K + (N // 128) * (K // 128) * 4 + N * K * 2          # 396,393,984 incl. scales
GEMM_FLOP = 2 * M * N * K                                                # 2,164,663,517,184


def act_quant_bytes(rows, k):
    return rows * k * 2 + rows * k + rows * (k // 128) * 4


def dequant_bytes(n, k, out_bytes=2):
    return n * k + (-(-n // 128)) * (-(-k // 128)) * 4 + n * k * out_bytes


def weight_quant_bytes(n, k):
    return n * k * 2 + n * k + (-(-n // 128)) * (-(-k // 128)) * 4


def decode_bytes(m, n, k):
    """Weight stream plus activation codes, scales and output of one decode GEMM."""
    return m * k + m * (k // 128) * 4 + n * k + (-(-n // 128)) * (k // 128) * 4 + m * n * 2


def parse(argv=None):
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--cpu-rows", type=int, default=6144,
                   help="activation rows in the CPU oracle sample of the step (0 skips it)")
    p.add_argument("--no-cpu", action="store_true", help="skip every CPU oracle timing")
    p.add_argument("--no-configs", action="store_true", help="time the step only")
    p.add_argument("--config-reps", type=int, default=50,
                   help="timed launches per bandwidth-bound workload")
    p.add_argument("--prefill-rows", type=int, default=128,
                   help="activation rows in the CPU oracle sample of each prefill GEMM")
    p.add_argument("--profile-workload", default=None,
                   choices=["act_quant", "act_quant_ue8m0", "dequant", "dequant_ragged", "weight_quant",
                            "weight_quant_ue8m0", "decode1", "decode8", "decode32", "decode64",
                            "act_quant_gemm1", "act_quant_gemm2", "act_quant_gemm8", "act_quant_gemm32",
                            "act_quant_gemm64", "prefill1", "prefill2", "step"],
                   help="run only this workload's kernels --iters times (for rocprofv3)")
    p.add_argument("--iters", type=int, default=20)
    p.add_argument("--calibrate-copy", action="store_true",
                   help="copy 1 GiB once with torch (counter calibration under rocprofv3)")
    return p.parse_args(argv)


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


def copies(t, nbytes_each, total=ROTATE_BYTES):
    """t and enough clones of it that all of them together span `total` bytes."""
    n = max(1, -(-total // max(1, nbytes_each)))
    return [t] + [t.clone() for _ in range(n - 1)]


class Rotation:
    """Cycles through a list of argument sets, one per call."""

    def __init__(self, items):
        self.items = items
        self.i = 0

    def next(self):
        self.i += 1
        return self.items[self.i % len(self.items)]


def profile_workload(name, iters):
    """Run one workload's kernels `iters` times, inputs resident in HBM; the
    bandwidth-bound ones cycle through >= 1 GB of buffer copies so that no
    launch is served from the Infinity Cache."""
    import torch

    import fp8_block_scaled_quant_amd as fb
    from inputs import gen

    dev = torch.device("cuda:0")
    if name.startswith("act_quant_gemm"):
        d = gen.decode_gemm(int(name[len("act_quant_gemm"):]))
        x = d["x"].to(dev)
        w0 = torch.from_numpy(d["w"]).to(dev)
        rot = Rotation(copies(w0, w0.numel()))
        ws = torch.from_numpy(d["w_s"]).to(dev)
        run = lambda: fb.act_quant_gemm(x, rot.next(), ws)
    elif name.startswith("act_quant"):
        x0 = gen.act_quant_workload()["x"].to(dev)
        rot = Rotation(copies(x0, act_quant_bytes(M, K)))
        fmt = "ue8m0" if name.endswith("ue8m0") else None
        run = lambda: fb.act_quant(rot.next(), 128, fmt)
    elif name.startswith("dequant"):
        n = 18440 if name.endswith("ragged") else 18432
        d = gen.dequant_workload(n=n)
        w0 = torch.from_numpy(d["w"]).to(dev)
        ws = torch.from_numpy(d["w_s"]).to(dev)
        rot = Rotation(copies(w0, dequant_bytes(n, K)))
        run = lambda: fb.weight_dequant(rot.next(), ws, 128, torch.bfloat16)
    elif name.startswith("weight_quant"):
        w0 = gen.weight_quant_workload()["w"].to(dev)
        rot = Rotation(copies(w0, weight_quant_bytes(N, K)))
        fmt = "ue8m0" if name.endswith("ue8m0") else None
        run = lambda: fb.weight_quant(rot.next(), 128, fmt)
    elif name.startswith("decode"):
        d = gen.decode_gemm(int(name[len("decode"):]))
        y, s = fb.act_quant(d["x"].to(dev))
        w0 = torch.from_numpy(d["w"]).to(dev)
        rot = Rotation(copies(w0, w0.numel()))
        ws = torch.from_numpy(d["w_s"]).to(dev)
        run = lambda: fb.fp8_gemm(y, s, rot.next(), ws, torch.bfloat16)
    elif name == "step":
        d = gen.prefill_gemm(1)
        x = d["x"].to(dev)
        w = torch.from_numpy(d["w"]).to(dev)
        ws = torch.from_numpy(d["w_s"]).to(dev)

        def run():
            y, s = fb.act_quant(x, 128, "ue8m0")
            fb.weight_dequant(w, ws, 128, torch.bfloat16)
            fb.fp8_gemm(y, s, w, ws, torch.bfloat16, "ue8m0")
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


_SLEEP_CYCLES_PER_MS = None


def hold_gpu_for(ms, stream):
    """Queue a spin kernel of about `ms` milliseconds on `stream` (torch's
    _sleep), so that the host can queue the timed launches behind it: they then
    run back to back, and no event interval holds host launch overhead."""
    global _SLEEP_CYCLES_PER_MS
    import torch
    with torch.cuda.stream(stream):
        if _SLEEP_CYCLES_PER_MS is None:
            ev = TimingEvents(2)
            torch.cuda._sleep(1000)
            ev.record(0, stream)
            torch.cuda._sleep(2_000_000)
            ev.record(1, stream)
            torch.cuda.synchronize()
            _SLEEP_CYCLES_PER_MS = 2_000_000 / max(ev.elapsed_ms(0, 1), 1e-3)
            ev.close()
        torch.cuda._sleep(int(min(ms, 100.0) * _SLEEP_CYCLES_PER_MS))


def time_launches(calls, reps, warmup, stream):
    """Mean and median microseconds of each call in `calls` (callables run in
    order, once per repetition), from events recorded between them on `stream`.
    Where the warm-up shows the host queuing a repetition in more than a third
    of the time the GPU takes to run it, the timed launches are queued behind a
    spin kernel long enough for the host to queue them all, so that they run
    back to back and no interval holds host launch overhead."""
    import numpy as np
    import torch
    wev = TimingEvents(2)
    wev.record(0, stream)
    t0 = time.perf_counter()
    for _ in range(warmup):
        for c in calls:
            c()
    host_ms = (time.perf_counter() - t0) * 1e3 / max(warmup, 1)
    wev.record(1, stream)
    torch.cuda.synchronize()
    gpu_ms = wev.elapsed_ms(0, 1) / max(warmup, 1)
    wev.close()
    nc = len(calls)
    ev = TimingEvents((nc + 1) * reps)
    if host_ms > gpu_ms / 3:
        hold_gpu_for(2 * reps * host_ms + 1.0, stream)
    for r in range(reps):
        base = (nc + 1) * r
        ev.record(base, stream)
        for i, c in enumerate(calls):
            c()
            ev.record(base + i + 1, stream)
    torch.cuda.synchronize()
    out = []
    for i in range(nc):
        t = np.array([ev.elapsed_ms((nc + 1) * r + i, (nc + 1) * r + i + 1) for r in range(reps)]) * 1e3
        out.append((float(t.mean()), float(np.median(t))))
    whole = np.array([ev.elapsed_ms((nc + 1) * r, (nc + 1) * r + nc) for r in range(reps)]) * 1e3
    ev.close()
    return out, (float(whole.mean()), float(np.median(whole)))


def timed_cpu(fn):
    t0 = time.perf_counter()
    out = fn()
    return out, time.perf_counter() - t0


def blas_info():
    """numpy and OpenBLAS versions and the BLAS thread count in this process."""
    import numpy as np
    info = {"numpy": np.__version__, "blas": None, "blas_version": None, "blas_threads": None,
            "OPENBLAS_NUM_THREADS": os.environ.get("OPENBLAS_NUM_THREADS")}
    try:
        from threadpoolctl import threadpool_info
        for i in threadpool_info():
            if i.get("user_api") == "blas":
                info.update(blas=i.get("internal_api"), blas_version=i.get("version"),
                            blas_threads=i.get("num_threads"))
                break
    except Exception:
        pass
    return info


def hbm_record(us, nbytes, extra=None):
    """Rate and HBM fraction of the mean launch time `us` (and of the median,
    when `extra` holds "median_us")."""
    gbs = nbytes / (us * 1e-6) / 1e9
    rec = {"us": us, "GB/s": gbs, "frac_hbm": gbs / PEAK_HBM_GBS, "bytes": nbytes}
    rec.update(extra or {})
    if "median_us" in rec:
        rec["frac_hbm_median"] = nbytes / (rec["median_us"] * 1e-6) / 1e9 / PEAK_HBM_GBS
    return rec


def oracle_record(seconds, what, nbytes=None, flop=None):
    rec = {"oracle_s": seconds, "oracle_sample": what}
    if nbytes:
        rec["oracle_GB/s"] = nbytes / seconds / 1e9
    if flop:
        rec["oracle_GFLOP/s"] = flop / seconds / 1e9
    return rec


def bench_configs(args, stream):
    """Per-workload records: GPU time and rate, roofline fraction, oracle time."""
    import numpy as np
    import torch

    import fp8_block_scaled_quant_amd as fb
    import oracle
    from inputs import gen

    dev = torch.device("cuda:0")
    reps, warm = args.config_reps, 20   # ~20 launches for the clock to settle after host-side work
    cpu = not args.no_cpu
    recs = {}

    def log(msg):
        print(f"[bench] {msg}", file=sys.stderr, flush=True)

    # 1. tiny GEMM: fp32 activations [16, 512] -> act_quant (None) -> GEMM, fp32 out
    d = gen.tiny_gemm()
    x = d["x"].to(dev)
    w = torch.from_numpy(d["w"]).to(dev)
    ws = torch.from_numpy(d["w_s"]).to(dev)
    y, s = fb.act_quant(x)
    (aq, gm), _ = time_launches([lambda: fb.act_quant(x), lambda: fb.fp8_gemm(y, s, w, ws, torch.float32)],
                                reps, warm, stream)
    rec = {"workload": "tiny: act_quant fp32 [16,512] (scale_fmt None) + block GEMM 16x256x512, fp32 out",
           "act_quant_us": aq[0], "gemm_us": gm[0], "gemm_flop": 2 * 16 * 256 * 512, "bound": "launch latency"}
    if cpu:
        xn = d["x"].numpy()
        _, t = timed_cpu(lambda: oracle.fp8_gemm(*oracle.act_quant(xn), d["w"], d["w_s"]))
        rec.update(oracle_record(t, "whole workload"))
    recs["tiny"] = rec
    log("tiny done")

    # 2. act_quant [8192, 7168] bf16, both scale formats, rotating >= 1 GB
    d = gen.act_quant_workload()
    nbytes = act_quant_bytes(M, K)
    xs = copies(d["x"].to(dev), nbytes)
    xn = d["x"].float().numpy() if cpu else None
    for fmt in (None, "ue8m0"):
        rot = Rotation(xs)
        (t,), _ = time_launches([lambda: fb.act_quant(rot.next(), 128, fmt)], reps, warm, stream)
        rec = hbm_record(t[0], nbytes, {"median_us": t[1], "rotation": len(xs),
                                        "workload": f"act_quant bf16 [8192,7168] scale_fmt={fmt}"})
        if cpu:
            _, tc = timed_cpu(lambda: oracle.act_quant(xn, 128, fmt))
            rec.update(oracle_record(tc, "whole tensor", nbytes=nbytes))
        recs[f"act_quant_{'ue8m0' if fmt else 'none'}"] = rec
    del xs, xn
    log("act_quant done")

    # 3. weight_dequant [18432, 7168] and ragged [18440, 7168] -> bf16, rotating >= 1 GB
    for n, key in ((18432, "dequant"), (18440, "dequant_ragged")):
        d = gen.dequant_workload(n=n)
        nbytes = dequant_bytes(n, K)
        wl = copies(torch.from_numpy(d["w"]).to(dev), nbytes)
        ws = torch.from_numpy(d["w_s"]).to(dev)
        rot = Rotation(wl)
        (t,), _ = time_launches([lambda: fb.weight_dequant(rot.next(), ws, 128, torch.bfloat16)], reps, warm,
                                stream)
        rec = hbm_record(t[0], nbytes, {"median_us": t[1], "rotation": len(wl),
                                        "workload": f"weight_dequant E4M3 [{n},7168] -> bf16"})
        if cpu:
            _, tc = timed_cpu(lambda: oracle.weight_dequant(d["w"], d["w_s"], 128, "bf16"))
            rec.update(oracle_record(tc, "whole tensor", nbytes=nbytes))
        recs[key] = rec
        del wl
    log("dequant done")

    # weight_quant (the GEMM's weight operand) bf16 [18432, 7168], rotating >= 1 GB
    d = gen.weight_quant_workload()
    nbytes = weight_quant_bytes(N, K)
    wl = copies(d["w"].to(dev), nbytes)
    for fmt in (None, "ue8m0"):
        rot = Rotation(wl)
        (t,), _ = time_launches([lambda: fb.weight_quant(rot.next(), 128, fmt)], reps, warm, stream)
        recs[f"weight_quant_{'ue8m0' if fmt else 'none'}"] = hbm_record(
            t[0], nbytes, {"median_us": t[1], "rotation": len(wl),
                           "workload": f"weight_quant bf16 [18432,7168] scale_fmt={fmt}"})
    del wl
    log("weight_quant done")

    # 4. decode GEMMs: weights cycle through >= 1 GB of copies
    for m in (1, 8, 32, 64):
        d = gen.decode_gemm(m)
        x = d["x"].to(dev)
        wl = copies(torch.from_numpy(d["w"]).to(dev), N * K)
        ws = torch.from_numpy(d["w_s"]).to(dev)
        y, s = fb.act_quant(x)
        rot = Rotation(wl)
        (gm,), _ = time_launches([lambda: fb.fp8_gemm(y, s, rot.next(), ws, torch.bfloat16)], reps, warm, stream)
        rot = Rotation(wl)
        (aq, gm2), pair = time_launches([lambda: fb.act_quant(x),
                                         lambda: fb.fp8_gemm(y, s, rot.next(), ws, torch.bfloat16)],
                                        reps, warm, stream)
        rot = Rotation(wl)
        (fu,), _ = time_launches([lambda: fb.act_quant_gemm(x, rot.next(), ws)], reps, warm, stream)
        nbytes = decode_bytes(m, N, K)
        flop = 2 * m * N * K
        rec = hbm_record(gm[0], nbytes, {
            "workload": f"decode GEMM M={m} N=18432 K=7168, bf16 out (activations quantized by act_quant, None)",
            "median_us": gm[1], "TFLOP/s": flop / (gm[0] * 1e-6) / 1e12, "rotation": len(wl),
            "act_quant_us": aq[0], "act_quant_then_gemm_us": pair[0],
            "act_quant_gemm_call_us": fu[0]})
        if cpu:
            xn = d["x"].float().numpy()
            _, tc = timed_cpu(lambda: oracle.fp8_gemm(*oracle.act_quant(xn), d["w"], d["w_s"]))
            rec.update(oracle_record(tc, "whole workload (act_quant + GEMM)", flop=flop))
        recs[f"decode_m{m}"] = rec
        del wl
    log("decode done")

    # 5. prefill GEMMs, ue8m0 activation scales, bf16 out (shape 2 may split its last round over K)
    for shape in (1, 2):
        d = gen.prefill_gemm(shape)
        n, k = d["w"].shape
        x = d["x"].to(dev)
        w = torch.from_numpy(d["w"]).to(dev)
        ws = torch.from_numpy(d["w_s"]).to(dev)
        y, s = fb.act_quant(x, 128, "ue8m0")
        # enough warm-up launches (~20 ms) for the clock to settle after the idle host-side work
        (aq, gm), _ = time_launches([lambda: fb.act_quant(x, 128, "ue8m0"),
                                     lambda: fb.fp8_gemm(y, s, w, ws, torch.bfloat16, "ue8m0")],
                                    max(5, reps // 2), 20, stream)
        flop = 2 * M * n * k
        tf = flop / (gm[0] * 1e-6) / 1e12
        rec = {"workload": f"prefill GEMM {M}x{n}x{k}, ue8m0 activation scales, bf16 out",
               "us": gm[0], "median_us": gm[1], "TFLOP/s": tf, "frac_mfma": tf / PEAK_FP8_TFLOPS,
               "frac_mfma_median": flop / (gm[1] * 1e-6) / 1e12 / PEAK_FP8_TFLOPS, "flop": flop,
               "act_quant_us": aq[0], "act_quant_bytes": act_quant_bytes(M, k)}
        if cpu and args.prefill_rows > 0:
            rows = args.prefill_rows
            xn = d["x"][:rows].float().numpy()
            _, tc = timed_cpu(lambda: oracle.fp8_gemm(*oracle.act_quant(xn, 128, "ue8m0"), d["w"], d["w_s"]))
            rec.update(oracle_record(tc, f"first {rows} of {M} rows (act_quant + GEMM, all {n} columns)",
                                     flop=2 * rows * n * k))
        recs[f"prefill_shape{shape}"] = rec
        del x, w, y
    log("prefill done")
    return recs


def cpu_baseline(x_bf16, w, ws, rows):
    """Time the oracle on the first `rows` rows (and rows/M of the weight)."""
    import numpy as np
    import oracle
    info = blas_info()
    x = x_bf16[:rows].float().numpy()
    wrows = max(128, (N * rows // M) // 128 * 128)
    t0 = time.perf_counter()
    a, a_s = oracle.act_quant(x, 128, "ue8m0")
    oracle.weight_dequant(w[:wrows], np.ascontiguousarray(ws[:wrows // 128]), 128, "bf16")
    oracle.fp8_gemm(a, a_s, w, ws)
    dt = time.perf_counter() - t0
    flop = 2.0 * rows * N * K
    cores = info["blas_threads"] or host_threads()
    return {
        "value": flop / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": cores,
        "kind": "oracle",
        "sample": (f"first {rows} of {M} activation rows through act_quant(ue8m0) + fp8_gemm "
                   f"(all {N} columns) and {wrows} of {N} weight rows through weight_dequant; "
                   f"{dt:.2f} s; value = 2*{rows}*N*K / time; {cores} BLAS threads "
                   f"(elementwise steps single-threaded numpy)"),
        "seconds": dt,
        "host": info,
    }


def main(argv=None):
    args = parse(argv)
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

    aq_t = [ev.elapsed_ms(4 * i, 4 * i + 1) for i in range(args.steps)]
    dq_t = [ev.elapsed_ms(4 * i + 1, 4 * i + 2) for i in range(args.steps)]
    gm_t = [ev.elapsed_ms(4 * i + 2, 4 * i + 3) for i in range(args.steps)]
    aq_ms, dq_ms, gm_ms = (float(np.mean(t)) for t in (aq_t, dq_t, gm_t))
    aq_med, dq_med, gm_med = (float(np.median(t)) for t in (aq_t, dq_t, gm_t))
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
            "workload": ("one pass of the hot path, three kernels: act_quant (ue8m0) of bf16 [8192,7168]; "
                         "weight_dequant of E4M3 [18432,7168] with [144,56] scales -> bf16 (not read by the "
                         "GEMM); block-scaled FP8 GEMM 8192x18432x7168 (fp8_block_gemm_ue8m0), bf16 out"),
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
                          "median_us": aq_med * 1e3,
                          "frac_hbm_median": ACT_QUANT_BYTES / (aq_med * 1e-3) / 1e9 / PEAK_HBM_GBS,
                          "bytes": ACT_QUANT_BYTES},
            "weight_dequant": {"us": dq_ms * 1e3, "GB/s": dq_gbs, "frac_hbm": dq_gbs / PEAK_HBM_GBS,
                               "median_us": dq_med * 1e3,
                               "frac_hbm_median": DEQUANT_BYTES / (dq_med * 1e-3) / 1e9 / PEAK_HBM_GBS,
                               "bytes": DEQUANT_BYTES},
            "block_gemm": {"us": gm_ms * 1e3, "TFLOP/s": gemm_tflops,
                           "frac_mfma": gemm_tflops / PEAK_FP8_TFLOPS, "median_us": gm_med * 1e3,
                           "frac_mfma_median": GEMM_FLOP / (gm_med * 1e-3) / 1e12 / PEAK_FP8_TFLOPS,
                           "flop": GEMM_FLOP},
        },
        "cpu_baseline": None,
    }
    del x, w
    if not args.no_configs:
        result["configs"] = bench_configs(args, stream)
    if not args.no_cpu and args.cpu_rows > 0:
        result["cpu_baseline"] = cpu_baseline(x_cpu, w_np, ws_np, args.cpu_rows)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
