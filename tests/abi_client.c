/*
 * abi_client.c -- a plain C caller of libfp8bsq (no Python, no PyTorch):
 * HIP runtime calls for memory and a stream, the library's C ABI for the
 * computation.  tests/test_gpu_c_client.py builds it with gcc, writes the
 * inputs, runs it, and checks what it writes against the oracle.
 *
 * usage: abi_client DIR M N K
 *   reads   DIR/x.bf16   bf16 activations [M, K] (raw bits)
 *           DIR/w.e4m3   E4M3 weight codes [N, K]
 *           DIR/ws.f32   weight block scales [ceil(N / 128), K / 128]
 *   writes  DIR/aq.e4m3, DIR/as.f32   fp8_act_quant (scale_fmt None)
 *           DIR/c.bf16                fp8_block_gemm of those, bf16 out
 *           DIR/wd.bf16               fp8_weight_dequant, bf16 out
 *           DIR/c2.f32, DIR/aq2.e4m3, DIR/as2.f32
 *                                     fp8_act_quant_gemm, ue8m0 scales, fp32 out
 * and checks that invalid arguments come back as the documented status codes.
 * Prints "ok" and exits 0, or prints the failing call and exits 1.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <hip/hip_runtime_api.h>

#include "fp8bsq.h"

static int fail(const char *what, const char *detail) {
  fprintf(stderr, "abi_client: %s: %s\n", what, detail);
  return 1;
}

#define HIP_OK(call)                                                       \
  do {                                                                     \
    hipError_t e_ = (call);                                                \
    if (e_ != hipSuccess) return fail(#call, hipGetErrorString(e_));       \
  } while (0)

#define LIB_OK(call)                                                       \
  do {                                                                     \
    int s_ = (call);                                                       \
    if (s_ != FP8BSQ_OK) return fail(#call, fp8bsq_strerror(s_));         \
  } while (0)

static void *read_file(const char *dir, const char *name, size_t bytes) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", dir, name);
  FILE *f = fopen(path, "rb");
  if (!f) return NULL;
  void *p = malloc(bytes ? bytes : 1);
  size_t got = p ? fread(p, 1, bytes, f) : 0;
  fclose(f);
  if (got != bytes) {
    free(p);
    return NULL;
  }
  return p;
}

static int write_file(const char *dir, const char *name, const void *p, size_t bytes) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", dir, name);
  FILE *f = fopen(path, "wb");
  if (!f) return 0;
  size_t put = fwrite(p, 1, bytes, f);
  return fclose(f) == 0 && put == bytes;
}

/* device buffer <- host buffer of the same size */
static int upload(void **dev, const void *host, size_t bytes) {
  if (hipMalloc(dev, bytes) != hipSuccess) return 0;
  return hipMemcpy(*dev, host, bytes, hipMemcpyHostToDevice) == hipSuccess;
}

static int download(const char *dir, const char *name, const void *dev, size_t bytes) {
  void *host = malloc(bytes);
  if (!host) return 0;
  int ok = hipMemcpy(host, dev, bytes, hipMemcpyDeviceToHost) == hipSuccess &&
           write_file(dir, name, host, bytes);
  free(host);
  return ok;
}

int main(int argc, char **argv) {
  if (argc != 5) return fail("usage", "abi_client DIR M N K");
  const char *dir = argv[1];
  const int64_t m = atoll(argv[2]), n = atoll(argv[3]), k = atoll(argv[4]);
  if (m <= 0 || n <= 0 || k <= 0 || k % 128) return fail("arguments", "M, N, K > 0 and K % 128 == 0");
  const int64_t gn = (n + 127) / 128, nkb = k / 128;
  const size_t x_bytes = (size_t)(m * k * 2), w_bytes = (size_t)(n * k), ws_bytes = (size_t)(gn * nkb * 4);

  void *x_h = read_file(dir, "x.bf16", x_bytes), *w_h = read_file(dir, "w.e4m3", w_bytes),
       *ws_h = read_file(dir, "ws.f32", ws_bytes);
  if (!x_h || !w_h || !ws_h) return fail("inputs", "missing or short input file");

  hipStream_t stream;
  HIP_OK(hipStreamCreate(&stream));
  void *x, *w, *ws;
  if (!upload(&x, x_h, x_bytes) || !upload(&w, w_h, w_bytes) || !upload(&ws, ws_h, ws_bytes))
    return fail("upload", "hipMalloc / hipMemcpy failed");
  void *aq, *as, *c, *wd, *c2, *aq2, *as2;
  HIP_OK(hipMalloc(&aq, (size_t)(m * k)));
  HIP_OK(hipMalloc(&as, (size_t)(m * nkb * 4)));
  HIP_OK(hipMalloc(&c, (size_t)(m * n * 2)));
  HIP_OK(hipMalloc(&wd, (size_t)(n * k * 2)));
  HIP_OK(hipMalloc(&c2, (size_t)(m * n * 4)));
  HIP_OK(hipMalloc(&aq2, (size_t)(m * k)));
  HIP_OK(hipMalloc(&as2, (size_t)(m * nkb * 4)));

  LIB_OK(fp8_act_quant(x, FP8BSQ_BF16, m, k, 128, FP8BSQ_SCALE_NONE, (uint8_t *)aq, (float *)as, stream));
  LIB_OK(fp8_block_gemm((const uint8_t *)aq, (const float *)as, (const uint8_t *)w, (const float *)ws, c,
                        FP8BSQ_BF16, m, n, k, stream));
  LIB_OK(fp8_weight_dequant((const uint8_t *)w, (const float *)ws, n, k, 128, wd, FP8BSQ_BF16, stream));
  LIB_OK(fp8_act_quant_gemm(x, FP8BSQ_BF16, FP8BSQ_SCALE_UE8M0, (const uint8_t *)w, (const float *)ws, NULL,
                            c2, FP8BSQ_F32, m, n, k, (uint8_t *)aq2, (float *)as2, stream));
  HIP_OK(hipStreamSynchronize(stream));

  /* rejected before any HIP call: nothing is queued */
  if (fp8_block_gemm((const uint8_t *)aq, (const float *)as, (const uint8_t *)w, (const float *)ws, c,
                     FP8BSQ_BF16, m, n, 100, stream) != FP8BSQ_ESHAPE)
    return fail("fp8_block_gemm(k = 100)", "expected FP8BSQ_ESHAPE");
  if (fp8_act_quant(x, FP8BSQ_BF16, m, k, 64, FP8BSQ_SCALE_NONE, (uint8_t *)aq, (float *)as, stream) !=
      FP8BSQ_EUNSUPPORTED)
    return fail("fp8_act_quant(block_size = 64)", "expected FP8BSQ_EUNSUPPORTED");
  if (fp8_weight_dequant((const uint8_t *)w, (const float *)ws, n, k, 128, (char *)wd + 1, FP8BSQ_BF16,
                         stream) != FP8BSQ_EALIGN)
    return fail("fp8_weight_dequant(misaligned y)", "expected FP8BSQ_EALIGN");
  if (fp8_block_gemm(NULL, NULL, NULL, NULL, NULL, FP8BSQ_BF16, 0, n, k, stream) != FP8BSQ_OK)
    return fail("fp8_block_gemm(m = 0)", "expected FP8BSQ_OK for an empty product");

  if (!download(dir, "aq.e4m3", aq, (size_t)(m * k)) || !download(dir, "as.f32", as, (size_t)(m * nkb * 4)) ||
      !download(dir, "c.bf16", c, (size_t)(m * n * 2)) || !download(dir, "wd.bf16", wd, (size_t)(n * k * 2)) ||
      !download(dir, "c2.f32", c2, (size_t)(m * n * 4)) || !download(dir, "aq2.e4m3", aq2, (size_t)(m * k)) ||
      !download(dir, "as2.f32", as2, (size_t)(m * nkb * 4)))
    return fail("download", "hipMemcpy or file write failed");

  void *bufs[] = {x, w, ws, aq, as, c, wd, c2, aq2, as2};
  for (size_t i = 0; i < sizeof bufs / sizeof bufs[0]; ++i) HIP_OK(hipFree(bufs[i]));
  HIP_OK(hipStreamDestroy(stream));
  free(x_h);
  free(w_h);
  free(ws_h);
  printf("ok %s\n", fp8bsq_version());
  return 0;
}
