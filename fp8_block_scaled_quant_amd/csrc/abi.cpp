// C ABI of the block-scaled FP8 library: argument validation and dispatch.
// Every check runs before any HIP call, so a rejected call queues nothing.
// A call whose outputs have no elements passes the enum and shape checks and
// then returns FP8BSQ_OK without looking at its pointers.
#include <stddef.h>
#include <stdint.h>

#include "fp8bsq.h"
#include "launch.h"

namespace {

constexpr int64_t kMaxDim = (int64_t)1 << 31;        // per-dimension limit of the launch grids
constexpr int64_t kMaxGemmRows = (int64_t)65535 * 64; // grid.y limit of the GEMM launch

bool aligned(const void *p, uintptr_t bytes) { return ((uintptr_t)p % bytes) == 0; }

int launch_status(hipError_t e) { return e == hipSuccess ? FP8BSQ_OK : FP8BSQ_ELAUNCH; }

}  // namespace

extern "C" {

int fp8_act_quant(const void *x, int x_dtype, int64_t rows, int64_t k, int block_size,
                  int scale_fmt, uint8_t *y, float *s, void *hip_stream) {
  if (rows < 0 || k < 0) return FP8BSQ_EINVAL;
  if (x_dtype != FP8BSQ_F32 && x_dtype != FP8BSQ_BF16) return FP8BSQ_EINVAL;
  if (scale_fmt != FP8BSQ_SCALE_NONE && scale_fmt != FP8BSQ_SCALE_UE8M0) return FP8BSQ_EINVAL;
  if (block_size != 128) return FP8BSQ_EUNSUPPORTED;
  if (k % block_size != 0) return FP8BSQ_ESHAPE;
  if (rows == 0 || k == 0) return FP8BSQ_OK;
  if (!x || !y || !s) return FP8BSQ_EINVAL;
  if (!aligned(x, 16) || !aligned(y, 8) || !aligned(s, 4)) return FP8BSQ_EALIGN;
  if (rows >= kMaxDim || k >= kMaxDim) return FP8BSQ_ERANGE;
  const int64_t nblocks = rows * (k / block_size);
  if ((nblocks + 31) / 32 >= kMaxDim) return FP8BSQ_ERANGE;
  return launch_status(fp8bsq::launch_act_quant(x, x_dtype == FP8BSQ_BF16, nblocks,
                                                scale_fmt == FP8BSQ_SCALE_UE8M0, y, s,
                                                (hipStream_t)hip_stream));
}

int fp8_weight_dequant(const uint8_t *x, const float *s, int64_t m, int64_t n, int block_size,
                       void *y, int y_dtype, void *hip_stream) {
  if (m < 0 || n < 0) return FP8BSQ_EINVAL;
  if (y_dtype != FP8BSQ_F32 && y_dtype != FP8BSQ_BF16) return FP8BSQ_EINVAL;
  if (block_size != 128) return FP8BSQ_EUNSUPPORTED;
  if (m == 0 || n == 0) return FP8BSQ_OK;
  if (!x || !s || !y) return FP8BSQ_EINVAL;
  if (!aligned(s, 4) || !aligned(y, y_dtype == FP8BSQ_F32 ? 4 : 2)) return FP8BSQ_EALIGN;
  if (m >= kMaxDim || n >= kMaxDim || m * n >= ((int64_t)1 << 50)) return FP8BSQ_ERANGE;
  return launch_status(fp8bsq::launch_weight_dequant(x, s, m, n, y, y_dtype == FP8BSQ_BF16,
                                                     (hipStream_t)hip_stream));
}

int fp8_weight_quant(const void *x, int x_dtype, int64_t m, int64_t n, int block_size,
                     int scale_fmt, uint8_t *y, float *s, void *hip_stream) {
  if (m < 0 || n < 0) return FP8BSQ_EINVAL;
  if (x_dtype != FP8BSQ_F32 && x_dtype != FP8BSQ_BF16) return FP8BSQ_EINVAL;
  if (scale_fmt != FP8BSQ_SCALE_NONE && scale_fmt != FP8BSQ_SCALE_UE8M0) return FP8BSQ_EINVAL;
  if (block_size != 128) return FP8BSQ_EUNSUPPORTED;
  if (m == 0 || n == 0) return FP8BSQ_OK;
  if (!x || !y || !s) return FP8BSQ_EINVAL;
  if (!aligned(x, x_dtype == FP8BSQ_F32 ? 4 : 2) || !aligned(s, 4)) return FP8BSQ_EALIGN;
  if (m >= kMaxDim || n >= kMaxDim || m * n >= ((int64_t)1 << 50)) return FP8BSQ_ERANGE;
  if ((m + 127) / 128 > 65535) return FP8BSQ_ERANGE;   // grid.y
  return launch_status(fp8bsq::launch_weight_quant(x, x_dtype == FP8BSQ_BF16, m, n,
                                                   scale_fmt == FP8BSQ_SCALE_UE8M0, y, s,
                                                   (hipStream_t)hip_stream));
}

namespace {

enum class GemmKernel { kDispatch, kDispatchPow2, kReference };

int block_gemm_checked(const uint8_t *a, const float *a_s, const uint8_t *b, const float *b_s,
                       void *c, int c_dtype, int64_t m, int64_t n, int64_t k, void *hip_stream,
                       GemmKernel kernel) {
  if (m < 0 || n < 0 || k <= 0) return FP8BSQ_EINVAL;
  if (c_dtype != FP8BSQ_F32 && c_dtype != FP8BSQ_BF16) return FP8BSQ_EINVAL;
  if (k % 128 != 0) return FP8BSQ_ESHAPE;
  if (m == 0 || n == 0) return FP8BSQ_OK;
  if (!a || !a_s || !b || !b_s || !c) return FP8BSQ_EINVAL;
  if (!aligned(a, 16) || !aligned(b, 16) || !aligned(a_s, 4) || !aligned(b_s, 4) ||
      !aligned(c, 4))
    return FP8BSQ_EALIGN;
  if (m > kMaxGemmRows || n >= kMaxDim || k >= kMaxDim) return FP8BSQ_ERANGE;
  const bool bf16 = c_dtype == FP8BSQ_BF16;
  const hipStream_t st = (hipStream_t)hip_stream;
  if (kernel == GemmKernel::kReference)
    return launch_status(fp8bsq::launch_block_gemm_reference(a, a_s, b, b_s, c, bf16, m, n, k, st));
  return launch_status(fp8bsq::launch_block_gemm(a, a_s, b, b_s, c, bf16, m, n, k, st, nullptr,
                                                 kernel == GemmKernel::kDispatchPow2));
}

}  // namespace

int fp8_block_gemm(const uint8_t *a, const float *a_s, const uint8_t *b, const float *b_s,
                   void *c, int c_dtype, int64_t m, int64_t n, int64_t k, void *hip_stream) {
  return block_gemm_checked(a, a_s, b, b_s, c, c_dtype, m, n, k, hip_stream, GemmKernel::kDispatch);
}

int fp8_block_gemm_ue8m0(const uint8_t *a, const float *a_s, const uint8_t *b, const float *b_s,
                         void *c, int c_dtype, int64_t m, int64_t n, int64_t k, void *hip_stream) {
  return block_gemm_checked(a, a_s, b, b_s, c, c_dtype, m, n, k, hip_stream,
                            GemmKernel::kDispatchPow2);
}

int fp8_block_gemm_reference(const uint8_t *a, const float *a_s, const uint8_t *b, const float *b_s,
                             void *c, int c_dtype, int64_t m, int64_t n, int64_t k, void *hip_stream) {
  return block_gemm_checked(a, a_s, b, b_s, c, c_dtype, m, n, k, hip_stream, GemmKernel::kReference);
}

size_t fp8_block_gemm_split_workspace(int64_t m, int64_t n, int64_t k) {
  if (m <= 0 || n <= 0 || k <= 0 || k % 128 != 0) return 0;   // rejected, or nothing to split
  if (m > kMaxGemmRows || n >= kMaxDim || k >= kMaxDim) return 0;
  return fp8bsq::block_gemm_split_bytes(m, n, k);
}

int fp8_block_gemm_split(const uint8_t *a, const float *a_s, const uint8_t *b, const float *b_s,
                         void *c, int c_dtype, int64_t m, int64_t n, int64_t k, int scale_fmt,
                         void *workspace, size_t workspace_bytes, void *hip_stream) {
  if (m < 0 || n < 0 || k <= 0) return FP8BSQ_EINVAL;
  if (c_dtype != FP8BSQ_F32 && c_dtype != FP8BSQ_BF16) return FP8BSQ_EINVAL;
  if (scale_fmt != FP8BSQ_SCALE_NONE && scale_fmt != FP8BSQ_SCALE_UE8M0) return FP8BSQ_EINVAL;
  if (k % 128 != 0) return FP8BSQ_ESHAPE;
  if (m == 0 || n == 0) return FP8BSQ_OK;
  if (!a || !a_s || !b || !b_s || !c) return FP8BSQ_EINVAL;
  if (!aligned(a, 16) || !aligned(b, 16) || !aligned(a_s, 4) || !aligned(b_s, 4) ||
      !aligned(c, 4) || !aligned(workspace, 256))
    return FP8BSQ_EALIGN;
  if (m > kMaxGemmRows || n >= kMaxDim || k >= kMaxDim) return FP8BSQ_ERANGE;
  return launch_status(fp8bsq::launch_block_gemm_split(
      a, a_s, b, b_s, c, c_dtype == FP8BSQ_BF16, m, n, k, (hipStream_t)hip_stream,
      scale_fmt == FP8BSQ_SCALE_UE8M0, workspace, workspace ? workspace_bytes : 0));
}

int fp8_block_gemm_split_noalloc(const uint8_t *a, const float *a_s, const uint8_t *b,
                                 const float *b_s, void *c, int c_dtype, int64_t m, int64_t n,
                                 int64_t k, int scale_fmt, void *hip_stream) {
  if (m < 0 || n < 0 || k <= 0) return FP8BSQ_EINVAL;
  if (c_dtype != FP8BSQ_F32 && c_dtype != FP8BSQ_BF16) return FP8BSQ_EINVAL;
  if (scale_fmt != FP8BSQ_SCALE_NONE && scale_fmt != FP8BSQ_SCALE_UE8M0) return FP8BSQ_EINVAL;
  if (k % 128 != 0) return FP8BSQ_ESHAPE;
  if (m == 0 || n == 0) return FP8BSQ_OK;
  if (!a || !a_s || !b || !b_s || !c) return FP8BSQ_EINVAL;
  if (!aligned(a, 16) || !aligned(b, 16) || !aligned(a_s, 4) || !aligned(b_s, 4) || !aligned(c, 4))
    return FP8BSQ_EALIGN;
  if (m > kMaxGemmRows || n >= kMaxDim || k >= kMaxDim) return FP8BSQ_ERANGE;
  bool too_big = false;
  const int rc = launch_status(fp8bsq::launch_block_gemm_split_noalloc(
      a, a_s, b, b_s, c, c_dtype == FP8BSQ_BF16, m, n, k, (hipStream_t)hip_stream,
      scale_fmt == FP8BSQ_SCALE_UE8M0, &too_big));
  return too_big ? FP8BSQ_ESCRATCH : rc;
}

int fp8_act_quant_gemm(const void *x, int x_dtype, int scale_fmt, const uint8_t *b,
                       const float *b_s, const void *bias, void *c, int c_dtype, int64_t m,
                       int64_t n, int64_t k, uint8_t *a_q, float *a_s, void *hip_stream) {
  if (m < 0 || n < 0 || k <= 0) return FP8BSQ_EINVAL;
  if (x_dtype != FP8BSQ_F32 && x_dtype != FP8BSQ_BF16) return FP8BSQ_EINVAL;
  if (c_dtype != FP8BSQ_F32 && c_dtype != FP8BSQ_BF16) return FP8BSQ_EINVAL;
  if (scale_fmt != FP8BSQ_SCALE_NONE && scale_fmt != FP8BSQ_SCALE_UE8M0) return FP8BSQ_EINVAL;
  if (k % 128 != 0) return FP8BSQ_ESHAPE;
  if (m == 0) return FP8BSQ_OK;
  // with no weight rows only the quantization has outputs: b, b_s, bias and c go unread
  const bool product = n > 0;
  if (!x || !a_q || !a_s || (product && (!b || !b_s || !c))) return FP8BSQ_EINVAL;
  if (!aligned(x, 16) || !aligned(a_q, 16) || !aligned(a_s, 4)) return FP8BSQ_EALIGN;
  if (product && (!aligned(b, 16) || !aligned(b_s, 4) || !aligned(c, 4) ||
                  !aligned(bias, c_dtype == FP8BSQ_F32 ? 4 : 2)))
    return FP8BSQ_EALIGN;
  if (m > kMaxGemmRows || n >= kMaxDim || k >= kMaxDim) return FP8BSQ_ERANGE;
  if ((m * (k / 128) + 31) / 32 >= kMaxDim) return FP8BSQ_ERANGE;
  const hipStream_t st = (hipStream_t)hip_stream;
  const bool x_bf16 = x_dtype == FP8BSQ_BF16, ue8m0 = scale_fmt == FP8BSQ_SCALE_UE8M0;
  if (!product) return launch_status(fp8bsq::launch_act_quant(x, x_bf16, m * (k / 128), ue8m0, a_q, a_s, st));
  if (fp8bsq::act_quant_gemm_fusable(x_bf16, m, k))
    return launch_status(fp8bsq::launch_act_quant_gemm_fused(x, ue8m0, b, b_s, bias, c,
                                                            c_dtype == FP8BSQ_BF16, m, n, k, a_q,
                                                            a_s, st));
  const int rc = launch_status(fp8bsq::launch_act_quant(x, x_bf16, m * (k / 128), ue8m0, a_q, a_s, st));
  if (rc != FP8BSQ_OK) return rc;
  return launch_status(fp8bsq::launch_block_gemm(a_q, a_s, b, b_s, c, c_dtype == FP8BSQ_BF16, m, n,
                                                 k, st, bias, ue8m0));
}

const char *fp8bsq_strerror(int status) {
  switch (status) {
    case FP8BSQ_OK: return "ok";
    case FP8BSQ_EINVAL: return "invalid argument (null pointer, negative size, K of 0 for a product, or unknown enum)";
    case FP8BSQ_ESHAPE: return "a dimension that must be a multiple of the block size is not";
    case FP8BSQ_EUNSUPPORTED: return "unsupported block size (only 128 is implemented)";
    case FP8BSQ_EALIGN: return "pointer is not aligned as the entry point requires";
    case FP8BSQ_ELAUNCH: return "HIP runtime error at kernel launch";
    case FP8BSQ_ERANGE: return "size exceeds the kernels' indexing limits";
    case FP8BSQ_ESCRATCH: return "the split needs more scratch than the library's static buffer holds";
    default: return "unknown status";
  }
}

const char *fp8bsq_version(void) { return "0.1.0"; }

}  // extern "C"
