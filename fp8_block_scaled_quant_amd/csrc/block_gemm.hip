// Block-scaled FP8 E4M3 GEMM for gfx950: C[m, n] = A[m, k] . B[n, k]^T.
//
// Method (page "How weight_dequant Handles Per-Block Scaling in DeepSeek-V3
// FP8 GEMM", section "Relationship to FP8 GEMM Operations": the scales are
// folded into the product instead of dequantizing the weight; page
// "DeepSeek-V3: How Selective FP8 Stays Stable", "Learning outcomes" and FAQ:
// partial sums are periodically promoted to FP32).  Here every 128-wide K
// block kb yields an FP32 partial from one E4M3 MFMA per 16x16 output tile,
//     P = sum_{k in kb} A[i, k] * B[j, k],
// which is multiplied by a_s[i, kb] * b_s[j / 128, kb] and added into an FP32
// accumulator held in registers.
//
// MFMA operands: v_mfma_f32_16x16x128_f8f6f4 takes, per lane, 32 bytes of a
// 16-row A fragment and 32 bytes of a 16-column B fragment.  Lane l supplies
// row (l % 16) and the 32-byte K slice (l / 16); A and B are loaded with the
// same lane/byte -> k assignment, so the product is the block's full dot
// product whatever order the hardware pairs the bytes in.  The 16x16 FP32
// result sits in lane l as column (l % 16), rows 4 * (l / 16) + 0..3.
#include "device_common.h"
#include "launch.h"

namespace fp8bsq {
namespace {

__device__ __forceinline__ f32x4 mfma_e4m3_16x16x128(const i32x8 &a, const i32x8 &b, f32x4 c) {
  // format 0 = E4M3 for both operands; scale operands unused (plain MFMA).
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ i32x8 load_frag(const uint8_t *p) {
  const uint4 lo = *(const uint4 *)p;
  const uint4 hi = *(const uint4 *)(p + 16);
  return i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z,
               (int)hi.w};
}

__device__ __forceinline__ void store_out(void *c, bool bf16, int64_t idx, float v) {
  if (bf16)
    ((uint16_t *)c)[idx] = (uint16_t)(pack_bf16x2(v, 0.0f) & 0xFFFFu);
  else
    ((float *)c)[idx] = v;
}

// Reference-structure kernel: 256 threads = 2 x 2 waves, each wave a 32 x 32
// output tile (2 x 2 MFMA tiles), fragments read straight from global memory.
// The 64-column workgroup tile never straddles a 128-row weight block, so the
// weight scale is workgroup-uniform.
template <bool kBf16Out>
__global__ __launch_bounds__(256) void block_gemm_simple_kernel(
    const uint8_t *__restrict__ a, const float *__restrict__ a_s, const uint8_t *__restrict__ b,
    const float *__restrict__ b_s, void *__restrict__ c, int64_t m, int64_t n, int64_t k) {
  const int nkb = (int)(k / kBlock);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t m0 = (int64_t)blockIdx.y * 64 + (wave >> 1) * 32;
  const int64_t n0 = (int64_t)blockIdx.x * 64 + (wave & 1) * 32;
  const int64_t b_row = ((int64_t)blockIdx.x * 64) / kBlock;
  const int lr = lane & 15, lk = (lane >> 4) * 32, lq = (lane >> 4) * 4;

  f32x4 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const i32x8 zero8 = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int kb = 0; kb < nkb; ++kb) {
    i32x8 af[2], bfr[2];
    float sa[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int64_t row = m0 + 16 * i + lr;
      af[i] = row < m ? load_frag(a + row * k + (int64_t)kb * kBlock + lk) : zero8;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t orow = m0 + 16 * i + lq + r;
        sa[i][r] = orow < m ? a_s[orow * nkb + kb] : 0.0f;
      }
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t col = n0 + 16 * j + lr;
      bfr[j] = col < n ? load_frag(b + col * k + (int64_t)kb * kBlock + lk) : zero8;
    }
    const float sb = b_s[b_row * nkb + kb];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const f32x4 p = mfma_e4m3_16x16x128(af[i], bfr[j], f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[i][j][r] = __builtin_fmaf(p[r], sa[i][r] * sb, acc[i][j][r]);
      }
  }

#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t col = n0 + 16 * j + lr;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t row = m0 + 16 * i + lq + r;
        if (row < m && col < n) store_out(c, kBf16Out, row * n + col, acc[i][j][r]);
      }
    }
}

}  // namespace

hipError_t launch_block_gemm(const uint8_t *a, const float *a_s, const uint8_t *b,
                             const float *b_s, void *c, bool c_bf16, int64_t m, int64_t n,
                             int64_t k, hipStream_t stream) {
  const dim3 grid((unsigned)((n + 63) / 64), (unsigned)((m + 63) / 64)), block(256);
  if (c_bf16)
    hipLaunchKernelGGL(block_gemm_simple_kernel<true>, grid, block, 0, stream, a, a_s, b, b_s, c,
                       m, n, k);
  else
    hipLaunchKernelGGL(block_gemm_simple_kernel<false>, grid, block, 0, stream, a, a_s, b, b_s, c,
                       m, n, k);
  return hipGetLastError();
}

}  // namespace fp8bsq
