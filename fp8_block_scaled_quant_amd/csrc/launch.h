// Internal launchers: one per kernel family.  Arguments are already validated
// by the C ABI layer (abi.cpp); each returns the HIP error of its launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fp8bsq {

// x: [nblocks, 128] bf16 or fp32 (16-byte aligned); y: [nblocks, 128] codes;
// s: [nblocks] scales.
hipError_t launch_act_quant(const void *x, bool x_bf16, int64_t nblocks, bool ue8m0, uint8_t *y,
                            float *s, hipStream_t stream);

// x: [m, n] codes; s: [ceil(m/128), ceil(n/128)]; y: [m, n] fp32 or bf16.
hipError_t launch_weight_dequant(const uint8_t *x, const float *s, int64_t m, int64_t n, void *y,
                                 bool y_bf16, hipStream_t stream);

// x: [m, n] bf16 or fp32; y: [m, n] codes; s: [ceil(m/128), ceil(n/128)] scales.
hipError_t launch_weight_quant(const void *x, bool x_bf16, int64_t m, int64_t n, bool ue8m0,
                               uint8_t *y, float *s, hipStream_t stream);

// C[m, n] = block-scaled A[m, k] . B[n, k]^T (+ bias[n] of C's dtype, if not null).
// a_s_pow2: every a_s is a power of two (act_quant ue8m0), so the tiled kernel
// may apply it inside the MX-scaled MFMA; when it does, a guard kernel queued
// after it sets to NaN every C row whose a_s row breaks that precondition.
hipError_t launch_block_gemm(const uint8_t *a, const float *a_s, const uint8_t *b,
                             const float *b_s, void *c, bool c_bf16, int64_t m, int64_t n,
                             int64_t k, hipStream_t stream, const void *bias = nullptr,
                             bool a_s_pow2 = false);

// The same product by the reference-structure kernel (fragments straight from
// global memory), for any shape: what shapes beyond the fast kernels' 32-bit
// offsets take.
hipError_t launch_block_gemm_reference(const uint8_t *a, const float *a_s, const uint8_t *b,
                                       const float *b_s, void *c, bool c_bf16, int64_t m, int64_t n,
                                       int64_t k, hipStream_t stream, const void *bias = nullptr);

// launch_block_gemm with split-K for a last round of tiles that would leave
// CUs idle.  workspace: block_gemm_split_bytes(m, n, k) bytes, 256-byte
// aligned, with no initial contents required: the call clears the tail's
// counters itself (in its first launch) and leaves them at the part count.
// With a smaller workspace (or when no split pays), the same launch as
// launch_block_gemm.
size_t block_gemm_split_bytes(int64_t m, int64_t n, int64_t k);
hipError_t launch_block_gemm_split(const uint8_t *a, const float *a_s, const uint8_t *b,
                                   const float *b_s, void *c, bool c_bf16, int64_t m, int64_t n,
                                   int64_t k, hipStream_t stream, bool a_s_pow2, void *workspace,
                                   size_t workspace_bytes);

// launch_block_gemm_split with the library's static per-device scratch
// (FP8BSQ_SPLIT_SCRATCH_BYTES) as its workspace; *too_big is set, and nothing
// queued, when the split needs more than that.
hipError_t launch_block_gemm_split_noalloc(const uint8_t *a, const float *a_s, const uint8_t *b,
                                           const float *b_s, void *c, bool c_bf16, int64_t m,
                                           int64_t n, int64_t k, hipStream_t stream, bool a_s_pow2,
                                           bool *too_big);

// Fused act_quant + decode GEMM (bf16 x [m, k], m small enough for
// act_quant_gemm_fusable): C = Q(x) . B^T (+ bias); a_q / a_s receive
// act_quant's codes and scales.
hipError_t launch_act_quant_gemm_fused(const void *x, bool ue8m0, const uint8_t *b,
                                      const float *b_s, const void *bias, void *c, bool c_bf16,
                                      int64_t m, int64_t n, int64_t k, uint8_t *a_q, float *a_s,
                                      hipStream_t stream);
bool act_quant_gemm_fusable(bool x_bf16, int64_t m, int64_t k);

}  // namespace fp8bsq
