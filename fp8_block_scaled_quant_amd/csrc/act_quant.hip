// Dynamic 1x128 activation quantization to E4M3 for gfx950.
//
// Method (page "Understanding Dynamic and Static Activation Quantization
// Schemes in DeepSeek-V3", section "How Dynamic Activation Quantization Works";
// page "DeepSeek-V3 quantization_config Parameters Explained", section "The
// activation_scheme Parameter"): for every 1 x 128 block along the last
// dimension, amax = max |x| clamped to at least 1e-4, s = amax / 448
// (optionally rounded up to a power of two, "ue8m0"), codes = E4M3(x / s).
//
// Layout: x is [rows, k] row-major with k % 128 == 0, so the blocks of the whole
// tensor form one contiguous sequence [nblocks, 128] and the scales one
// contiguous [nblocks] vector.  The kernel works on that flat sequence.
//
// Work split (bf16 input): sixteen lanes own one block, 8 elements (16 bytes)
// each, so every load instruction of a wave reads 1 KiB of four consecutive
// blocks and every code store writes their 512 contiguous bytes: both cover
// whole cache lines, so loads and stores both stream past the caches.  A wave
// covers 8 blocks in two such instructions (fewer in flight per wave and more
// waves measured faster than four or eight); the block's amax is reduced over
// its 16-lane row with four DPP row rotations.  (fp32 inputs, used only for
// small activations, keep four lanes per block.)
//
// The scale and the exact quotient E4M3(fl32(x / s)) come from quant_common.h.
#include "launch.h"
#include "quant_common.h"

#pragma clang fp contract(off)

namespace fp8bsq {
namespace {

// Blocks handled per wave: kWaveBlocks = 4 rows x kChunks load instructions.
constexpr int kChunks = 2, kWaveBlocks = 4 * kChunks, kWgBlocks = 4 * kWaveBlocks;

template <bool kUe8m0>
__global__ __launch_bounds__(256) void act_quant_bf16_kernel(const u32x4 *__restrict__ x,
                                                              u32x2 *__restrict__ y,
                                                              float *__restrict__ scales,
                                                              int64_t nblocks) {
  const int lane = threadIdx.x & 63;
  const int row = lane >> 4, sub = lane & 15;
  const int64_t blk0 = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * kWaveBlocks + row;

  u32x4 v[kChunks];
#pragma unroll
  for (int i = 0; i < kChunks; ++i) {
    const int64_t blk = blk0 + 4 * i;                 // 16 chunks of 8 bf16 per block
    v[i] = blk < nblocks ? load_stream(x + blk * 16 + sub) : u32x4{0, 0, 0, 0};
  }
#pragma unroll
  for (int i = 0; i < kChunks; ++i) {
    const int64_t blk = blk0 + 4 * i;
    // |x| max on the packed bf16 halves: clearing the sign bits leaves
    // magnitudes whose integer order is their numeric order.
    u16x2 m2 = {0, 0};
    const uint32_t d[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
#pragma unroll
    for (int j = 0; j < 4; ++j)
      m2 = __builtin_elementwise_max(m2, __builtin_bit_cast(u16x2, d[j] & 0x7FFF7FFFu));
    const uint32_t amax = row_max_u32((uint32_t)(m2.x > m2.y ? m2.x : m2.y) << 16);
    float s, r;
    block_scale_fast(amax, kUe8m0, s, r);
    if (blk < nblocks) {
      // 16 lanes x 8 codes = one whole 128-byte line per block: stream it out
      __builtin_nontemporal_store(encode_chunk_bf16(v[i], s, r), y + blk * 16 + sub);
      if (sub == 0) scales[blk] = s;
    }
  }
}

template <bool kUe8m0>
__global__ __launch_bounds__(256) void act_quant_f32_kernel(const u32x4 *__restrict__ x,
                                                             uint32_t *__restrict__ y,
                                                             float *__restrict__ scales,
                                                             int64_t nblocks) {
  const int lane = threadIdx.x & 63;
  const int64_t blk = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * 16 + (lane >> 2);
  const int sub = lane & 3;
  const bool valid = blk < nblocks;

  u32x4 v[8];
  if (valid) {
    const u32x4 *xb = x + blk * 32;          // 32 chunks of 4 fp32
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = xb[4 * i + sub];
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = u32x4{0, 0, 0, 0};
  }

  uint32_t amax = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t d[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t a = d[j] & 0x7FFFFFFFu;
      amax = amax > a ? amax : a;
    }
  }
  amax = quad_max_u32(amax);

  float s, r;
  block_scale(amax, kUe8m0, s, r);

  if (valid) {
    uint32_t *yb = y + blk * 32;             // 32 groups of 4 codes
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint32_t c = cvt_pk_e4m3<false>(quotient_f32(__uint_as_float(v[i].x), s),
                                      quotient_f32(__uint_as_float(v[i].y), s), 0u);
      c = cvt_pk_e4m3<true>(quotient_f32(__uint_as_float(v[i].z), s),
                            quotient_f32(__uint_as_float(v[i].w), s), c);
      yb[4 * i + sub] = c;
    }
    if (sub == 0) scales[blk] = s;
  }
}

}  // namespace

hipError_t launch_act_quant(const void *x, bool x_bf16, int64_t nblocks, bool ue8m0, uint8_t *y,
                            float *s, hipStream_t stream) {
  const dim3 block(256);
  if (x_bf16) {
    const dim3 grid((unsigned)((nblocks + kWgBlocks - 1) / kWgBlocks));
    if (ue8m0)
      hipLaunchKernelGGL(act_quant_bf16_kernel<true>, grid, block, 0, stream,
                         (const u32x4 *)x, (u32x2 *)y, s, nblocks);
    else
      hipLaunchKernelGGL(act_quant_bf16_kernel<false>, grid, block, 0, stream,
                         (const u32x4 *)x, (u32x2 *)y, s, nblocks);
  } else {
    const dim3 grid((unsigned)((nblocks + 63) / 64));
    if (ue8m0)
      hipLaunchKernelGGL(act_quant_f32_kernel<true>, grid, block, 0, stream,
                         (const u32x4 *)x, (uint32_t *)y, s, nblocks);
    else
      hipLaunchKernelGGL(act_quant_f32_kernel<false>, grid, block, 0, stream,
                         (const u32x4 *)x, (uint32_t *)y, s, nblocks);
  }
  return hipGetLastError();
}

}  // namespace fp8bsq
