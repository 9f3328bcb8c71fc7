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
// Exact quotient: the codes must equal E4M3(fl32(x / s)).  For bf16 inputs
// the per-element division is replaced by r = fl32(1 / s) (one IEEE division
// per block) and a residual correction:
//     q0 = x * r;  e = q0 * s - x (fused);  q = q0 - e * r (fused).
// This returns fl32(x / s) for every bf16 significand and every fp32 scale
// significand (checked exhaustively, 2^30 pairs, by tests/division_identity.c);
// residuals are exact whenever |x| >= 2^-102, and below that |x / s| < 2^-80
// encodes to zero either way.  The sign convention of e keeps x = -0 at -0.
// The scale itself, fl32(amax / 448), is computed the same way from the
// constant fl32(1/448); the same file checks that against the IEEE division
// for every fp32 amax from fl32(1e-4) to the largest finite value.  Under
// ue8m0 the scale is a power of two and its reciprocal is exact bit arithmetic.
// fp32 inputs use the IEEE division directly.
#include "device_common.h"
#include "launch.h"

#pragma clang fp contract(off)

namespace fp8bsq {
namespace {

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

constexpr float kFp8Max = 448.0f;
constexpr float kAmaxFloor = 1e-4f;   // fl32(1e-4) = 0x38D1B717
constexpr float kInv448 = 0x1.24924Ap-9f;   // fl32(1/448) = 0x3B124925

// DPP row rotations (within each 16-lane row).
constexpr int kDppRowRor8 = 0x128, kDppRowRor4 = 0x124, kDppRowRor2 = 0x122, kDppRowRor1 = 0x121;

__device__ __forceinline__ uint32_t row_max_u32(uint32_t v) {
  uint32_t o = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppRowRor8, 0xF, 0xF, false);
  v = v > o ? v : o;
  o = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppRowRor4, 0xF, 0xF, false);
  v = v > o ? v : o;
  o = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppRowRor2, 0xF, 0xF, false);
  v = v > o ? v : o;
  o = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppRowRor1, 0xF, 0xF, false);
  return v > o ? v : o;
}

// s = fl32(amax / 448) and r = fl32(1 / s), amax given as the bits of a
// non-negative fp32 (bf16 path: reciprocal-and-residual form of the division).
__device__ __forceinline__ void block_scale_fast(uint32_t amax_bits, bool ue8m0, float &s, float &r) {
  float amax = __uint_as_float(amax_bits);
  amax = amax > kAmaxFloor ? amax : kAmaxFloor;
  const float q0 = amax * kInv448;
  const float e = __builtin_fmaf(q0, kFp8Max, -amax);
  s = __builtin_fmaf(-e, kInv448, q0);
  if (ue8m0) {
    // smallest power of two >= s; its reciprocal is the mirrored exponent
    const uint32_t p = (__float_as_uint(s) + 0x007FFFFFu) & 0xFF800000u;
    s = __uint_as_float(p);
    r = __uint_as_float(0x7F000000u - p);
  } else {
    r = 1.0f / s;                                         // IEEE, correctly rounded
  }
}

// s and r = fl32(1/s) from the block's amax (given as the bits of a
// non-negative fp32).
__device__ __forceinline__ void block_scale(uint32_t amax_bits, bool ue8m0, float &s, float &r) {
  float amax = __uint_as_float(amax_bits);
  amax = amax > kAmaxFloor ? amax : kAmaxFloor;
  s = amax / kFp8Max;                                     // IEEE, correctly rounded
  if (ue8m0) {
    // smallest power of two >= s (s is a positive normal here): carry any
    // nonzero mantissa into the exponent, then clear the mantissa.
    s = __uint_as_float((__float_as_uint(s) + 0x007FFFFFu) & 0xFF800000u);
  }
  r = 1.0f / s;                                           // IEEE, correctly rounded
}

__device__ __forceinline__ float quotient_bf16(float x, float s, float r) {
  float q0 = x * r;
  float e = __builtin_fmaf(q0, s, -x);
  float q = __builtin_fmaf(-e, r, q0);
  return __builtin_amdgcn_fmed3f(q, -kFp8Max, kFp8Max);
}

__device__ __forceinline__ float quotient_f32(float x, float s) {
  return __builtin_amdgcn_fmed3f(x / s, -kFp8Max, kFp8Max);
}

// 8 bf16 (one 16-byte chunk) -> 8 codes (two dwords).
__device__ __forceinline__ u32x2 encode_chunk_bf16(u32x4 w, float s, float r) {
  const uint32_t d[4] = {w.x, w.y, w.z, w.w};
  uint32_t out[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint32_t a = d[2 * h], b = d[2 * h + 1];
    const float x0 = __uint_as_float(a << 16), x1 = __uint_as_float(a & 0xFFFF0000u);
    const float x2 = __uint_as_float(b << 16), x3 = __uint_as_float(b & 0xFFFF0000u);
    uint32_t c = cvt_pk_e4m3<false>(quotient_bf16(x0, s, r), quotient_bf16(x1, s, r), 0u);
    c = cvt_pk_e4m3<true>(quotient_bf16(x2, s, r), quotient_bf16(x3, s, r), c);
    out[h] = c;
  }
  return u32x2{out[0], out[1]};
}

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
