// Scale and quotient arithmetic shared by the two quantizers (1 x 128
// activation blocks and 128 x 128 weight tiles).  Both compute, per block,
//     s = fl32(max(amax, fl32(1e-4)) / 448)   (optionally the smallest power
//                                               of two >= s, "ue8m0")
//     code = E4M3(fl32(x / s))                 (round to nearest even)
// with the IEEE results reproduced exactly.
//
// Exact quotient: for bf16 inputs the per-element division is replaced by
// r = fl32(1 / s) (one IEEE division per block) and a residual correction:
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
//
// Include only from translation units compiled with FP contraction off.
#pragma once

#include "device_common.h"

namespace fp8bsq {

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

// 4 fp32 (one 16-byte chunk) -> 4 codes (one dword), IEEE division.
__device__ __forceinline__ uint32_t encode_chunk_f32(u32x4 w, float s) {
  uint32_t c = cvt_pk_e4m3<false>(quotient_f32(__uint_as_float(w.x), s),
                                  quotient_f32(__uint_as_float(w.y), s), 0u);
  return cvt_pk_e4m3<true>(quotient_f32(__uint_as_float(w.z), s),
                           quotient_f32(__uint_as_float(w.w), s), c);
}

}  // namespace fp8bsq
