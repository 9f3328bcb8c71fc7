// Device-side helpers shared by the HIP kernels of the block-scaled FP8 library.
// gfx950 (CDNA4) only: wave64, OCP E4M3 conversions, MFMA f8f6f4.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8bsq {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kBlock = 128;   // the only block size implemented

// DPP controls (quad permutations act inside groups of four lanes).
constexpr int kDppQuadSwap1 = 0xB1;   // quad_perm [1,0,3,2]
constexpr int kDppQuadSwap2 = 0x4E;   // quad_perm [2,3,0,1]

// Max of a uint32 over the four lanes of each quad (all lanes active).
__device__ __forceinline__ uint32_t quad_max_u32(uint32_t v) {
  uint32_t o = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppQuadSwap1, 0xF, 0xF, false);
  v = v > o ? v : o;
  o = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppQuadSwap2, 0xF, 0xF, false);
  return v > o ? v : o;
}

// Two fp32 -> two E4M3 codes (round to nearest even) written into the low
// (kHi=false) or high (kHi=true) 16 bits of `old`.  Callers keep |v| <= 448.
template <bool kHi>
__device__ __forceinline__ uint32_t cvt_pk_e4m3(float a, float b, uint32_t old) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)old, kHi);
}

// Four E4M3 codes packed in a dword -> four fp32 (exact).
__device__ __forceinline__ f32x4 e4m3x4_to_f32(uint32_t w) {
  f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
  f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
  return f32x4{lo.x, lo.y, hi.x, hi.y};
}

// Two fp32 -> packed bf16x2, round to nearest even.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2 h = __builtin_convertvector(f32x2{a, b}, bf16x2);
  return __builtin_bit_cast(uint32_t, h);
}

// Streaming (nontemporal) loads for inputs read exactly once.  Only used where
// each load instruction of a wave covers whole cache lines: a line read in
// parts by several streaming instructions would be fetched more than once.
__device__ __forceinline__ u32x4 load_stream(const u32x4 *p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ u32x2 load_stream(const u32x2 *p) { return __builtin_nontemporal_load(p); }

}  // namespace fp8bsq
