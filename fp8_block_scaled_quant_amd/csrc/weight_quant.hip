// 128x128 block weight quantization to E4M3 for gfx950: the inverse of the
// block-scaled weight dequantization.
//
// Method (page "DeepSeek-V3 quantization_config Parameters Explained",
// section "The weight_block_size Parameter"; page "How weight_dequant Handles
// Per-Block Scaling in DeepSeek-V3 FP8 GEMM", sections "Per-Block Scaling
// Architecture" and "Grid Mapping and Scale Lookup"): weights are held as E4M3
// codes in 128 x 128 tiles, each with one FP32 scale (weight_scale_inv) in a
// row-major [ceil(m/128), ceil(n/128)] grid, and dequantize as y = code * s.
// The pages print no rule for producing them; this library applies the
// activation rule to the tile (page "Understanding Dynamic and Static
// Activation Quantization Schemes in DeepSeek-V3", section "How Dynamic
// Activation Quantization Works"): amax over the tile's elements, clamped to
// at least 1e-4, s = amax / 448 (optionally rounded up to a power of two,
// "ue8m0"), codes = E4M3(x / s).  Edge tiles use their valid elements only.
//
// One 256-thread workgroup per tile.  Sixteen lanes cover one 128-element row
// of the tile (8 elements each), so a wave's load instruction reads four
// whole rows (bf16: 256 bytes each) and a code store writes four whole
// 128-byte lines; 16 rows per pass, 8 passes, all loads issued before any
// arithmetic.  The tile amax is reduced over each 16-lane row with DPP, over
// the wave with two lane exchanges, and over the four waves through LDS; the
// codes are then formed from the registers, so the weight is read once.
//
// Shapes with n % 8 != 0, or unaligned pointers, take an element-wise kernel.
#include "launch.h"
#include "quant_common.h"

#pragma clang fp contract(off)

namespace fp8bsq {
namespace {

// Max of the tile: per-lane value in, workgroup-uniform value out.
__device__ __forceinline__ uint32_t tile_max_u32(uint32_t v, uint32_t *red) {
  v = row_max_u32(v);                                   // within 16-lane rows
  uint32_t o = (uint32_t)__shfl_xor((int)v, 16);
  v = v > o ? v : o;
  o = (uint32_t)__shfl_xor((int)v, 32);
  v = v > o ? v : o;
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  const uint32_t a = red[0] > red[1] ? red[0] : red[1];
  const uint32_t b = red[2] > red[3] ? red[2] : red[3];
  return a > b ? a : b;
}

template <bool kBf16In, bool kUe8m0>
__global__ __launch_bounds__(256) void weight_quant_tile_kernel(const void *__restrict__ x,
                                                                uint8_t *__restrict__ y,
                                                                float *__restrict__ scales,
                                                                int64_t m, int64_t n,
                                                                int64_t grid_n) {
  __shared__ uint32_t red[4];
  constexpr int kLoads = kBf16In ? 1 : 2;             // 16-byte loads per 8 elements
  const int64_t tile_c = blockIdx.x, tile_r = blockIdx.y;
  const int tid = threadIdx.x;
  const int64_t col = tile_c * kBlock + (tid & 15) * 8;
  const int64_t row0 = tile_r * kBlock + (tid >> 4);
  const bool col_ok = col < n;                        // n % 8 == 0: chunks never straddle the edge
  const int elem = kBf16In ? 2 : 4;

  u32x4 v[8][kLoads];
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    const int64_t row = row0 + 16 * p;
    const u32x4 *src = (const u32x4 *)((const uint8_t *)x + (row * n + col) * elem);
#pragma unroll
    for (int h = 0; h < kLoads; ++h)
      v[p][h] = (col_ok && row < m) ? load_stream(src + h) : u32x4{0, 0, 0, 0};
  }

  uint32_t amax = 0;
  if (kBf16In) {
    // |x| max on the packed bf16 halves: clearing the sign bits leaves
    // magnitudes whose integer order is their numeric order.
    u16x2 m2 = {0, 0};
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      const uint32_t d[4] = {v[p][0].x, v[p][0].y, v[p][0].z, v[p][0].w};
#pragma unroll
      for (int j = 0; j < 4; ++j)
        m2 = __builtin_elementwise_max(m2, __builtin_bit_cast(u16x2, d[j] & 0x7FFF7FFFu));
    }
    amax = (uint32_t)(m2.x > m2.y ? m2.x : m2.y) << 16;
  } else {
#pragma unroll
    for (int p = 0; p < 8; ++p)
#pragma unroll
      for (int h = 0; h < kLoads; ++h) {
        const uint32_t d[4] = {v[p][h].x, v[p][h].y, v[p][h].z, v[p][h].w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t a = d[j] & 0x7FFFFFFFu;
          amax = amax > a ? amax : a;
        }
      }
  }
  amax = tile_max_u32(amax, red);

  float s, r;
  if (kBf16In)
    block_scale_fast(amax, kUe8m0, s, r);
  else
    block_scale(amax, kUe8m0, s, r);

  // a full tile row is one whole 128-byte line of codes: stream it out
  const bool full_rows = tile_c * kBlock + kBlock <= n;
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    const int64_t row = row0 + 16 * p;
    if (!col_ok || row >= m) continue;
    u32x2 c;
    if (kBf16In)
      c = encode_chunk_bf16(v[p][0], s, r);
    else
      c = u32x2{encode_chunk_f32(v[p][0], s), encode_chunk_f32(v[p][1], s)};
    u32x2 *dst = (u32x2 *)(y + row * n + col);
    if (full_rows)
      __builtin_nontemporal_store(c, dst);
    else
      *dst = c;
  }
  if (tid == 0) scales[tile_r * grid_n + tile_c] = s;
}

// Any shape and alignment: element by element, the tile read twice.
template <bool kBf16In, bool kUe8m0>
__global__ __launch_bounds__(256) void weight_quant_elementwise_kernel(
    const void *__restrict__ x, uint8_t *__restrict__ y, float *__restrict__ scales, int64_t m,
    int64_t n, int64_t grid_n) {
  __shared__ uint32_t red[4];
  const int64_t tile_c = blockIdx.x, tile_r = blockIdx.y;
  const int64_t r0 = tile_r * kBlock, c0 = tile_c * kBlock;
  auto load = [&](int64_t i) -> float {
    return kBf16In ? __uint_as_float((uint32_t)((const uint16_t *)x)[i] << 16)
                   : ((const float *)x)[i];
  };
  uint32_t amax = 0;
  for (int e = threadIdx.x; e < kBlock * kBlock; e += 256) {
    const int64_t row = r0 + e / kBlock, col = c0 + e % kBlock;
    if (row < m && col < n) {
      const uint32_t a = __float_as_uint(load(row * n + col)) & 0x7FFFFFFFu;
      amax = amax > a ? amax : a;
    }
  }
  amax = tile_max_u32(amax, red);
  float s, r;
  if (kBf16In)
    block_scale_fast(amax, kUe8m0, s, r);
  else
    block_scale(amax, kUe8m0, s, r);
  for (int e = threadIdx.x; e < kBlock * kBlock; e += 256) {
    const int64_t row = r0 + e / kBlock, col = c0 + e % kBlock;
    if (row < m && col < n) {
      const float v = load(row * n + col);
      const float q = kBf16In ? quotient_bf16(v, s, r) : quotient_f32(v, s);
      y[row * n + col] = (uint8_t)(cvt_pk_e4m3<false>(q, 0.0f, 0u) & 0xFFu);
    }
  }
  if (threadIdx.x == 0) scales[tile_r * grid_n + tile_c] = s;
}

template <bool kBf16In, bool kUe8m0>
void launch_typed(const void *x, int64_t m, int64_t n, uint8_t *y, float *s, hipStream_t stream) {
  const int64_t grid_n = (n + kBlock - 1) / kBlock, grid_m = (m + kBlock - 1) / kBlock;
  const dim3 grid((unsigned)grid_n, (unsigned)grid_m), block(256);
  const bool vec = (n % 8 == 0) && ((uintptr_t)x % 16 == 0) && ((uintptr_t)y % 8 == 0);
  if (vec)
    hipLaunchKernelGGL((weight_quant_tile_kernel<kBf16In, kUe8m0>), grid, block, 0, stream, x, y,
                       s, m, n, grid_n);
  else
    hipLaunchKernelGGL((weight_quant_elementwise_kernel<kBf16In, kUe8m0>), grid, block, 0, stream,
                       x, y, s, m, n, grid_n);
}

}  // namespace

hipError_t launch_weight_quant(const void *x, bool x_bf16, int64_t m, int64_t n, bool ue8m0,
                               uint8_t *y, float *s, hipStream_t stream) {
  if (x_bf16) {
    if (ue8m0) launch_typed<true, true>(x, m, n, y, s, stream);
    else launch_typed<true, false>(x, m, n, y, s, stream);
  } else {
    if (ue8m0) launch_typed<false, true>(x, m, n, y, s, stream);
    else launch_typed<false, false>(x, m, n, y, s, stream);
  }
  return hipGetLastError();
}

}  // namespace fp8bsq
