// 128x128 block-scaled weight dequantization for gfx950.
//
// Method (page "How weight_dequant Handles Per-Block Scaling in DeepSeek-V3
// FP8 GEMM", sections "Grid Mapping and Scale Lookup" and "Dequantization
// Computation"): one program per 128x128 tile reads the tile's single FP32
// scale at s[tile_row * ceil(n/128) + tile_col], converts each E4M3 code to
// FP32 and multiplies, y = x * s; rows and columns past the matrix edge are
// masked.
//
// The tile-per-workgroup structure is kept because it makes the scale a
// workgroup-uniform value (one scalar load).  Inside the tile, 16 lanes cover
// one 128-column row segment, 8 codes each: every 8-byte load instruction then
// reads whole 128-byte lines of codes (so the loads can stream past the
// caches) and every 16-byte bf16 store writes whole lines.  A 256-thread
// workgroup covers 16 rows per pass; all eight passes' loads are issued
// before any conversion.  Codes go to FP32 with the hardware E4M3 conversion
// (exact), one FP32 multiply, then the hardware round-to-nearest-even BF16
// pack for BF16 output.
//
// Shapes with n % 8 != 0, or unaligned pointers, take an element-wise kernel.
#include "device_common.h"
#include "launch.h"

#pragma clang fp contract(off)

namespace fp8bsq {
namespace {

template <bool kBf16Out>
__global__ __launch_bounds__(256) void dequant_tile_kernel(const uint8_t *__restrict__ x,
                                                           const float *__restrict__ s,
                                                           void *__restrict__ y, int64_t m,
                                                           int64_t n, int64_t grid_n) {
  const int64_t tile_c = blockIdx.x, tile_r = blockIdx.y;
  const float sc = s[tile_r * grid_n + tile_c];
  const int tid = threadIdx.x;
  const int64_t col = tile_c * kBlock + (tid & 15) * 8;
  if (col >= n) return;                        // n % 8 == 0: chunks never straddle the edge
  const int64_t row0 = tile_r * kBlock + (tid >> 4);

  u32x2 v[8];
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    const int64_t row = row0 + 16 * p;
    v[p] = row < m ? load_stream((const u32x2 *)(x + row * n + col)) : u32x2{0, 0};
  }
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    const int64_t row = row0 + 16 * p;
    if (row >= m) break;
    const f32x4 lo = e4m3x4_to_f32(v[p].x), hi = e4m3x4_to_f32(v[p].y);
    const float f[8] = {lo.x * sc, lo.y * sc, lo.z * sc, lo.w * sc,
                        hi.x * sc, hi.y * sc, hi.z * sc, hi.w * sc};
    if (kBf16Out) {
      u32x4 *dst = (u32x4 *)((uint16_t *)y + row * n + col);
      *dst = u32x4{pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]),
                   pack_bf16x2(f[6], f[7])};
    } else {
      u32x4 *dst = (u32x4 *)((float *)y + row * n + col);
      dst[0] = u32x4{__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]),
                     __float_as_uint(f[3])};
      dst[1] = u32x4{__float_as_uint(f[4]), __float_as_uint(f[5]), __float_as_uint(f[6]),
                     __float_as_uint(f[7])};
    }
  }
}

template <bool kBf16Out>
__global__ __launch_bounds__(256) void dequant_elementwise_kernel(const uint8_t *__restrict__ x,
                                                                  const float *__restrict__ s,
                                                                  void *__restrict__ y,
                                                                  int64_t m, int64_t n,
                                                                  int64_t grid_n) {
  const int64_t total = m * n;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
    const int64_t row = i / n, col = i - row * n;
    const float sc = s[(row / kBlock) * grid_n + col / kBlock];
    const float v = e4m3x4_to_f32(x[i]).x * sc;
    if (kBf16Out)
      ((uint16_t *)y)[i] = (uint16_t)(pack_bf16x2(v, 0.0f) & 0xFFFFu);
    else
      ((float *)y)[i] = v;
  }
}

}  // namespace

hipError_t launch_weight_dequant(const uint8_t *x, const float *s, int64_t m, int64_t n, void *y,
                                 bool y_bf16, hipStream_t stream) {
  const int64_t grid_n = (n + kBlock - 1) / kBlock, grid_m = (m + kBlock - 1) / kBlock;
  const bool vec = (n % 8 == 0) && ((uintptr_t)x % 8 == 0) && ((uintptr_t)y % 16 == 0) &&
                   grid_m <= 65535;
  if (vec) {
    const dim3 grid((unsigned)grid_n, (unsigned)grid_m), block(256);
    if (y_bf16)
      hipLaunchKernelGGL(dequant_tile_kernel<true>, grid, block, 0, stream, x, s, y, m, n, grid_n);
    else
      hipLaunchKernelGGL(dequant_tile_kernel<false>, grid, block, 0, stream, x, s, y, m, n, grid_n);
  } else {
    int64_t wgs = (m * n + 255) / 256;
    if (wgs > 65536) wgs = 65536;
    const dim3 grid((unsigned)wgs), block(256);
    if (y_bf16)
      hipLaunchKernelGGL(dequant_elementwise_kernel<true>, grid, block, 0, stream, x, s, y, m, n,
                         grid_n);
    else
      hipLaunchKernelGGL(dequant_elementwise_kernel<false>, grid, block, 0, stream, x, s, y, m, n,
                         grid_n);
  }
  return hipGetLastError();
}

}  // namespace fp8bsq
