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


// ---------------------------------------------------------------------------
// Tiled kernel for large M.
//
// Workgroup tile 256 (M) x 128 (N), 512 threads = 8 waves arranged 4 x 2, each
// wave a 64 x 64 output tile (4 x 4 MFMA tiles).  Per 128-wide K block the
// workgroup needs A[256 x 128] and B[128 x 128] (48 KiB of E4M3 codes) plus the
// 256 activation scales of that K block.  They arrive in LDS by direct
// global->LDS loads (global_load_lds_dwordx4 / _dword), which need no staging
// registers, into a three-stage ring: while K block kb is computed, blocks kb+1
// and kb+2 are in flight, so each load has two K blocks of compute to land.
// The loads are issued from inline assembly with explicit vmcnt waits: the
// compiler's own handling of LDS DMA waits for every outstanding transfer
// before any LDS read, which would serialize the ring.  Each wave issues the
// same seven transfers per stage, so "vmcnt <= 7" means its part of stage kb
// has landed; the barrier after the wait makes that true for all waves.
//
// A 128-column N tile lies inside one 128-row weight block, so b_s is one
// scalar per K block.
//
// LDS rows are 128 bytes (eight 16-byte chunks); chunk c of row r is stored at
// chunk slot c ^ swz(r), which spreads the 16 rows a fragment read touches
// over all banks.  A DMA instruction writes 64 consecutive 16-byte slots (8
// rows), so lane p fetches the global chunk that belongs in slot p.
//
// Tile order is XCD-aware: workgroup ids are dealt round-robin to the eight
// XCDs, so consecutive tiles of the grouped raster order (4 M tiles by the N
// tiles) are given to ids of the same XCD and share its L2.
// ---------------------------------------------------------------------------
constexpr int kTileM = 256, kTileN = 128, kThreads = 512, kStages = 3;
constexpr int kDmaPerStage = 7;   // per wave: 4 (A) + 2 (B) + 1 (scales)

struct RingSmem {
  uint8_t a[kStages][kTileM * kBlock];
  uint8_t b[kStages][kTileN * kBlock];
  float as[kStages][kTileM];
};

__device__ __forceinline__ int swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return (uint32_t)(uintptr_t)((const __attribute__((address_space(3))) void *)p);
}

// 64 lanes x 16 bytes from per-lane global addresses to LDS [lds, lds + 1024).
__device__ __forceinline__ void lds_dma16(const void *src, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(lds)
               : "memory", "m0");
}

// active lanes x 4 bytes from per-lane global addresses to LDS [lds + 4 * lane].
__device__ __forceinline__ void lds_dma4(const void *src, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off" ::"v"(src), "s"(lds)
               : "memory", "m0");
}

__device__ __forceinline__ void wait_dma_all_but_one_stage() {
  asm volatile("s_waitcnt vmcnt(7)" ::: "memory");
  static_assert(kDmaPerStage == 7, "the vmcnt immediate above must equal kDmaPerStage");
}
__device__ __forceinline__ void wait_dma_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
__device__ __forceinline__ void workgroup_barrier() { asm volatile("s_barrier" ::: "memory"); }

__device__ __forceinline__ void tile_coords(int wg, int tiles_m, int tiles_n, int &tm, int &tn) {
  const int ntiles = tiles_m * tiles_n;
  // XCD-aware remap: ids wg = 8 * local + xcd; give XCD x a contiguous range of tiles.
  int tile = wg;
  if (ntiles % 8 == 0) tile = (wg % 8) * (ntiles / 8) + wg / 8;
  // grouped raster: groups of kGroupM M tiles walk across N
  constexpr int kGroupM = 4;
  const int group = tile / (kGroupM * tiles_n);
  const int first_m = group * kGroupM;
  const int gm = min(tiles_m - first_m, kGroupM);
  const int idx = tile - group * kGroupM * tiles_n;
  tm = first_m + idx % gm;
  tn = idx / gm;
}

template <bool kBf16Out>
__global__ __launch_bounds__(kThreads) void block_gemm_tile_kernel(
    const uint8_t *__restrict__ a, const float *__restrict__ a_s, const uint8_t *__restrict__ b,
    const float *__restrict__ b_s, void *__restrict__ c, int64_t m, int64_t n, int64_t k,
    int tiles_m, int tiles_n) {
  __shared__ __attribute__((aligned(1024))) RingSmem sm;
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  int tm, tn;
  tile_coords(blockIdx.x, tiles_m, tiles_n, tm, tn);
  const int64_t m0 = (int64_t)tm * kTileM, n0 = (int64_t)tn * kTileN;
  const int nkb = (int)(k / kBlock);
  const float *bs_row = b_s + (n0 / kBlock) * nkb;

  // DMA plan.  A: 8-row groups g = wave + 8 i (i < 4); B: g = wave + 8 i (i < 2).
  // Lane p of a group fills slot p: row 8 g + p / 8, chunk slot p % 8.  Rows
  // past the matrix edge re-read the last row (their outputs are never stored).
  const int dr = lane >> 3, ds = lane & 7;
  const uint8_t *a_src[4];
  const uint8_t *b_src[2];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = 8 * (wave + 8 * i) + dr;
    const int64_t grow = min(m0 + row, m - 1);
    a_src[i] = a + grow * k + ((ds ^ swz(row)) << 4);
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int row = 8 * (wave + 8 * i) + dr;
    const int64_t grow = min(n0 + row, n - 1);
    b_src[i] = b + grow * k + ((ds ^ swz(row)) << 4);
  }
  // scales: wave w, lanes 0..31 -> rows 32 w + lane
  const int64_t srow = min(m0 + 32 * wave + (lane & 31), m - 1);
  const float *as_src = a_s + srow * nkb;

  auto issue = [&](int kb, int s) {
    const int64_t off = (int64_t)kb * kBlock;
    const uint32_t abase = lds_addr(&sm.a[s][0]), bbase = lds_addr(&sm.b[s][0]);
#pragma unroll
    for (int i = 0; i < 4; ++i) lds_dma16(a_src[i] + off, abase + (wave + 8 * i) * 1024);
#pragma unroll
    for (int i = 0; i < 2; ++i) lds_dma16(b_src[i] + off, bbase + (wave + 8 * i) * 1024);
    if (lane < 32) lds_dma4(as_src + kb, lds_addr(&sm.as[s][32 * wave]));
  };

  const int wm = (wave >> 1) * 64, wn = (wave & 1) * 64;
  const int fr = lane & 15, fq = lane >> 4;

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  issue(0, 0);
  if (nkb > 1) issue(1, 1);

  int cur = 0;
  for (int kb = 0; kb < nkb; ++kb) {
    if (kb + 1 < nkb)
      wait_dma_all_but_one_stage();
    else
      wait_dma_all();
    workgroup_barrier();
    if (kb + 2 < nkb) issue(kb + 2, cur == 0 ? 2 : cur - 1);

    const float sb = bs_row[kb];
    float sc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f32x4 v = *(const f32x4 *)(&sm.as[cur][wm + 16 * i + 4 * fq]);
#pragma unroll
      for (int e = 0; e < 4; ++e) sc[i][e] = v[e] * sb;
    }
    i32x8 af[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = wm + 16 * i + fr;
      const uint4 *base = (const uint4 *)&sm.a[cur][r * kBlock];
      const uint4 lo = base[(2 * fq) ^ swz(r)];
      const uint4 hi = base[(2 * fq + 1) ^ swz(r)];
      af[i] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = wn + 16 * j + fr;
      const uint4 *base = (const uint4 *)&sm.b[cur][r * kBlock];
      const uint4 lo = base[(2 * fq) ^ swz(r)];
      const uint4 hi = base[(2 * fq + 1) ^ swz(r)];
      const i32x8 bfr = {(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const f32x4 p = mfma_e4m3_16x16x128(af[i], bfr, f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[i][j][e] = __builtin_fmaf(p[e], sc[i][e], acc[i][j][e]);
      }
    }
    cur = cur == kStages - 1 ? 0 : cur + 1;
  }

#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t col = n0 + wn + 16 * j + fr;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t row = m0 + wm + 16 * i + 4 * fq + e;
        if (row < m && col < n) store_out(c, kBf16Out, row * n + col, acc[i][j][e]);
      }
    }
}

}  // namespace

hipError_t launch_block_gemm(const uint8_t *a, const float *a_s, const uint8_t *b,
                             const float *b_s, void *c, bool c_bf16, int64_t m, int64_t n,
                             int64_t k, hipStream_t stream) {
  if (m > 64) {
    const int tiles_m = (int)((m + kTileM - 1) / kTileM), tiles_n = (int)((n + kTileN - 1) / kTileN);
    const dim3 grid((unsigned)(tiles_m * tiles_n)), block(kThreads);
    if (c_bf16)
      hipLaunchKernelGGL(block_gemm_tile_kernel<true>, grid, block, 0, stream, a, a_s, b, b_s, c, m,
                         n, k, tiles_m, tiles_n);
    else
      hipLaunchKernelGGL(block_gemm_tile_kernel<false>, grid, block, 0, stream, a, a_s, b, b_s, c,
                         m, n, k, tiles_m, tiles_n);
    return hipGetLastError();
  }
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
