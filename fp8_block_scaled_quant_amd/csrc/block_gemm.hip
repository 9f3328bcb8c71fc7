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
#include <atomic>

#include "fp8bsq.h"
#include "launch.h"
#include "quant_common.h"

namespace fp8bsq {
namespace {

__device__ __forceinline__ f32x4 mfma_e4m3_16x16x128(const i32x8 &a, const i32x8 &b, f32x4 c) {
  // format 0 = E4M3 for both operands; the literal zero scale operands select
  // the unscaled instruction (no block scaling inside the matrix core).
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// The same MFMA with each A row scaled by 2^(e - 127) inside the matrix core:
// lane l supplies the E8M0 exponent e of the row it feeds (row l % 16); the B
// scale is 1 (E8M0 127).
__device__ __forceinline__ f32x4 mfma_e4m3_16x16x128_mx(const i32x8 &a, const i32x8 &b, int e8m0_a) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0,
                                                          e8m0_a, 0, 127);
}

__device__ __forceinline__ i32x8 load_frag(const uint8_t *p) {
  const uint4 lo = *(const uint4 *)p;
  const uint4 hi = *(const uint4 *)(p + 16);
  return i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z,
               (int)hi.w};
}

// Optional bias of the output's dtype, added to the FP32 accumulator before
// the output rounding; `bias` may be null.
__device__ __forceinline__ float bias_at(const void *bias, bool bf16, int64_t col) {
  if (!bias) return 0.0f;
  return bf16 ? __uint_as_float((uint32_t)((const uint16_t *)bias)[col] << 16)
              : ((const float *)bias)[col];
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
    const float *__restrict__ b_s, void *__restrict__ c, int64_t m, int64_t n, int64_t k,
    const void *__restrict__ bias) {
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
      const float bv = col < n ? bias_at(bias, kBf16Out, col) : 0.0f;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t row = m0 + 16 * i + lq + r;
        if (row < m && col < n) store_out(c, kBf16Out, row * n + col, acc[i][j][r] + bv);
      }
    }
}


// ---------------------------------------------------------------------------
// Tiled kernel for large M.
//
// Workgroup tile 256 (M) x 256 (N), 512 threads = 8 waves arranged 4 x 2; each
// wave owns a 64 x 128 output tile (4 x 8 MFMA tiles, 128 FP32 accumulators
// per lane).  The tile size is set by the operand feed: every K block brings
// (256 + 256) x 128 bytes of E4M3 codes from L2 into LDS, and on this part the
// L2 -> LDS path, not the matrix cores, is what runs out first, so the widest
// tile whose accumulators still fit in registers moves the fewest bytes per
// MFMA.
//
// Operands reach LDS by direct global->LDS loads (global_load_lds_dwordx4)
// into a two-stage ring: K block kb+1 is loaded while kb is computed.  The
// loads are issued from inline assembly with an explicit vmcnt wait, because
// the compiler's own handling of LDS DMA waits for every outstanding transfer
// before any LDS read.  Global addresses are a per-lane 32-bit offset on a
// wave-uniform 64-bit base, so advancing to the next K block costs scalar adds
// only.
//
// The CU accepts these transfers at about one instruction per 16-18 cycles,
// and a wave that issues them waits until they are accepted, so where they
// are issued decides who waits.  The next K block's A (32 instructions) is
// issued by waves 0-3 at the top of the block, while waves 4-7 (one per SIMD)
// start computing; its B (32) by all eight waves, four each, after their
// first two columns of MFMAs, by which time the A transfers have been
// accepted and the waves have MFMAs in flight.  B still lands well before the
// next block's wait.  (All 64 issued at the top by waves 0-3 kept those waves
// out of the matrix pipe for ~1,160 cycles per block and was 3% slower.)
//
// Activation scales (kTab): the kernel keeps a table of kTabKb K blocks'
// scales per row, loaded in 16-byte pieces one chunk ahead (double-buffered).
// Without it (K / 128 not a multiple of 4, or a_s not 16-byte aligned) the 256
// scales of each K block are gathered one 4-byte transfer per row, eight
// times the transfers for the same bytes.
//
// Each wave's 128 columns lie inside one 128-row weight block, so b_s is one
// scalar per wave and K block.  The per-K-block rescale (4 FMAs per MFMA) is
// software-pipelined by hand three MFMAs behind the MFMA that produced its
// partial, which keeps four partials live and lets the FMAs read them without
// hazard wait states; the scheduler would otherwise hoist all 32 MFMAs of a K
// block and run out of registers.
//
// LDS rows are 128 bytes (eight 16-byte chunks); chunk c of row r is stored at
// slot c ^ swz(r), so the 16 rows a fragment read touches hit distinct banks.
// A DMA instruction fills 64 consecutive 16-byte slots (8 rows): lane p
// fetches the global chunk that belongs in slot p.
//
// Tile order is XCD-aware: workgroup ids are dealt round-robin to the eight
// XCDs, so consecutive tiles of the grouped raster order (4 M tiles by the N
// tiles) go to ids of the same XCD and share its L2.
//
// Launches: one persistent workgroup per CU walks the tiles; with
// launch_block_gemm_split a last round of tiles that would leave CUs idle
// runs in a second launch, split over K (kSplit).
// ---------------------------------------------------------------------------
constexpr int kTileM = 256, kTileN = 256, kThreads = 512;

// K blocks per chunk of the power-of-two scale table
constexpr int kTabKb = 8;

// most parts a split-K tile is computed in
constexpr int kSplitMax = 4;

struct TileSmem {
  uint8_t a[2][kTileM * kBlock];
  uint8_t b[2][kTileN * kBlock];
  union {
    float as[2][kTileM];              // generic: the K block's a_s, per stage
    float tab[2][kTileM * kTabKb];    // power-of-two a_s: [32-row block][half][row][4 K blocks]
  };
};

__device__ __forceinline__ int swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return (uint32_t)(uintptr_t)((const __attribute__((address_space(3))) void *)p);
}

// 64 lanes x 16 bytes from base + voff (per lane) into LDS [lds, lds + 1024).
__device__ __forceinline__ void lds_dma16(const void *base, uint32_t voff, uint32_t lds) {
  asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(base), "{m0}"(lds) : "memory");
}

// active lanes x 4 bytes from base + voff into LDS [lds + 4 * lane].
__device__ __forceinline__ void lds_dma4(const void *base, uint32_t voff, uint32_t lds) {
  asm volatile("global_load_lds_dword %0, %1" ::"v"(voff), "s"(base), "{m0}"(lds) : "memory");
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

__device__ __forceinline__ i32x8 frag_from_lds(const uint8_t *row_base, int fq, int r) {
  const uint4 *base = (const uint4 *)row_base;
  const uint4 lo = base[(2 * fq) ^ swz(r)];
  const uint4 hi = base[(2 * fq + 1) ^ swz(r)];
  return i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}

// kSplit: this launch computes tiles tile0, tile0 + 1, ... of the tile order,
// each in nsplit parts over consecutive K ranges.  Every part stores its FP32
// partial tile to ws, then counts itself in counters[tile] (zeroed by an
// earlier launch on the stream); the part that counts last adds the partials
// in part order (P0 + P1 + ...) and finishes the tile as the unsplit kernel
// would.  No workgroup waits for another.  Unsplit launches with zero_n > 0
// have workgroup 0 clear zero_ptr[0, zero_n) for a split launch that follows.
template <bool kBf16Out, bool kMxA, bool kTab, bool kSplit = false>
__global__ __launch_bounds__(kThreads) void block_gemm_tile_kernel(
    const uint8_t *__restrict__ a, const float *__restrict__ a_s, const uint8_t *__restrict__ b,
    const float *__restrict__ b_s, void *__restrict__ c, int64_t m, int64_t n, int64_t k,
    int tiles_m, int tiles_n, const void *__restrict__ bias, int tile0 = 0, int nsplit = 1,
    float *__restrict__ ws = nullptr, uint32_t *__restrict__ counters = nullptr,
    uint32_t *__restrict__ zero_ptr = nullptr, int zero_n = 0, int tile_end = 0) {
  __shared__ __attribute__((aligned(1024))) TileSmem sm;
  if (!kSplit && blockIdx.x == 0)
    for (int i = threadIdx.x; i < zero_n; i += kThreads) zero_ptr[i] = 0u;
  __shared__ int split_last;
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int nkb = (int)(k / kBlock);
  // Unsplit launches are persistent: one workgroup per CU walks tiles
  // blockIdx.x, + gridDim.x, ... below tile_end, and issues a tile's first
  // transfers before the previous tile's output stores, with no workgroup
  // launch in between.  A split launch runs one tile part per workgroup.
  bool prologue_done = false;
  for (int tile_it = blockIdx.x;; tile_it += gridDim.x) {
    if (!kSplit && tile_it >= tile_end) break;
    int tm, tn, tslot = 0, part = 0, kb_begin = 0, kb_end = nkb;
    if (kSplit) {
      // Workgroups are dealt to the 8 XCDs round-robin.  With whole XCD shares
      // of the tail, workgroup w of XCD w % 8 takes tile 8 u + w % 8 of the
      // tail (its home XCD in the tile order, next to the tiles it shares A and
      // B rows with) and part (w / 8) / (tail / 8): that XCD's tiles, part by part.
      const int ntail = gridDim.x / nsplit;
      if (ntail % 8 == 0 && tile0 % 8 == 0) {
        const int local = blockIdx.x / 8, per = ntail / 8;
        part = local / per;
        tslot = 8 * (local % per) + blockIdx.x % 8;
      } else {
        tslot = blockIdx.x / nsplit;
        part = blockIdx.x % nsplit;
      }
      // whole chunks of the scale table per part
      const int per = ((nkb + kTabKb - 1) / kTabKb + nsplit - 1) / nsplit * kTabKb;
      kb_begin = min(nkb, part * per);
      kb_end = min(nkb, kb_begin + per);
      tile_coords(tile0 + tslot, tiles_m, tiles_n, tm, tn);
    } else {
      tile_coords(tile_it, tiles_m, tiles_n, tm, tn);
    }
    const int64_t m0 = (int64_t)tm * kTileM, n0 = (int64_t)tn * kTileN;
    const int wm = (wave >> 1) * 64, wn = (wave & 1) * 128;
    const int64_t grid_n = (n + kBlock - 1) / kBlock;
    const float *bs_row = b_s + min((n0 + wn) / kBlock, grid_n - 1) * nkb;

    // DMA plan, in 8-row groups (one instruction each; lane p of a group fills
    // slot p: row 8 g + p / 8, chunk slot p % 8): A group 8 d + g (g < 8) by
    // wave d < 4, B group 4 w + h (h < 4) by every wave w.  Rows past the matrix
    // edge re-read the last row; their outputs are never stored.
    const bool dma_wave = wave < 4;
    const int dw = wave & 3;
    const int dr = lane >> 3, ds = lane & 7;
    uint32_t a_off[8], b_off[4], s_off[2];
    // scales of the 32-row blocks dw and dw + 4: generic, lanes 0..31 -> rows;
    // table, lane p -> row p % 32 and K blocks 4 (p / 32) .. +3 of the chunk
    auto set_offsets = [&](int64_t tm0, int64_t tn0) {
#pragma unroll
      for (int g = 0; g < 8; ++g) {
        const int row = 8 * (8 * dw + g) + dr;
        a_off[g] = (uint32_t)(min(tm0 + row, m - 1) * k + ((ds ^ swz(row)) << 4));
      }
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const int row = 8 * (4 * wave + h) + dr;
        b_off[h] = (uint32_t)(min(tn0 + row, n - 1) * k + ((ds ^ swz(row)) << 4));
      }
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int64_t row = min(tm0 + 32 * (dw + 4 * h) + (lane & 31), m - 1);
        s_off[h] = (uint32_t)(row * nkb * 4 + (kTab ? (lane >> 5) * 16 : 0));
      }
    };
    set_offsets(m0, n0);
    const uint32_t lds_a = lds_addr(&sm.a[0][0]), lds_b = lds_addr(&sm.b[0][0]),
                   lds_s = lds_addr(&sm.as[0][0]);

    // K block kb's A (and, without the table, its scales) into stage s: waves 0-3
    auto issue_a = [&](int kb, int s) {
      const uint8_t *ab = a + (int64_t)kb * kBlock;
#pragma unroll
      for (int g = 0; g < 8; ++g)
        lds_dma16(ab, a_off[g], lds_a + s * (kTileM * kBlock) + (8 * dw + g) * 1024);
      if (!kTab) {
#pragma unroll
        for (int h = 0; h < 2; ++h)
          if (lane < 32) lds_dma4(a_s + kb, s_off[h], lds_s + s * (kTileM * 4) + 32 * (dw + 4 * h) * 4);
      }
    };
    // K block kb's B into stage s: every wave
    auto issue_b = [&](int kb, int s) {
      const uint8_t *bb = b + (int64_t)kb * kBlock;
#pragma unroll
      for (int h = 0; h < 4; ++h)
        lds_dma16(bb, b_off[h], lds_b + s * (kTileN * kBlock) + (4 * wave + h) * 1024);
    };
    // chunk c of the scale table (K blocks kTabKb c ..), into buffer c & 1; in
    // a last, half-filled chunk the upper lanes re-read their row's first four
    // scales (in bounds, never used)
    auto issue_tab = [&](int c) {
      const int kb0 = kTabKb * c;
      const bool inside = kb0 + 4 * (lane >> 5) < nkb;
#pragma unroll
      for (int h = 0; h < 2; ++h)
        lds_dma16(a_s, inside ? s_off[h] + (uint32_t)kb0 * 4 : s_off[h] - (uint32_t)(lane >> 5) * 16,
                  lds_s + (c & 1) * (kTileM * kTabKb * 4) + (dw + 4 * h) * 1024);
    };

    const int fr = lane & 15, fq = lane >> 4;
    f32x4 acc[4][8];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // MFMA q = 4 j + i of a K block; its rescale runs three MFMAs later (a ring
    // of 4 partials).  With kMxA the rescale of a block's last three MFMAs runs
    // at the top of the next block, behind that block's fragment reads (and
    // after the tile's last block); the partials start at zero so that the
    // first block of a tile adds nothing for a previous one.  (The generic
    // kernel keeps it at the end of the block: carrying its row scales into the
    // next block would spill.)
    constexpr bool kDefer = kMxA;
    f32x4 prt[4];
    float sc[4][4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      prt[q] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int e = 0; e < 4; ++e) sc[q][e] = 0.f;
    }
    float sb_prev = 0.f;
    auto finish_block = [&]() {
#pragma unroll
      for (int qp = 29; qp < 32; ++qp) {
        const int ip = qp % 4, jp = qp / 4;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          acc[ip][jp][e] = __builtin_fmaf(prt[qp % 4][e], kMxA ? sb_prev : sc[ip][e], acc[ip][jp][e]);
      }
    };

    // landed: stage cur is known to have landed for every wave (the first block
    // of a persistent tile, whose transfers were waited for before the previous
    // tile's output stores)
    auto step = [&](int kb, int cur, bool landed) {
      const float sbv = bs_row[kb];   // scalar load, issued ahead of the wait below
      if (!landed) {
        wait_dma_all();
        workgroup_barrier();   // stage cur landed for every wave; stage cur^1 no longer read
      }
      if (dma_wave) {
        if (kb + 1 < kb_end) issue_a(kb + 1, cur ^ 1);
        // the table buffer of chunk c + 1 was last read in chunk c - 1
        if (kTab && kb % kTabKb == 0 && kb + kTabKb < kb_end) issue_tab(kb / kTabKb + 1);
      }
      // Retire the scalar load now (the empty asm consumes its value): scalar and
      // LDS results share one counter and the scalar one may return out of order,
      // so while it is outstanding every LDS wait would have to be a full drain.
      asm volatile("" ::"s"(sbv));
      // kMxA (activation scales that are powers of two, act_quant's ue8m0): the
      // MFMA applies a_s of the A row a lane feeds (its E8M0 exponent, the fp32
      // exponent field), leaving the rescale a multiply by the wave-uniform b_s.
      // P * 2^e is exact, so fma(P * a_s, b_s, acc) equals the generic
      // fma(P, a_s * b_s, acc) bit for bit.
      f32x4 sav[4];
      int ea[4];
      const float *tab = &sm.tab[(kb / kTabKb) & 1][((kb % kTabKb) >> 2) * 128 + (kb & 3)];
      // table row r = wm + 16 i + x lies in 32-row block wm / 32 + i / 2, at row
      // 16 (i % 2) + x of it; the MFMA scale wants x = fr, the rescale x = 4 fq + e
      auto tab_row = [&](int i) { return tab + (wm / 32 + i / 2) * 256 + 16 * (i % 2) * 4; };
      // Reads in the order the first MFMAs use them -- the MFMA scales, B's first
      // fragment, then A's fragments one by one -- so the first MFMA waits for
      // three of them rather than all; the rescale's row scales come last.
      uint32_t ew[4];   // the scale words; their exponent fields are taken after the reads go out
      if (kMxA) {
#pragma unroll
        for (int i = 0; i < 4; ++i) ew[i] = __float_as_uint(tab_row(i)[fr * 4]);
      }
      auto read_b = [&](int j) {
        const int r = wn + 16 * j + fr;
        return frag_from_lds(&sm.b[cur][r * kBlock], fq, r);
      };
      i32x8 bcur = read_b(0), bnext;
      __builtin_amdgcn_sched_barrier(0);
      i32x8 af[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = wm + 16 * i + fr;
        af[i] = frag_from_lds(&sm.a[cur][r * kBlock], fq, r);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (!kMxA) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (kTab) {
#pragma unroll
            for (int e = 0; e < 4; ++e) sav[i][e] = tab_row(i)[(4 * fq + e) * 4];
          } else {
            sav[i] = *(const f32x4 *)(&sm.as[cur][wm + 16 * i + 4 * fq]);
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      if (kMxA) {
#pragma unroll
        for (int i = 0; i < 4; ++i) ea[i] = (int)((ew[i] >> 23) & 0xFFu);
      }
      // the previous block's last rescale, while these reads are in flight
      if (kDefer) finish_block();
      __builtin_amdgcn_sched_barrier(0);
      // The row scales a_s * b_s are formed at their first use (q - 3 < 4), so
      // their LDS reads never hold up the first MFMAs.
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (j + 1 < 8) bnext = read_b(j + 1);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int q = 4 * j + i;
          prt[q % 4] = kMxA ? mfma_e4m3_16x16x128_mx(af[i], bcur, ea[i])
                             : mfma_e4m3_16x16x128(af[i], bcur, f32x4{0.f, 0.f, 0.f, 0.f});
          // the next block's B, unconditionally so that no branch splits the
          // unrolled loop (the last block re-reads itself into the stage no one
          // reads again; drained after the loop)
          if (j == 2 && i == 0) issue_b(min(kb + 1, kb_end - 1), cur ^ 1);
          if (q >= 3) {
            const int qp = q - 3, ip = qp % 4, jp = qp / 4;
            if (!kMxA && qp < 4) {
#pragma unroll
              for (int e = 0; e < 4; ++e) sc[ip][e] = sav[ip][e] * sbv;
            }
#pragma unroll
            for (int e = 0; e < 4; ++e)
              acc[ip][jp][e] = __builtin_fmaf(prt[qp % 4][e], kMxA ? sbv : sc[ip][e], acc[ip][jp][e]);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
        if (j + 1 < 8) bcur = bnext;
      }
      sb_prev = sbv;
      if (!kDefer) finish_block();
    };

    if (!prologue_done) {
      if (dma_wave) {
        issue_a(kb_begin, 0);
        if (kTab) issue_tab(kb_begin / kTabKb);
      }
      issue_b(kb_begin, 0);
    }
    const bool stage0_landed = prologue_done;
#pragma nounroll
    for (int kb = kb_begin; kb < kb_end; ++kb) step(kb, (kb - kb_begin) & 1, kb == kb_begin && stage0_landed);
    if (kDefer) finish_block();
    wait_dma_all();

    // persistent: once every wave is done with LDS, the next tile's first
    // transfers (stage 0, table chunk 0) go out and are waited for, and only
    // then this tile's output stores: the next tile's first block then starts
    // without a wait, and its stores drain while that block computes (a wait
    // for transfers issued after the stores would wait for them too)
    prologue_done = false;
    if (!kSplit && tile_it + (int)gridDim.x < tile_end) {
      workgroup_barrier();
      int ntm, ntn;
      tile_coords(tile_it + gridDim.x, tiles_m, tiles_n, ntm, ntn);
      set_offsets((int64_t)ntm * kTileM, (int64_t)ntn * kTileN);
      if (dma_wave) {
        issue_a(0, 0);
        if (kTab) issue_tab(0);
      }
      issue_b(0, 0);
      wait_dma_all();
      workgroup_barrier();
      prologue_done = true;
    }

    if (kSplit) {
      // partials in the lanes' own order: [tile][part][wave][i][j][lane][4]
      const size_t tile_floats = (size_t)kTileM * kTileN;
      float *base = ws + (size_t)tslot * nsplit * tile_floats + (size_t)wave * (tile_floats / 8) + lane * 4;
      float *mine = base + (size_t)part * tile_floats;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) *(f32x4 *)(mine + (i * 8 + j) * 256) = acc[i][j];
      // Every wave's stores complete (in L2) before the barrier; one device-scope
      // fence then publishes the workgroup's partial ahead of its count, and the
      // last part's fence makes the others' partials visible before it reads
      // them.  (Each fence writes back or invalidates a whole L2, so one per
      // workgroup, not one per thread.)
      wait_dma_all();
      __syncthreads();
      if (t == 0) {
        __threadfence();
        split_last = atomicAdd(&counters[tslot], 1u) == (uint32_t)(nsplit - 1);
        if (split_last) __threadfence();
      }
      __syncthreads();
      if (!split_last) return;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          // Two parts: own + other, the same either way round (FP32 addition
          // commutes).  More: every part from the workspace in part order, this
          // one's included; a select between acc and a loaded value would pin
          // acc to memory for the whole kernel.
          if (nsplit == 2) {
            acc[i][j] += *(const f32x4 *)(base + (size_t)(part ^ 1) * tile_floats + (i * 8 + j) * 256);
          } else {
            f32x4 sum = *(const f32x4 *)(base + (i * 8 + j) * 256);
#pragma unroll
            for (int p = 1; p < kSplitMax; ++p)
              if (p < nsplit) sum += *(const f32x4 *)(base + (size_t)p * tile_floats + (i * 8 + j) * 256);
            acc[i][j] = sum;
          }
        }
    }

#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int64_t col = n0 + wn + 16 * j + fr;
        const float bv = col < n ? bias_at(bias, kBf16Out, col) : 0.0f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int64_t row = m0 + wm + 16 * i + 4 * fq + e;
          if (row < m && col < n) store_out(c, kBf16Out, row * n + col, acc[i][j][e] + bv);
        }
      }
    if (kSplit || !prologue_done) break;
  }
}

// ---------------------------------------------------------------------------
// Decode kernel for M <= 32 (the weight B [n, k] streams from HBM once and
// dominates the traffic; the wide kernel below takes 32 < M <= 64).
//
// A workgroup owns 80 weight rows, one 16-row MFMA tile per compute wave
// (waves 0-4), and all of them walk the same K blocks.  A last wave only
// moves A: it DMAs each K block of A (all its activation rows x 128 bytes, in
// whole-line 16-byte pieces, with the XOR swizzle of the tiled kernel) and
// their activation scales into an LDS ring, kLead blocks ahead (kLead + 1
// slots), waiting on its own transfers only, and one barrier per K block
// hands the ring on.
//
// The weight streams from HBM per compute wave (below), so the only
// vector-memory transfers a compute wave waits on are its own weight loads.
// (A first design split K across four waves instead: every workgroup then
// pulled all of A through fragment-shaped loads, and because a wave's loads
// complete in order, each wait for an A fragment also drained its weight
// prefetch ring; it was 20-45% slower at every M.)
//
// Fused act_quant (kFuseQ, M <= kFusedMaxM, bf16 activations): every
// workgroup quantizes all of x [m, k] into LDS with act_quant's arithmetic,
// and workgroup 0 also publishes the codes and scales; there is no mover and
// no per-block barrier.  Helper waves (the workgroup's sixteen waves less the
// compute waves) do the quantization while the compute waves already stream
// their weights: the helpers take x's
// blocks in K order and count each finished block in LDS, and a compute wave
// waits for a K block's count before it reads that block's codes.  The
// compute waves do the same arithmetic in the same order as on the two-call
// path, so both give bit-identical outputs.
// ---------------------------------------------------------------------------
constexpr int kDecodeMaxM = 64;
// Longest K (in K blocks) of the fused path, whose scales sit in LDS for the
// whole run.
constexpr int kDecodeMaxKb = 160;
// Activations quantized inside the decode kernel (fused act_quant) for up to
// this many rows (one 16-row MFMA tile), within the code limits below: every
// workgroup quantizes all of them, but on helper waves that overlap the
// weight stream, so the redundant work stays off the critical path.  The
// workgroup has kFusedWaves waves, four per SIMD: the compute waves (one to
// five, as the decode kernel chooses them for N) and helpers.  Fewer compute
// waves per workgroup at narrow N measured 9-18% faster at N = 4096 and 7168
// (M = 1-16), as the grid grows from 90 to 224 or 256 workgroups, even though
// every workgroup repeats the quantization.
constexpr int kFusedMaxM = 16;
constexpr int kFusedWaves = 16;
// Most bytes of codes the fused path keeps in LDS, beside the five weight
// rings and the scales: 80 KB keeps the workgroup within 160 KB.  Up to that
// many codes (m * k) all of x stays in LDS; beyond it, up to
// kFusedRingMaxCodes, the codes go through a ring of fused_ring_blocks(m) K
// blocks that the helpers refill as the compute waves finish reading them.
// Past that limit the redundant quantization outweighs the saved kernel
// boundary (measured against the two kernels: m = 16 at K = 7168 (112 K codes)
// 7-12% slower at N = 4096-12288, m = 6 at K = 18432 (108 K) 9% slower at
// N = 7168).
constexpr int64_t kFusedMaxCodes = 80 * 1024;
constexpr int64_t kFusedRingMaxCodes = 96 * 1024;
// K blocks of m rows' codes in the ring: the largest power of two that fits.
__host__ __device__ constexpr int fused_ring_blocks(int m) {
  int r = 1;
  while (2 * r * m * kBlock <= kFusedMaxCodes) r *= 2;
  return r;
}

// Fused act_quant on the helper waves (hq = thread index among them):
// quantize x [m, k] bf16 per 1 x 128 block exactly as the act_quant kernel
// does -- sixteen lanes per block, 8 elements each, amax over the 16-lane row,
// the same scale and quotient arithmetic -- into LDS codes aq [m][k] and
// scales as_t [kb][row].  Blocks go in K order (flat index kb * m + row, four
// blocks' loads in flight per lane), so the K blocks the compute waves need
// first are done first.  After a block's codes and scale are in LDS, its
// first lane adds one to done[kb] and to done[kDecodeMaxKb] (all blocks) with
// workgroup-scope release; a reader that sees done[kb] == m with acquire sees
// the whole K block.  With kRing, block kb's codes go to ring slot
// kb & ring_mask, and a helper first waits until every compute wave has
// finished reading the slot's previous block (prog[w]: K blocks compute wave
// w of kNC has read).  Workgroup 0 also writes the codes and scales to a_q /
// a_s_out, bit-identical to fp8_act_quant.  The helpers start at a raised
// wave priority for their first batch, whose blocks the compute waves wait
// for first, and drop to the normal priority after it (measured: 2-4% faster
// at M = 1-16 than either priority throughout).
template <int kRows, int kThreadsQ, bool kRing, int kNC, int kBatchQ = 4>
__device__ __forceinline__ void fused_act_quant(const u32x4 *__restrict__ x, int m, int nkb, int hq,
                                                bool ue8m0, uint8_t *aq, float (*as_t)[kRows], int *done,
                                                const int *prog, int ring_mask, uint8_t *__restrict__ a_q,
                                                float *__restrict__ a_s_out, bool publish) {
  const int group = hq >> 4, sub = hq & 15;
  int seen = 0;   // K blocks every compute wave has read, as last looked up
  const int nblocks = m * nkb;
  constexpr int kStride = kThreadsQ / 16;
  // The sixteen lanes of a block share every condition below, as the row
  // reduction needs.
  for (int base = group; base < nblocks; base += kBatchQ * kStride) {
    u32x4 v[kBatchQ];
#pragma unroll
    for (int u = 0; u < kBatchQ; ++u) {
      const int idx = base + u * kStride;
      if (idx < nblocks) {
        const int kb = idx / m, row = idx - kb * m;
        v[u] = x[((int64_t)row * nkb + kb) * 16 + sub];
      }
    }
#pragma unroll
    for (int u = 0; u < kBatchQ; ++u) {
      const int idx = base + u * kStride;
      if (idx >= nblocks) break;
      const int kb = idx / m, row = idx - kb * m;
      const int64_t blk = (int64_t)row * nkb + kb;
      u16x2 m2 = {0, 0};
      const uint32_t d[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
      for (int j = 0; j < 4; ++j)
        m2 = __builtin_elementwise_max(m2, __builtin_bit_cast(u16x2, d[j] & 0x7FFF7FFFu));
      const uint32_t amax = row_max_u32((uint32_t)(m2.x > m2.y ? m2.x : m2.y) << 16);
      float sc, r;
      block_scale_fast(amax, ue8m0, sc, r);
      const u32x2 codes = encode_chunk_bf16(v[u], sc, r);
      if constexpr (kRing) {
        // the compute waves only wait on the helpers' older blocks, so this
        // ends; the bound only keeps a wave from spinning forever
        if (kb > seen + ring_mask) {
          for (int spin = 0; spin < (1 << 20); ++spin) {
            int lo = __hip_atomic_load(&prog[0], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP);
#pragma unroll
            for (int w = 1; w < kNC; ++w)
              lo = min(lo, __hip_atomic_load(&prog[w], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP));
            seen = lo;
            if (kb <= seen + ring_mask) break;
            __builtin_amdgcn_s_sleep(2);
          }
        }
        *(u32x2 *)(aq + ((int64_t)(kb & ring_mask) * m + row) * kBlock + 8 * sub) = codes;
      } else {
        *(u32x2 *)(aq + blk * kBlock + 8 * sub) = codes;
      }
      if (sub == 0) as_t[kb][row] = sc;
      if (publish) {
        *(u32x2 *)(a_q + blk * kBlock + 8 * sub) = codes;
        if (sub == 0) a_s_out[blk] = sc;
      }
      if (sub == 0) {
        __hip_atomic_fetch_add(&done[kb], 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
        __hip_atomic_fetch_add(&done[kDecodeMaxKb], 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
      }
    }
    __builtin_amdgcn_s_setprio(0);
  }
}

constexpr int kDecodeCompute = 5;                // most compute waves per workgroup (plus the mover)
constexpr int kDecodeRows = 16 * kDecodeCompute;   // weight rows per workgroup at that width
constexpr int kDecodeLead = 6;                   // K blocks of A in flight ahead of use (ring: one more slot)
constexpr int kDecodeDepth = 6;                  // weight ring depth per compute wave
// The fused path at one or two compute waves per workgroup (narrow N) keeps
// more weight blocks in flight per wave: 10 measured 3-5% faster than 6 at
// N = 7168 (M = 1-4), and 14 no better.  The decode kernel, whose waves also
// meet once per K block at the mover's barrier, measured 2-5% slower with it.
constexpr int kFusedNarrowDepth = 10;

template <int kMT>
struct DecodeSlot {
  uint8_t a[16 * kMT * kBlock];   // [row][16-byte chunk slot], swizzled
  float s[16 * kMT];              // a_s of the K block, per row
};

// Workgroup size (kCW compute waves): each workgroup fetches its K blocks of
// A and their scales once, and the CU's vector-memory issue rate (not HBM)
// bounded the kernel, so the wider the workgroup the fewer fetches per weight
// row.  Five compute waves give 231 workgroups for N = 18432, one per CU;
// three gave 384, two on half the CUs, whose mover then sat ~1000 cycles per
// K block in DMA issue (M = 64 with weights streaming from HBM, measured when
// this kernel still served M = 64: 50.7 us at three, 38.5 at five, 40.7 at
// six).  A narrower weight leaves CUs idle at five waves (N = 7168: 90
// workgroups), so the launch takes the fewest waves that keep the grid within
// one workgroup per CU: two at N = 7168 (224 workgroups) measured 19-21%
// faster than five at M = 1-32, and 8-10% faster than one (448) or three
// (150), bit-identical.
//
// Activation scales (kTab): as in the tiled kernel, a double-buffered table of
// kTabKb K blocks' scales per row, loaded one chunk ahead in 16-byte pieces;
// otherwise each K block's kRows scales travel in its ring slot, one 4-byte
// transfer per row.
template <bool kBf16Out, int kMT, int kDepth, bool kTab, bool kFuseQ = false, bool kRing = false,
          int kCW = kDecodeCompute>
__global__ __launch_bounds__(kFuseQ ? 64 * kFusedWaves : 64 * (kCW + 1)) void block_gemm_decode_kernel(
    const uint8_t *__restrict__ a, const float *__restrict__ a_s, const uint8_t *__restrict__ b,
    const float *__restrict__ b_s, void *__restrict__ c, int64_t m, int64_t n, int64_t k,
    const void *__restrict__ bias, bool ue8m0 = false, uint8_t *__restrict__ a_q = nullptr,
    float *__restrict__ a_s_out = nullptr) {
  static_assert(kCW >= 1 && kCW <= kDecodeCompute, "one to five compute waves");
  static_assert(!kFuseQ || (kMT == 1 && kFusedMaxM <= 16), "the fused path: one 16-row tile");
  static_assert(!kRing || kFuseQ, "the ring belongs to the fused path");
  static_assert(kMT <= 2, "up to 32 activation rows");
  constexpr int kRows = 16 * kMT;
  constexpr int kLead = kDecodeLead;   // A blocks in flight ahead
  constexpr int kSlots = kLead + 1;
  constexpr int kDmaPerBlock = kRows / 8 + (kTab ? 0 : 1);   // A row groups of 8 (+ the scales)
  // table: [32-row block][half][row][4 K blocks], as the DMA lanes lay it down
  constexpr int kTabRows = (kRows + 31) / 32 * 32;   // whole 32-row blocks (one DMA each)
  __shared__ __attribute__((aligned(1024))) DecodeSlot<kMT> ring[kFuseQ ? 1 : kSlots];
  // fused: codes [m][k] (dynamic; with kRing [slot][m][128]) and scales
  // [kb][row] of all of x
  extern __shared__ __attribute__((aligned(16))) uint8_t aq[];
  __shared__ float as_t[kFuseQ ? kDecodeMaxKb : 1][kRows];
  // fused: blocks of x quantized, per K block and (last) in all
  __shared__ int q_done[kFuseQ ? kDecodeMaxKb + 1 : 1];
  // fused with the ring: K blocks each compute wave has finished reading
  __shared__ int q_prog[kRing ? kCW : 1];
  __shared__ __attribute__((aligned(16))) float stab[kTab ? 2 : 1][kTab ? kTabRows * kTabKb : 1];
  // weights: each compute wave DMAs its 16 weight rows into its own LDS ring
  // (whole-line transfers, half the vector-memory issue of fragment-shaped
  // loads)
  __shared__ __attribute__((aligned(1024))) uint8_t bring[kCW][kDepth][16 * kBlock];
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const bool mover = !kFuseQ && wave == kCW;
  const int nkb = (int)(k / kBlock);

  // mover: lane p of row group g fills chunk slot p % 8 of row 8 g + p / 8;
  // rows past m re-read row m - 1 and scale lanes past kRows sit idle
  const int dr = lane >> 3, ds = lane & 7;
  uint32_t a_off[kRows / 8];
#pragma unroll
  for (int g = 0; g < kRows / 8; ++g) {
    const int row = 8 * g + dr;
    a_off[g] = (uint32_t)(min((int64_t)row, m - 1) * k + ((ds ^ swz(row)) << 4));
  }
  const uint32_t s_off = (uint32_t)(min((int64_t)lane, m - 1) * nkb * 4);
  const uint32_t lds_ring = lds_addr(&ring[0]);
  auto issue = [&](int kb) {
    const uint32_t slot = lds_ring + (uint32_t)((kb % kSlots) * sizeof(DecodeSlot<kMT>));
#pragma unroll
    for (int g = 0; g < kRows / 8; ++g) lds_dma16(a + (int64_t)kb * kBlock, a_off[g], slot + g * 1024);
    if (!kTab && lane < kRows) lds_dma4(a_s + kb, s_off, slot + kRows * kBlock);
  };
  // table chunk c into buffer c & 1: instruction i, lane p -> row 32 i + p % 32
  // and K blocks 4 (p / 32) .. +3 of the chunk; in a half-filled last chunk the
  // upper half re-reads the row's first four scales (in bounds, never used)
  const int trow = lane & 31, thalf = lane >> 5;
  uint32_t t_off[kTabRows / 32];
#pragma unroll
  for (int i = 0; i < kTabRows / 32; ++i)
    t_off[i] = (uint32_t)(min((int64_t)(32 * i + trow), m - 1) * nkb * 4);
  const uint32_t lds_tab = lds_addr(&stab[0][0]);
  auto issue_tab = [&](int ch) {
    const int kb0 = kTabKb * ch;
    const uint32_t piece = kb0 + 4 * thalf < nkb ? (uint32_t)(kb0 + 4 * thalf) * 4 : 0u;
#pragma unroll
    for (int i = 0; i < kTabRows / 32; ++i)
      if (32 * i + trow < kRows)
        lds_dma16(a_s, t_off[i] + piece, lds_tab + (ch & 1) * (kTabRows * kTabKb * 4) + i * 1024);
  };
  // wait until a K block's transfers have landed, given how many blocks were
  // issued after it (transfers complete in issue order)
  static_assert(kLead <= 6 && 5 * kDmaPerBlock < 64, "one vmcnt case per block behind");
  auto wait_block = [&](int behind) {
    switch (behind) {
      case 1: asm volatile("s_waitcnt vmcnt(%0)" ::"n"(1 * kDmaPerBlock) : "memory"); break;
      case 2: asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * kDmaPerBlock) : "memory"); break;
      case 3: asm volatile("s_waitcnt vmcnt(%0)" ::"n"(3 * kDmaPerBlock) : "memory"); break;
      case 4: asm volatile("s_waitcnt vmcnt(%0)" ::"n"(4 * kDmaPerBlock) : "memory"); break;
      case 5: asm volatile("s_waitcnt vmcnt(%0)" ::"n"(5 * kDmaPerBlock) : "memory"); break;
      default: wait_dma_all(); break;
    }
  };

  const int64_t n0 = (int64_t)blockIdx.x * (16 * kCW) + 16 * (mover ? 0 : wave);
  const int fr = lane & 15, fq = lane >> 4;
  const float *bs_row = b_s + min(n0 / kBlock, (n - 1) / kBlock) * nkb;
  // Each compute wave DMAs its own 16 weight rows of a K block (two
  // whole-line transfers, same lane plan and swizzle as A) into its own
  // kDepth-slot LDS ring; no other wave reads them, so they need no barrier.
  // Addresses are 32-bit lane offsets from the wave's first (clamped) row.
  const int64_t nb0 = min(n0, n - 1);
  const uint8_t *b_wave = b + nb0 * k;
  uint32_t b_off[2];
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    const int row = 8 * g + dr;
    b_off[g] = (uint32_t)((min(n0 + row, n - 1) - nb0) * k + ((ds ^ swz(row)) << 4));
  }
  const uint32_t lds_b = lds_addr(&bring[mover ? 0 : wave][0][0]);
  auto issue_b = [&](int kb) {
    const uint32_t slot = lds_b + (uint32_t)((kb % kDepth) * 16 * kBlock);
#pragma unroll
    for (int g = 0; g < 2; ++g) lds_dma16(b_wave + (int64_t)kb * kBlock, b_off[g], slot + g * 1024);
  };
  const int sw = swz(fr);   // rows 16 mt + fr share their swizzle
  const uint32_t a_lo = (uint32_t)(fr * kBlock + ((fq ^ sw) << 4));
  const uint32_t a_hi = (uint32_t)(fr * kBlock + (((4 + fq) ^ sw) << 4));

  // The mover and the compute waves run separate loops with one barrier per K
  // block plus one after the prologue.  The compute waves' main loop is
  // branch-free: the compiler's count of weight loads in flight stays exact,
  // and no ring register is merged across paths (either would make it wait
  // for every load in flight).
  const int ring_mask = kRing ? fused_ring_blocks((int)m) - 1 : 0;
  if constexpr (kFuseQ) {
    // `a` holds the bf16 activations; scale rows m..kRows-1 stay 0
    for (int i = t; i < kDecodeMaxKb * kRows; i += 64 * kFusedWaves) as_t[i / kRows][i % kRows] = 0.0f;
    for (int i = t; i <= kDecodeMaxKb; i += 64 * kFusedWaves) q_done[i] = 0;
    if (kRing && t < kCW) q_prog[t] = 0;
    __syncthreads();
    // the helper waves only quantize; the fused K loop has no barrier to miss
    if (wave >= kCW) {
      __builtin_amdgcn_s_setprio(3);
      fused_act_quant<kRows, 64 * (kFusedWaves - kCW), kRing, kCW>((const u32x4 *)a, (int)m, nkb, t - 64 * kCW,
                                                        ue8m0, aq, as_t, q_done, q_prog, ring_mask, a_q, a_s_out,
                                                        blockIdx.x == 0);
      return;
    }
  }
  if (mover) {
    // the compute waves read block kb + 1 while they compute kb, so by the
    // barrier that ends block kb, block kb + 2 must have landed
    if (kTab) issue_tab(0);
    for (int kb = 0; kb < kLead && kb < nkb; ++kb) issue(kb);
    wait_block(min(kLead, nkb) - 1 - min(1, nkb - 1));
    workgroup_barrier();
    for (int kb = 0; kb < nkb; ++kb) {
      // the slot of kb + lead was last read during block kb - 2
      if (kb + kLead < nkb) issue(kb + kLead);
      // chunk c + 1 into the buffer chunk c - 1 used (last read during block
      // kb - 2); it is older than block kb + 7's transfers, which are waited
      // for (two blocks ahead of their use) before its first read
      if (kTab && kb % kTabKb == 0 && kb + kTabKb < nkb) issue_tab(kb / kTabKb + 1);
      if (kb + 2 < nkb) wait_block(min(kb + kLead, nkb - 1) - (kb + 2));
      workgroup_barrier();
    }
    wait_dma_all();
    return;
  }

  f32x4 acc[kMT];
#pragma unroll
  for (int mt = 0; mt < kMT; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  // A fragments, row scales and b_s of one K block, double-buffered: block
  // kb + 1's are read from the ring while block kb's feed the MFMAs
  i32x8 af[2][kMT];
  f32x4 sa[2][kMT];
  float sb[2];
  const bool a_row_live = fr < m;   // fused: rows past m are zero fragments
  int ready = 0;                     // fused: K blocks known to be quantized (wave-uniform)
  const uint8_t *a_lds = aq + (int64_t)(a_row_live ? fr : 0) * (kRing ? kBlock : k) + 16 * fq;
  auto read_a = [&](int kb, int buf) {   // kb may be nkb (a stale slot, never used)
    if constexpr (kFuseQ) {
      const int kbc = min(kb, nkb - 1);
      if (kbc >= ready) {
        // wait for the helpers to finish K block kbc (they wait on nothing,
        // so this ends within microseconds; the bound only keeps a wave from
        // spinning forever); once every block is done, stop checking
        for (int spin = 0; spin < (1 << 20); ++spin) {
          if (__builtin_amdgcn_readfirstlane(__hip_atomic_load(&q_done[kbc], __ATOMIC_ACQUIRE,
                                                               __HIP_MEMORY_SCOPE_WORKGROUP)) >= m) break;
          __builtin_amdgcn_s_sleep(1);
        }
        ready = __builtin_amdgcn_readfirstlane(__hip_atomic_load(&q_done[kDecodeMaxKb], __ATOMIC_ACQUIRE,
                                                                 __HIP_MEMORY_SCOPE_WORKGROUP)) >= m * nkb
                    ? nkb : kbc + 1;
      }
      af[buf][0] = i32x8{0, 0, 0, 0, 0, 0, 0, 0};
      if (a_row_live) {
        const uint8_t *codes = kRing ? a_lds + (kbc & ring_mask) * (int)m * kBlock : a_lds + (int64_t)kbc * kBlock;
        const uint4 lo = *(const uint4 *)codes;
        const uint4 hi = *(const uint4 *)(codes + 64);
        af[buf][0] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      }
      sa[buf][0] = *(const f32x4 *)&as_t[kbc][4 * fq];
      sb[buf] = bs_row[kbc];
      return;
    }
    const DecodeSlot<kMT> &sl = ring[kb % kSlots];
#pragma unroll
    for (int mt = 0; mt < kMT; ++mt) {
      const int tile = mt;
      const uint4 lo = *(const uint4 *)(&sl.a[tile * 16 * kBlock + a_lo]);
      const uint4 hi = *(const uint4 *)(&sl.a[tile * 16 * kBlock + a_hi]);
      af[buf][mt] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      if (kTab) {
        const float *tb = &stab[(kb / kTabKb) & 1][((kb % kTabKb) >> 2) * 128 + (kb & 3)];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 16 * tile + 4 * fq + e;
          sa[buf][mt][e] = tb[(r >> 5) * 256 + (r & 31) * 4];
        }
      } else {
        sa[buf][mt] = *(const f32x4 *)&sl.s[16 * tile + 4 * fq];
      }
    }
    sb[buf] = bs_row[min(kb, nkb - 1)];
  };
  auto compute = [&](const i32x8 &bf, int buf) {
#pragma unroll
    for (int mt = 0; mt < kMT; ++mt) {
      const f32x4 p = mfma_e4m3_16x16x128(af[buf][mt], bf, f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[mt][e] = __builtin_fmaf(p[e], sa[buf][mt][e] * sb[buf], acc[mt][e]);
    }
  };
  i32x8 bf[2];
  auto read_b = [&](int kb, int buf) {   // kb may be nkb (a stale slot, never used)
    const uint8_t *sl = &bring[wave][kb % kDepth][0];
    const uint4 lo = *(const uint4 *)(sl + a_lo), hi = *(const uint4 *)(sl + a_hi);
    bf[buf] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
  };
  // one K block: block kb + 1's weight transfers (issued kDepth - 1 blocks
  // ago) have landed once at most kDepth - 2 younger blocks' remain; read
  // its fragments and A's while block kb's feed the MFMAs, then refill the
  // slot block kb came from (its fragments were read a block ago) with
  // block kb + kDepth, clamped so that every block issues the same two
  // transfers
  static_assert(2 * (kDepth - 1) < 64, "vmcnt range");
  auto step = [&](int kb, int cur) {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * (kDepth - 2)) : "memory");
    read_a(kb + 1, cur ^ 1);
    read_b(kb + 1, cur ^ 1);
    compute(bf[cur], cur);
    issue_b(min(kb + kDepth, nkb - 1));
    if (!kFuseQ) workgroup_barrier();   // hands the mover's A ring on
    // fused, ring: blocks 0..kb are read (block kb's codes fed this step's
    // MFMA; the release orders those reads before the helpers' refill)
    if (kRing) __hip_atomic_store(&q_prog[wave], kb + 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
  };
#pragma unroll
  for (int d = 0; d < kDepth; ++d) issue_b(min(d, nkb - 1));
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * (kDepth - 1)) : "memory");
  if (!kFuseQ) workgroup_barrier();
  read_a(0, 0);
  read_b(0, 0);
  const int neven = nkb & ~1;
  for (int kb = 0; kb < neven; kb += 2) {
    step(kb, 0);
    step(kb + 1, 1);
  }
  if (nkb & 1) step(neven, 0);
  wait_dma_all();   // the clamped refills past the last block, before the workgroup's LDS is released

  const int64_t col = n0 + fr;
  const float bv = col < n ? bias_at(bias, kBf16Out, col) : 0.0f;
#pragma unroll
  for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int64_t row = 16 * mt + 4 * fq + e;
      if (row < m && col < n) store_out(c, kBf16Out, row * n + col, acc[mt][e] + bv);
    }
}

// ---------------------------------------------------------------------------
// Wide decode kernel for 32 < M <= 64: the weight tiles are shared, the
// activation tiles are not.  A workgroup owns kWT 16-row weight tiles (up to
// five, 80 rows) and all of A's row tiles (kAT = 3 or 4); compute wave w owns
// A's row tile w and runs it against all kWT weight tiles, so each K block a
// wave reads one A fragment and kWT weight fragments, and the MFMA and
// rescale work sits evenly on the four SIMDs.  Two mover waves fill a
// kWideSlots-slot LDS ring kWideLead blocks ahead: one DMAs each K block's A
// rows and (without the table) their scales, the other its weight rows.  Each waits on its
// own transfers only, and one barrier per K block hands the ring on, as in the
// decode kernel.  (One mover for both measured 1-3% slower.)  Against two
// compute waves per weight tile, each DMAing its own copy of the tile's rows,
// this measured 7-11% faster at M = 33-64 with bit-identical outputs (each
// output element sees the same FMAs in the same order); at M <= 32 it
// measured no faster than the decode kernel, and at M <= 16 2% slower.  As
// for the decode kernel, the launch takes the fewest weight tiles that keep
// the grid within one workgroup per CU: at N = 4096 and 7168 (one and two
// tiles) 24-27% faster than five tiles, at 12288 (three) 16%.
// ---------------------------------------------------------------------------
constexpr int kWideTiles = 5;                    // most weight tiles per workgroup
constexpr int kWideRows = 16 * kWideTiles;       // weight rows per workgroup at that width
constexpr int kWideLead = 5;                     // K blocks in flight ahead of use
constexpr int kWideSlots = kWideLead + 1;

template <int kAT, int kWT>
struct WideSlot {
  uint8_t a[16 * kAT * kBlock];    // [row][16-byte chunk slot], swizzled
  uint8_t b[16 * kWT * kBlock];    // the same for the weight rows
  float s[16 * kAT];               // a_s of the K block, per row (no table)
};

template <bool kBf16Out, int kAT, bool kTab, int kWT = kWideTiles>
__global__ __launch_bounds__(64 * (kAT + 2)) void block_gemm_decode_wide_kernel(
    const uint8_t *__restrict__ a, const float *__restrict__ a_s, const uint8_t *__restrict__ b,
    const float *__restrict__ b_s, void *__restrict__ c, int64_t m, int64_t n, int64_t k,
    const void *__restrict__ bias) {
  constexpr int kRows = 16 * kAT;
  constexpr int kWRows = 16 * kWT;
  // transfers per K block of the A mover and of the weight mover
  constexpr int kDmaA = kRows / 8 + (kTab ? 0 : 1), kDmaB = kWRows / 8;
  static_assert((kWideLead - 2) * kDmaB < 64 && (kWideLead - 2) * kDmaA < 64, "the wait counter's range");
  constexpr int kTabRows = (kRows + 31) / 32 * 32;
  __shared__ __attribute__((aligned(1024))) WideSlot<kAT, kWT> ring[kWideSlots];
  __shared__ __attribute__((aligned(16))) float stab[kTab ? 2 : 1][kTab ? kTabRows * kTabKb : 1];
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const bool mover = wave >= kAT, bmover = wave == kAT + 1;
  const int nkb = (int)(k / kBlock);
  const int64_t n0 = (int64_t)blockIdx.x * kWRows;

  if (mover) {
    // lane p of row group g fills chunk slot p % 8 of row 8 g + p / 8; A rows
    // past m re-read row m - 1, weight rows past n row n - 1
    const int dr = lane >> 3, ds = lane & 7;
    uint32_t a_off[kRows / 8], b_off[kWRows / 8];
#pragma unroll
    for (int g = 0; g < kRows / 8; ++g) {
      const int row = 8 * g + dr;
      a_off[g] = (uint32_t)(min((int64_t)row, m - 1) * k + ((ds ^ swz(row)) << 4));
    }
    const int64_t nb0 = min(n0, n - 1);
    const uint8_t *b_base = b + nb0 * k;
#pragma unroll
    for (int g = 0; g < kWRows / 8; ++g) {
      const int row = 8 * g + dr;
      b_off[g] = (uint32_t)((min(n0 + row, n - 1) - nb0) * k + ((ds ^ swz(row)) << 4));
    }
    const uint32_t s_off = (uint32_t)(min((int64_t)lane, m - 1) * nkb * 4);
    const uint32_t lds_ring = lds_addr(&ring[0]);
    auto issue = [&](int kb) {
      const uint32_t slot = lds_ring + (uint32_t)((kb % kWideSlots) * sizeof(WideSlot<kAT, kWT>));
      if (!bmover) {
#pragma unroll
        for (int g = 0; g < kRows / 8; ++g) lds_dma16(a + (int64_t)kb * kBlock, a_off[g], slot + g * 1024);
        if (!kTab && lane < kRows) lds_dma4(a_s + kb, s_off, slot + (kRows + kWRows) * kBlock);
      } else {
#pragma unroll
        for (int g = 0; g < kWRows / 8; ++g)
          lds_dma16(b_base + (int64_t)kb * kBlock, b_off[g], slot + kRows * kBlock + g * 1024);
      }
    };
    // table chunk c into buffer c & 1, as in the decode kernel
    const int trow = lane & 31, thalf = lane >> 5;
    uint32_t t_off[kTabRows / 32];
#pragma unroll
    for (int i = 0; i < kTabRows / 32; ++i)
      t_off[i] = (uint32_t)(min((int64_t)(32 * i + trow), m - 1) * nkb * 4);
    const uint32_t lds_tab = lds_addr(&stab[0][0]);
    auto issue_tab = [&](int ch) {
      const int kb0 = kTabKb * ch;
      const uint32_t piece = kb0 + 4 * thalf < nkb ? (uint32_t)(kb0 + 4 * thalf) * 4 : 0u;
#pragma unroll
      for (int i = 0; i < kTabRows / 32; ++i)
        if (32 * i + trow < kRows)
          lds_dma16(a_s, t_off[i] + piece, lds_tab + (ch & 1) * (kTabRows * kTabKb * 4) + i * 1024);
    };
    // a block's transfers landed, `behind` younger blocks issued (the A
    // mover's table chunks only make its waits stricter)
    auto wait_block = [&](int behind) {
#define FP8BSQ_WAIT_BEHIND(D)                                                     \
  switch (behind) {                                                               \
    case 1: asm volatile("s_waitcnt vmcnt(%0)" ::"n"(1 * (D)) : "memory"); break; \
    case 2: asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * (D)) : "memory"); break; \
    case 3: asm volatile("s_waitcnt vmcnt(%0)" ::"n"(3 * (D)) : "memory"); break; \
    case 4: asm volatile("s_waitcnt vmcnt(%0)" ::"n"(4 * (D)) : "memory"); break; \
    default: wait_dma_all(); break;                                               \
  }
      if (bmover) {
        FP8BSQ_WAIT_BEHIND(kDmaB)
      } else {
        FP8BSQ_WAIT_BEHIND(kDmaA)
      }
#undef FP8BSQ_WAIT_BEHIND
    };
    static_assert(kWideLead - 2 <= 4, "one wait case per block behind");
    // the compute waves read block kb + 1 while they compute kb, so by the
    // barrier that ends block kb, block kb + 2 must have landed
    if (kTab && !bmover) issue_tab(0);
    for (int kb = 0; kb < kWideLead && kb < nkb; ++kb) issue(kb);
    wait_block(min(kWideLead, nkb) - 1 - min(1, nkb - 1));
    workgroup_barrier();
    for (int kb = 0; kb < nkb; ++kb) {
      // the slot of kb + lead was last read during block kb - 2
      if (kb + kWideLead < nkb) issue(kb + kWideLead);
      // table chunk c + 1 into the buffer chunk c - 1 used (last read during
      // block kb - 2); older than the transfers waited for below
      if (kTab && !bmover && kb % kTabKb == 0 && kb + kTabKb < nkb) issue_tab(kb / kTabKb + 1);
      if (kb + 2 < nkb) wait_block(min(kb + kWideLead, nkb - 1) - (kb + 2));
      workgroup_barrier();
    }
    wait_dma_all();
    return;
  }

  // compute wave: A's row tile `wave` against the five weight tiles
  const int fr = lane & 15, fq = lane >> 4;
  const int sw = swz(fr);
  const uint32_t f_lo = (uint32_t)(fr * kBlock + ((fq ^ sw) << 4));
  const uint32_t f_hi = (uint32_t)(fr * kBlock + (((4 + fq) ^ sw) << 4));
  // b_s rows of the (at most two) weight blocks the workgroup's rows fall in
  const int64_t grid_n = (n + kBlock - 1) / kBlock;
  const int64_t nblk0 = min(n0 / kBlock, grid_n - 1);
  const float *bs0 = b_s + nblk0 * nkb;
  const float *bs1 = b_s + min(nblk0 + 1, grid_n - 1) * nkb;
  f32x4 acc[kWT];
#pragma unroll
  for (int j = 0; j < kWT; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  i32x8 af[2], bf[2][kWT];
  f32x4 sa[2];
  float sb0[2], sb1[2];
  auto frag = [&](const uint8_t *rows) {
    const uint4 lo = *(const uint4 *)(rows + f_lo), hi = *(const uint4 *)(rows + f_hi);
    return i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
  };
  auto read = [&](int kb, int buf) {   // kb may be nkb (a stale slot, never used)
    const WideSlot<kAT, kWT> &sl = ring[kb % kWideSlots];
    af[buf] = frag(&sl.a[wave * 16 * kBlock]);
#pragma unroll
    for (int j = 0; j < kWT; ++j) bf[buf][j] = frag(&sl.b[j * 16 * kBlock]);
    if (kTab) {
      const float *tb = &stab[(kb / kTabKb) & 1][((kb % kTabKb) >> 2) * 128 + (kb & 3)];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 16 * wave + 4 * fq + e;
        sa[buf][e] = tb[(r >> 5) * 256 + (r & 31) * 4];
      }
    } else {
      sa[buf] = *(const f32x4 *)&sl.s[16 * wave + 4 * fq];
    }
    const int kbc = min(kb, nkb - 1);
    sb0[buf] = bs0[kbc];
    sb1[buf] = bs1[kbc];
  };
  auto compute = [&](int buf) {
#pragma unroll
    for (int j = 0; j < kWT; ++j) {
      const f32x4 p = mfma_e4m3_16x16x128(af[buf], bf[buf][j], f32x4{0.f, 0.f, 0.f, 0.f});
      // tile j's weight block: the workgroup's first, or the next one
      const float sb = (n0 + 16 * j) / kBlock == nblk0 ? sb0[buf] : sb1[buf];
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[j][e] = __builtin_fmaf(p[e], sa[buf][e] * sb, acc[j][e]);
    }
  };
  workgroup_barrier();   // blocks 0 and 1 landed
  read(0, 0);
  auto step = [&](int kb, int cur) {
    read(kb + 1, cur ^ 1);
    compute(cur);
    workgroup_barrier();   // hands the ring on
  };
  const int neven = nkb & ~1;
  for (int kb = 0; kb < neven; kb += 2) {
    step(kb, 0);
    step(kb + 1, 1);
  }
  if (nkb & 1) step(neven, 0);

#pragma unroll
  for (int j = 0; j < kWT; ++j) {
    const int64_t col = n0 + 16 * j + fr;
    const float bv = col < n ? bias_at(bias, kBf16Out, col) : 0.0f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int64_t row = 16 * wave + 4 * fq + e;
      if (row < m && col < n) store_out(c, kBf16Out, row * n + col, acc[j][e] + bv);
    }
  }
}

}  // namespace

// Compute units of the current device, asked of the runtime once per device;
// 0 if the runtime cannot say.
static int current_device_cus() {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cached[kMaxDevices];   // 0: not asked yet
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < kMaxDevices) {
    const int c = cached[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    return 0;
  if (dev < kMaxDevices) cached[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

// Compute waves of the decode kernel and the fused path, or weight tiles of
// the wide decode kernel, per workgroup for a weight of n rows: the fewest
// (one to five) that keep the grid within one workgroup per CU; five if the
// CU count is unknown.
static int decode_width(int64_t n) {
  const int64_t cus = current_device_cus();
  const int64_t want = cus > 0 ? (n + 16 * cus - 1) / (16 * cus) : kDecodeCompute;
  return want < 1 ? 1 : want > kDecodeCompute ? kDecodeCompute : (int)want;
}

// the tiled kernel serves m > 64 while A, B and a_s fit its 32-bit per-lane offsets
static bool tiled_path(int64_t m, int64_t n, int64_t k) {
  return m > 64 && m * k < ((int64_t)1 << 32) && n * k < ((int64_t)1 << 32);
}

// The tiled kernel applies power-of-two activation scales inside the
// MX-scaled MFMA when they come from the scale table (K / 128 a multiple of 4,
// a_s 16-byte aligned); otherwise it applies a_s in the FP32 rescale.
static bool mx_kernel_used(int64_t k, const float *a_s, bool a_s_pow2) {
  return a_s_pow2 && (k / kBlock) % 4 == 0 && ((uintptr_t)a_s & 15) == 0;
}

// Tiled kernel: unsplit, tiles [0, grid) by min(grid, CUs) persistent
// workgroups; split, `grid` workgroups (see block_gemm_tile_kernel for tile0,
// nsplit, ws and counters).
static hipError_t launch_tiles(const uint8_t *a, const float *a_s, const uint8_t *b,
                               const float *b_s, void *c, bool c_bf16, int64_t m, int64_t n,
                               int64_t k, hipStream_t stream, const void *bias, bool a_s_pow2,
                               unsigned grid, bool split, int tile0, int nsplit, float *ws,
                               uint32_t *counters, int zero_n = 0) {
  const int tiles_m = (int)((m + kTileM - 1) / kTileM), tiles_n = (int)((n + kTileN - 1) / kTileN);
  const dim3 block(kThreads);
  int cus = current_device_cus();
  if (cus <= 0) cus = 256;
  const unsigned pgrid = grid < (unsigned)cus ? grid : (unsigned)cus;
#define FP8BSQ_TILE(BF16, MX, TAB)                                                                      \
  do {                                                                                                   \
    if (split)                                                                                           \
      hipLaunchKernelGGL((block_gemm_tile_kernel<BF16, MX, TAB, true>), dim3(grid), block, 0, stream, a, \
                         a_s, b, b_s, c, m, n, k, tiles_m, tiles_n, bias, tile0, nsplit, ws, counters);  \
    else                                                                                                 \
      hipLaunchKernelGGL((block_gemm_tile_kernel<BF16, MX, TAB, false>), dim3(pgrid), block, 0, stream,  \
                         a, a_s, b, b_s, c, m, n, k, tiles_m, tiles_n, bias, 0, 1, nullptr, nullptr,     \
                         counters, zero_n, (int)grid);                                                   \
  } while (0)
  // the scale table loads each row's scales in 16-byte pieces; the MX-scaled
  // kernel reads its exponents from it
  const bool tab = (k / kBlock) % 4 == 0 && ((uintptr_t)a_s & 15) == 0;
  const bool mx = mx_kernel_used(k, a_s, a_s_pow2);
  if (c_bf16) {
    if (mx) FP8BSQ_TILE(true, true, true);
    else if (tab) FP8BSQ_TILE(true, false, true);
    else FP8BSQ_TILE(true, false, false);
  } else {
    if (mx) FP8BSQ_TILE(false, true, true);
    else if (tab) FP8BSQ_TILE(false, false, true);
    else FP8BSQ_TILE(false, false, false);
  }
#undef FP8BSQ_TILE
  return hipGetLastError();
}

__global__ void zero_u32_kernel(uint32_t *p, int n) {
  for (int i = threadIdx.x; i < n; i += blockDim.x) p[i] = 0u;
}

// Guard of the MX-scaled kernel, which applies each activation scale as the
// E8M0 exponent field of its fp32 bits: a row of a_s [m, nkb] holding any
// value that is not a positive normal power of two (bits other than e << 23,
// 1 <= e <= 254) gets NaN in every column of its C row.  Runs after the GEMM
// on the same stream.  One lane per 16 bytes (four scales) of a_s, which the
// MX-scaled kernel's preconditions (nkb % 4 == 0, 16-byte aligned a_s) keep
// inside one row: a single load per lane when every scale is good, and a lane
// that finds a stray scale fills its row with NaN itself.
template <bool kBf16Out>
__global__ __launch_bounds__(256) void ue8m0_guard_kernel(const u32x4 *__restrict__ a_s4, int64_t nvec,
                                                          int vec_per_row, void *__restrict__ c, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= nvec) return;
  const u32x4 v = a_s4[i];
  const uint32_t stray = (v.x | v.y | v.z | v.w) & 0x807FFFFFu;   // sign or mantissa bits
  const uint32_t lo = min(min(v.x, v.y), min(v.z, v.w));            // zero or subnormal exponent
  if (stray == 0u && lo >= 0x00800000u) return;
  const int64_t row = i / vec_per_row;
  for (int64_t j = 0; j < n; ++j) {
    if (kBf16Out)
      ((uint16_t *)c)[row * n + j] = 0x7FC0u;
    else
      ((uint32_t *)c)[row * n + j] = 0x7FC00000u;
  }
}

static hipError_t launch_ue8m0_guard(const float *a_s, int64_t m, int64_t k, void *c, bool c_bf16,
                                     int64_t n, hipStream_t stream) {
  const int vec_per_row = (int)(k / kBlock / 4);
  const int64_t nvec = m * vec_per_row;
  const dim3 grid((unsigned)((nvec + 255) / 256)), block(256);
  if (c_bf16)
    hipLaunchKernelGGL(ue8m0_guard_kernel<true>, grid, block, 0, stream, (const u32x4 *)a_s, nvec, vec_per_row,
                       c, n);
  else
    hipLaunchKernelGGL(ue8m0_guard_kernel<false>, grid, block, 0, stream, (const u32x4 *)a_s, nvec,
                       vec_per_row, c, n);
  return hipGetLastError();
}

// Split-K plan: when the tiles leave a last round that fills at most half the
// CUs, those `tail` tiles run in `parts` parts over K (whole scale-table
// chunks of at least kSplitMinKb K blocks each), `parts` times as many
// workgroups for 1/parts of the work each.  The full rounds run unsplit.
constexpr int kSplitMinKb = 16;
struct SplitPlan {
  int full = 0, tail = 0, parts = 1;
  size_t counter_bytes = 0, bytes = 0;   // bytes = 0: no split
};
static SplitPlan split_plan(int64_t m, int64_t n, int64_t k) {
  SplitPlan p;
  if (!tiled_path(m, n, k)) return p;
  const int cus = current_device_cus();
  if (cus <= 0) return p;
  const int64_t tiles = ((m + kTileM - 1) / kTileM) * ((n + kTileN - 1) / kTileN);
  const int full = (int)(tiles / cus * cus), tail = (int)(tiles - full);
  const int nkb = (int)(k / kBlock), nch = (nkb + kTabKb - 1) / kTabKb;
  if (tail == 0) return p;
  int parts = min(min(cus / tail, kSplitMax), min(nch, nkb / kSplitMinKb));
  if (parts < 2) return p;
  const int per = (nch + parts - 1) / parts;   // chunks per part, as the kernel divides them
  parts = (nch + per - 1) / per;               // parts that get any
  if (parts < 2) return p;
  p.full = full;
  p.tail = tail;
  p.parts = parts;
  p.counter_bytes = ((size_t)tail * 4 + 255) / 256 * 256;
  p.bytes = p.counter_bytes + (size_t)tail * parts * kTileM * kTileN * sizeof(float);
  return p;
}

size_t block_gemm_split_bytes(int64_t m, int64_t n, int64_t k) { return split_plan(m, n, k).bytes; }

hipError_t launch_block_gemm_split(const uint8_t *a, const float *a_s, const uint8_t *b,
                                   const float *b_s, void *c, bool c_bf16, int64_t m, int64_t n,
                                   int64_t k, hipStream_t stream, bool a_s_pow2, void *workspace,
                                   size_t workspace_bytes) {
  const SplitPlan p = split_plan(m, n, k);
  if (p.bytes == 0 || workspace_bytes < p.bytes)
    return launch_block_gemm(a, a_s, b, b_s, c, c_bf16, m, n, k, stream, nullptr, a_s_pow2);
  uint32_t *counters = (uint32_t *)workspace;
  float *partials = (float *)((uint8_t *)workspace + p.counter_bytes);
  // the full rounds, whose workgroup 0 clears the tail's counters; without
  // full rounds, a one-workgroup fill does
  if (p.full > 0) {
    const hipError_t e = launch_tiles(a, a_s, b, b_s, c, c_bf16, m, n, k, stream, nullptr, a_s_pow2,
                                      (unsigned)p.full, false, 0, 1, nullptr, counters, p.tail);
    if (e != hipSuccess) return e;
  } else {
    hipLaunchKernelGGL(zero_u32_kernel, dim3(1), dim3(256), 0, stream, counters, p.tail);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const hipError_t e = launch_tiles(a, a_s, b, b_s, c, c_bf16, m, n, k, stream, nullptr, a_s_pow2,
                                    (unsigned)(p.tail * p.parts), true, p.full, p.parts, partials,
                                    counters);
  if (e != hipSuccess || !mx_kernel_used(k, a_s, a_s_pow2)) return e;
  return launch_ue8m0_guard(a_s, m, k, c, c_bf16, n, stream);
}

// Split-K scratch of launch_block_gemm_split_noalloc: one array per GPU,
// living as long as the process.  A split's partials take tail * parts tiles
// of 256 x 256 FP32 with tail * parts <= CUs, and its counters one word per
// tail tile (tail <= CUs / 2), so 256 CUs need at most 512 B + 64 MiB.
static_assert(FP8BSQ_SPLIT_SCRATCH_BYTES ==
                  512 + (size_t)256 * kTileM * kTileN * sizeof(float),
              "scratch size");
static __device__ __align__(256) uint8_t scratch[FP8BSQ_SPLIT_SCRATCH_BYTES];

// Device address of the current device's scratch, looked up on the first
// call there (the array's name is a host-side stand-in, not that address).
static hipError_t scratch_address(void **out) {
  constexpr int kMaxDevices = 64;
  static std::atomic<void *> address[kMaxDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void *p = address[dev].load(std::memory_order_acquire);
  if (!p) {
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    address[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return hipSuccess;
}

hipError_t launch_block_gemm_split_noalloc(const uint8_t *a, const float *a_s, const uint8_t *b,
                                           const float *b_s, void *c, bool c_bf16, int64_t m,
                                           int64_t n, int64_t k, hipStream_t stream, bool a_s_pow2,
                                           bool *too_big) {
  const size_t need = split_plan(m, n, k).bytes;
  *too_big = need > FP8BSQ_SPLIT_SCRATCH_BYTES;
  if (*too_big) return hipSuccess;
  if (need == 0)   // no split pays: the unsplit launch, which uses no scratch
    return launch_block_gemm(a, a_s, b, b_s, c, c_bf16, m, n, k, stream, nullptr, a_s_pow2);
  void *ws = nullptr;
  const hipError_t e = scratch_address(&ws);
  if (e != hipSuccess) return e;
  return launch_block_gemm_split(a, a_s, b, b_s, c, c_bf16, m, n, k, stream, a_s_pow2, ws,
                                 FP8BSQ_SPLIT_SCRATCH_BYTES);
}

hipError_t launch_block_gemm(const uint8_t *a, const float *a_s, const uint8_t *b,
                             const float *b_s, void *c, bool c_bf16, int64_t m, int64_t n,
                             int64_t k, hipStream_t stream, const void *bias, bool a_s_pow2) {
  if (tiled_path(m, n, k)) {
    const int64_t tiles = ((m + kTileM - 1) / kTileM) * ((n + kTileN - 1) / kTileN);
    const hipError_t e = launch_tiles(a, a_s, b, b_s, c, c_bf16, m, n, k, stream, bias, a_s_pow2,
                                      (unsigned)tiles, false, 0, 1, nullptr, nullptr);
    if (e != hipSuccess || !mx_kernel_used(k, a_s, a_s_pow2)) return e;
    return launch_ue8m0_guard(a_s, m, k, c, c_bf16, n, stream);
  }
  // the decode kernels' A and weight transfers use 32-bit lane offsets (from
  // A's base, and from the first weight row of a wave or a workgroup)
  if (m <= kDecodeMaxM && m * k < ((int64_t)1 << 32) && kWideRows * k < ((int64_t)1 << 32)) {
    const bool tab = (k / kBlock) % 4 == 0 && ((uintptr_t)a_s & 15) == 0;
    const int cw = decode_width(n);   // compute waves, or the wide kernel's weight tiles
    const dim3 dgrid((unsigned)((n + 16 * cw - 1) / (16 * cw)));
    // up to 32 rows: the decode kernel with MT activation row tiles per
    // compute wave; above: the wide kernel with AT row tiles, one per wave
#define FP8BSQ_DECODE_W(MT, TAB, CW)                                                                        \
  do {                                                                                                       \
    const dim3 block(64 * ((CW) + 1));                                                                       \
    if (c_bf16)                                                                                              \
      hipLaunchKernelGGL((block_gemm_decode_kernel<true, MT, kDecodeDepth, TAB, false, false, CW>), dgrid,   \
                         block, 0, stream, a, a_s, b, b_s, c, m, n, k, bias);                                \
    else                                                                                                     \
      hipLaunchKernelGGL((block_gemm_decode_kernel<false, MT, kDecodeDepth, TAB, false, false, CW>), dgrid,  \
                         block, 0, stream, a, a_s, b, b_s, c, m, n, k, bias);                                \
  } while (0)
#define FP8BSQ_DECODE_T(MT, TAB)                                                                            \
  do {                                                                                                       \
    switch (cw) {                                                                                            \
      case 1: FP8BSQ_DECODE_W(MT, TAB, 1); break;                                                            \
      case 2: FP8BSQ_DECODE_W(MT, TAB, 2); break;                                                            \
      case 3: FP8BSQ_DECODE_W(MT, TAB, 3); break;                                                            \
      case 4: FP8BSQ_DECODE_W(MT, TAB, 4); break;                                                            \
      default: FP8BSQ_DECODE_W(MT, TAB, kDecodeCompute); break;                                              \
    }                                                                                                        \
  } while (0)
#define FP8BSQ_DECODE(MT)                                                                                   \
  do {                                                                                                       \
    if (tab) FP8BSQ_DECODE_T(MT, true); else FP8BSQ_DECODE_T(MT, false);                                   \
  } while (0)
#define FP8BSQ_WIDE_W(AT, TAB, WT)                                                                          \
  do {                                                                                                       \
    const dim3 block(64 * (AT + 2)), wgrid((unsigned)((n + 16 * (WT) - 1) / (16 * (WT))));                  \
    if (c_bf16)                                                                                              \
      hipLaunchKernelGGL((block_gemm_decode_wide_kernel<true, AT, TAB, WT>), wgrid, block, 0, stream, a, a_s, \
                         b, b_s, c, m, n, k, bias);                                                          \
    else                                                                                                     \
      hipLaunchKernelGGL((block_gemm_decode_wide_kernel<false, AT, TAB, WT>), wgrid, block, 0, stream, a,    \
                         a_s, b, b_s, c, m, n, k, bias);                                                     \
  } while (0)
#define FP8BSQ_WIDE_T(AT, TAB)                                                                              \
  do {                                                                                                       \
    switch (cw) {                                                                                            \
      case 1: FP8BSQ_WIDE_W(AT, TAB, 1); break;                                                              \
      case 2: FP8BSQ_WIDE_W(AT, TAB, 2); break;                                                              \
      case 3: FP8BSQ_WIDE_W(AT, TAB, 3); break;                                                              \
      case 4: FP8BSQ_WIDE_W(AT, TAB, 4); break;                                                              \
      default: FP8BSQ_WIDE_W(AT, TAB, kWideTiles); break;                                                    \
    }                                                                                                        \
  } while (0)
#define FP8BSQ_WIDE(AT)                                                                                     \
  do {                                                                                                       \
    if (tab) FP8BSQ_WIDE_T(AT, true); else FP8BSQ_WIDE_T(AT, false);                                       \
  } while (0)
    switch ((m + 15) / 16) {
      case 1: FP8BSQ_DECODE(1); break;
      case 2: FP8BSQ_DECODE(2); break;
      case 3: FP8BSQ_WIDE(3); break;
      default: FP8BSQ_WIDE(4); break;
    }
#undef FP8BSQ_WIDE
#undef FP8BSQ_WIDE_T
#undef FP8BSQ_WIDE_W
#undef FP8BSQ_DECODE
#undef FP8BSQ_DECODE_T
#undef FP8BSQ_DECODE_W
    return hipGetLastError();
  }
  return launch_block_gemm_reference(a, a_s, b, b_s, c, c_bf16, m, n, k, stream, bias);
}

hipError_t launch_block_gemm_reference(const uint8_t *a, const float *a_s, const uint8_t *b,
                                       const float *b_s, void *c, bool c_bf16, int64_t m, int64_t n,
                                       int64_t k, hipStream_t stream, const void *bias) {
  const dim3 grid((unsigned)((n + 63) / 64), (unsigned)((m + 63) / 64)), block(256);
  if (c_bf16)
    hipLaunchKernelGGL(block_gemm_simple_kernel<true>, grid, block, 0, stream, a, a_s, b, b_s, c,
                       m, n, k, bias);
  else
    hipLaunchKernelGGL(block_gemm_simple_kernel<false>, grid, block, 0, stream, a, a_s, b, b_s, c,
                       m, n, k, bias);
  return hipGetLastError();
}

hipError_t launch_act_quant_gemm_fused(const void *x, bool ue8m0, const uint8_t *b,
                                      const float *b_s, const void *bias, void *c, bool c_bf16,
                                      int64_t m, int64_t n, int64_t k, uint8_t *a_q, float *a_s,
                                      hipStream_t stream) {
  // no mover: the compute waves, and the helpers that quantize x
  const int cw = decode_width(n);
  const dim3 grid((unsigned)((n + 16 * cw - 1) / (16 * cw))), block(64 * kFusedWaves);
#define FP8BSQ_FUSED_W(RING, LDS, CW, DEPTH)                                                                  \
  do {                                                                                                         \
    if (c_bf16)                                                                                                \
      hipLaunchKernelGGL((block_gemm_decode_kernel<true, 1, DEPTH, false, true, RING, CW>), grid, block,        \
                         (LDS), stream, (const uint8_t *)x, nullptr, b, b_s, c, m, n, k, bias, ue8m0, a_q, a_s); \
    else                                                                                                       \
      hipLaunchKernelGGL((block_gemm_decode_kernel<false, 1, DEPTH, false, true, RING, CW>), grid, block,       \
                         (LDS), stream, (const uint8_t *)x, nullptr, b, b_s, c, m, n, k, bias, ue8m0, a_q, a_s); \
  } while (0)
#define FP8BSQ_FUSED(RING, LDS)                                                                               \
  do {                                                                                                         \
    switch (cw) {                                                                                              \
      case 1: FP8BSQ_FUSED_W(RING, LDS, 1, kFusedNarrowDepth); break;                                          \
      case 2: FP8BSQ_FUSED_W(RING, LDS, 2, kFusedNarrowDepth); break;                                          \
      case 3: FP8BSQ_FUSED_W(RING, LDS, 3, kDecodeDepth); break;                                               \
      case 4: FP8BSQ_FUSED_W(RING, LDS, 4, kDecodeDepth); break;                                               \
      default: FP8BSQ_FUSED_W(RING, LDS, kDecodeCompute, kDecodeDepth); break;                                 \
    }                                                                                                          \
  } while (0)
  if (m * k <= kFusedMaxCodes)
    FP8BSQ_FUSED(false, (size_t)(m * k));
  else
    FP8BSQ_FUSED(true, (size_t)fused_ring_blocks((int)m) * m * kBlock);
#undef FP8BSQ_FUSED
#undef FP8BSQ_FUSED_W
  return hipGetLastError();
}

bool act_quant_gemm_fusable(bool x_bf16, int64_t m, int64_t k) {
  return x_bf16 && m <= kFusedMaxM && k / kBlock <= kDecodeMaxKb && m * k <= kFusedRingMaxCodes;
}

}  // namespace fp8bsq
