/*
 * fp8bsq.h -- C ABI of the block-scaled FP8 library for AMD Instinct MI355X
 * (gfx950): dynamic 1x128 activation quantization, 128x128 block-scaled
 * weight dequantization, the block-scaled FP8 E4M3 GEMM those two feed, and
 * the 128x128 weight quantization that produces the GEMM's weight operand.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every data pointer is a DEVICE pointer (hipMalloc'd or a PyTorch CUDA
 *    tensor's data_ptr) owned by the caller, who keeps it alive until the work
 *    queued on `hip_stream` has finished.  The library allocates nothing; its
 *    only state is a per-device cache of the compute-unit count and the
 *    static scratch of fp8_block_gemm_split_noalloc.  Calls are re-entrant
 *    and thread-safe, except fp8_block_gemm_split_noalloc calls that overlap
 *    on one GPU, which race on that scratch.
 *  - All tensors are dense and row-major.  E4M3 codes are bytes in the OCP
 *    E4M3FN encoding (PyTorch's torch.float8_e4m3fn).  Scales are FP32.
 *  - Work is queued on `hip_stream` (a hipStream_t; NULL = the default stream)
 *    and the call returns without synchronizing.
 *  - The return value is FP8BSQ_OK or an fp8bsq_status code.  Arguments are
 *    validated before any HIP call; on a validation error nothing is queued.
 *    FP8BSQ_ELAUNCH reports an error from the HIP runtime after the launch.
 *  - Empty inputs: a call whose outputs have no elements (a row or column
 *    count of 0) passes the enum and shape checks, then returns FP8BSQ_OK
 *    without queuing anything or reading its pointers, which may be NULL.  A
 *    negative size is FP8BSQ_EINVAL, and so is k = 0 for a product.
 *  - Inputs must be finite.  NaN/Inf inputs or scales give unspecified (but
 *    memory-safe) outputs.
 *  - block_size is an argument because the format makes it configurable; only
 *    128 is implemented (FP8BSQ_EUNSUPPORTED otherwise).
 *
 * Citations name the web page and the section the operation is defined in.
 */
#ifndef FP8BSQ_H
#define FP8BSQ_H

#include <stddef.h>
#include <stdint.h>

#define FP8BSQ_API __attribute__((visibility("default")))

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FP8BSQ_OK = 0,
  FP8BSQ_EINVAL = 1,       /* null pointer, negative dimension (or k = 0 for a product), unknown enum */
  FP8BSQ_ESHAPE = 2,       /* a dimension that must be a multiple of block_size is not */
  FP8BSQ_EUNSUPPORTED = 3, /* block_size != 128 */
  FP8BSQ_EALIGN = 4,       /* a pointer lacks the alignment stated for it */
  FP8BSQ_ELAUNCH = 5,      /* the HIP runtime reported an error for the launch */
  FP8BSQ_ERANGE = 6,       /* a size does not fit the kernels' 32-bit indexing limits */
  FP8BSQ_ESCRATCH = 7      /* the product needs more scratch than the static buffer holds */
} fp8bsq_status;

typedef enum { FP8BSQ_F32 = 0, FP8BSQ_BF16 = 1 } fp8bsq_dtype;

typedef enum {
  FP8BSQ_SCALE_NONE = 0,  /* scale_fmt=None: s = fl32(amax / 448) */
  FP8BSQ_SCALE_UE8M0 = 1  /* scale_fmt="ue8m0": s rounded up to a power of two */
} fp8bsq_scale_fmt;

/*
 * fp8_act_quant -- dynamic activation quantization, one scale per 1 x 128 block.
 *
 * Defined on the page "Understanding Dynamic and Static Activation
 * Quantization Schemes in DeepSeek-V3", section "How Dynamic Activation
 * Quantization Works" (act_quant(x, block_size=128, scale_fmt=None) -> (y, s)),
 * and on "DeepSeek-V3 quantization_config Parameters Explained", section "The
 * activation_scheme Parameter": per block, amax = max |x| clamped to at least
 * 1e-4, s = amax / 448, y = x / s in E4M3.
 *
 *   x          [rows, k] activations, dtype x_dtype (FP8BSQ_F32 or FP8BSQ_BF16),
 *              16-byte aligned.
 *   rows, k    rows >= 0, k >= 0 and k % block_size == 0 (else FP8BSQ_ESHAPE);
 *              either 0: nothing to do.
 *   scale_fmt  FP8BSQ_SCALE_NONE or FP8BSQ_SCALE_UE8M0 (smallest power of two
 *              >= fl32(amax/448)).
 *   y          [rows, k] E4M3 codes out, 8-byte aligned:
 *              y = RNE_E4M3(fl32(x / s)), saturating at +-448, sign kept on zero.
 *   s          [rows, k / block_size] FP32 scales out, 4-byte aligned.
 *
 * Results are bit-identical to the CPU oracle for finite x.
 */
FP8BSQ_API int fp8_act_quant(const void *x, int x_dtype, int64_t rows, int64_t k, int block_size,
                  int scale_fmt, uint8_t *y, float *s, void *hip_stream);

/*
 * fp8_weight_dequant -- 128x128 block-scaled weight dequantization.
 *
 * Defined on the page "How weight_dequant Handles Per-Block Scaling in
 * DeepSeek-V3 FP8 GEMM", sections "Per-Block Scaling Architecture", "Grid
 * Mapping and Scale Lookup" and "Dequantization Computation": each
 * block_size x block_size tile of x is converted to FP32 and multiplied by its
 * own scale, y = x * s; edge tiles are masked.
 *
 *   x        [m, n] E4M3 codes (m weight rows, n columns), any alignment.
 *   s        [ceil(m / block_size), ceil(n / block_size)] FP32 scales
 *            (weight_scale_inv), row-major: tile (i, j) at i * ceil(n/bs) + j.
 *   m, n     >= 0 (either 0: nothing to do); need not be multiples of block_size.
 *   y        [m, n] out, dtype y_dtype: FP8BSQ_F32 gives fl32(DEC(x) * s);
 *            FP8BSQ_BF16 gives that product rounded to nearest even bf16.
 *
 * Results are bit-identical to the CPU oracle for finite scales.  Inputs with
 * n % 8 == 0, 8-byte-aligned x and 16-byte-aligned y take the vectorized path.
 */
FP8BSQ_API int fp8_weight_dequant(const uint8_t *x, const float *s, int64_t m, int64_t n, int block_size,
                       void *y, int y_dtype, void *hip_stream);

/*
 * fp8_weight_quant -- 128x128 block weight quantization (fp8_weight_dequant's
 * inverse).
 *
 * The storage format is defined on the page "DeepSeek-V3 quantization_config
 * Parameters Explained", section "The weight_block_size Parameter" (E4M3
 * codes in 128 x 128 blocks, each with its own inverse scale,
 * weight_scale_inv) and on "How weight_dequant Handles Per-Block Scaling in
 * DeepSeek-V3 FP8 GEMM", sections "Per-Block Scaling Architecture" and "Grid
 * Mapping and Scale Lookup" (the scale grid and y = x * s).  The pages give
 * no formula for producing the codes; this entry point applies the
 * activation rule of fp8_act_quant to each tile: amax = max |x| over the
 * tile's elements clamped to at least 1e-4, s = fl32(amax / 448) (or the
 * smallest power of two >= that under FP8BSQ_SCALE_UE8M0),
 * y = RNE_E4M3(fl32(x / s)) saturating at +-448, sign kept on zero.
 *
 *   x          [m, n] weights, dtype x_dtype (FP8BSQ_F32 or FP8BSQ_BF16),
 *              aligned to its element size.
 *   m, n       >= 0 (either 0: nothing to do); need not be multiples of
 *              block_size (edge tiles use their valid elements only);
 *              m <= 65535 * 128 (else FP8BSQ_ERANGE).
 *   y          [m, n] E4M3 codes out.
 *   s          [ceil(m / block_size), ceil(n / block_size)] FP32 scales out,
 *              row-major, 4-byte aligned; fp8_weight_dequant(y, s) maps the
 *              codes back to within half an E4M3 ulp of x / s, times s.
 *
 * Results are bit-identical to the CPU oracle for finite x.  Inputs with
 * n % 8 == 0, 16-byte-aligned x and 8-byte-aligned y take the vectorized path.
 */
FP8BSQ_API int fp8_weight_quant(const void *x, int x_dtype, int64_t m, int64_t n, int block_size,
                     int scale_fmt, uint8_t *y, float *s, void *hip_stream);

/*
 * fp8_block_gemm -- block-scaled FP8 GEMM, C = A . B^T.
 *
 * Defined on the page "How weight_dequant Handles Per-Block Scaling in
 * DeepSeek-V3 FP8 GEMM", section "Relationship to FP8 GEMM Operations"
 * (fp8_gemm(a, a_s, b, b_s): the per-block scales are applied inside the
 * product, no dequantized weight is materialized), with the weight used as in
 * F.linear(x, W) ("Practical Usage Example"), and on the page "DeepSeek-V3:
 * How Selective FP8 Stays Stable" ("Learning outcomes", FAQ and "Lower
 * precision is a constrained budget"): partial sums are promoted to FP32
 * periodically and outputs are BF16 or FP32.  Here the promotion happens once
 * per 128-wide K block: for each K block kb,
 *     C[i, j] += (sum_{k in kb} A[i, k] * B[j, k]) * a_s[i, kb] * b_s[j / 128, kb].
 *
 *   a      [m, k] E4M3 activation codes (act_quant's y), 16-byte aligned.
 *   a_s    [m, k / 128] FP32 activation scales (act_quant's s).
 *   b      [n, k] E4M3 weight codes ([out, in]), 16-byte aligned.
 *   b_s    [ceil(n / 128), k / 128] FP32 weight block scales.
 *   c      [m, n] out, dtype c_dtype (FP8BSQ_F32 or FP8BSQ_BF16, RNE from the
 *          FP32 accumulator); 4-byte aligned.
 *   m, n   >= 0 (either 0: nothing to do); k >= 128 and k % 128 == 0 (else
 *          FP8BSQ_ESHAPE; k = 0 is FP8BSQ_EINVAL).
 *
 * Accumulation order is not specified; every element is within
 * 1e-3 * sum_k |a_k * b_k| of the exact result (plus one bf16 ulp for BF16).
 */
FP8BSQ_API int fp8_block_gemm(const uint8_t *a, const float *a_s, const uint8_t *b, const float *b_s,
                   void *c, int c_dtype, int64_t m, int64_t n, int64_t k, void *hip_stream);

/*
 * fp8_block_gemm_ue8m0 -- fp8_block_gemm for activation scales that are
 * powers of two (fp8_act_quant with FP8BSQ_SCALE_UE8M0).
 *
 * The page "Understanding Dynamic and Static Activation Quantization Schemes
 * in DeepSeek-V3", section "How Dynamic Activation Quantization Works", gives
 * the ue8m0 option: scales rounded to powers of two for hardware
 * compatibility.  On gfx950 such a scale is an E8M0 number the MX-scaled
 * matrix instruction applies itself: each A row's a_s is applied inside the
 * MFMA and the per-K-block rescale multiplies by b_s alone.  Since scaling by
 * a power of two is exact, the result is bit-identical to fp8_block_gemm on
 * the same inputs.
 *
 * Arguments, layouts and errors as for fp8_block_gemm.  Precondition: every
 * a_s value is a positive normal power of two.  Where the MX-scaled kernel
 * runs (m > 64, k / 128 a multiple of 4, a_s 16-byte aligned) the call checks
 * it with a second kernel queued after the product: every C row whose a_s row
 * holds any other value is set to NaN in all n columns.  Other shapes run
 * fp8_block_gemm's kernels, which apply any a_s exactly.
 */
FP8BSQ_API int fp8_block_gemm_ue8m0(const uint8_t *a, const float *a_s, const uint8_t *b,
                         const float *b_s, void *c, int c_dtype, int64_t m, int64_t n, int64_t k,
                         void *hip_stream);

/*
 * fp8_block_gemm_reference -- fp8_block_gemm by its reference-structure
 * kernel, for testing: each wave reads its MFMA fragments straight from
 * global memory (no LDS staging, no persistent tiles).  This kernel is also
 * what fp8_block_gemm runs for shapes beyond its fast kernels' 32-bit lane
 * offsets (A or B of 4 GiB or more); this entry point runs it for any shape,
 * so that path can be checked on small problems.
 *
 * Same product, arguments, layouts, bound and errors as fp8_block_gemm (page
 * "How weight_dequant Handles Per-Block Scaling in DeepSeek-V3 FP8 GEMM",
 * section "Relationship to FP8 GEMM Operations").  Slow: not for production.
 */
FP8BSQ_API int fp8_block_gemm_reference(const uint8_t *a, const float *a_s, const uint8_t *b,
                             const float *b_s, void *c, int c_dtype, int64_t m, int64_t n,
                             int64_t k, void *hip_stream);

/*
 * fp8_block_gemm_split -- fp8_block_gemm / fp8_block_gemm_ue8m0 (scale_fmt
 * FP8BSQ_SCALE_NONE / FP8BSQ_SCALE_UE8M0) with split-K for a last round of
 * tiles that would leave compute units idle.
 *
 * Same product as fp8_block_gemm (per 128-wide K block, the partial times
 * a_s * b_s accumulated in FP32; the page "How weight_dequant Handles
 * Per-Block Scaling in DeepSeek-V3 FP8 GEMM", section "Relationship to FP8
 * GEMM Operations").  When the 256 x 256 output tiles fill the device's compute
 * units in whole rounds plus a last round of at most half of them, that last
 * round's tiles are computed in 2-4 parts over consecutive K ranges, and
 * their FP32 partial tiles are added in part order (P0 + P1 + ...) before the
 * output rounding.  Only the summation order differs from fp8_block_gemm, so
 * results meet the same bound but need not be bit-identical to it.
 *
 *   workspace        device memory of fp8_block_gemm_split_workspace(m, n, k)
 *                    bytes, 256-byte aligned, owned by the caller: scratch
 *                    for the partial tiles and per-tile counters, with no
 *                    initial contents required (the call clears the counters
 *                    itself, in the first of its launches).  Calls in flight
 *                    at the same time need separate workspaces.
 *   workspace_bytes  its size.  NULL or a smaller size runs the unsplit launch
 *                    of fp8_block_gemm (same results up to summation order).
 *
 * Other arguments, layouts and errors as for fp8_block_gemm; workspace must be
 * 256-byte aligned (FP8BSQ_EALIGN).
 */
FP8BSQ_API int fp8_block_gemm_split(const uint8_t *a, const float *a_s, const uint8_t *b,
                         const float *b_s, void *c, int c_dtype, int64_t m, int64_t n, int64_t k,
                         int scale_fmt, void *workspace, size_t workspace_bytes, void *hip_stream);

/*
 * fp8_block_gemm_split_workspace -- bytes of workspace fp8_block_gemm_split
 * uses for an [m, k] x [n, k] product on the current HIP device: 0 when no
 * split pays for this shape there (the call then needs no workspace), for an
 * empty product, or for arguments fp8_block_gemm would reject.  Queries the device's compute-unit
 * count; queues no work.
 */
FP8BSQ_API size_t fp8_block_gemm_split_workspace(int64_t m, int64_t n, int64_t k);

/*
 * fp8_block_gemm_split_noalloc -- fp8_block_gemm_split without a workspace
 * argument, for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc).
 *
 * Same product, arguments (less workspace and workspace_bytes), layouts,
 * bound and errors as fp8_block_gemm_split.  The split-K scratch (partial
 * tiles and per-tile counters) lives in a static device array of
 * FP8BSQ_SPLIT_SCRATCH_BYTES bytes inside the library, one per GPU, held until
 * the process ends; its address is looked up once per device, on the first
 * call there.  The call allocates nothing and clears the counters it uses
 * itself (with a kernel, no memset).  A product whose split needs more than
 * FP8BSQ_SPLIT_SCRATCH_BYTES (fp8_block_gemm_split_workspace(m, n, k) larger;
 * not possible on a 256-CU device) returns FP8BSQ_ESCRATCH and queues nothing.
 * Every call on one GPU shares that GPU's array: calls that may overlap on
 * one GPU (other streams, other threads) race on it and must be ordered by
 * the caller, or use fp8_block_gemm_split with separate workspaces.
 */
#define FP8BSQ_SPLIT_SCRATCH_BYTES ((size_t)67109376) /* 512 + 256 * 256 * 256 * 4: 64 MiB + 512 B */
FP8BSQ_API int fp8_block_gemm_split_noalloc(const uint8_t *a, const float *a_s, const uint8_t *b,
                                 const float *b_s, void *c, int c_dtype, int64_t m, int64_t n,
                                 int64_t k, int scale_fmt, void *hip_stream);

/*
 * fp8_act_quant_gemm -- a linear layer's forward product in one call:
 * quantize the activations, then multiply by the block-scaled weight.
 *
 * The page "Understanding Dynamic and Static Activation Quantization Schemes
 * in DeepSeek-V3", section "How Dynamic Activation Quantization Works",
 * describes the linear wrapper calling act_quant on the activations during
 * the forward pass before the FP8 GEMM; page "How weight_dequant Handles
 * Per-Block Scaling in DeepSeek-V3 FP8 GEMM", section "Relationship to FP8
 * GEMM Operations", gives the GEMM.  This entry point computes
 *     (a_q, a_s) = fp8_act_quant(x, scale_fmt);
 *     c          = fp8_block_gemm(a_q, a_s, b, b_s)  (+ bias)
 * with outputs bit-identical to those two calls when bias is null.  For bf16 x with m <= 16,
 * k <= 20480 and m * k <= 98304 (the decode case) both happen in one kernel: in every workgroup helper
 * waves quantize x into LDS while the GEMM's waves stream the weight, and workgroup 0 also
 * writes a_q and a_s.  Otherwise
 * the two kernels are queued back to back on hip_stream (with
 * FP8BSQ_SCALE_UE8M0, the GEMM is fp8_block_gemm_ue8m0's).
 *
 *   x          [m, k] activations, dtype x_dtype (FP8BSQ_F32 or FP8BSQ_BF16),
 *              16-byte aligned.
 *   scale_fmt  as for fp8_act_quant.
 *   b, b_s     [n, k] E4M3 weight (16-byte aligned) and its
 *              [ceil(n / 128), k / 128] FP32 block scales, as for fp8_block_gemm.
 *   bias       [n] of c's dtype, or NULL; added to the FP32 accumulator
 *              before the output rounding.
 *   c          [m, n] out, dtype c_dtype (FP8BSQ_F32 or FP8BSQ_BF16).
 *   m, n, k    m, n >= 0; k >= 128 and k % 128 == 0 (else FP8BSQ_ESHAPE; k = 0
 *              is FP8BSQ_EINVAL).  m = 0: nothing to do.  n = 0: only a_q and
 *              a_s are written (act_quant alone); b, b_s, bias and c are not
 *              read and may be NULL.
 *   a_q        [m, k] E4M3 codes out (16-byte aligned): act_quant's y.
 *   a_s        [m, k / 128] FP32 scales out (4-byte aligned): act_quant's s.
 *
 * c meets fp8_block_gemm's bound (around the exact product plus bias); a_q and
 * a_s are bit-identical to the oracle.
 */
FP8BSQ_API int fp8_act_quant_gemm(const void *x, int x_dtype, int scale_fmt, const uint8_t *b,
                       const float *b_s, const void *bias, void *c, int c_dtype, int64_t m,
                       int64_t n, int64_t k, uint8_t *a_q, float *a_s, void *hip_stream);

/* Short English text for a status code; never NULL. */
FP8BSQ_API const char *fp8bsq_strerror(int status);

/* Library version, "major.minor.patch". */
FP8BSQ_API const char *fp8bsq_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FP8BSQ_H */
