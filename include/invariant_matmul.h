/*
 * invariant_matmul.h -- C ABI of a batch-invariant GEMM library for AMD
 * MI355X (gfx950).
 *
 * It computes C = scale_a * scale_b * (A x B) with A [M,K], B [K,N] and
 * C [M,N], all row-major and contiguous (leading dimensions K, N and N), from
 * fp16, bf16 or OCP fp8 (e4m3fn / e5m2) inputs with fp32 accumulation.  The
 * problem statement, the matrix shapes and the element formula follow the
 * Tencent engineer article on deterministic LLM inference ("AI インフラの深化：
 * 大規模モデルに確定的な出力を実現する方法"), section "Batch Invariance の由来"
 * (C = A x B with A [M,K], B [K,N]; C_ij is the dot product of row i of A and
 * column j of B over k).
 *
 * Batch invariance.  The same article (same section) shows that the
 * spatial tile sizes and the workgroup order do not change any bit, while the
 * reduction step and the split of K do.  This library therefore fixes the
 * matrix-core instruction per input dtype and fixes the K order, the K-step
 * and the split of K from (N, K, dtypes, explicit options) alone -- never
 * from M.  For one plan key the bits of row i of C are a function of row i of
 * A and of B only: they do not depend on M, on other rows, on concurrently
 * running work, on the stream or on how often the call has run.
 *
 * Calls, their passages (each call's own comment below repeats its passage):
 *   gemm_plan, gemm_plan_ex, gemm_plan_ex2
 *                     the problem statement C = A x B with A [M,K], B [K,N],
 *                     C [M,N] and a configuration fixed from (N, K, dtypes)
 *                     alone (article, section "Batch Invariance の由来"; section
 *                     "演算子チューニング" shows the M-driven tile and split
 *                     choices this planner does not make).
 *   gemm_plan_info    the configuration a plan fixed: BLOCK_M / BLOCK_N /
 *                     BLOCK_K, SPLIT_K, GROUP_M and the waves (the tuning
 *                     parameters of section "演算子チューニング").
 *   gemm_workspace_size
 *                     bytes of the [split_k, M, N] fp32 partial-sum workspace
 *                     (section "Split-K").
 *   gemm_plan_tile_of the workgroup -> output tile order (section "GROUP_M -
 *                     Swizzle L2 Cache").
 *   gemm_run          one workgroup per output tile running the K loop
 *                     (section "Tiling - 分塊行列乗算": accumulator init,
 *                     load/compute/accumulate per K step, one write-back);
 *                     tiles visited in GROUP_M order (section "GROUP_M -
 *                     Swizzle L2 Cache").
 *   gemm_run_bias, gemm_splitk_run_bias
 *                     the same plus the bias of a linear layer (the vLLM
 *                     batch-invariant linear operator listed in the article's
 *                     closing section).
 *   gemm_splitk_run   split-K through a [split_k, M, N] fp32 workspace and a
 *                     separate reduction kernel on the same stream, no atomics
 *                     (section "Split-K", the workspace variant).
 *   ozaki_*           the fp64 product by the Ozaki scheme (Insight Edge blog
 *                     on cuTile Python, section "倍精度行列積エミュレーション").
 *   gemm_plan_destroy, ozaki_plan_destroy, gemm_status_string,
 *   gemm_last_hip_error
 *                     library housekeeping (freeing a host plan, naming a
 *                     status, the last HIP error); no passage defines them.
 *
 * Conventions for every call:
 *   - All matrices and the workspace are DEVICE memory owned by the caller; the
 *     library never allocates device memory.  A plan is host memory owned by
 *     the caller (free it with gemm_plan_destroy).  Plans are immutable and
 *     may be used from several host threads / streams at once (each concurrent
 *     split-K call needs its own workspace).
 *   - `stream` is a hipStream_t passed as void* (NULL means the null stream),
 *     so that a caller needs no HIP header to include this one; a hipStream_t
 *     converts to void* implicitly in C and C++.  Run calls only enqueue work
 *     on it: they never synchronise the host.
 *   - Inputs are read-only.  C is fully overwritten (there is no beta).  The
 *     workspace holds no meaningful data after the call.
 *   - Every argument is validated before anything is enqueued (the checks
 *     that need no runtime come first, so they also run without a GPU); on
 *     error nothing is enqueued and C is untouched.  A status other than
 *     GEMM_OK is returned:
 *       GEMM_ERR_INVALID_VALUE  negative size, NULL pointer for a non-empty
 *                               operand, pointer not 16-byte aligned, NULL
 *                               plan or output handle; on a machine with a
 *                               GPU also an operand that does not lie
 *                               wholly inside one device allocation of the
 *                               current device (host memory, another
 *                               device's memory, or a buffer shorter than
 *                               the operand), checked with the runtime's
 *                               pointer queries before anything is enqueued;
 *       GEMM_ERR_UNSUPPORTED    unsupported dtype pair, N or K not a multiple of
 *                               16 bytes' worth of elements (8 for 16-bit
 *                               inputs, 16 for fp8), bad option value;
 *       GEMM_ERR_WORKSPACE      workspace NULL or smaller than
 *                               gemm_workspace_size();
 *       GEMM_ERR_HIP            no usable GPU, or a launch failed (the HIP
 *                               error is then available from hipGetLastError
 *                               semantics inside the library: call
 *                               gemm_last_hip_error() for its code).
 *   - Empty products: M == 0 or N == 0 enqueue nothing and return GEMM_OK;
 *     K == 0 writes C = 0.
 */
#ifndef INVARIANT_MATMUL_H
#define INVARIANT_MATMUL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GEMM_OK = 0,
  GEMM_ERR_INVALID_VALUE = 1,
  GEMM_ERR_UNSUPPORTED = 2,
  GEMM_ERR_WORKSPACE = 3,
  GEMM_ERR_HIP = 4
} gemm_status;

/* Element types.  Inputs: F16, BF16, F8_E4M3 (OCP e4m3fn), F8_E5M2 (OCP e5m2).
 * Outputs: F32, BF16 or F16 (round to nearest, ties to even; fp16 keeps
 * subnormals and overflows to infinity). */
typedef enum {
  GEMM_F16 = 0,
  GEMM_BF16 = 1,
  GEMM_F8_E4M3 = 2,
  GEMM_F8_E5M2 = 3,
  GEMM_F32 = 4,
  GEMM_I8 = 5   /* int8, as Ozaki-scheme slices only (ozaki_plan) */
} gemm_dtype;

/* Output-tile shapes (rows x columns of C per workgroup).  All tiles of one
 * input dtype use the same matrix-core instruction and the same K order, so
 * for a fixed split of K they produce identical bits; the choice only moves
 * work in space. */
typedef enum {
  GEMM_TILE_DEFAULT = 0,    /* chosen from (N, K, dtype) */
  GEMM_TILE_256x256 = 1,    /* 8 waves, LDS ring filled by buffer->LDS DMA */
  GEMM_TILE_128x128 = 2,    /* 4 waves, register-staged LDS tiles */
  GEMM_TILE_32x128 = 3,     /* 4 waves, register-staged LDS tiles */
  GEMM_TILE_256x256_RS = 4, /* 8 waves, register-staged LDS tiles */
  GEMM_TILE_32x256 = 5,     /* 4 waves, DMA ring; narrow tile for skinny or
                               reduction-dominated shapes */
  GEMM_TILE_64x256 = 6,     /* 4 waves, DMA ring */
  GEMM_TILE_128x256 = 7,    /* 8 waves, DMA ring of 3 stages */
  GEMM_TILE_32x64 = 8,      /* 2 waves, DMA ring of 3 stages of 256 bytes of
                               K (two workgroups per compute unit); fp16 /
                               bf16 only: narrow tile for small M (4x the
                               workgroups of 32x256) */
  GEMM_TILE_64x64 = 9,      /* 2 waves, DMA ring of 2 stages of 256 bytes of
                               K (two workgroups per compute unit); fp16 /
                               bf16 only */
  GEMM_TILE_32x32 = 10      /* 2 waves, DMA ring of 3 stages of 256 bytes of
                               K (three workgroups per compute unit); fp16 /
                               bf16 only: twice the workgroups of 32x64 for
                               small M */
} gemm_tile;

/* Plan flags (gemm_plan_ex2). */
typedef enum {
  /* B is given transposed: a [N, K] row-major matrix W with B = W^T (the
   * weight layout of a linear layer, y = x W^T + b, as in the vLLM
   * batch-invariant operators the Tencent article lists in its closing
   * section).  Only the DMA tiles (256x256, 128x256, 64x256, 32x256, 64x64, 32x64,
   * 32x32) read this layout;
   * the bits of C are those of the [K, N] layout holding the same values. */
  GEMM_PLAN_B_TRANSPOSED = 1,
  /* gemm_run / gemm_run_bias with the 256x256 tile launch at most one
   * workgroup per compute unit, each walking the tiles of the one-tile-per-
   * workgroup grid in the same raster order, with its LDS pipeline running
   * on from one tile into the next (the persistent batch-invariant matmul of
   * the Tencent article's closing section).  The bits of C are those of the
   * plan without the flag; other tiles and the split-K path ignore it. */
  GEMM_PLAN_PERSISTENT = 2,
  /* gemm_run / gemm_run_bias take their tile from M instead of from (N, K,
   * dtype): the DMA tile (32x32, 32x64, 64x64, 32x256, 64x256, 128x256 or
   * 256x256; fp8 inputs skip the first three) with the least estimated time,
   * rounds of 256 workgroups times a per-tile time that grows with the
   * tile's size.  gemm_splitk_run of a wide reduction-dominated shape
   * (K >= 2N, N > 512) takes from M the tile with the fewest row tiles (32-row,
   * 64x256, 128x256 or 256x256); the split of K stays the one (N, K, dtype)
   * gives.  Every tile uses the same matrix-core instruction and K order, so
   * C is bitwise that of the plan without the flag for every M (tile sizes do
   * not change bits: the Tencent article, "Batch Invariance の由来"); only the
   * time changes.  An explicit tile, and the split-K path of other shapes,
   * ignore it. */
  GEMM_PLAN_TILE_BY_M = 4,
  /* fp8 inputs (GEMM_F8_E4M3, GEMM_F8_E5M2) only: every fp8 value is widened
   * to fp16 in registers (exactly: both formats are subsets of fp16) and the
   * products are accumulated by the 16x16x32 fp16 matrix-core step in fp32,
   * in ascending K, instead of by the 16x16x128 fp8 step.  The fp8 step adds
   * each group of 8 consecutive products in a window that drops what lies
   * more than 13 binades below the group's largest product, so its error is
   * bounded by K * 2^-24 * sum |a||b| (the fp32 accumulation the Tencent
   * article's "背景" assumes) only for long K or benign inputs; with this flag
   * that bound holds for every K and every input.  The bits are this mode's
   * own (equal to those of the fp8 step only where no product is dropped) and
   * are batch-invariant by the same rule as every plan: one instruction and
   * one K order for every tile and M.  It runs the fp8 data at the fp16
   * matrix rate.  DMA tiles only: an explicit register-staged tile, or a K so
   * large that the DMA tiles' 32-bit offsets overflow, gives
   * GEMM_ERR_UNSUPPORTED, as does another input dtype. */
  GEMM_PLAN_FP8_FP32_ACCUM = 8
} gemm_plan_flags;

typedef struct gemm_plan_s* gemm_plan_t;

/* A plan holds one tile for each entry point: tile / block_m / block_n /
 * waves / tiles_m / tiles_n describe gemm_splitk_run's partial kernel, the
 * run_* fields gemm_run's single pass.  Both are chosen from (N, K, dtype,
 * options) alone (with GEMM_PLAN_TILE_BY_M, also from M), and the bits of C
 * depend on neither: only split_k and k_per_split, which never depend on M,
 * decide them. */
typedef struct {
  int64_t M, N, K;
  int32_t in_dtype, out_dtype;  /* gemm_dtype values */
  int32_t tile;                 /* gemm_tile value of the split-K path */
  int32_t block_m, block_n;     /* its output tile */
  int32_t block_k;              /* K elements staged per main-loop step */
  int32_t mfma_m, mfma_n, mfma_k; /* matrix-core instruction shape */
  int32_t waves;                /* 64-lane wavefronts per workgroup (split-K path) */
  int32_t group_m;              /* GROUP_M of the tile raster */
  int32_t split_k;              /* K slices used by gemm_splitk_run */
  int64_t k_per_split;          /* K elements per slice (multiple of block_k) */
  int64_t tiles_m, tiles_n;     /* output tiles along M and N (split-K path) */
  int64_t grid_run;             /* workgroups launched by gemm_run */
  int64_t grid_splitk;          /* workgroups of the split-K partial kernel */
  uint64_t workspace_bytes;     /* split_k * M * N * 4 */
  float scale_a, scale_b;
  int32_t run_tile;             /* gemm_tile value of gemm_run */
  int32_t run_block_m, run_block_n;
  int32_t run_waves;
  int64_t run_tiles_m, run_tiles_n;
} gemm_plan_info_t;

/* Plan C[M,N] = A[M,K] x B[K,N] (Tencent article, "Batch Invariance の由来":
 * the problem statement, and the conclusion that the K step and the split of
 * K must not follow the batch size) with default options: fp32 output for
 * fp16 / bf16 inputs and bf16 output for fp8 inputs, split and tile chosen
 * from (N, K, dtype), GROUP_M = 8, scales 1.0.  M only sizes the grid and the
 * workspace.  On success *out receives a new plan (host memory; free it with
 * gemm_plan_destroy). */
gemm_status gemm_plan(int64_t M, int64_t N, int64_t K, gemm_dtype in, gemm_plan_t* out);

/* As gemm_plan with explicit options (same passage).  out_dtype: GEMM_F32,
 * GEMM_BF16 or GEMM_F16.
 * split_k: 0 = default, else 1..4096 (the slice length is rounded up to a
 * multiple of block_k; the split actually used is reported by
 * gemm_plan_info).  group_m: 0 = default (8), else >= 1.  scale_a, scale_b:
 * per-tensor scales multiplied into the result (their fp32 product is applied
 * to the fp32 sum before the output conversion); must be finite. */
gemm_status gemm_plan_ex(int64_t M, int64_t N, int64_t K, gemm_dtype in, gemm_dtype out,
                         int split_k, int group_m, float scale_a, float scale_b,
                         gemm_plan_t* plan);

/* As gemm_plan_ex with an explicit output tile and plan flags (same passage;
 * the tile is the article's BLOCK_M / BLOCK_N, which it shows changes no bit).
 * tile: a gemm_tile value (GEMM_TILE_DEFAULT: chosen from (N, K, dtype)).
 * flags: a bitwise OR of gemm_plan_flags; unknown bits give
 * GEMM_ERR_UNSUPPORTED.  With GEMM_PLAN_B_TRANSPOSED, B is read as [N, K]
 * row-major; an explicit register-staged tile, or a K so large that the DMA
 * tiles' 32-bit offsets overflow, gives GEMM_ERR_UNSUPPORTED. */
gemm_status gemm_plan_ex2(int64_t M, int64_t N, int64_t K, gemm_dtype in, gemm_dtype out,
                          int split_k, int group_m, int tile, float scale_a, float scale_b,
                          unsigned flags, gemm_plan_t* plan);

/* The configuration a plan fixed (Tencent article, "演算子チューニング": the
 * tile sizes, the K step, SPLIT_K and GROUP_M of its parameter table), into
 * *info.  Pure host call.  GEMM_ERR_INVALID_VALUE for a NULL argument. */
gemm_status gemm_plan_info(gemm_plan_t plan, gemm_plan_info_t* info);

/* Bytes of workspace gemm_splitk_run needs: split_k * M * N * sizeof(float),
 * the [split_k, M, N] fp32 partial sums (Tencent article, "Split-K").  0 for
 * a NULL plan. */
size_t gemm_workspace_size(gemm_plan_t plan);

/* Tile raster: the (k_slice, pid_m, pid_n) that workgroup `workgroup` of the
 * split-K partial kernel computes (k_slice is 0 for gemm_run's grid), after
 * the XCD remap and the GROUP_M order (Tencent article, "GROUP_M - Swizzle L2
 * Cache").  Pure host function, exposed so the raster can be checked to be a
 * bijection.  GEMM_ERR_INVALID_VALUE for a workgroup outside the grid. */
gemm_status gemm_plan_tile_of(gemm_plan_t plan, int64_t workgroup, int64_t* k_slice,
                              int64_t* pid_m, int64_t* pid_n);

/* C = A x B in one pass: one workgroup per output tile, full K in order
 * (Tencent article, "Tiling - 分塊行列乗算").  A, B, C: device memory,
 * row-major, 16-byte aligned; enqueued on `stream`. */
gemm_status gemm_run(gemm_plan_t plan, const void* A, const void* B, void* C, void* stream);

/* As gemm_run plus a bias: C[i, j] = convert(scale * sum_ij + bias[j]), one
 * fp32 add after the scale.  bias: device fp32 [N], 4-byte aligned, or NULL
 * (then exactly gemm_run).  The bias term of a linear layer (the vLLM
 * batch-invariant linear operator in the Tencent article's closing section). */
gemm_status gemm_run_bias(gemm_plan_t plan, const void* A, const void* B, const float* bias,
                          void* C, void* stream);

/* C = A x B through the split-K workspace (Tencent article, "Split-K", the
 * workspace variant): the partial kernel writes slice s of K to
 * workspace[s, :, :] (fp32, no atomics), then a reduction kernel sums the
 * slices in ascending s and writes C.  With split_k == 1 the result is
 * bitwise identical to gemm_run.  workspace: device memory of at least
 * gemm_workspace_size(plan) bytes, 16-byte aligned, owned by the caller. */
gemm_status gemm_splitk_run(gemm_plan_t plan, const void* A, const void* B, void* C,
                            void* workspace, size_t workspace_bytes, void* stream);

/* As gemm_splitk_run plus a bias, added by the reduction kernel after the
 * ascending-slice sum and the scale (same rule as gemm_run_bias). */
gemm_status gemm_splitk_run_bias(gemm_plan_t plan, const void* A, const void* B,
                                 const float* bias, void* C, void* workspace,
                                 size_t workspace_bytes, void* stream);

/* Frees a host plan (NULL is ignored).  Housekeeping: no passage. */
void gemm_plan_destroy(gemm_plan_t plan);

/* The largest split-K workspace gemm_splitk_run_noalloc serves: 64 MiB (for
 * example the decode product 128 x 4096 x 14336 bf16 at its default 16 slices
 * needs 32 MiB; 256 x 4096 x 14336 needs 64 MiB exactly). */
#define GEMM_NOALLOC_WORKSPACE_BYTES ((size_t)64 << 20)

/* For callers that cannot allocate device memory -- code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc: as
 * gemm_splitk_run, with the [split_k, M, N] fp32 workspace taken from an array
 * inside the library instead of from the caller.  The library holds one such
 * array of GEMM_NOALLOC_WORKSPACE_BYTES on every GPU it runs on, from the
 * first call on that GPU until the process ends; the call itself allocates
 * nothing.  C is bitwise what gemm_splitk_run gives for the same plan.
 * Errors: as gemm_splitk_run; GEMM_ERR_WORKSPACE if gemm_workspace_size(plan)
 * exceeds GEMM_NOALLOC_WORKSPACE_BYTES (nothing is enqueued).  All calls on
 * one GPU share its array: calls that overlap on one GPU (other streams or
 * host threads) race and must be serialised by the caller. */
gemm_status gemm_splitk_run_noalloc(gemm_plan_t plan, const void* A, const void* B, void* C,
                                    void* stream);

/* ---------------------------------------------------------------------------
 * fp64 matrix product by the Ozaki scheme: C = A x B with A [M,K], B [K,N]
 * and C [M,N] in fp64 (row-major, contiguous), computed on the matrix cores
 * from low-precision slices: bf16 or fp8 e4m3 with fp32 accumulation, or
 * int8 with int32 accumulation.  Insight Edge blog on
 * cuTile Python, section "倍精度行列積エミュレーション":
 *   split ("分解(Split)", equations (1)-(5)): every row of A and every column
 *     of B is cut into `slices` Type2 slices (bf16, fp8 e4m3 or int8) with
 *     c0 = ceil(log2 max|x|) of that row / column, c_p = c0 - p*delta,
 *     sigma = 0.75*2^(rho+c_p), v = (x+sigma)-sigma, x -= v,
 *     slice_p = Type2(v*2^-c_p);
 *   product ("行列積の計算", equations (10), (11)): for each slice pair (p,q),
 *     p ascending then q ascending, without the pairs with p+q >= d ("Fast
 *     Mode（GEMMの削減）"), the fp32 product of the two slices, scaled by
 *     2^(c_p(row) + c_q(column)), is added to an fp64 sum starting at +0.
 * K is cut into chunks of `chunk` products; for each pair the exact fp32
 * product of every chunk is added to the fp64 sum in ascending chunk order
 * (the page's exactness argument in "最適化後の結果" is per K tile).
 * Precision parameter ("分解(Split)"): rho = max(gamma, xi),
 * gamma = ceil(53 - (m_Type3 - log2 k)/2), xi = 53 - m_Type2 (m_Type2 = 8 for
 * bf16, 4 for e4m3, 6 for int8 -- an int8 entry n * 2^-b needs |n| <= 2^b <=
 * 127; m_Type3 = 24 for fp32, 31 for int32 accumulation), with k = min(K,
 * chunk) the length of one accumulation chain.  A slice
 * carries b = 53 - rho bits, so every fp32 chunk product is exact and the
 * result does not depend on any summation order inside the matrix cores: it
 * is a bitwise function of row i of A, of B, of K and of (type2, slices, d,
 * chunk).  delta = b + 1.
 * Defaults: chunk = 2^(m_Type3 - 2 m_Type2), the longest exact chain with
 * all of Type2's bits (256 for bf16, 65536 for e4m3, 2^19 for int8);
 * slices = min(ceil(53 / b), 20) (7 for bf16, 14 for e4m3, 9 for int8; 20 is
 * the most the page's split routine makes),
 * d = slices + 2 (39 products for 7 bf16 slices, 130 for 14 e4m3 slices, the
 * page's "最適化後の結果" tables; 60 for 9 int8 slices).
 * Domain: finite inputs whose nonzero row / column maxima lie in
 * [2^-300, 2^300].  There every slice value, scaled term and partial sum is
 * a normal fp64 number, so the kernel may apply 2^(c0(row) + c0(column)) once
 * at the end instead of to every term without changing a bit.  A row of A or
 * a column of B outside it (holding a NaN or an infinity, a magnitude above
 * 2^300, or a nonzero maximum below 2^-300) gets the exponent -2^30 in the
 * workspace and zero slices, and its whole row / column of C is NaN; every
 * other entry of C is unaffected (no error is reported).
 *
 * Workspace (device memory, caller-owned, 16-byte aligned, at least
 * ozaki_workspace_size bytes), with the offsets that ozaki_plan_info reports:
 *   a_slices  [slices, M, k_pad] Type2, row-major (k_pad = K rounded up to 16)
 *   b_slices  [slices, k_pad, n_pad] Type2 (n_pad = N rounded up to 16)
 *   a_exp     [M] int32 c0 of each row of A
 *   b_exp     [n_pad] int32 c0 of each column of B
 *   scratch   column maxima of B
 * Padding entries of the slices are zero.  The contents stay valid after a
 * call until the workspace is used again.
 * ------------------------------------------------------------------------- */
typedef struct ozaki_plan_s* ozaki_plan_t;

typedef struct {
  int64_t M, N, K;
  int32_t type2;              /* GEMM_BF16, GEMM_F8_E4M3 or GEMM_I8 */
  int32_t rho, bits, delta;   /* precision parameter, bits per slice, exponent step */
  int32_t slices, d, pairs;   /* slices per operand, Fast Mode threshold, products */
  int64_t chunk;              /* products per exact fp32 chain */
  int32_t tile_m, tile_n;     /* output tile of the product kernel */
  int64_t k_pad, n_pad;
  int64_t grid;               /* workgroups of the product kernel */
  uint64_t workspace_bytes;
  uint64_t a_slices_offset, b_slices_offset, a_exp_offset, b_exp_offset, scratch_offset;
} ozaki_plan_info_t;

/* Plan an Ozaki-scheme product.  type2: GEMM_BF16, GEMM_F8_E4M3 or GEMM_I8.
 * slices: 0 = default, else 1..20; d: 0 = default, else >= 1; chunk: 0 =
 * default, else a multiple of 128 (at most 2^22).  M, N, K >= 0; K below 2^23
 * (bf16), 2^25 (e4m3) or 2^24 (int8), N below 2^23 (32-bit offsets inside one
 * tile).
 * Errors: GEMM_ERR_INVALID_VALUE (negative size, NULL
 * handle), GEMM_ERR_UNSUPPORTED (other type2, slices, d or chunk out of range,
 * sizes too large). */
gemm_status ozaki_plan(int64_t M, int64_t N, int64_t K, gemm_dtype type2, int slices, int d,
                       int64_t chunk, ozaki_plan_t* plan);

gemm_status ozaki_plan_info(ozaki_plan_t plan, ozaki_plan_info_t* info);

size_t ozaki_workspace_size(ozaki_plan_t plan);

/* The split of one operand into the workspace: operand 0 = A (x is [M, K]),
 * 1 = B (x is [K, N]); x is device fp64, 8-byte aligned.  Enqueues the
 * exponent and split kernels on `stream`. */
gemm_status ozaki_split(ozaki_plan_t plan, int operand, const double* x, void* workspace,
                        size_t workspace_bytes, void* stream);

/* The slice-pair product from a workspace holding both operands' slices and
 * exponents (after ozaki_split of A and of B): writes C (device fp64 [M, N],
 * 8-byte aligned). */
gemm_status ozaki_multiply(ozaki_plan_t plan, const void* workspace, size_t workspace_bytes,
                           double* C, void* stream);

/* ozaki_split(A), ozaki_split(B), ozaki_multiply on one stream. */
gemm_status ozaki_run(ozaki_plan_t plan, const double* A, const double* B, double* C,
                      void* workspace, size_t workspace_bytes, void* stream);

void ozaki_plan_destroy(ozaki_plan_t plan);

/* Name of a status ("GEMM_OK", ...); a static string.  Housekeeping. */
const char* gemm_status_string(gemm_status status);

/* HIP error code (hipError_t as int) of the most recent GEMM_ERR_HIP return on
 * this host thread, 0 if none. */
int gemm_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* INVARIANT_MATMUL_H */
