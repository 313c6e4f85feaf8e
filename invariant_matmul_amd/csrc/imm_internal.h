// Internal declarations shared by the host library (api.cpp) and the kernels.
//
// Citations: [TDI] = Tencent engineer article on deterministic LLM inference
// ("AI インフラの深化：大規模モデルに確定的な出力を実現する方法").
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "invariant_matmul.h"

namespace imm {

// Every tile configuration of an input dtype uses the same matrix-core
// instruction (a 16x16 output block with K of 32 for 16-bit inputs, with K of
// 128 for fp8) and walks K in ascending order in steps of that
// instruction, so configurations differ only in how output elements are
// spread over workgroups and waves -- which [TDI] "Batch Invariance の由来"
// (BLOCK_M / BLOCK_N, num_warps paragraphs) shows has no effect on bits.

// Bytes of K staged per main-loop step: 64 fp16/bf16 elements or 128 fp8.
constexpr int kTileKBytes = 128;

inline int elem_bytes(int dt) { return (dt == GEMM_F8_E4M3 || dt == GEMM_F8_E5M2) ? 1 : 2; }
inline int block_k_elems(int dt) { return kTileKBytes / elem_bytes(dt); }
// Shape of the matrix-core step the GEMM kernels use for an input dtype:
// 16 x 16 x 32 for fp16 / bf16, 16 x 16 x 128 for fp8.
inline int mfma_mn(int) { return 16; }
inline int mfma_k(int dt) { return elem_bytes(dt) == 1 ? 128 : 32; }

// Kernel input codes of fp8 data under GEMM_PLAN_FP8_FP32_ACCUM: fp8 bytes in
// memory and LDS, widened to fp16 in registers for the 16x16x32 fp16 step.
constexpr int kInWiden = 0x10;
constexpr int kInE4M3W = kInWiden | GEMM_F8_E4M3;
constexpr int kInE5M2W = kInWiden | GEMM_F8_E5M2;

}  // namespace imm

struct gemm_plan_s {
  int64_t M, N, K;
  int in, out;
  // Tile of the split-K path (gemm_splitk_run) ...
  int tile;             // gemm_tile actually used
  int bm, bn, bk;       // bk in elements
  int waves_m, waves_n;
  int64_t tiles_m, tiles_n;
  // ... and of the single pass (gemm_run).  Both are chosen from (N, K,
  // dtype, options); the bits do not depend on either.
  int run_tile;
  int run_bm, run_bn;
  int run_waves_m, run_waves_n;
  int64_t run_tiles_m, run_tiles_n;
  bool b_trans;         // B is given as [N, K] row-major (DMA tiles only)
  bool f8_fp32;         // fp8 through the fp16 step (DMA tiles only)
  bool persistent;      // gemm_run: at most one workgroup per compute unit
  int group_m;
  int split_k;          // slices actually used (after rounding)
  int64_t k_per_split;  // elements, multiple of bk
  float scale_a, scale_b;
  float scale;          // fp32 product applied in the epilogue
};

namespace imm {

// Workgroup -> (k_slice, pid_m, pid_n).
//
// Step 1 (XCD remap): the dispatcher hands workgroup w to XCD w % 8, and each
// XCD has its own L2.  Renumber so that every XCD works on one contiguous run
// of logical ids, so tiles that share A rows / B columns share one L2.
// Step 2: the K slice is the slowest-moving coordinate.
// Step 3 (GROUP_M, [TDI] "GROUP_M - Swizzle L2 Cache"): within a slice, tiles
// are taken group_m rows of tiles at a time, column by column, so that
// consecutive workgroups reuse the same A rows and B columns from L2.
// Every step is a bijection of [0, G); none of them affects any bit of C.
__host__ __device__ inline void raster_tile(int64_t w, int64_t G, int64_t tiles_m,
                                            int64_t tiles_n, int64_t group_m,
                                            int64_t* k_slice, int64_t* pid_m,
                                            int64_t* pid_n) {
  const int64_t per = G / 8, rem = G % 8;
  const int64_t x = w % 8, loc = w / 8;
  const int64_t logical = (x < rem) ? x * (per + 1) + loc : rem * (per + 1) + (x - rem) * per + loc;
  const int64_t tiles = tiles_m * tiles_n;
  *k_slice = logical / tiles;
  const int64_t t = logical % tiles;
  const int64_t width = group_m * tiles_n;
  const int64_t first_m = (t / width) * group_m;
  const int64_t rows_left = tiles_m - first_m;
  const int64_t gm = rows_left < group_m ? rows_left : group_m;
  const int64_t in_group = t % width;
  *pid_m = first_m + in_group % gm;
  *pid_n = in_group / gm;
}

// The same mapping in 32-bit arithmetic for grids without a K split
// (k_slice = 0) and fewer than 2^31 workgroups: cheap enough to evaluate once
// per tile inside a kernel's main loop (64-bit divisions expand into long
// vector-ALU sequences there).
__host__ __device__ inline void raster_tile32(uint32_t w, uint32_t G, uint32_t tiles_m,
                                              uint32_t tiles_n, uint32_t group_m, uint32_t* pid_m,
                                              uint32_t* pid_n) {
  const uint32_t per = G / 8, rem = G % 8;
  const uint32_t x = w % 8, loc = w / 8;
  const uint32_t t = (x < rem) ? x * (per + 1) + loc : rem * (per + 1) + (x - rem) * per + loc;
  const uint32_t width = group_m * tiles_n;
  const uint32_t grp = t / width;
  const uint32_t first_m = grp * group_m;
  const uint32_t rows_left = tiles_m - first_m;
  const uint32_t gm = rows_left < group_m ? rows_left : group_m;
  const uint32_t in_group = t - grp * width;
  const uint32_t q = in_group / gm;
  *pid_m = first_m + (in_group - q * gm);
  *pid_n = q;
}

// Kernel arguments (passed by value).
struct GemmArgs {
  const void* A;
  const void* B;
  void* C;              // output (store-C mode) or workspace (slice mode)
  const float* bias;    // fp32 [N] added in the epilogue, or null (store-C mode only)
  int64_t M, N, K;
  int64_t k_per_split;  // elements per K slice (K itself when not split)
  int64_t tiles_m, tiles_n;
  int64_t grid;         // total workgroups
  int64_t group_m;
  float scale;
};

// Arguments of the Ozaki-scheme slice-pair product (the DMA kernel in its
// slice-pair mode).  A and B point at the first slice of each operand; slice
// p of A starts slice_a bytes after slice p-1 (likewise B).  K and N are the
// slices' padded sizes (their leading dimensions); n_out and ldc describe the
// fp64 output.
struct OzGemmArgs : GemmArgs {
  int64_t slice_a, slice_b;
  int64_t n_out, ldc;
  const int32_t* ea;    // exponent of each row of A (M values)
  const int32_t* eb;    // exponent of each column of B (n_out values)
  int32_t slices, d, npairs, delta;
  int32_t chunk_stages;  // K stages per exact fp32 chain
};

// Arguments of the persistent single pass: `grid` (and tiles_m, tiles_n)
// describe the one-tile-per-workgroup raster, `wgs` the workgroups launched.
struct PersistArgs : GemmArgs {
  int64_t wgs;
};

struct ReduceArgs {
  const float* ws;
  void* C;
  const float* bias;    // fp32 [N] or null
  int64_t MN;           // M * N
  int64_t N;
  int split_k;
  float scale;
};

// Launchers (gemm_kernels.hip).  They only enqueue; they return the launch
// status.  `slice_mode` selects the split-K partial kernel (fp32 workspace
// output, raw sums, no scale) instead of the final store.
hipError_t launch_gemm(const gemm_plan_s& p, int tile, const GemmArgs& a, bool slice_mode,
                       hipStream_t s);
hipError_t launch_reduce(const gemm_plan_s& p, const ReduceArgs& a, hipStream_t s);
// The DMA-fed kernels (gemm_dma.hip); launch_gemm forwards the DMA tiles to it.
hipError_t launch_gemm_dma(const gemm_plan_s& p, int tile, const GemmArgs& a, bool slice_mode,
                           hipStream_t s);
// The persistent single pass on the 256 x 256 DMA tile (gemm_dma.hip).
hipError_t launch_gemm_persist(const gemm_plan_s& p, const PersistArgs& a, hipStream_t s);
// The Ozaki slice-pair product on the DMA kernel (gemm_dma.hip); type2 is
// GEMM_BF16, GEMM_F8_E4M3 or GEMM_I8.  Output tile oz_tile_m(type2) x 256.
constexpr int kOzTileN = 256;
// Exponent of a row of A or a column of B outside the Ozaki domain (a NaN or
// an infinity, a magnitude above 2^300, or a nonzero maximum below 2^-300):
// its slices are zero and its row / column of C is NaN.
constexpr int kOzBadExp = -(1 << 30);
constexpr double kOzMaxMag = 0x1p300, kOzMinMax = 0x1p-300;
inline int oz_tile_m(int type2) { return type2 == GEMM_F8_E4M3 ? 64 : 128; }
hipError_t launch_ozaki_gemm(int type2, const OzGemmArgs& a, hipStream_t s);
// The Ozaki split (ozaki.hip): exponents of the rows of x [R, C] ...
hipError_t launch_oz_row_exp(const double* x, int64_t R, int64_t C, int32_t* e, hipStream_t s);
// ... of its columns (maxima over chunks of rc rows into part [ceil(R/rc), C],
// then combined) ...
hipError_t launch_oz_col_exp(const double* x, int64_t R, int64_t C, int64_t rc, double* part,
                             int32_t* e, hipStream_t s);
// ... and the slices [slices, Ro, Co] of x with one exponent per row
// (per_row) or per column.
hipError_t launch_oz_split(int type2, bool per_row, const double* x, int64_t R, int64_t C,
                           int64_t Ro, int64_t Co, const int32_t* e, int slices, int rho, int delta,
                           void* out, hipStream_t s);

}  // namespace imm
