// GEMM kernels for gfx950 (CDNA4): tiled main loop on the matrix cores and
// the fixed-order split-K reduction.
//
// Citations:
//   [TDI] Tencent engineer article on deterministic LLM inference
//         ("AI インフラの深化：大規模モデルに確定的な出力を実現する方法").
//   [GKM] "GEMM kernels" memo on GPU matrix multiply basics (qsysarch).
//
// Data flow of one workgroup ([TDI] "Tiling - 分塊行列乗算"): it owns one
// BM x BN tile of C (or of one K slice of it), clears its accumulators, and
// walks its K range in ascending steps of 128 bytes of K: the A and B blocks
// of the step are read from HBM with 16-byte coalesced loads into registers
// (the next step's loads are in flight while the current step computes),
// written to a double-buffered LDS tile, and fed to the matrix cores from
// LDS.  The accumulators never leave registers until the single write-back.
//
// Bits.  Each output element is one accumulation chain: its 16x16 MFMA block
// is updated once per instruction-K step (32 elements for fp16/bf16, 128 for
// fp8) in ascending k, starting from +0.  The instruction is fixed per input
// dtype and the chain does not depend on BM, BN, the wave layout or the tile
// order ([TDI] "Batch Invariance の由来": BLOCK_M/BLOCK_N and GROUP_M change
// no bits, the K step does).  Rows past M load as zero and are never stored,
// so row i of C depends on row i of A and on B only.
//
// LDS layout.  Both operands are stored K-contiguous, 128 bytes of K per row
// (one row per M row of A and per N column of B), as 8 chunks of 16 bytes;
// chunk c of row r lives at slot c ^ ((r ^ r >> 3) & 7).  The XOR spreads
// the 16-byte fragment reads of 8 consecutive rows, and the transposed
// writes of B (8 columns apart), over distinct bank groups.
//
// B is row-major [K, N] (N contiguous) but the matrix core wants K-contiguous
// data per lane, so each thread loads a 4 x 16-byte block of B (4 K rows)
// and transposes it in registers before writing it to LDS ([GKM] discusses
// the non-coalesced column access of B that this avoids).
#include "kernel_common.h"

namespace imm {
namespace {
using namespace dev;

constexpr int ROWB = kTileKBytes;  // bytes of K per LDS row per stage
constexpr int CHUNKS = ROWB / 16;  // 16-byte chunks per LDS row

template <int IN>
struct TileT {
  static constexpr int EB = InT<IN>::EB;
  static constexpr bool M16 = EB == 2;                   // 16x16x32 step (16-bit inputs)
  static constexpr bool F8 = EB == 1;                    // 16x16x128 step (fp8 inputs)
  static constexpr int BLK = 16;                         // MFMA output block edge
  static constexpr int NACC = BLK * BLK / 64;            // accumulators per lane per block
  static constexpr int KSTEP = M16 ? 64 : 128;           // bytes of K per MFMA step
  static constexpr int BKE = ROWB / EB;                  // K elements per stage
  static constexpr int NKK = ROWB / KSTEP;               // MFMA steps per stage
  static constexpr int FRAG = M16 ? 1 : 2;               // 16-byte chunks per lane
  using Acc = f32x4;
};

__device__ __forceinline__ int swz(int r) { return (r ^ (r >> 3)) & 7; }

// Transpose a 4 (K) x 16-byte (N) block of B held as rows q[0..3] into
// K-major pieces: for 16-bit elements, 8 columns x 4 K values (8 bytes each);
// for 8-bit elements, 16 columns x 4 K values (4 bytes each).
template <int EB>
__device__ __forceinline__ void transpose_b(const i32x4 (&q)[4], i32x2 (&o16)[8], int (&o8)[16]) {
  if constexpr (EB == 2) {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const unsigned r0 = q[0][p], r1 = q[1][p], r2 = q[2][p], r3 = q[3][p];
      // column 2p takes the low halves, column 2p+1 the high halves
      o16[2 * p][0] = (int)((r0 & 0xffffu) | (r1 << 16));
      o16[2 * p][1] = (int)((r2 & 0xffffu) | (r3 << 16));
      o16[2 * p + 1][0] = (int)((r0 >> 16) | (r1 & 0xffff0000u));
      o16[2 * p + 1][1] = (int)((r2 >> 16) | (r3 & 0xffff0000u));
    }
  } else {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const unsigned r0 = q[0][p], r1 = q[1][p], r2 = q[2][p], r3 = q[3][p];
      // interleave bytes of rows 0/1 and 2/3, then 16-bit halves of those
      const unsigned lo01 = __builtin_amdgcn_perm(r1, r0, 0x05010400u);  // r0.b0 r1.b0 r0.b1 r1.b1
      const unsigned hi01 = __builtin_amdgcn_perm(r1, r0, 0x07030602u);  // r0.b2 r1.b2 r0.b3 r1.b3
      const unsigned lo23 = __builtin_amdgcn_perm(r3, r2, 0x05010400u);
      const unsigned hi23 = __builtin_amdgcn_perm(r3, r2, 0x07030602u);
      o8[4 * p + 0] = (int)__builtin_amdgcn_perm(lo23, lo01, 0x05040100u);
      o8[4 * p + 1] = (int)__builtin_amdgcn_perm(lo23, lo01, 0x07060302u);
      o8[4 * p + 2] = (int)__builtin_amdgcn_perm(hi23, hi01, 0x05040100u);
      o8[4 * p + 3] = (int)__builtin_amdgcn_perm(hi23, hi01, 0x07060302u);
    }
  }
}

template <int IN, int OUT, int BM, int BN, int WAVES_M, int WAVES_N, bool SLICE>
__global__ __launch_bounds__(WAVES_M* WAVES_N * 64) void gemm_tile_kernel(GemmArgs g) {
  using T = TileT<IN>;
  constexpr int THREADS = WAVES_M * WAVES_N * 64;
  constexpr int EB = T::EB;
  constexpr int BKE = T::BKE;
  constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N;  // wave tile
  constexpr int BLK = T::BLK;
  constexpr int FM = WTM / BLK, FN = WTN / BLK;
  constexpr int A_CH = BM * CHUNKS / THREADS;            // A chunks per thread
  constexpr int NB = BN * EB / 16;                       // 16-byte column groups of B
  constexpr int B_TASKS = (BKE / 4) * NB;                // 4-row blocks of B
  static_assert(WTM % BLK == 0 && WTN % BLK == 0, "wave tile must be a multiple of the block");
  static_assert(BM * CHUNKS % THREADS == 0 && B_TASKS == THREADS, "staging layout");
  constexpr int STAGE = (BM + BN) * ROWB;

  __shared__ __attribute__((aligned(16))) char lds[2 * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  const int lb = lane % BLK, hq = lane / BLK;  // row / column in the block, K piece

  int64_t ks, pm, pn;
  raster_tile(blockIdx.x, g.grid, g.tiles_m, g.tiles_n, g.group_m, &ks, &pm, &pn);
  const int64_t m0 = pm * BM, n0 = pn * BN;
  const int64_t kbeg = ks * g.k_per_split;
  const int64_t kend = (g.K < kbeg + g.k_per_split) ? g.K : kbeg + g.k_per_split;
  const int nt = kend > kbeg ? (int)((kend - kbeg + BKE - 1) / BKE) : 0;

  const char* A = static_cast<const char*>(g.A);
  const char* B = static_cast<const char*>(g.B);

  i32x4 ra[A_CH];
  i32x4 rb[4];
  // B task of this thread: column group nb, 4-row group kq.
  const int nb = tid % NB, kq = tid / NB;

  auto load_tile = [&](int t) {
    const int64_t kb = kbeg + (int64_t)t * BKE;
#pragma unroll
    for (int i = 0; i < A_CH; ++i) {
      const int c = tid + i * THREADS;
      const int r = c / CHUNKS, ch = c % CHUNKS;
      const int64_t row = m0 + r;
      const int64_t k = kb + ch * (16 / EB);
      if (row < g.M && k < kend)
        ra[i] = *reinterpret_cast<const i32x4*>(A + (row * g.K + k) * EB);
      else
        ra[i] = i32x4{0, 0, 0, 0};
    }
    const int64_t col = n0 + nb * (16 / EB);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int64_t k = kb + kq * 4 + q;
      if (k < kend && col < g.N)
        rb[q] = *reinterpret_cast<const i32x4*>(B + (k * g.N + col) * EB);
      else
        rb[q] = i32x4{0, 0, 0, 0};
    }
  };

  auto store_tile = [&](int st) {
    char* sa = lds + st * STAGE;
    char* sb = sa + BM * ROWB;
#pragma unroll
    for (int i = 0; i < A_CH; ++i) {
      const int c = tid + i * THREADS;
      const int r = c / CHUNKS, ch = c % CHUNKS;
      *reinterpret_cast<i32x4*>(sa + r * ROWB + ((ch ^ swz(r)) << 4)) = ra[i];
    }
    i32x2 o16[8];
    int o8[16];
    transpose_b<EB>(rb, o16, o8);
    if constexpr (EB == 2) {
      // 4 K values (8 bytes) for each of 8 columns; byte offset kq*8 in the row
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const int n = nb * 8 + t;
        *reinterpret_cast<i32x2*>(sb + n * ROWB + (((kq >> 1) ^ swz(n)) << 4) + ((kq & 1) << 3)) =
            o16[t];
      }
    } else {
      // 4 K values (4 bytes) for each of 16 columns; byte offset kq*4 in the row
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        const int n = nb * 16 + t;
        *reinterpret_cast<int*>(sb + n * ROWB + (((kq >> 2) ^ swz(n)) << 4) + ((kq & 3) << 2)) =
            o8[t];
      }
    }
  };

  typename T::Acc acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = typename T::Acc{};

  if (nt > 0) {
    load_tile(0);
    store_tile(0);
    __syncthreads();
  }
  for (int t = 0; t < nt; ++t) {
    const int cur = t & 1;
    if (t + 1 < nt) load_tile(t + 1);
    const char* sa = lds + cur * STAGE;
    const char* sb = sa + BM * ROWB;
#pragma unroll
    for (int kk = 0; kk < T::NKK; ++kk) {
      i32x4 af[FM][T::FRAG], bfr[FN][T::FRAG];
      // chunk of K piece f of this lane in step kk
      auto chunk = [&](int f) { return kk * (T::KSTEP / 16) + hq * T::FRAG + f; };
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int r = wm * WTM + i * BLK + lb;
#pragma unroll
        for (int f = 0; f < T::FRAG; ++f)
          af[i][f] = *reinterpret_cast<const i32x4*>(sa + r * ROWB + ((chunk(f) ^ swz(r)) << 4));
      }
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int n = wn * WTN + j * BLK + lb;
#pragma unroll
        for (int f = 0; f < T::FRAG; ++f)
          bfr[j][f] = *reinterpret_cast<const i32x4*>(sb + n * ROWB + ((chunk(f) ^ swz(n)) << 4));
      }
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          if constexpr (T::M16) {
            acc[i][j] = mfma16_v<IN>(af[i][0], bfr[j][0], acc[i][j]);
          } else {
            const i32x8 av = __builtin_shufflevector(af[i][0], af[i][1], 0, 1, 2, 3, 4, 5, 6, 7);
            const i32x8 bv = __builtin_shufflevector(bfr[j][0], bfr[j][1], 0, 1, 2, 3, 4, 5, 6, 7);
            acc[i][j] = mfma16_f8<IN>(av, bv, acc[i][j]);
          }
        }
    }
    if (t + 1 < nt) store_tile(cur ^ 1);
    __syncthreads();
  }

  // Write-back.  Accumulator layout of a 16x16 block: lane l, register r holds
  // row 4*(l/16) + r, column l%16.
#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int64_t col = n0 + wn * WTN + j * BLK + lb;
#pragma unroll
      for (int r = 0; r < T::NACC; ++r) {
        const int64_t row = m0 + wm * WTM + i * BLK + 4 * hq + r;
        if (row < g.M && col < g.N) {
          const float v = acc[i][j][r];
          if constexpr (SLICE) {
            static_cast<float*>(g.C)[(ks * g.M + row) * g.N + col] = v;
          } else {
            store_final<OUT>(g.C, row * g.N + col, v, g.scale, g.bias, col);
          }
        }
      }
    }
  }
}

// C = convert(scale * (((ws[0] + ws[1]) + ws[2]) + ... + ws[S-1]) [+ bias]),
// fp32 adds in ascending slice order for every element ([TDI] "Split-K": the separate
// reduction kernel that sums the workspace over split_k).  Four consecutive
// elements per thread, grid-stride.  The slices are loaded in groups of RG
// before they are added (in order), so a thread waits for one memory latency
// per group instead of one per slice: one group for the decode splits.
template <int OUT>
__global__ __launch_bounds__(64) void splitk_reduce_kernel(ReduceArgs r) {
  constexpr int RG = 16;
  const int64_t n4 = r.MN / 4;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const f32x4* ws = reinterpret_cast<const f32x4*>(r.ws);
  const int64_t slice4 = r.MN / 4;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride) {
    f32x4 v = ws[i];
    for (int s0 = 1; s0 < r.split_k; s0 += RG) {
      f32x4 w[RG];
#pragma unroll
      for (int j = 0; j < RG; ++j)
        if (s0 + j < r.split_k) w[j] = ws[(int64_t)(s0 + j) * slice4 + i];
#pragma unroll
      for (int j = 0; j < RG; ++j) {
        if (s0 + j < r.split_k) {
          v[0] = v[0] + w[j][0];
          v[1] = v[1] + w[j][1];
          v[2] = v[2] + w[j][2];
          v[3] = v[3] + w[j][3];
        }
      }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int64_t idx = i * 4 + e;
      store_final<OUT>(r.C, idx, v[e], r.scale, r.bias, idx % r.N);
    }
  }
}

template <int IN, int OUT, int BM, int BN, int WM, int WN>
hipError_t launch_cfg(const GemmArgs& a, bool slice, hipStream_t s) {
  const dim3 grid((unsigned)a.grid), block(WM * WN * 64);
  if (slice)
    hipLaunchKernelGGL((gemm_tile_kernel<IN, GEMM_F32, BM, BN, WM, WN, true>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((gemm_tile_kernel<IN, OUT, BM, BN, WM, WN, false>), grid, block, 0, s, a);
  return hipGetLastError();
}

template <int IN, int OUT>
hipError_t launch_tile(int tile, const GemmArgs& a, bool slice, hipStream_t s) {
  switch (tile) {
    case GEMM_TILE_256x256_RS: return launch_cfg<IN, OUT, 256, 256, 2, 4>(a, slice, s);
    case GEMM_TILE_128x128: return launch_cfg<IN, OUT, 128, 128, 2, 2>(a, slice, s);
    case GEMM_TILE_32x128: return launch_cfg<IN, OUT, 32, 128, 1, 4>(a, slice, s);
    default: return hipErrorInvalidValue;
  }
}

template <int IN>
hipError_t launch_in(const gemm_plan_s& p, int tile, const GemmArgs& a, bool slice, hipStream_t s) {
  if (p.out == GEMM_F32) return launch_tile<IN, GEMM_F32>(tile, a, slice, s);
  if (p.out == GEMM_F16) return launch_tile<IN, GEMM_F16>(tile, a, slice, s);
  return launch_tile<IN, GEMM_BF16>(tile, a, slice, s);
}

}  // namespace

hipError_t launch_gemm(const gemm_plan_s& p, int tile, const GemmArgs& a, bool slice_mode,
                       hipStream_t s) {
  if (tile == GEMM_TILE_256x256 || tile == GEMM_TILE_128x256 || tile == GEMM_TILE_32x256 ||
      tile == GEMM_TILE_64x256 || tile == GEMM_TILE_32x64 || tile == GEMM_TILE_64x64 ||
      tile == GEMM_TILE_32x32)
    return launch_gemm_dma(p, tile, a, slice_mode, s);
  if (p.f8_fp32) return hipErrorInvalidValue;  // the planner keeps such plans on DMA tiles
  switch (p.in) {
    case GEMM_F16: return launch_in<GEMM_F16>(p, tile, a, slice_mode, s);
    case GEMM_BF16: return launch_in<GEMM_BF16>(p, tile, a, slice_mode, s);
    case GEMM_F8_E4M3: return launch_in<GEMM_F8_E4M3>(p, tile, a, slice_mode, s);
    case GEMM_F8_E5M2: return launch_in<GEMM_F8_E5M2>(p, tile, a, slice_mode, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_reduce(const gemm_plan_s& p, const ReduceArgs& a, hipStream_t s) {
  // One-wave workgroups: a small output (decode) spreads over more compute
  // units, so each issues fewer of the slice loads.
  constexpr int kThreads = 64;
  const int64_t n4 = a.MN / 4;
  int64_t blocks = (n4 + kThreads - 1) / kThreads;
  if (blocks > 16384) blocks = 16384;
  if (blocks < 1) blocks = 1;
  if (p.out == GEMM_F32)
    hipLaunchKernelGGL(splitk_reduce_kernel<GEMM_F32>, dim3((unsigned)blocks), dim3(kThreads), 0, s, a);
  else if (p.out == GEMM_F16)
    hipLaunchKernelGGL(splitk_reduce_kernel<GEMM_F16>, dim3((unsigned)blocks), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL(splitk_reduce_kernel<GEMM_BF16>, dim3((unsigned)blocks), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace imm
