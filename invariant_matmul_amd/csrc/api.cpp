// Host side of the C ABI: planning, argument validation, launches.
//
// Citations: [TDI] = Tencent engineer article on deterministic LLM inference
// ("AI インフラの深化：大規模モデルに確定的な出力を実現する方法").
//
// The plan is a pure function of (N, K, input dtype, output dtype, explicit
// options).  M is stored only to size the grid and the workspace.  [TDI]
// "Batch Invariance の由来" concludes that a configuration which changes the
// K step or the split of K with the batch size is what breaks batch
// invariance, and [TDI] "演算子チューニング" describes exactly such M-driven
// tile and split heuristics; by default this planner never reads M for any
// decision.  The one exception is opt-in and bits-neutral: with
// GEMM_PLAN_TILE_BY_M the single pass takes its output tile from M, which
// [TDI] "Batch Invariance の由来" shows does not change bits (and every tile
// here uses the same instruction and K order).
#include <hip/hip_runtime.h>

#include <climits>
#include <cmath>
#include <cstring>
#include <initializer_list>
#include <new>

#include "host_internal.h"

using namespace imm;

namespace {

thread_local int g_last_hip_error = 0;

constexpr int kMaxSplit = 4096;

bool valid_in(int dt) {
  return dt == GEMM_F16 || dt == GEMM_BF16 || dt == GEMM_F8_E4M3 || dt == GEMM_F8_E5M2;
}
bool valid_out(int dt) { return dt == GEMM_F32 || dt == GEMM_BF16 || dt == GEMM_F16; }

void tile_shape(int tile, int* bm, int* bn, int* wm, int* wn) {
  switch (tile) {
    case GEMM_TILE_256x256: *bm = 256; *bn = 256; *wm = 2; *wn = 4; break;
    case GEMM_TILE_256x256_RS: *bm = 256; *bn = 256; *wm = 2; *wn = 4; break;
    case GEMM_TILE_128x128: *bm = 128; *bn = 128; *wm = 2; *wn = 2; break;
    case GEMM_TILE_32x256: *bm = 32; *bn = 256; *wm = 1; *wn = 4; break;
    case GEMM_TILE_64x256: *bm = 64; *bn = 256; *wm = 1; *wn = 4; break;
    case GEMM_TILE_128x256: *bm = 128; *bn = 256; *wm = 2; *wn = 4; break;
    case GEMM_TILE_32x64: *bm = 32; *bn = 64; *wm = 2; *wn = 1; break;
    case GEMM_TILE_64x64: *bm = 64; *bn = 64; *wm = 2; *wn = 1; break;
    case GEMM_TILE_32x32: *bm = 32; *bn = 32; *wm = 2; *wn = 1; break;
    default: *bm = 32; *bn = 128; *wm = 1; *wn = 4; break;  // GEMM_TILE_32x128
  }
}

// Reduction-dominated shapes (K at least twice N): the regime where the
// output has few tiles and split-K is the tool ([TDI] "Split-K": tiny M x N,
// huge K; the parameter table restricts SPLIT_K to such shapes).  Wide ones
// (decode-like, N > 512) get the narrow 32 x 128 tile, whose time is the
// stream of B; narrow ones (N <= 512) get the 128 x 256 DMA tile, which reads
// each slice of B once per 128 rows.  The rest get the large tile.
bool reduction_dominated(int64_t N, int64_t K) { return K >= 2 * N; }

// Small B (at most 4 MB, the L2 of one XCD): 256 x 256 tiles leave most of
// the machine idle unless M is large (1024^3 has 16 of them), so these
// shapes take the tile whose worst case over M is least: 64 x 64 for 16-bit
// inputs, 128 x 256 for fp8 (which the narrow tiles do not take).  Measured
// (us; fp16, fp32 out; 32 x 32 / 32 x 64 / 64 x 64 / 32 x 256 / 128 x 256 /
// 256 x 256) on N = K = 1024: M = 1: 8.2 / 9.9 / 11.4 / 14.8 / 16.5 / 23.9;
// M = 1024: 15.4 / 11.4 / 11.7 / 15.7 / 17.7 / 25.4; M = 4096: 37.9 / 34.0 /
// 23.1 / 28.2 / 19.7 / 27.9; M = 16384: 131.6 / 119.5 / 77.0 / 99.7 / 48.7 /
// 40.0.  Worst case against the fastest tile at each M, over N = K = 1024,
// N = 2048 K = 1024 and N = 1024 K = 2048, both B layouts: 64 x 64 2.07x
// (large M), 128 x 256 2.31x (small M), the others 2.9x and more.  On
// N = K = 2048 e5m2 (us, 32 x 256 / 128 x 256 / 256 x 256): M = 1024: 15.0 /
// 18.4 / 25.8; M = 4096: 44.4 / 23.4 / 28.8; M = 16384: 163.2 / 77.6 / 67.3.
// Bits do not depend on the tile, and these shapes are never split.
bool small_b(int64_t N, int64_t K, int eb) { return N * K * eb <= ((int64_t)4 << 20); }

bool dma_offsets_fit(int tile, int64_t N, int64_t K, int eb, bool b_trans);

// The narrow DMA tiles (64 and 32 columns) take 16-bit inputs only: their
// 256-byte K stages hold two fp8 k-steps where the fp8 schedule runs one per
// stage, and a 32-column fp8 row would be 32 bytes, below the four 16-byte
// slots the B swizzle needs.
bool is_narrow_tile(int tile) {
  return tile == GEMM_TILE_32x64 || tile == GEMM_TILE_64x64 || tile == GEMM_TILE_32x32;
}

int small_b_tile(int eb) { return eb == 2 ? GEMM_TILE_64x64 : GEMM_TILE_128x256; }

// Tile of the split-K path.  Past the K where a 128-row tile's 32-bit A
// offsets overflow, narrow shapes keep a DMA tile of 64 rows (the split,
// and so the bits, depend only on the tile's 256 columns).
int default_tile(int64_t N, int64_t K, int eb) {
  if (!reduction_dominated(N, K)) return small_b(N, K, eb) ? small_b_tile(eb) : GEMM_TILE_256x256;
  if (N > 512) return GEMM_TILE_32x128;
  return dma_offsets_fit(GEMM_TILE_128x256, N, K, eb, false) ? GEMM_TILE_128x256 : GEMM_TILE_64x256;
}

// Tile of the single pass.  Without a split, a 32-row tile only pays off
// when M is small, and the plan does not look at M: a reduction-dominated
// shape with a large M (4096 x 4096 x 8192) ran at 440 TFLOP/s with the
// 32 x 128 tile and at over 1100 with 256 x 256.  So the single pass keeps
// the large tile except for small B (as above) and narrow N (N <= 512, where
// 256 columns already cover all of N).
int default_run_tile(int64_t N, int64_t K, int eb) {
  if (small_b(N, K, eb)) return small_b_tile(eb);
  if (reduction_dominated(N, K) && N <= 512) return GEMM_TILE_64x256;
  return GEMM_TILE_256x256;
}

// GEMM_PLAN_TILE_BY_M: the DMA tile with the least estimated time.  A grid
// runs in rounds of 256 workgroups (a 256-CU MI355X), and one round of a
// tile takes about the same time whatever the shape: it is a workgroup's
// walk through K.  The narrow tiles' rings let c workgroups share a compute
// unit (c = 3 for 32x32, 2 for 32x64 and 64x64, 1 for the others), so their
// rounds come in waves of c, and a round that shares its compute units with
// the wave's first costs much less than a new wave.  Estimated time (in
// units of 0.2 us) = waves x wave cost + (rounds - waves) x shared-round
// cost, per tile and B layout, fitted on a sweep at K = 4096 (M = 1 ...
// 2048; N = 1024, 4096, 6144, 14336; both B layouts; 112 shapes, identical
// bits from every tile): there it picks the fastest tile, or one within
// 3 % of it, at 105 shapes, and one at most 11 % slower at the others.  The
// smaller tile wins a tie.  The 64- and 32-column tiles take 16-bit inputs
// only.  Bits do not depend on the tile.
int tile_by_m(int64_t M, int64_t N, int eb, bool b_trans) {
  struct Cand {
    int tile, rows, cols, per_cu;
    int wave[2], shared[2];  // [K, N] B, transposed B
  };
  static const Cand kCands[7] = {
      {GEMM_TILE_32x32, 32, 32, 3, {106, 81}, {14, 12}},
      {GEMM_TILE_32x64, 32, 64, 2, {112, 99}, {16, 19}},
      {GEMM_TILE_64x64, 64, 64, 2, {172, 156}, {14, 9}},
      {GEMM_TILE_32x256, 32, 256, 1, {219, 208}, {0, 0}},
      {GEMM_TILE_64x256, 64, 256, 1, {279, 256}, {0, 0}},
      {GEMM_TILE_128x256, 128, 256, 1, {274, 269}, {0, 0}},
      {GEMM_TILE_256x256, 256, 256, 1, {443, 429}, {0, 0}}};
  const int l = b_trans ? 1 : 0;
  int best = -1;
  int64_t best_cost = -1;
  for (int i = 0; i < 7; ++i) {
    const Cand& c = kCands[i];
    if (is_narrow_tile(c.tile) && eb != 2) continue;
    const int64_t wgs = ((M + c.rows - 1) / c.rows) * ((N + c.cols - 1) / c.cols);
    const int64_t rounds = (wgs + 255) / 256;
    const int64_t waves = (rounds + c.per_cu - 1) / c.per_cu;
    const int64_t cost = waves * c.wave[l] + (rounds - waves) * c.shared[l];
    if (best_cost < 0 || cost < best_cost) {
      best = i;
      best_cost = cost;
    }
  }
  return kCands[best].tile;
}

// GEMM_PLAN_TILE_BY_M on the split-K path of wide reduction-dominated shapes
// (K >= 2N, N > 512: the decode-like default, a 32-row tile): the tile with
// the fewest row tiles, the fewer rows on a tie.  There the time is B's
// stream, which every row tile reads again; the split (the default's, from
// N and K alone) gives every tile enough workgroups.  Measured on the decode
// shape N = 4096, K = 14336: M = 128 takes 38 us on 128 x 256 against 63 us on
// 32 x 128, M = 256 takes 54 us on 256 x 256 against 111 us; M <= 32 stays
// on the 32-row tile.  Bits do not depend on the tile.
int split_tile_by_m(int64_t M, int narrow) {
  static const int kRows[4] = {32, 64, 128, 256};
  const int tiles[4] = {narrow, GEMM_TILE_64x256, GEMM_TILE_128x256, GEMM_TILE_256x256};
  int best = 0;
  for (int i = 1; i < 4; ++i)
    if ((M + kRows[i] - 1) / kRows[i] < (M + kRows[best] - 1) / kRows[best]) best = i;
  return tiles[best];
}

bool is_dma_tile(int tile) {
  return tile == GEMM_TILE_256x256 || tile == GEMM_TILE_128x256 || tile == GEMM_TILE_32x256 ||
         tile == GEMM_TILE_64x256 || tile == GEMM_TILE_32x64 || tile == GEMM_TILE_64x64 ||
         tile == GEMM_TILE_32x32;
}


// The DMA kernels address one A tile (bm rows of K) and one B stage (128
// bytes of K, 256 on the 32x32 tile: that many / eb rows of N elements, or
// with B transposed bn rows of K) with 32-bit offsets.
bool dma_offsets_fit(int tile, int64_t N, int64_t K, int eb, bool b_trans) {
  int bm, bn, wm, wn;
  tile_shape(tile, &bm, &bn, &wm, &wn);
  const int64_t lim = ((int64_t)1 << 31) - 256;
  const int64_t stage = is_narrow_tile(tile) ? 256 : 128;
  return bm * K * eb < lim && (b_trans ? bn * K * eb < lim : stage * N < lim);
}

// A DMA tile whose offsets would overflow falls back to a register-staged
// tile of the same bits; plans that only the DMA tiles run (transposed B,
// widened fp8) get -1 instead.
int checked_tile(int tile, int64_t N, int64_t K, int eb, bool b_trans, bool dma_only) {
  if (!is_dma_tile(tile)) return dma_only ? -1 : tile;
  if (dma_offsets_fit(tile, N, K, eb, b_trans)) return tile;
  if (dma_only) return -1;
  if (tile == GEMM_TILE_256x256) return GEMM_TILE_256x256_RS;
  return (tile == GEMM_TILE_128x256 || tile == GEMM_TILE_64x64) ? GEMM_TILE_128x128
                                                                 : GEMM_TILE_32x128;
}

// Workgroups the default split aims for per row of output tiles.  Wide
// shapes: two per compute unit of a 256-CU MI355X (512).  Narrow shapes
// (N <= 512): 64, because there the row tiles multiply it and more slices
// add workspace traffic; 128 where every slice still keeps at least
// kLongSliceSteps main-loop steps.  Measured on the 128 x 256 tile (fp16,
// N = 128 / 256 / 512): at K = 131072 the larger split takes 24-28 us at
// M <= 32 against 30-35 and is level or ahead at M = 256; at K = 32768 (4- and
// 8-step slices) it lost 10-35 % at M >= 256.  Constants, not device
// queries, so a plan (and therefore the bits) never depends on the machine
// it was made on.
constexpr int64_t kLongSliceSteps = 16;
int64_t target_workgroups(int64_t N) { return N <= 512 ? 64 : 512; }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }


// Default split: only for reduction-dominated shapes; the largest power of two
// that brings one tile-row of the grid to about target_workgroups(N) while
// every slice keeps at least 4 main-loop steps; for narrow shapes, one more
// doubling if every slice still keeps kLongSliceSteps steps.
int default_split(int64_t N, int64_t K, int bn, int bk) {
  if (!reduction_dominated(N, K)) return 1;
  const int64_t tiles_n = ceil_div(N, bn);
  const int64_t steps = ceil_div(K, bk);
  const int64_t target = target_workgroups(N);
  int s = 1;
  while (s * 2 <= kMaxSplit && tiles_n * s * 2 <= target && steps / (s * 2) >= 4) s *= 2;
  if (N <= 512 && s * 2 <= kMaxSplit && tiles_n * s * 2 <= 2 * target &&
      steps / (s * 2) >= kLongSliceSteps)
    s *= 2;
  return s;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

gemm_status hip_fail(hipError_t e) {
  g_last_hip_error = (int)e;
  return GEMM_ERR_HIP;
}

// 0 if a HIP device is usable from this thread, else the HIP error.
hipError_t device_ready() {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  int n = 0;
  e = hipGetDeviceCount(&n);
  if (e != hipSuccess) return e;
  return n > 0 ? hipSuccess : hipErrorNoDevice;
}

// One operand of a call: its first byte and the bytes the kernels touch.
struct Span {
  const void* p;
  size_t bytes;
};

// True if the span lies in device memory that kernels on device `dev` may
// access: inside one allocation made on that device, or in managed memory.
// A pointer the runtime does not know (pageable host memory), host memory,
// another device's memory or a span running past the end of its allocation
// is rejected: a kernel touching it would take a memory fault.
bool on_device(const Span& s, int dev) {
  hipPointerAttribute_t at;
  if (hipPointerGetAttributes(&at, s.p) != hipSuccess) {
    (void)hipGetLastError();  // clear the lookup's error: it is not a failed call
    return false;
  }
  if (at.type == hipMemoryTypeManaged || at.isManaged) return true;
  if (at.type != hipMemoryTypeDevice || at.device != dev) return false;
  hipDeviceptr_t base = nullptr;
  size_t size = 0;
  if (hipMemGetAddressRange(&base, &size, const_cast<void*>(s.p)) != hipSuccess) {
    (void)hipGetLastError();
    return false;
  }
  const uintptr_t b = reinterpret_cast<uintptr_t>(base), q = reinterpret_cast<uintptr_t>(s.p);
  return q >= b && q - b <= size && s.bytes <= size - (q - b);
}

// After device_ready(): every span with a non-null pointer must lie in device
// memory of the current device (GEMM_ERR_INVALID_VALUE otherwise, nothing
// enqueued).
gemm_status check_device_spans(std::initializer_list<Span> spans) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e);
  for (const Span& sp : spans)
    if (sp.p && !on_device(sp, dev)) return GEMM_ERR_INVALID_VALUE;
  return GEMM_OK;
}

// The spans of a GEMM call's operands (A and B only when K > 0).
gemm_status check_gemm_spans(const gemm_plan_s* p, const void* A, const void* B, const void* C,
                             const float* bias, const void* ws, size_t ws_bytes) {
  const size_t eb = (size_t)elem_bytes(p->in);
  const size_t ob = p->out == GEMM_F32 ? 4 : 2;
  const size_t M = (size_t)p->M, N = (size_t)p->N, K = (size_t)p->K;
  return check_device_spans({{K > 0 ? A : nullptr, M * K * eb},
                             {K > 0 ? B : nullptr, K * N * eb},
                             {C, M * N * ob},
                             {bias, N * sizeof(float)},
                             {ws, ws_bytes}});
}

gemm_status check_operands(const gemm_plan_s* p, const void* A, const void* B, const void* C) {
  if (!p) return GEMM_ERR_INVALID_VALUE;
  if (p->M == 0 || p->N == 0) return GEMM_OK;
  if (!C || !aligned16(C)) return GEMM_ERR_INVALID_VALUE;
  if (p->K > 0) {
    if (!A || !B || !aligned16(A) || !aligned16(B)) return GEMM_ERR_INVALID_VALUE;
  }
  return GEMM_OK;
}

GemmArgs make_args(const gemm_plan_s* p, const void* A, const void* B, void* out, bool split) {
  GemmArgs a;
  a.A = A;
  a.B = B;
  a.C = out;
  a.bias = nullptr;
  a.M = p->M;
  a.N = p->N;
  a.K = p->K;
  a.k_per_split = split ? p->k_per_split : (p->K > 0 ? p->K : p->bk);
  a.tiles_m = split ? p->tiles_m : p->run_tiles_m;
  a.tiles_n = split ? p->tiles_n : p->run_tiles_n;
  a.grid = a.tiles_m * a.tiles_n * (split ? p->split_k : 1);
  a.group_m = p->group_m;
  a.scale = p->scale;
  return a;
}

// ---- Ozaki scheme ----------------------------------------------------------

constexpr int kOzMaxSlices = 20;  // as many as the page's split routine makes at most
// Rows per partial column maximum of B: 256, more when K is so large that
// the chunk count (the second grid dimension) would pass kOzMaxColChunks.
constexpr int64_t kOzColChunk = 256;
constexpr int64_t kOzMaxColChunks = 16384;

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
bool aligned8(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 7u) == 0; }

// Largest b with k * 4^b <= 2^m3: the bits per slice for which a k-term sum
// of slice products is exact in an accumulator of m3 bits (24: fp32, 31:
// int32); gamma = 53 - b_max of the Insight Edge blog's "分解(Split)" formula
// gamma = ceil(53 - (m3 - log2 k) / 2).
int oz_exact_bits(int64_t k, int m3) {
  if (k < 1) k = 1;
  int b = 0;
  while (b < 16 && k * ((int64_t)1 << (2 * (b + 1))) <= ((int64_t)1 << m3)) ++b;
  return b;
}

}  // namespace

namespace imm {

gemm_status record_hip_error(hipError_t e) { return hip_fail(e); }

gemm_status check_run_args(const gemm_plan_s* p, const void* A, const void* B, const void* C,
                           const float* bias) {
  gemm_status st = check_operands(p, A, B, C);
  if (st != GEMM_OK) return st;
  if (bias && !aligned4(bias)) return GEMM_ERR_INVALID_VALUE;
  return GEMM_OK;
}

gemm_status splitk_run(const gemm_plan_s* p, const void* A, const void* B, const float* bias,
                       void* C, void* workspace, size_t workspace_bytes, bool check_ws,
                       hipStream_t s) {
  gemm_status st = check_run_args(p, A, B, C, bias);
  if (st != GEMM_OK || p->M == 0 || p->N == 0) return st;
  if (!workspace || workspace_bytes < gemm_workspace_size(const_cast<gemm_plan_s*>(p)))
    return GEMM_ERR_WORKSPACE;
  if (!aligned16(workspace)) return GEMM_ERR_INVALID_VALUE;
  hipError_t e = device_ready();
  if (e != hipSuccess) return hip_fail(e);
  const size_t ws_need = gemm_workspace_size(const_cast<gemm_plan_s*>(p));
  st = check_gemm_spans(p, A, B, C, bias, check_ws ? workspace : nullptr, ws_need);
  if (st != GEMM_OK) return st;
  e = launch_gemm(*p, p->tile, make_args(p, A, B, workspace, true), true, s);
  if (e != hipSuccess) return hip_fail(e);
  ReduceArgs r;
  r.ws = static_cast<const float*>(workspace);
  r.C = C;
  r.bias = bias;
  r.MN = p->M * p->N;
  r.N = p->N;
  r.split_k = p->split_k;
  r.scale = p->scale;
  e = launch_reduce(*p, r, s);
  if (e != hipSuccess) return hip_fail(e);
  return GEMM_OK;
}

}  // namespace imm

struct ozaki_plan_s {
  int64_t M, N, K;
  int type2, eb;
  int rho, b, delta, slices, d, npairs;
  int64_t chunk;
  int64_t kp, np;
  int64_t tiles_m, tiles_n, grid;
  int64_t col_rows, col_chunks;
  size_t off_sa, off_sb, off_ea, off_eb, off_part, ws_bytes;
};

extern "C" {

gemm_status gemm_plan_ex(int64_t M, int64_t N, int64_t K, gemm_dtype in, gemm_dtype out,
                         int split_k, int group_m, float scale_a, float scale_b,
                         gemm_plan_t* plan) {
  return gemm_plan_ex2(M, N, K, in, out, split_k, group_m, GEMM_TILE_DEFAULT, scale_a, scale_b, 0,
                       plan);
}

gemm_status gemm_plan_ex2(int64_t M, int64_t N, int64_t K, gemm_dtype in, gemm_dtype out,
                          int split_k, int group_m, int tile, float scale_a, float scale_b,
                          unsigned flags, gemm_plan_t* plan) {
  if (!plan) return GEMM_ERR_INVALID_VALUE;
  *plan = nullptr;
  if (M < 0 || N < 0 || K < 0) return GEMM_ERR_INVALID_VALUE;
  if (M > INT_MAX || N > INT_MAX || K > INT_MAX) return GEMM_ERR_UNSUPPORTED;
  if (!valid_in(in) || !valid_out(out)) return GEMM_ERR_UNSUPPORTED;
  if (split_k < 0 || split_k > kMaxSplit || group_m < 0) return GEMM_ERR_UNSUPPORTED;
  if (tile < GEMM_TILE_DEFAULT || tile > GEMM_TILE_32x32) return GEMM_ERR_UNSUPPORTED;
  if (is_narrow_tile(tile) && elem_bytes(in) != 2) return GEMM_ERR_UNSUPPORTED;
  if (!std::isfinite(scale_a) || !std::isfinite(scale_b)) return GEMM_ERR_UNSUPPORTED;
  if (flags & ~(unsigned)(GEMM_PLAN_B_TRANSPOSED | GEMM_PLAN_PERSISTENT | GEMM_PLAN_TILE_BY_M |
                          GEMM_PLAN_FP8_FP32_ACCUM))
    return GEMM_ERR_UNSUPPORTED;
  const bool bt = (flags & GEMM_PLAN_B_TRANSPOSED) != 0;
  const bool f8w = (flags & GEMM_PLAN_FP8_FP32_ACCUM) != 0;
  if (f8w && in != GEMM_F8_E4M3 && in != GEMM_F8_E5M2) return GEMM_ERR_UNSUPPORTED;
  const bool dma_only = bt || f8w;
  // 16-byte vector access of every row of A and B needs K and N to be
  // multiples of 16 bytes' worth of elements.
  const int eb = elem_bytes(in);
  const int vec = 16 / eb;
  if (K % vec != 0 || N % vec != 0) return GEMM_ERR_UNSUPPORTED;

  gemm_plan_s* p = new (std::nothrow) gemm_plan_s();
  if (!p) return GEMM_ERR_INVALID_VALUE;
  p->M = M;
  p->N = N;
  p->K = K;
  p->in = in;
  p->out = out;
  p->b_trans = bt;
  p->f8_fp32 = f8w;
  p->persistent = (flags & GEMM_PLAN_PERSISTENT) != 0;
  int split_tile = tile == GEMM_TILE_DEFAULT ? default_tile(N, K, eb) : tile;
  // Transposed B and widened fp8 run on the DMA tiles only; their decode-like
  // default is the 32-row DMA tile.
  if (dma_only && tile == GEMM_TILE_DEFAULT && split_tile == GEMM_TILE_32x128)
    split_tile = GEMM_TILE_32x256;
  if (tile == GEMM_TILE_DEFAULT && (flags & GEMM_PLAN_TILE_BY_M) && reduction_dominated(N, K) &&
      N > 512) {
    // the flag never makes a plan fail: a tile whose offsets would not fit
    // (transposed B with a very long K) leaves the default in place
    const int by_m = split_tile_by_m(M, split_tile);
    if (checked_tile(by_m, N, K, eb, bt, dma_only) >= 0) split_tile = by_m;
  }
  p->tile = checked_tile(split_tile, N, K, eb, bt, dma_only);
  int run_tile = tile;
  if (tile == GEMM_TILE_DEFAULT)
    run_tile = (flags & GEMM_PLAN_TILE_BY_M) ? tile_by_m(M, N, eb, bt) : default_run_tile(N, K, eb);
  p->run_tile = checked_tile(run_tile, N, K, eb, bt, dma_only);
  if (p->tile < 0 || p->run_tile < 0) {
    delete p;
    return GEMM_ERR_UNSUPPORTED;
  }
  tile_shape(p->tile, &p->bm, &p->bn, &p->waves_m, &p->waves_n);
  tile_shape(p->run_tile, &p->run_bm, &p->run_bn, &p->run_waves_m, &p->run_waves_n);
  p->bk = block_k_elems(in);
  p->group_m = group_m == 0 ? 8 : group_m;
  const int64_t steps = ceil_div(K, p->bk);
  // The default split (which decides bits) comes from (N, K, dtype) alone:
  // it is computed for the default split-path tile of the [K, N] layout,
  // whatever tile or B layout this plan runs, so an explicit tile or a
  // transposed B never changes the bits.
  int def_bm, def_bn, def_wm, def_wn;
  tile_shape(default_tile(N, K, eb), &def_bm, &def_bn, &def_wm, &def_wn);
  int s = split_k == 0 ? default_split(N, K, def_bn, p->bk) : split_k;
  // Slices are contiguous, equal multiples of bk ([TDI] "Split-K" leaves the
  // segment boundaries open; this is the plain reading).  Drop trailing empty
  // slices so every slice has work.
  int64_t steps_per = steps > 0 ? ceil_div(steps, s) : 1;
  if (steps > 0) s = (int)ceil_div(steps, steps_per);
  p->split_k = s;
  p->k_per_split = steps_per * p->bk;
  p->tiles_m = ceil_div(M, p->bm);
  p->tiles_n = ceil_div(N, p->bn);
  p->run_tiles_m = ceil_div(M, p->run_bm);
  p->run_tiles_n = ceil_div(N, p->run_bn);
  p->scale_a = scale_a;
  p->scale_b = scale_b;
  p->scale = (float)((double)scale_a * (double)scale_b);
  const int64_t threads = (int64_t)p->waves_m * p->waves_n * 64;
  const int64_t run_threads = (int64_t)p->run_waves_m * p->run_waves_n * 64;
  if (p->tiles_m * p->tiles_n * p->split_k * threads >= ((int64_t)1 << 32) ||
      p->run_tiles_m * p->run_tiles_n * run_threads >= ((int64_t)1 << 32)) {
    delete p;
    return GEMM_ERR_UNSUPPORTED;
  }
  *plan = p;
  return GEMM_OK;
}

gemm_status gemm_plan(int64_t M, int64_t N, int64_t K, gemm_dtype in, gemm_plan_t* out) {
  const gemm_dtype od = (in == GEMM_F8_E4M3 || in == GEMM_F8_E5M2) ? GEMM_BF16 : GEMM_F32;
  return gemm_plan_ex(M, N, K, in, od, 0, 0, 1.0f, 1.0f, out);
}

gemm_status gemm_plan_info(gemm_plan_t p, gemm_plan_info_t* info) {
  if (!p || !info) return GEMM_ERR_INVALID_VALUE;
  std::memset(info, 0, sizeof(*info));
  info->M = p->M;
  info->N = p->N;
  info->K = p->K;
  info->in_dtype = p->in;
  info->out_dtype = p->out;
  info->tile = p->tile;
  info->block_m = p->bm;
  info->block_n = p->bn;
  info->block_k = p->bk;
  info->mfma_m = mfma_mn(p->in);
  info->mfma_n = mfma_mn(p->in);
  info->mfma_k = p->f8_fp32 ? 32 : mfma_k(p->in);
  info->waves = p->waves_m * p->waves_n;
  info->group_m = p->group_m;
  info->split_k = p->split_k;
  info->k_per_split = p->k_per_split;
  info->tiles_m = p->tiles_m;
  info->tiles_n = p->tiles_n;
  info->grid_run = p->run_tiles_m * p->run_tiles_n;
  info->grid_splitk = p->tiles_m * p->tiles_n * p->split_k;
  info->run_tile = p->run_tile;
  info->run_block_m = p->run_bm;
  info->run_block_n = p->run_bn;
  info->run_waves = p->run_waves_m * p->run_waves_n;
  info->run_tiles_m = p->run_tiles_m;
  info->run_tiles_n = p->run_tiles_n;
  info->workspace_bytes = gemm_workspace_size(p);
  info->scale_a = p->scale_a;
  info->scale_b = p->scale_b;
  return GEMM_OK;
}

size_t gemm_workspace_size(gemm_plan_t p) {
  if (!p) return 0;
  return (size_t)p->split_k * (size_t)p->M * (size_t)p->N * sizeof(float);
}

gemm_status gemm_plan_tile_of(gemm_plan_t p, int64_t w, int64_t* k_slice, int64_t* pid_m,
                              int64_t* pid_n) {
  if (!p || !k_slice || !pid_m || !pid_n) return GEMM_ERR_INVALID_VALUE;
  const int64_t G = p->tiles_m * p->tiles_n * p->split_k;
  if (w < 0 || w >= G) return GEMM_ERR_INVALID_VALUE;
  raster_tile(w, G, p->tiles_m, p->tiles_n, p->group_m, k_slice, pid_m, pid_n);
  return GEMM_OK;
}

gemm_status gemm_run_bias(gemm_plan_t p, const void* A, const void* B, const float* bias,
                          void* C, void* stream) {
  gemm_status st = check_operands(p, A, B, C);
  if (st != GEMM_OK || p->M == 0 || p->N == 0) return st;
  if (bias && !aligned4(bias)) return GEMM_ERR_INVALID_VALUE;
  hipError_t e = device_ready();
  if (e != hipSuccess) return hip_fail(e);
  st = check_gemm_spans(p, A, B, C, bias, nullptr, 0);
  if (st != GEMM_OK) return st;
  GemmArgs a = make_args(p, A, B, C, false);
  a.bias = bias;
  // The persistent kernel evaluates the raster in 32-bit arithmetic and
  // needs whole K stages (its transfers carry no K check); otherwise the
  // plan runs one tile per workgroup, with the same bits.
  const bool raster32 = a.grid < INT_MAX && a.group_m * a.tiles_n < INT_MAX;
  if (p->persistent && p->run_tile == GEMM_TILE_256x256 && p->K > 0 && p->K % p->bk == 0 &&
      raster32) {
    // One workgroup per compute unit (a multiple of 8, the XCD count, so
    // that every virtual workgroup stays on the XCD the raster assigns it);
    // the device query only places work, it never changes a bit.
    int dev = 0, cus = 0;
    e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return hip_fail(e);
    PersistArgs pa;
    static_cast<GemmArgs&>(pa) = a;
    const int64_t slots = cus >= 8 ? cus / 8 * 8 : 8;
    pa.wgs = a.grid < slots ? a.grid : slots;
    e = launch_gemm_persist(*p, pa, static_cast<hipStream_t>(stream));
  } else {
    e = launch_gemm(*p, p->run_tile, a, false, static_cast<hipStream_t>(stream));
  }
  if (e != hipSuccess) return hip_fail(e);
  return GEMM_OK;
}

gemm_status gemm_run(gemm_plan_t p, const void* A, const void* B, void* C, void* stream) {
  return gemm_run_bias(p, A, B, nullptr, C, stream);
}

gemm_status gemm_splitk_run(gemm_plan_t p, const void* A, const void* B, void* C,
                            void* workspace, size_t workspace_bytes, void* stream) {
  return gemm_splitk_run_bias(p, A, B, nullptr, C, workspace, workspace_bytes, stream);
}

gemm_status gemm_splitk_run_bias(gemm_plan_t p, const void* A, const void* B, const float* bias,
                                 void* C, void* workspace, size_t workspace_bytes, void* stream) {
  return imm::splitk_run(p, A, B, bias, C, workspace, workspace_bytes, true,
                         static_cast<hipStream_t>(stream));
}

void gemm_plan_destroy(gemm_plan_t p) { delete p; }

gemm_status ozaki_plan(int64_t M, int64_t N, int64_t K, gemm_dtype type2, int slices, int d,
                       int64_t chunk, ozaki_plan_t* plan) {
  if (!plan) return GEMM_ERR_INVALID_VALUE;
  *plan = nullptr;
  if (M < 0 || N < 0 || K < 0) return GEMM_ERR_INVALID_VALUE;
  if (type2 != GEMM_BF16 && type2 != GEMM_F8_E4M3 && type2 != GEMM_I8) return GEMM_ERR_UNSUPPORTED;
  if (slices < 0 || slices > kOzMaxSlices || d < 0) return GEMM_ERR_UNSUPPORTED;
  if (chunk < 0 || chunk % 128 != 0 || chunk > ((int64_t)1 << 22)) return GEMM_ERR_UNSUPPORTED;
  if (M > INT_MAX || K > INT_MAX || N >= ((int64_t)1 << 23)) return GEMM_ERR_UNSUPPORTED;
  // rho = max(gamma, xi): b = min(exact bits of one chain, bits of a Type2
  // slice entry); the default chain is the longest that keeps all of
  // Type2's bits, 2^(m_Type3 - 2 m_Type2).  int8 entries n with |n| <= 2^b
  // need b <= 6; int8 products accumulate in int32 (31 bits).
  const int m_type2 = type2 == GEMM_BF16 ? 8 : type2 == GEMM_I8 ? 6 : 4;
  const int m_type3 = type2 == GEMM_I8 ? 31 : 24;
  const int64_t kc = chunk ? chunk : ((int64_t)1 << (m_type3 - 2 * m_type2));
  const int bx = oz_exact_bits(K < kc ? K : kc, m_type3);
  const int b = bx < m_type2 ? bx : m_type2;
  if (b < 1) return GEMM_ERR_UNSUPPORTED;
  ozaki_plan_s* p = new (std::nothrow) ozaki_plan_s();
  if (!p) return GEMM_ERR_INVALID_VALUE;
  p->M = M;
  p->N = N;
  p->K = K;
  p->type2 = type2;
  p->eb = type2 == GEMM_BF16 ? 2 : 1;
  p->b = b;
  p->chunk = kc;
  p->rho = 53 - b;
  p->delta = b + 1;
  p->slices = slices ? slices : (53 + b - 1) / b;
  if (p->slices > kOzMaxSlices) p->slices = kOzMaxSlices;
  p->d = d ? d : p->slices + 2;
  int n = 0;
  for (int i = 0; i < p->slices; ++i) {
    const int c = p->d - i < p->slices ? p->d - i : p->slices;
    if (c > 0) n += c;
  }
  p->npairs = n;
  // slices padded so every row starts on 16 bytes (and fp8 rows on 16 elements)
  p->kp = (K + 15) / 16 * 16;
  p->np = (N + 15) / 16 * 16;
  p->tiles_m = ceil_div(M, oz_tile_m(type2));
  p->tiles_n = ceil_div(p->np, kOzTileN);
  p->grid = p->tiles_m * p->tiles_n;
  p->col_rows = kOzColChunk;
  if (ceil_div(K, p->col_rows) > kOzMaxColChunks) p->col_rows = ceil_div(K, kOzMaxColChunks);
  p->col_chunks = ceil_div(K, p->col_rows);
  const size_t sa = (size_t)p->slices * M * p->kp * p->eb;
  const size_t sb = (size_t)p->slices * p->kp * p->np * p->eb;
  p->off_sa = 0;
  p->off_sb = align256(sa);
  p->off_ea = p->off_sb + align256(sb);
  p->off_eb = p->off_ea + align256((size_t)M * 4);
  p->off_part = p->off_eb + align256((size_t)p->np * 4);
  p->ws_bytes = p->off_part + align256((size_t)p->col_chunks * N * 8);
  // DMA offsets of one A tile and one stage of B stay below 2^31, and so does
  // the kernel's stage count (stages per pair times pairs)
  const int64_t stages = ceil_div(p->kp, 128 / p->eb) * p->npairs;
  // the split kernels run one thread per 8 slice entries of one operand
  const int64_t split_a = ceil_div(M * p->kp, 8 * 256), split_b = ceil_div(p->kp * p->np, 8 * 256);
  const int64_t split_blocks = split_a > split_b ? split_a : split_b;
  if (oz_tile_m(type2) * p->kp * p->eb >= ((int64_t)1 << 31) - 256 ||
      p->grid * 512 >= ((int64_t)1 << 32) || stages >= ((int64_t)1 << 31) ||
      split_blocks >= ((int64_t)1 << 31)) {
    delete p;
    return GEMM_ERR_UNSUPPORTED;
  }
  *plan = p;
  return GEMM_OK;
}

gemm_status ozaki_plan_info(ozaki_plan_t p, ozaki_plan_info_t* info) {
  if (!p || !info) return GEMM_ERR_INVALID_VALUE;
  std::memset(info, 0, sizeof(*info));
  info->M = p->M;
  info->N = p->N;
  info->K = p->K;
  info->type2 = p->type2;
  info->rho = p->rho;
  info->bits = p->b;
  info->delta = p->delta;
  info->slices = p->slices;
  info->d = p->d;
  info->pairs = p->npairs;
  info->chunk = p->chunk;
  info->tile_m = oz_tile_m(p->type2);
  info->tile_n = kOzTileN;
  info->k_pad = p->kp;
  info->n_pad = p->np;
  info->grid = p->grid;
  info->workspace_bytes = p->ws_bytes;
  info->a_slices_offset = p->off_sa;
  info->b_slices_offset = p->off_sb;
  info->a_exp_offset = p->off_ea;
  info->b_exp_offset = p->off_eb;
  info->scratch_offset = p->off_part;
  return GEMM_OK;
}

size_t ozaki_workspace_size(ozaki_plan_t p) { return p ? p->ws_bytes : 0; }

namespace {

gemm_status oz_check_ws(ozaki_plan_t p, const void* ws, size_t bytes) {
  if (!ws || bytes < p->ws_bytes) return GEMM_ERR_WORKSPACE;
  if (!aligned16(ws)) return GEMM_ERR_INVALID_VALUE;
  return GEMM_OK;
}

gemm_status oz_split(ozaki_plan_t p, int operand, const double* x, void* ws, hipStream_t s) {
  char* w = static_cast<char*>(ws);
  hipError_t e;
  if (operand == 0) {
    int32_t* ea = reinterpret_cast<int32_t*>(w + p->off_ea);
    e = launch_oz_row_exp(x, p->M, p->K, ea, s);
    if (e == hipSuccess)
      e = launch_oz_split(p->type2, true, x, p->M, p->K, p->M, p->kp, ea, p->slices, p->rho,
                          p->delta, w + p->off_sa, s);
  } else {
    int32_t* eb = reinterpret_cast<int32_t*>(w + p->off_eb);
    e = launch_oz_col_exp(x, p->K, p->N, p->col_rows, reinterpret_cast<double*>(w + p->off_part),
                          eb, s);
    if (e == hipSuccess)
      e = launch_oz_split(p->type2, false, x, p->K, p->N, p->kp, p->np, eb, p->slices, p->rho,
                          p->delta, w + p->off_sb, s);
  }
  return e == hipSuccess ? GEMM_OK : hip_fail(e);
}

}  // namespace

gemm_status ozaki_split(ozaki_plan_t p, int operand, const double* x, void* ws, size_t bytes,
                        void* stream) {
  if (!p || (operand != 0 && operand != 1)) return GEMM_ERR_INVALID_VALUE;
  const int64_t n = operand == 0 ? p->M * p->K : p->K * p->N;
  if (n > 0 && (!x || !aligned8(x))) return GEMM_ERR_INVALID_VALUE;
  gemm_status st = oz_check_ws(p, ws, bytes);
  if (st != GEMM_OK) return st;
  hipError_t e = device_ready();
  if (e != hipSuccess) return hip_fail(e);
  st = check_device_spans({{n > 0 ? x : nullptr, (size_t)n * 8}, {ws, p->ws_bytes}});
  if (st != GEMM_OK) return st;
  return oz_split(p, operand, x, ws, static_cast<hipStream_t>(stream));
}

gemm_status ozaki_multiply(ozaki_plan_t p, const void* ws, size_t bytes, double* C, void* stream) {
  if (!p) return GEMM_ERR_INVALID_VALUE;
  if (p->M == 0 || p->N == 0) return GEMM_OK;
  if (!C || !aligned8(C)) return GEMM_ERR_INVALID_VALUE;
  gemm_status st = oz_check_ws(p, ws, bytes);
  if (st != GEMM_OK) return st;
  hipError_t e = device_ready();
  if (e != hipSuccess) return hip_fail(e);
  st = check_device_spans({{ws, p->ws_bytes}, {C, (size_t)p->M * p->N * 8}});
  if (st != GEMM_OK) return st;
  const char* w = static_cast<const char*>(ws);
  OzGemmArgs a;
  a.A = w + p->off_sa;
  a.B = w + p->off_sb;
  a.C = C;
  a.bias = nullptr;
  a.M = p->M;
  a.N = p->np;
  a.K = p->kp;
  a.k_per_split = p->kp;
  a.tiles_m = p->tiles_m;
  a.tiles_n = p->tiles_n;
  a.grid = p->grid;
  a.group_m = 8;
  a.scale = 1.0f;
  a.slice_a = p->M * p->kp * p->eb;
  a.slice_b = p->kp * p->np * p->eb;
  a.n_out = p->N;
  a.ldc = p->N;
  a.ea = reinterpret_cast<const int32_t*>(w + p->off_ea);
  a.eb = reinterpret_cast<const int32_t*>(w + p->off_eb);
  a.slices = p->slices;
  a.d = p->d;
  a.npairs = p->npairs;
  a.delta = p->delta;
  a.chunk_stages = (int32_t)(p->chunk / (128 / p->eb));  // 128-byte K stages
  e = launch_ozaki_gemm(p->type2, a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? GEMM_OK : hip_fail(e);
}

gemm_status ozaki_run(ozaki_plan_t p, const double* A, const double* B, double* C, void* ws,
                      size_t bytes, void* stream) {
  if (!p) return GEMM_ERR_INVALID_VALUE;
  if (p->M == 0 || p->N == 0) return GEMM_OK;
  if (!C || !aligned8(C)) return GEMM_ERR_INVALID_VALUE;
  if (p->K > 0 && (!A || !B || !aligned8(A) || !aligned8(B))) return GEMM_ERR_INVALID_VALUE;
  gemm_status st = oz_check_ws(p, ws, bytes);
  if (st != GEMM_OK) return st;
  hipError_t e = device_ready();
  if (e != hipSuccess) return hip_fail(e);
  st = check_device_spans({{p->K > 0 ? A : nullptr, (size_t)p->M * p->K * 8},
                           {p->K > 0 ? B : nullptr, (size_t)p->K * p->N * 8},
                           {C, (size_t)p->M * p->N * 8},
                           {ws, p->ws_bytes}});
  if (st != GEMM_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if ((st = oz_split(p, 0, A, ws, s)) != GEMM_OK) return st;
  if ((st = oz_split(p, 1, B, ws, s)) != GEMM_OK) return st;
  return ozaki_multiply(p, ws, bytes, C, stream);
}

void ozaki_plan_destroy(ozaki_plan_t p) { delete p; }

const char* gemm_status_string(gemm_status s) {
  switch (s) {
    case GEMM_OK: return "GEMM_OK";
    case GEMM_ERR_INVALID_VALUE: return "GEMM_ERR_INVALID_VALUE";
    case GEMM_ERR_UNSUPPORTED: return "GEMM_ERR_UNSUPPORTED";
    case GEMM_ERR_WORKSPACE: return "GEMM_ERR_WORKSPACE";
    case GEMM_ERR_HIP: return "GEMM_ERR_HIP";
    default: return "GEMM_ERR_UNKNOWN";
  }
}

int gemm_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"
