// Large-tile GEMM main loop for gfx950 fed by buffer->LDS DMA.
//
// Citations: [TDI] = Tencent engineer article on deterministic LLM inference
// ("AI インフラの深化：大規模モデルに確定的な出力を実現する方法").
//
// One workgroup of 8 waves (two per SIMD) owns a 256 x 256 tile of C (or of
// one K slice of it); each wave owns a 128 x 64 block held in 128 fp32
// accumulators per lane, as 8 x 4 blocks of 16 x 16 (the 16x16x32 matrix-core
// step for 16-bit inputs, 16x16x128 for fp8).  K is walked in ascending
// stages ([TDI] "Tiling - 分塊行列乗算": load, compute, accumulate per K step,
// one write-back at the end).  Two waves per SIMD, because a single wave serialises its own LDS and
// DMA instructions with its MFMAs while a second wave's memory instructions
// overlap the first wave's MFMAs (both measured).
//
// Memory pipeline ([TDI] "演算子チューニング": latency is hidden by
// multi-buffering rather than by occupancy).  A ring of 2 LDS stages of 128
// bytes of K per row (64 KB each: 32 KB of A, 32 KB of B) is filled by
// buffer_load ... lds: every lane moves 16 bytes straight from L2/HBM into
// LDS, no registers, no LDS-store instructions, and an out-of-range offset
// writes zeros (used for rows past M, columns past N and K past the end of
// the slice).  128-byte rows make every A request one whole cache line
// (64-byte rows, which would allow a 4-deep ring, measured slower, as did a
// 3-slot A ring beside a 2-slot B ring and L2 prefetching of later stages).
//
// LDS layouts.  A is stored K-contiguous (128 bytes per row in 16-byte
// slots, slot c of row r at c ^ ((r >> 1) & 7); the narrow tiles' 256-byte
// rows at c ^ (r & 15)), read with ds_read_b128.
// B is stored as it lies in memory, N-contiguous (512 bytes per K row for
// 16-bit, 256 for fp8), and read with the gfx950 transposing LDS reads
// (ds_read_b64_tr_b16 / _b8), which hand each lane the K-contiguous column
// piece the matrix core needs.  16-byte slot c of B row k lives at
// c ^ ((k & 3) << 2) ^ (((k >> 3) & 1) << 1) (16-bit) or c ^ ((k & 7) << 1)
// (fp8), and narrower rows by swizzles of their own (bswz below), so that
// the rows and columns each quarter-wave reads fall on different banks.  The
// swizzles are applied
// on the global side: each DMA lane fetches the chunk that belongs in its
// fixed LDS slot.
//
// Synchronisation.  Each wave waits (vmcnt) for its own DMA of the next stage,
// then one s_barrier makes every wave's data visible and certifies that every
// wave has finished reading the stage about to be refilled.  The barrier sits
// at the start of the stage's last MFMA k-step (fp8: half-way through its one
// k-step), so the refill and the fragment reads of the next stage overlap the
// remaining MFMAs.  The fp8 tiles and the 16-bit 256 x 256 tile issue their
// LDS reads in the order the next MFMAs use them, spread between MFMAs, and
// wait for exactly the reads each MFMA row needs, with one MFMA issued before
// the barrier (F8Sched, M16Sched); the other tiles spread the reads of a
// k-step evenly and wait for all of them at its start.
//
// Bits: the per-element chain is the same as in every other kernel of the
// library (same instruction per input dtype, MFMA K steps in ascending k from
// +0), so this kernel's output is bitwise identical to theirs.
#include <type_traits>

#include "kernel_common.h"

namespace imm {
namespace {
using namespace dev;

constexpr int WIDE_TBN = 256;  // tile columns of the wide tiles, the persistent and Ozaki modes

// What a workgroup does with its tile.
//   MODE_STORE: the product, scaled, converted, stored to C.
//   MODE_SLICE: the raw fp32 sum of one K slice, stored to the workspace.
//   MODE_OZAKI: the Ozaki-scheme product (Insight Edge cuTile blog, "行列積の
//     計算" and its fused kernel listing): for every slice pair (p, q) of the
//     pair list, the full K loop over slice p of A and slice q of B into the
//     fp32 accumulators; after every chunk of K (chunk_stages stages, the
//     length of an exact fp32 chain) and at the end of the pair they are
//     scaled by 2^-(p+q)*delta, added to an fp64 accumulator and cleared.  At
//     the end the row and column exponents are applied and fp64 C is stored.
//     The LDS ring runs on across pair boundaries (the stage sequence is
//     pair-major).
//   MODE_PERSIST: MODE_STORE with a grid of at most one workgroup per compute
//     unit: workgroup b computes the tiles of virtual workgroups b, b + wgs,
//     b + 2 wgs, ... of the one-tile-per-workgroup raster (the persistent
//     batch-invariant kernel of the Tencent article's closing section).  The
//     LDS ring runs on across tiles, so the next tile's first stages load
//     while the current one finishes and stores.  Each output element still
//     gets the same instruction chain from +0 in the same K order, so the
//     bits are those of MODE_STORE.
enum { MODE_STORE = 0, MODE_SLICE = 1, MODE_OZAKI = 2, MODE_PERSIST = 3 };

// Position in the Ozaki stage sequence: slice pair (p, q) -- p ascending,
// then q ascending with q < min(s, d - p) (Fast Mode skips p + q >= d) --
// and stage kt of its K pass.  Advanced one stage at a time, no divisions.
struct OzCursor {
  int p = 0, q = 0, kt = 0;
  __device__ __forceinline__ bool live(int s) const { return p < s; }
  // returns true when the step ends the pair
  __device__ __forceinline__ bool step(int ntp, int s, int d) {
    if (++kt < ntp) return false;
    kt = 0;
    if (++q >= min(s, d - p)) {
      ++p;
      q = 0;
      if (d - p <= 0) p = s;  // no pair left with p + q < d
    }
    return true;
  }
};

// Issue plan of the fp8 stage (one 16x16x128 k-step per stage, fragments
// single-buffered), for a wave tile of FM x FN blocks with RA LDS reads per A
// block, RB per B block and DPW DMA instructions per stage.  H = FN / 2.
//   Phase 1: the MFMAs (i, j < H), i-major.  After MFMA p (p < SP) the late
//     B reads [late_lo(p), late_hi(p)) of this stage: the pieces of blocks
//     j >= H, whose registers phase 2 of the previous stage freed.
//   Then MFMA (0, H), the LDS wait and the barrier (the stage change).
//   Phase 2: the MFMAs (i, j >= H), i-major.  Slot s follows its MFMA s and
//     carries DMA instructions [dma_lo(s), dma_hi(s)) of stage t + NS, the
//     early B reads [early_lo(s), early_hi(s)) of stage t + 1 (blocks j < H,
//     free since phase 1), and, at the end of a row (s % H == H - 1), the RA
//     reads of A block s / H of stage t + 1.
// LDS reads complete in issue order, so each use waits until at most the
// reads issued after the last one it needs are still in flight (capped at 15,
// the counter field, which only waits longer).
template <int FM, int FN, int RA, int RB, int DPW>
struct F8Sched {
  static constexpr int H = FN / 2;
  static constexpr int NP = FM * H;             // MFMAs per phase
  static constexpr int NB = H * RB;             // reads of half the B blocks
  static constexpr int SP = NP < 16 ? NP : 16;  // slots the spread-out work covers
  // item k of n spread over the SP slots goes to slot floor(k SP / n): slot s
  // holds items [lo(s, n), lo(s + 1, n))
  static constexpr int lo(int s, int n) { return s < SP ? (s * n + SP - 1) / SP : n; }
  static constexpr int late_lo(int p) { return lo(p, NB); }
  static constexpr int late_hi(int p) { return lo(p + 1, NB); }
  static constexpr int early_lo(int s) { return lo(s, NB); }
  static constexpr int early_hi(int s) { return lo(s + 1, NB); }
  static constexpr int dma_lo(int s) { return lo(s, DPW); }
  static constexpr int dma_hi(int s) { return lo(s + 1, DPW); }
  static constexpr bool a_at(int s) { return s % H == H - 1; }
  // LDS reads phase 2 issues in slots 0 .. s
  static constexpr int reads_thru(int s) {
    int n = 0;
    for (int u = 0; u <= s; ++u) n += early_hi(u) - early_lo(u) + (a_at(u) ? RA : 0);
    return n;
  }
  static constexpr int NR2 = reads_thru(NP - 1);
  // phase-2 issue index of the last read of A block i, of the last early read
  static constexpr int a_last(int i) { return reads_thru(i * H + H - 1) - 1; }
  static constexpr int early_last() {
    constexpr int sl = (NB - 1) * SP / NB;  // the slot of the last early read
    return (sl > 0 ? reads_thru(sl - 1) : 0) + early_hi(sl) - early_lo(sl) - 1;
  }
  static constexpr int cap(int n) { return n > 15 ? 15 : n; }
  // stage start: the early B reads and A block 0
  static constexpr int need0() { return early_last() > a_last(0) ? early_last() : a_last(0); }
  static constexpr int wait_start() { return cap(NR2 - 1 - need0()); }
  // before row i of phase 1: A block i (-1: already covered)
  static constexpr int wait_row(int i) {
    return a_last(i) <= need0() ? -1 : cap(NR2 - 1 - a_last(i) + late_lo(i * H));
  }
  // before MFMA (0, H): the late reads of block H (the first RB)
  static constexpr int wait_mid() { return cap(NB - RB); }
  // Replays the plan over one stage with in-order completion and checks that
  // every read has landed before the MFMA that first uses it.
  static constexpr bool verified() {
    // issue times: phase-2 reads of the previous stage 0 .. NR2 - 1, then the
    // late reads of this stage NR2 .. NR2 + NB - 1; `done` reads have landed
    int issued = NR2, done = 0;
    auto wait = [&](int n) {
      if (issued - done > n) done = issued - n;
    };
    wait(wait_start());
    if (early_last() >= done) return false;
    for (int p = 0; p < NP; ++p) {
      const int i = p / H;
      if (p % H == 0 && i > 0) {
        if (wait_row(i) >= 0) wait(wait_row(i));
        if (a_last(i) >= done) return false;
      }
      if (p == 0 && a_last(0) >= done) return false;
      issued += late_hi(p) - late_lo(p);
    }
    wait(wait_mid());
    return NR2 + RB - 1 < done;
  }
};

// Issue plan of the 16-bit stage: two 16x16x32 k-steps per stage on
// double-buffered fragments, FM x FN blocks per wave, RA LDS reads per A block
// and RB per B block, DPW DMA instructions per stage.  The reads of one
// k-step go out B blocks first, then A blocks 0 .. FM-1: the first row of
// MFMAs needs every B block and A block 0, row i only A block i more.
//   k-step 0: the MFMAs on F0, i-major; after MFMA p the reads
//     [lo0(p), lo0(p + 1)) of k-step 1 into F1, spread over the first SW0
//     MFMAs so that the last of them lands before the stage change.
//   Then MFMA 0 of k-step 1, the LDS wait and the barrier.
//   k-step 1: MFMAs 1 .. NM-1 on F1; slot s after MFMA s carries the DMA
//     instructions [dlo(s), dlo(s + 1)) of stage t + NS and the reads
//     [lo1(s), lo1(s + 1)) of k-step 0 of stage t + 1 into F0.
// As in F8Sched, each use waits for exactly the reads it needs.
template <int FM, int FN, int RA, int RB, int DPW>
struct M16Sched {
  static constexpr int NM = FM * FN;           // MFMAs per k-step
  static constexpr int NBR = FN * RB;          // B reads per k-step (issued first)
  static constexpr int NR = NBR + FM * RA;     // reads per k-step
  static constexpr int SW0 = NM > 4 ? NM - NM / 4 : NM;
  static constexpr int SW1 = NM - 1 > 3 ? (NM - 1) - (NM - 1) / 4 : NM - 1;
  static constexpr int spread(int s, int n, int w) { return s < w ? (s * n + w - 1) / w : n; }
  static constexpr int lo0(int p) { return spread(p, NR, SW0); }
  static constexpr int lo1(int s) { return spread(s, NR, SW1); }
  static constexpr int dlo(int s) { return spread(s, DPW, SW1); }
  static constexpr int cap(int n) { return n > 15 ? 15 : n; }
  static constexpr int a_last(int i) { return NBR + (i + 1) * RA - 1; }  // in a k-step's read order
  // start of either k-step: its B reads and A block 0 (nothing issued since)
  static constexpr int wait_start() { return cap(NR - 1 - a_last(0)); }
  // before row i of k-step 0: A block i of F0, with the F1 reads issued so far
  static constexpr int wait_row(int i) { return cap(NR - 1 - a_last(i) + lo0(i * FN)); }
  static constexpr bool verified() {
    if (SW1 < 1 || lo0(SW0) != NR || lo1(SW1) != NR || dlo(SW1) != DPW) return false;
    // k-step 0: F0's reads 0 .. NR-1 issued, then F1's NR .. 2NR-1 interleaved
    int issued = NR, done = 0;
    auto wait = [&](int n) {
      if (issued - done > n) done = issued - n;
    };
    wait(wait_start());
    if (a_last(0) >= done) return false;
    for (int p = 0; p < NM; ++p) {
      const int i = p / FN;
      if (p % FN == 0 && i > 0) {
        wait(wait_row(i));
        if (a_last(i) >= done) return false;
      }
      issued += lo0(p + 1) - lo0(p);
    }
    // k-step 1 start: F1's B reads and A block 0
    wait(wait_start());
    return NR + a_last(0) < done;
  }
};

// Bytes of K per row per stage: 128 (whole cache lines of A rows), and 256
// on the narrow tiles (64 and 32 columns, 16-bit inputs), whose small-M time
// is one workgroup's walk through K: there each stage costs a fixed latency
// (LDS waits, the barrier, the DMA wait) whatever it holds, so fewer, larger
// stages shorten the walk.
template <int TBN>
constexpr int stage_kbytes() {
  return TBN <= 64 ? 256 : 128;
}
constexpr unsigned OOB = 0x80000000u;
constexpr int NREC = 0x7fffffff;
constexpr int RSRC_FLAGS = 0x00020000;

// Fragments of one MFMA k-step of one wave: FM blocks of A (rows), FN of B.
template <int IN, int FM, int FN>
struct Frag {
  typename FragOf<IN>::type a[FM];
  typename FragOf<IN>::type b[FN];
};

// Transposing reads at a compile-time row offset (immediate field); `rows`
// is constant after unrolling, the switch folds away.
template <int BROW>
__device__ __forceinline__ i32x2 tr16_rows(unsigned p0, int rows) {
  switch (rows) {
    case 0: return ds_read_tr16_b64<0>(p0);
    case 4: return ds_read_tr16_b64<4 * BROW>(p0);
    case 16: return ds_read_tr16_b64<16 * BROW>(p0);
    case 20: return ds_read_tr16_b64<20 * BROW>(p0);
    case 32: return ds_read_tr16_b64<32 * BROW>(p0);
    case 36: return ds_read_tr16_b64<36 * BROW>(p0);
    case 48: return ds_read_tr16_b64<48 * BROW>(p0);
    case 52: return ds_read_tr16_b64<52 * BROW>(p0);
    case 64: return ds_read_tr16_b64<64 * BROW>(p0);
    case 68: return ds_read_tr16_b64<68 * BROW>(p0);
    case 96: return ds_read_tr16_b64<96 * BROW>(p0);
    default: return ds_read_tr16_b64<100 * BROW>(p0);
  }
}
// int8 steps are 32 K rows: two reads of 8 rows per half-step
template <int BROW>
__device__ __forceinline__ i32x2 tr8_rows_k32(unsigned p0, int rows) {
  switch (rows) {
    case 0: return ds_read_tr8_b64<0>(p0);
    case 8: return ds_read_tr8_b64<8 * BROW>(p0);
    case 32: return ds_read_tr8_b64<32 * BROW>(p0);
    case 40: return ds_read_tr8_b64<40 * BROW>(p0);
    case 64: return ds_read_tr8_b64<64 * BROW>(p0);
    case 72: return ds_read_tr8_b64<72 * BROW>(p0);
    case 96: return ds_read_tr8_b64<96 * BROW>(p0);
    default: return ds_read_tr8_b64<104 * BROW>(p0);
  }
}
template <int BROW>
__device__ __forceinline__ i32x2 tr8_rows(unsigned p0, int rows) {
  switch (rows) {
    case 0: return ds_read_tr8_b64<0>(p0);
    case 8: return ds_read_tr8_b64<8 * BROW>(p0);
    case 16: return ds_read_tr8_b64<16 * BROW>(p0);
    case 24: return ds_read_tr8_b64<24 * BROW>(p0);
    case 64: return ds_read_tr8_b64<64 * BROW>(p0);
    case 72: return ds_read_tr8_b64<72 * BROW>(p0);
    case 80: return ds_read_tr8_b64<80 * BROW>(p0);
    default: return ds_read_tr8_b64<88 * BROW>(p0);
  }
}

// TBM x TBN tile of C per workgroup of WM x WN waves; NS stages in the ring.
//   256 x 256, WM = 2, WN = 4, NS = 2: the large tile (wave tile 128 x 64);
//   128 x 256, WM = 2, WN = 4, NS = 3: the half-height tile (wave tile
//     64 x 64) for grids that 256 x 256 tiles would leave under-filled;
//   64 x 256 / 32 x 256, WM = 1, WN = 4, NS = 4: short tiles for
//     reduction-dominated shapes (wave tile 64 x 64 / 32 x 64), where the time
//     is the stream of B;
//   64 x 64 / 32 x 64 / 32 x 32, WM = 2, WN = 1, NS = 2 / 3 / 3, with 256-byte
//     K stages: narrow tiles (16-bit inputs) for small M, where N / 256
//     column tiles would leave most compute units idle.  A workgroup's
//     stream of B runs at a rate of its own (about 20 GB/s on the 64-column
//     tiles with 128-byte stages, whatever the grid), so at small M the time
//     is one workgroup's walk through K, which fewer, larger stages and more,
//     narrower column tiles shorten.  Their rings (64, 72 and 48 KB) let two,
//     two and three workgroups share a compute unit, which gains more at
//     mid M than deeper rings gain at M = 1 (measured against 128-byte
//     stages with 6-10 stage rings: the 64 x 64 tile at M = 1 / 256 on the
//     fused-QKV shape 39.9 / 76.2 us before, 30.1 / 35.7 after).
// Two workgroups share a CU when their rings fit in half the LDS; the
// register budget then has to allow two waves per SIMD.  A four-wave
// workgroup alone on its CU has one wave per SIMD and the whole register file.
template <int TBM, int TBN, int WM, int WN, int NS>
constexpr int waves_per_simd() {
  return WM * WN == 4 && NS * (TBM + TBN) * stage_kbytes<TBN>() > 80 * 1024 ? 1 : 2;
}

// BT: B is given transposed, as [N, K] row-major (the weight layout of a
// linear layer).  Its rows are then K-contiguous like those of A, so B is
// staged and read exactly like A (128-byte rows, ds_read_b128); the matrix
// core sees the same values in the same K order, so the bits are those of
// the [K, N] layout.
template <int IN, int OUT, int MODE, int TBM, int TBN, int WM, int WN, int NS, bool BT, class ARGS>
__global__ __launch_bounds__(WM * WN * 64, (waves_per_simd<TBM, TBN, WM, WN, NS>())) void gemm_dma_kernel(ARGS g) {
  using T = InT<IN>;
  constexpr int EB = T::EB;
  constexpr int WAVES = WM * WN;
  constexpr int WTM = TBM / WM;              // wave tile rows
  constexpr int WTN = TBN / WN;              // wave tile columns
  // 16-bit inputs: the 16x16x32 step; fp8: the 16x16x128 step; int8 and the
  // exact Ozaki chains (whose bits no instruction changes): the 32x32 step
  constexpr bool M16 = EB == 2 && MODE != MODE_OZAKI;
  // fp8 data widened to fp16 in registers (GEMM_PLAN_FP8_FP32_ACCUM): the
  // 16x16x32 fp16 step over the fp8 LDS layout, 8 bytes of K per lane
  constexpr bool W16 = T::W16;
  static_assert(!W16 || MODE != MODE_OZAKI, "widened fp8 in an Ozaki pass");
  constexpr bool F8S = EB == 1 && !T::I8 && !W16 && MODE != MODE_OZAKI;
  constexpr bool B16 = M16 || F8S || W16;    // 16 x 16 output blocks
  constexpr int BLK = B16 ? 16 : 32;         // MFMA output block edge
  constexpr int NACC = BLK * BLK / 64;       // accumulators per lane per block
  using AccT = typename std::conditional<B16, f32x4, f32x16>::type;
  constexpr int KSTEP = F8S ? 128 : (M16 ? 64 : (W16 ? 32 : T::KSTEP_B));  // bytes of K per MFMA step
  constexpr int FM = WTM / BLK;              // MFMA row blocks per wave
  constexpr int FN = WTN / BLK;              // MFMA column blocks per wave
  constexpr int NM = FM * FN;                // MFMAs per k-step per wave
  constexpr int SKB = stage_kbytes<TBN>();   // bytes of K per row per stage
  static_assert(SKB == 128 || (EB == 2 && !T::I8 && !W16 && MODE != MODE_OZAKI), "256-byte stages");
  constexpr int A_STAGE = TBM * SKB;         // bytes of A per stage
  constexpr int B_STAGE = TBN * SKB;         // bytes of B per stage (32 KB)
  constexpr int STAGE = A_STAGE + B_STAGE;
  constexpr int BKE = SKB / EB;              // K elements (= B rows) per stage
  constexpr int KS = SKB / KSTEP;           // MFMA k-steps per stage
  constexpr int ACH = SKB / 16;              // 16-byte slots per A row
  constexpr int AROWS_PER_DMA = 1024 / SKB;  // A rows written by one DMA instruction
  constexpr int BROW = TBN * EB;             // bytes per B row in LDS
  constexpr int BSLOTS = BROW / 16;
  constexpr int BROWS_PER_DMA = 1024 / BROW; // B rows written by one DMA instruction
  constexpr int DA = A_STAGE / 1024 / WAVES; // DMA instructions per wave per stage: A ...
  constexpr int DB = B_STAGE / 1024 / WAVES; // ... and B
  constexpr int DPW = DA + DB;
  static_assert(DA * WAVES * 1024 == A_STAGE && DB * WAVES * 1024 == B_STAGE, "DMA split");
  static_assert(FM * BLK * WM == TBM, "tile rows");
  constexpr bool I8 = T::I8;                 // int8: 16-bit-like A reads, 8-bit B reads
  constexpr int NRA = (T::FRAG == 1 || W16) ? FM : 2 * FM;  // fragment reads per k-step: A ...
  constexpr int NRB = W16 ? FN : BT ? (T::FRAG == 1 ? FN : 2 * FN) : (EB == 2 || I8 ? 2 * FN : 4 * FN);  // ... B
  constexpr int NREAD = NRA + NRB;
  constexpr int LDS_BYTES = NS * STAGE;
  static_assert(LDS_BYTES <= 160 * 1024, "LDS ring too large");
  // fp8 (one 128-byte k-step per stage): single-buffered fragments; the
  // other paths alternate two fragment sets over an even number of k-steps
  static_assert(F8S ? KS == 1 : KS % 2 == 0, "k-steps per stage");
  // wave tiles are 64 columns wide (a 128-wide fp8 wave tile, one wave per
  // SIMD on the 256 x 256 tile, compiles too but measured 6-13 % slower);
  // the 32-column tile of 16-bit inputs has 32-column wave tiles
  static_assert(WN * WTN == TBN && (WTN == 64 || (WTN == 32 && EB == 2 && !T::I8)), "wave tile width");

  __shared__ __attribute__((aligned(1024))) char lds[LDS_BYTES];
  // LDS offsets of the A and B blocks of stage t.
  auto a_slot = [](int t) { return (t % NS) * STAGE; };
  auto b_slot = [](int t) { return (t % NS) * STAGE + A_STAGE; };

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index (uniform)
  const int wm = w / WN, wn = w % WN;
  const int lb = lane % BLK, hq = lane / BLK;  // row / column in the MFMA block, K piece

  int64_t ksl, pm, pn;
  raster_tile(blockIdx.x, g.grid, g.tiles_m, g.tiles_n, g.group_m, &ksl, &pm, &pn);
  const int64_t m0 = pm * TBM, n0 = pn * TBN;  // first (MODE_PERSIST) or only tile
  const int64_t kbeg = ksl * g.k_per_split;
  const int64_t kend = (g.K < kbeg + g.k_per_split) ? g.K : kbeg + g.k_per_split;
  // stages of one K pass; the Ozaki mode makes one pass per slice pair
  const int ntp = kend > kbeg ? (int)((kend - kbeg + BKE - 1) / BKE) : 0;
  int nt = ntp;
  if constexpr (MODE == MODE_OZAKI) nt = ntp * g.npairs;
  // tiles of this workgroup (MODE_PERSIST): virtual ids blockIdx.x + j * wgs
  int ntiles = 1;
  if constexpr (MODE == MODE_PERSIST) {
    ntiles = (int)((g.grid - blockIdx.x + g.wgs - 1) / g.wgs);
    nt = ntp * ntiles;
  }
  // origin of tile j of this workgroup
  auto tile_origin = [&](int j, int64_t* tm0, int64_t* tn0) {
    if constexpr (MODE == MODE_PERSIST) {
      uint32_t pm_, pn_;
      raster_tile32(blockIdx.x + (uint32_t)j * (uint32_t)g.wgs, (uint32_t)g.grid,
                    (uint32_t)g.tiles_m, (uint32_t)g.tiles_n, (uint32_t)g.group_m, &pm_, &pn_);
      *tm0 = (int64_t)pm_ * TBM;
      *tn0 = (int64_t)pn_ * TBN;
    }
  };
  const char* A = static_cast<const char*>(g.A);
  const char* B = static_cast<const char*>(g.B);

  // A row r keeps its 16-byte slot c at c ^ aswz(r): 128-byte rows put rows
  // r and r + 2 on the same banks, 256-byte rows every row, so the 16 rows a
  // quarter-wave reads take 8 or 16 different slots.
  auto aswz = [](int r) {
    if constexpr (SKB == 256) return r & 15;
    else return (r >> 1) & 7;
  };
  // B row k (the [K, N] layout) keeps its 16-byte slot c at c ^ bswz(k): a
  // bijection of the row's BSLOTS slots, chosen so that the K rows one
  // transposing read gathers lie on different banks.  A lane's transposing
  // reads of one stage reach rows k + (row offset) through the instruction's
  // immediate offset, with the slot computed once for row k, so bswz may only
  // use bits of k that those offsets never change: 16-bit inputs add 4 r and
  // 32 ks to k = 8 grp + t (t < 4), leaving bits 0, 1, 3 and 4; fp8 adds
  // 8 r and 64 ks to k = 32 h + t (t < 8), leaving bits 0 - 2 and 5; int8
  // adds 8, 32 and 64 multiples to k = 16 h + t, leaving bits 0 - 2 and 4.
  auto bswz = [](int k) {
    if constexpr (EB == 2) {
      if constexpr (BSLOTS >= 16) return ((k & 3) << 2) ^ (((k >> 3) & 1) << 1);
      else if constexpr (BSLOTS == 8) return ((k & 3) << 1) ^ ((k >> 3) & 1);
      // 64-byte rows (32 columns): rows k and k + 8 of one half-wave's read
      // share banks unless their two slots are swapped over
      else return ((k >> 3) & 1) << 1;
    } else {
      if constexpr (BSLOTS >= 16) return (k & 7) << 1;
      else if constexpr (BSLOTS == 8) return k & 7;
      else return (k & 3) ^ ((k >> 2) & 1);
    }
  };
  static_assert(BSLOTS >= 4, "B row of at least four 16-byte slots");

  // ---- DMA geometry of this lane (the same for every stage).  Offsets of
  // rows past M / columns past N are replaced by an out-of-range offset once;
  // the K check only matters in a partial stage.  MODE_PERSIST changes tiles,
  // so there the row / column checks are made per transfer, against bit
  // masks of the stage's tile (tile_masks).
  constexpr bool PER_TILE = MODE == MODE_PERSIST;
  unsigned a_off[DA], b_off[DB];
  int a_kel[DA], b_k[DB];
#pragma unroll
  for (int i = 0; i < DA; ++i) {
    const int idx = w * DA + i;
    const int row = AROWS_PER_DMA * idx + lane / ACH;
    const int c = (lane % ACH) ^ aswz(row);
    a_off[i] = (PER_TILE || m0 + row < g.M) ? (unsigned)(row * g.K * EB + c * 16) : OOB;
    a_kel[i] = c * (16 / EB);
  }
#pragma unroll
  for (int i = 0; i < DB; ++i) {
    const int idx = w * DB + i;
    if constexpr (BT) {
      // row n of B^T (column n of B), laid out like a row of A
      const int row = AROWS_PER_DMA * idx + lane / ACH;
      const int c = (lane % ACH) ^ aswz(row);
      b_off[i] = (PER_TILE || n0 + row < g.N) ? (unsigned)(row * g.K * EB + c * 16) : OOB;
      b_k[i] = c * (16 / EB);  // first K element of the chunk
    } else {
      const int k = BROWS_PER_DMA * idx + lane / BSLOTS;
      const int s = lane % BSLOTS;
      const int cb = s ^ bswz(k);
      b_off[i] = (PER_TILE || n0 + cb * (16 / EB) < g.N) ? (unsigned)(k * g.N * EB + cb * 16) : OOB;
      b_k[i] = k;  // K row of the chunk
    }
  }
  // MODE_PERSIST: bit i set if this lane's A (B) transfer i of a stage of the
  // tile at (tm0, tn0) lies inside M (N); recomputed from the lane index once
  // per tile, so no per-transfer row or column is kept in registers.
  auto tile_masks = [&](int64_t tm0, int64_t tn0, unsigned* am, unsigned* bm) {
    *am = 0;
    *bm = 0;
#pragma unroll
    for (int i = 0; i < DA; ++i) {
      const int row = AROWS_PER_DMA * (w * DA + i) + lane / ACH;
      *am |= (unsigned)(tm0 + row < g.M) << i;
    }
#pragma unroll
    for (int i = 0; i < DB; ++i) {
      int col;
      if constexpr (BT) {
        col = AROWS_PER_DMA * (w * DB + i) + lane / ACH;
      } else {
        const int k = BROWS_PER_DMA * (w * DB + i) + lane / BSLOTS;
        const int sl = lane % BSLOTS;
        col = (sl ^ bswz(k)) * (16 / EB);
      }
      *bm |= (unsigned)(tn0 + col < g.N) << i;
    }
  };

  struct StageSrc {
    const char* pa;  // first byte of the stage's A block (row m0)
    const char* pb;  // first byte of the stage's B block (column n0)
    int rem;         // K elements of this stage inside the slice (BKE for a full stage)
    unsigned amask, bmask;  // MODE_PERSIST: transfers inside M / N (tile_masks)
  };
  auto stage_src = [&](int t) {
    StageSrc q;
    const int64_t kst = kbeg + (int64_t)t * BKE;
    q.pa = A + (m0 * g.K + kst) * EB;
    q.pb = BT ? B + (n0 * g.K + kst) * EB : B + (kst * g.N + n0) * EB;
    q.rem = kend - kst < BKE ? (int)(kend - kst) : BKE;
    return q;
  };
  // Ozaki and persistent modes: the stages are requested strictly in
  // sequence (prologue, then one refill per stage), so the source of the next
  // one comes from a cursor; past the last pair / tile it is a zero fill.
  OzCursor pf;
  int pf_tile = 0, pf_kt = 0;
  int64_t pf_m0 = m0, pf_n0 = n0;
  unsigned pf_am = 0, pf_bm = 0;
  if constexpr (PER_TILE) tile_masks(m0, n0, &pf_am, &pf_bm);
  auto next_src = [&]() {
    StageSrc q;
    q.pa = A;
    q.pb = B;
    q.rem = 0;
    q.amask = 0;
    q.bmask = 0;
    if constexpr (MODE == MODE_PERSIST) {
      if (pf_tile < ntiles) {
        const int64_t kst = (int64_t)pf_kt * BKE;
        q.pa = A + (pf_m0 * g.K + kst) * EB;
        q.pb = BT ? B + (pf_n0 * g.K + kst) * EB : B + (kst * g.N + pf_n0) * EB;
        q.rem = g.K - kst < BKE ? (int)(g.K - kst) : BKE;
        q.amask = pf_am;
        q.bmask = pf_bm;
        if (++pf_kt == ntp) {
          pf_kt = 0;
          if (++pf_tile < ntiles) {
            tile_origin(pf_tile, &pf_m0, &pf_n0);
            tile_masks(pf_m0, pf_n0, &pf_am, &pf_bm);
          }
        }
      }
    }
    if constexpr (MODE == MODE_OZAKI) {
      if (pf.live(g.slices)) {
        const int64_t kst = (int64_t)pf.kt * BKE;
        q.pa = A + pf.p * g.slice_a + (m0 * g.K + kst) * EB;
        q.pb = B + pf.q * g.slice_b + (kst * g.N + n0) * EB;
        q.rem = g.K - kst < BKE ? (int)(g.K - kst) : BKE;
        pf.step(ntp, g.slices, g.d);
      }
    }
    return q;
  };
  // DMA instruction x of this wave for stage t (source q): x < DA: A rows,
  // else B rows.
  auto dma_one = [&](const StageSrc& q, int t, int x) {
    if (x < DA) {
      // MODE_PERSIST runs only where K is a multiple of the stage (every stage
      // is whole) and past the last tile the masks are clear: the masks
      // alone decide.
      bool ok;
      if constexpr (PER_TILE)
        ok = (q.amask >> x) & 1u;
      else
        ok = a_kel[x] < q.rem;
      const unsigned off = ok ? a_off[x] : OOB;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          __builtin_amdgcn_make_buffer_rsrc((void*)q.pa, 0, NREC, RSRC_FLAGS),
          IMM_LDS(lds + a_slot(t) + (w * DA + x) * 1024), 16, off, 0, 0, 0);
    } else {
      const int i = x - DA;
      bool ok;
      if constexpr (PER_TILE)
        ok = (q.bmask >> i) & 1u;
      else
        ok = b_k[i] < q.rem;
      const unsigned off = ok ? b_off[i] : OOB;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          __builtin_amdgcn_make_buffer_rsrc((void*)q.pb, 0, NREC, RSRC_FLAGS),
          IMM_LDS(lds + b_slot(t) + (w * DB + i) * 1024), 16, off, 0, 0, 0);
    }
  };

  // ---- fragment read offsets within a stage.
  const int asw = aswz(lb);  // rows of a fragment differ from lb by multiples of 16
  int a_rd[FM];
#pragma unroll
  for (int i = 0; i < FM; ++i) a_rd[i] = (wm * WTM + i * BLK + lb) * SKB;
  const int grp = lane >> 4, gi = lane & 15;
  int b_rd[FN];  // per column block j: byte offset of its first read
  if constexpr (BT) {
#pragma unroll
    for (int j = 0; j < FN; ++j) b_rd[j] = (wn * WTN + j * BLK + lb) * SKB;
  } else if constexpr (EB == 2) {
    // each group of 16 lanes reads 4 K rows x 16 columns per transposing read:
    // 16x16 blocks, the column block and K rows 8 grp ..; 32x32 blocks, column
    // half grp & 1 and K rows 8 (grp >> 1) ..
    const int t_ = gi >> 2, q = gi & 3;
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int n = M16 ? wn * WTN + j * 16 + 4 * q : wn * WTN + j * 32 + 16 * (grp & 1) + 4 * q;
      const int k = (M16 ? 8 * grp : 8 * (grp >> 1)) + t_;
      b_rd[j] = k * BROW + (((n >> 3) ^ bswz(k)) << 4) + (q & 1) * 8;
    }
  } else {
    // each group of 16 lanes reads 8 K rows x 16 columns per transposing read:
    // 16x16 blocks (fp8), the column block and K rows 32 grp ..; 32x32 blocks,
    // column half grp & 1 and K rows 32 (grp >> 1) .. (16 for int8)
    // (widened fp8: the column block and K rows 8 grp .., one read per k-step)
    const int t_ = gi >> 1, q = gi & 1;
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int n = (F8S || W16) ? wn * WTN + j * 16 + 8 * q : wn * WTN + j * 32 + 16 * (grp & 1) + 8 * q;
      const int k = F8S ? 32 * grp + t_ : W16 ? 8 * grp + t_ : (I8 ? 16 : 32) * (grp >> 1) + t_;
      b_rd[j] = k * BROW + (((n >> 4) ^ bswz(k)) << 4) + q * 8;
    }
  }

  // LDS byte address of the ring (for the transposing reads).
  const unsigned lds_addr = (unsigned)(uintptr_t)((__attribute__((address_space(3))) char*)lds);

  // Fragment read x of k-step ks of the stage whose A and B blocks sit at LDS
  // offsets as and bs, into F.
  //   16-bit: x < FM -> A block i = x (one ds_read_b128);
  //           else B block j = (x-FM)/2, half r = (x-FM)%2 (K elements 4r..4r+3).
  //   fp8:    x < 2FM -> A block i = x/2, half x%2 (16 bytes of K each);
  //           else B block j = (x-2FM)/4, piece r = (x-2FM)%4 (8 K values).
  //   B given transposed: B block j is read like an A block (x-NRA = j for
  //   16-bit, 2j + half for fp8).
  auto read_one = [&](Frag<IN, FM, FN>& F, int as, int bs, int ks, int x) {
    const char* sb = lds + as;
    if constexpr (W16) {
      // widened fp8: 8 bytes of K (32 ks + 8 hq ..) per lane and block, A and
      // B^T rows by plain 8-byte reads, B by one 8-row transposing read
      const int c = 2 * ks + (hq >> 1), h = (hq & 1) * 8;
      if (x < NRA) {
        F.a[x] = *reinterpret_cast<const i32x2*>(sb + a_rd[x] + ((c ^ asw) << 4) + h);
      } else if constexpr (BT) {
        const int j = x - NRA;
        F.b[j] = *reinterpret_cast<const i32x2*>(lds + bs + b_rd[j] + ((c ^ asw) << 4) + h);
      } else {
        const int j = x - NRA;
        F.b[j] = tr8_rows_k32<BROW>(lds_addr + bs + b_rd[j], 32 * ks);
      }
      return;
    }
    if constexpr (I8 && !BT) {
      // int8: A as for 16-bit inputs (one 16-byte slot per k-step half), B by
      // two 8-bit transposing reads of 8 K rows each.
      if (x < NRA) {
        const int c = ks * 2 + hq;
        F.a[x] = *reinterpret_cast<const i32x4*>(sb + a_rd[x] + ((c ^ asw) << 4));
      } else {
        const int j = (x - NRA) >> 1, r = (x - NRA) & 1;
        const i32x2 v = tr8_rows_k32<BROW>(lds_addr + bs + b_rd[j], ks * 32 + 8 * r);
        F.b[j][2 * r] = v[0];
        F.b[j][2 * r + 1] = v[1];
      }
      return;
    }
    if constexpr (BT) {
      if (x >= NRA) {
        const char* sbb = lds + bs;
        if constexpr (EB == 2) {
          const int j = x - NRA, c = ks * (KSTEP / 16) + hq;
          F.b[j] = *reinterpret_cast<const i32x4*>(sbb + b_rd[j] + ((c ^ asw) << 4));
        } else {
          const int j = (x - NRA) >> 1, f = (x - NRA) & 1;
          const int c = ks * (KSTEP / 16) + 2 * hq + f;
          const i32x4 v = *reinterpret_cast<const i32x4*>(sbb + b_rd[j] + ((c ^ asw) << 4));
#pragma unroll
          for (int e = 0; e < 4; ++e) F.b[j][4 * f + e] = v[e];
        }
        return;
      }
    }
    if constexpr (EB == 2) {
      if (x < NRA) {
        const int c = ks * (KSTEP / 16) + hq;
        F.a[x] = *reinterpret_cast<const i32x4*>(sb + a_rd[x] + ((c ^ asw) << 4));
      } else {
        const int j = (x - NRA) >> 1, r = (x - NRA) & 1;
        const i32x2 v = tr16_rows<BROW>(lds_addr + bs + b_rd[j], ks * (KSTEP / 2) + 4 * r);
        F.b[j][2 * r] = v[0];
        F.b[j][2 * r + 1] = v[1];
      }
    } else {
      if (x < NRA) {
        const int i = x >> 1, f = x & 1;
        const int c = ks * (KSTEP / 16) + 2 * hq + f;
        const i32x4 v = *reinterpret_cast<const i32x4*>(sb + a_rd[i] + ((c ^ asw) << 4));
#pragma unroll
        for (int e = 0; e < 4; ++e) F.a[i][4 * f + e] = v[e];
      } else {
        const int j = (x - NRA) >> 2, r = (x - NRA) & 3;
        const i32x2 v = tr8_rows<BROW>(lds_addr + bs + b_rd[j], ks * KSTEP + 8 * r);
        F.b[j][2 * r] = v[0];
        F.b[j][2 * r + 1] = v[1];
      }
    }
  };

  // The B fragments come from inline-assembly reads the compiler does not
  // track, so MFMAs that use freshly read fragments are preceded by an
  // explicit lgkmcnt(0) wait, fenced with sched_barrier.
  auto fence = [&]() { __builtin_amdgcn_sched_barrier(0); };
  auto lds_wait = [&]() {
    fence();
    __builtin_amdgcn_s_waitcnt(lgkmcnt_imm(0));
    fence();
  };
  // wait until at most N LDS reads are in flight (N a compile-time constant)
  auto lgkm_wait = [&](auto N) {
    fence();
    __builtin_amdgcn_s_waitcnt(lgkmcnt_imm(decltype(N)::value));
    fence();
  };

  AccT acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = AccT{};
  // widened fp8: the fp16 operands of the current A row block and of every B
  // block, widened at first use (after the k-step's LDS wait)
  i32x4 w16_a, w16_b[FN];
  auto mfma_x = [&](const Frag<IN, FM, FN>& F, int x) {
    if constexpr (W16) {
      const int i = x / FN, j = x % FN;
      if (j == 0) w16_a = widen_f8<T::F8>(F.a[i]);
      if (i == 0) w16_b[j] = widen_f8<T::F8>(F.b[j]);
      acc[i][j] = mfma16_v<GEMM_F16>(w16_a, w16_b[j], acc[i][j]);
    } else if constexpr (M16)
      acc[x / FN][x % FN] = mfma16_v<IN>(F.a[x / FN], F.b[x % FN], acc[x / FN][x % FN]);
    else if constexpr (F8S)
      acc[x / FN][x % FN] = mfma16_f8<IN>(F.a[x / FN], F.b[x % FN], acc[x / FN][x % FN]);
    else
      acc[x / FN][x % FN] = mfma_v<IN>(F.a[x / FN], F.b[x % FN], acc[x / FN][x % FN]);
  };
  // Ozaki mode: fp64 sum over the slice pairs (dead code otherwise).
  double acc64[FM][FN][16];
  if constexpr (MODE == MODE_OZAKI) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc64[i][j][r] = 0.0;
  }
  // End of a chunk of the slice pair at level p + q: its exact fp32 sums,
  // scaled by 2^-(p+q)*delta, join the fp64 sum in (pair, chunk) order; the
  // fp32 accumulators restart from +0.
  auto oz_flush = [&](int level) {
    if constexpr (MODE == MODE_OZAKI) {
      // int8 slices hold the integers n of the entries n * 2^-b, so their
      // int32 sums carry a further 2^-2b (b = delta - 1)
      const int sh = -level * g.delta - (I8 ? 2 * (g.delta - 1) : 0);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            // int8 slices accumulate in int32, held in the registers' bits (the
            // element is copied out first: a bit cast of a vector element
            // expression reads the vector's first element)
            const float f = acc[i][j][r];
            const double v = I8 ? (double)__float_as_int(f) : (double)f;
            acc64[i][j][r] += ldexp(v, sh);
          }
          acc[i][j] = AccT{};
        }
    }
  };

  // Write-back of the tile at (tm0, tn0).  Accumulator layouts: 16x16 blocks,
  // lane l, register r holds row 4*(l/16) + r, column l%16 of the block; 32x32
  // blocks, row 8*(r/4) + 4*(l/32) + r%4, column l%32.
  auto store_tile = [&](int64_t tm0, int64_t tn0) {
    // Inside the stage loop (MODE_PERSIST) the per-element offsets below are
    // loop-invariant; opaque lane bases keep the compiler from hoisting them
    // out of the loop (where they would sit in registers or scratch).
    int lrow = wm * WTM + 4 * hq, lcol = wn * WTN + lb;
    if constexpr (PER_TILE) asm volatile("" : "+v"(lrow), "+v"(lcol));
    if constexpr (MODE != MODE_OZAKI) {
      // A tile wholly inside C whose byte offsets from its first element fit
      // in 31 bits: every element is a uniform row address plus one 32-bit
      // offset per lane (plus a constant), with no bounds checks.  The
      // values, and the order of operations that makes them, are those of
      // the general path below.  (Transposing 4 x 4 pieces within quads of
      // lanes, for one 8- or 16-byte store per four elements, measured
      // slower: the exchanges cost more than the stores they save.)
      constexpr int OB = (MODE == MODE_SLICE || OUT == GEMM_F32) ? 4 : 2;
      if (tm0 + TBM <= g.M && tn0 + TBN <= g.N && g.N * (TBM * OB) < (int64_t(1) << 31)) {
        const int64_t row0 = MODE == MODE_SLICE ? ksl * g.M + tm0 : tm0;
        char* const base = static_cast<char*>(g.C) + (row0 * g.N + tn0) * OB;
        const unsigned loff = (unsigned)(lrow * (int)g.N + lcol) * OB;
        auto body = [&](auto plain) {
#pragma clang fp contract(off)
          float bv[FN];
          if constexpr (!decltype(plain)::value) {
#pragma unroll
            for (int j = 0; j < FN; ++j) bv[j] = g.bias ? g.bias[tn0 + lcol + j * BLK] : 0.0f;
          }
#pragma unroll
          for (int i = 0; i < FM; ++i) {
#pragma unroll
            for (int r = 0; r < NACC; ++r) {
              const int rr = i * BLK + (B16 ? r : 8 * (r >> 2) + (r & 3));
              char* const rb = base + (int64_t)rr * g.N * OB;
#pragma unroll
              for (int j = 0; j < FN; ++j) {
                float v = acc[i][j][r];
                if constexpr (!decltype(plain)::value) {
                  v = g.scale == 1.0f ? v : v * g.scale;
                  if (g.bias) v = v + bv[j];
                }
                char* const p = rb + j * BLK * OB + loff;
                if constexpr (MODE == MODE_SLICE)
                  *reinterpret_cast<float*>(p) = v;
                else
                  store_at<OUT>(p, v);
              }
            }
          }
        };
        if (MODE == MODE_SLICE || (g.scale == 1.0f && !g.bias))
          body(std::true_type{});
        else if constexpr (MODE != MODE_SLICE)
          body(std::false_type{});
        return;
      }
    }
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int64_t col = tn0 + lcol + j * BLK;
#pragma unroll
        for (int r = 0; r < NACC; ++r) {
          const int64_t row = tm0 + lrow + i * BLK + (B16 ? r : 8 * (r >> 2) + (r & 3));
          if constexpr (MODE == MODE_OZAKI) {
            // C = 2^(ea[row] + eb[col]) * sum: the same bits as scaling every
            // pair's term by its full exponent while no value leaves fp64's
            // normal range; NaN where the row or the column is outside it
            if (row < g.M && col < g.n_out) {
              const int er = g.ea[row], ec = g.eb[col];
              static_cast<double*>(g.C)[row * g.ldc + col] =
                  (er == kOzBadExp || ec == kOzBadExp) ? __builtin_nan("")
                                                       : ldexp(acc64[i][j][r], er + ec);
            }
          } else if (row < g.M && col < g.N) {
            const float v = acc[i][j][r];
            if constexpr (MODE == MODE_SLICE) {
              static_cast<float*>(g.C)[(ksl * g.M + row) * g.N + col] = v;
            } else {
              store_final<OUT>(g.C, row * g.N + col, v, g.scale, g.bias, col);
            }
          }
        }
      }
    }
  };

  // Issue order.  Stages are requested whole (A rows, then B rows) in
  // ascending stage index: the prologue requests stages 0 .. NS-1, every
  // refill stage t+NS.  Before stage t+1 is used, the NS - 2 stages after it
  // may still be in flight.  DMA is issued for every stage index (past the
  // end of the slice it only writes zeros), so these counts never change.
  constexpr int WAIT_FIRST = (NS - 1) * DPW;
  constexpr int WAIT_NEXT = (NS - 2) * DPW;
  Frag<IN, FM, FN> F0, F1;

  // fp8: fragment reads with compile-time block indices, so that the block
  // offsets are immediates and every wait is placed by the schedule
  // (F8Sched).  A (and B given transposed) rows: two 16-byte halves per lane
  // at f8_row[f] + (block row) * SKB; B in the [K, N] layout: four
  // transposing reads of 8 K rows per block.
  constexpr int RA8 = F8S ? NRA / FM : 1, RB8 = F8S ? NRB / FN : 1;
  unsigned f8_arow[2], f8_brow[2];
#pragma unroll
  for (int f = 0; f < 2; ++f) {
    const unsigned sl = (unsigned)((((2 * hq + f) ^ asw) << 4));
    f8_arow[f] = lds_addr + (unsigned)((wm * WTM + lb) * SKB) + sl;
    f8_brow[f] = lds_addr + (unsigned)((wn * WTN + lb) * SKB) + sl;
  }
  auto f8_read_a = [&](auto I, int as) {  // both halves of A block I
    constexpr int i = decltype(I)::value;
    static_for<0, 2>([&](auto Fh) {
      constexpr int f = decltype(Fh)::value;
      const i32x4 v = ds_read_b128_at<i * BLK * SKB>(f8_arow[f] + as);
#pragma unroll
      for (int e = 0; e < 4; ++e) F0.a[i][4 * f + e] = v[e];
    });
  };
  auto f8_read_b = [&](auto X, int bs) {  // B read X: block X / RB8, piece X % RB8
    constexpr int x = decltype(X)::value;
    constexpr int j = x / RB8, r = x % RB8;
    if constexpr (BT) {
      const i32x4 v = ds_read_b128_at<j * BLK * SKB>(f8_brow[r] + bs);
#pragma unroll
      for (int e = 0; e < 4; ++e) F0.b[j][4 * r + e] = v[e];
    } else {
      const i32x2 v = ds_read_tr8_b64<8 * r * BROW>(lds_addr + b_rd[j] + bs);
      F0.b[j][2 * r] = v[0];
      F0.b[j][2 * r + 1] = v[1];
    }
  };
  // before stage 0: the B blocks j < FN / 2 and every A block, all landed
  auto f8_prologue_reads = [&]() {
    if constexpr (F8S) {
      static_for<0, (FN / 2) * RB8>([&](auto X) { f8_read_b(X, b_slot(0)); });
      static_for<0, FM>([&](auto I) { f8_read_a(I, a_slot(0)); });
      lds_wait();
    }
  };

  // 16-bit inputs: the same immediate-offset reads for the 16x16x32 steps
  // (M16Sched).  Read X of a k-step: X < NRB the B reads (transposing reads of
  // 4 K rows, two per block, or one 16-byte read per block given
  // transposed), then one 16-byte read per A block at m16_arow[ks] +
  // (block row) * SKB.
  // Used on the 256 x 256 tile: there it measured 1.7 % faster than the
  // evenly spread k-steps below (8192^3 fp16); on the 128 x 256 tile it
  // measured about 1 % slower, so the smaller tiles keep those.
  constexpr bool M16S = M16 && FM == 8;
  constexpr int RA16 = M16 ? NRA / FM : 1, RB16 = M16 ? NRB / FN : 1;
  unsigned m16_arow[2], m16_brow[2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    const unsigned sl = (unsigned)(((((KSTEP / 16) * ks + hq) ^ asw) << 4));
    m16_arow[ks] = lds_addr + (unsigned)((wm * WTM + lb) * SKB) + sl;
    m16_brow[ks] = lds_addr + (unsigned)((wn * WTN + lb) * SKB) + sl;
  }
  auto m16_read = [&](auto KS_, auto X, Frag<IN, FM, FN>& F, int as, int bs) {
    constexpr int ks = decltype(KS_)::value, x = decltype(X)::value;
    if constexpr (x < NRB) {
      constexpr int j = x / RB16, r = x % RB16;
      if constexpr (BT) {
        F.b[j] = ds_read_b128_at<j * BLK * SKB>(m16_brow[ks] + bs);
      } else {
        const i32x2 v = ds_read_tr16_b64<(ks * (KSTEP / 2) + 4 * r) * BROW>(lds_addr + b_rd[j] + bs);
        F.b[j][2 * r] = v[0];
        F.b[j][2 * r + 1] = v[1];
      }
    } else {
      constexpr int i = x - NRB;
      F.a[i] = ds_read_b128_at<i * BLK * SKB>(m16_arow[ks] + as);
    }
  };
  if (nt > 0) {
    for (int p = 0; p < NS; ++p) {
      const StageSrc q = (MODE == MODE_OZAKI || PER_TILE) ? next_src() : stage_src(p);
#pragma unroll
      for (int x = 0; x < DPW; ++x) dma_one(q, p, x);
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(WAIT_FIRST));
    __builtin_amdgcn_s_barrier();
    fence();
    if constexpr (F8S) {
      f8_prologue_reads();
    } else if constexpr (M16S) {
      // k-step 0 of stage 0 into F0, all landed
      static_for<0, NREAD>([&](auto X) {
        m16_read(std::integral_constant<int, 0>{}, X, F0, a_slot(0), b_slot(0));
      });
      lds_wait();
    } else {
#pragma unroll
      for (int x = 0; x < NREAD; ++x) read_one(F0, a_slot(0), b_slot(0), 0, x);
    }
  }

  // The stage change sits at the start of the last k-step of stage t: once a
  // wave's fragment reads of that k-step have landed it has read all of stage
  // t, so after it waits for its own DMA of stage t+1 a single barrier
  // certifies that (a) stage t+1 is in LDS for every wave and (b) no wave
  // reads the slot of stage t any more.  The whole last k-step then
  // overlaps the refill of that slot with stage t+NS and the fragment reads
  // of stage t+1.
  auto stage_change = [&]() {
    fence();
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(WAIT_NEXT));
    __builtin_amdgcn_s_barrier();
    fence();
  };
  // MFMAs of one k-step on Fc, with (if refill) the DMA of stage t+NS and the
  // fragment reads of k-step ks of stage tr into Fn spread between them.  Every stage runs the same instructions: a refill past the
  // end of the slice has only out-of-range offsets (zero fill, no memory
  // traffic) and the reads past the last stage land in registers that are
  // never used.
  auto kstep = [&](bool refill, const Frag<IN, FM, FN>& Fc, int t, Frag<IN, FM, FN>& Fn, int tr,
                   int ks) {
    StageSrc q;
    if constexpr (MODE == MODE_OZAKI || PER_TILE) {
      if (refill) q = next_src();
    } else {
      q = stage_src(t + NS);
    }
    const int as = a_slot(tr), bs = b_slot(tr);
    // A wave issuing its refill runs at raised priority, so its DMA goes out
    // ahead of the other wave's MFMAs on the SIMD (measured about 1 % faster
    // on the large tile; bits unchanged).
    if (refill) __builtin_amdgcn_s_setprio(3);
#pragma unroll
    for (int x = 0; x < NM; ++x) {
      mfma_x(Fc, x);
      if (refill) {
#pragma unroll
        for (int y = x * DPW / NM; y < (x + 1) * DPW / NM; ++y) dma_one(q, t + NS, y);
      }
#pragma unroll
      for (int y = x * NREAD / NM; y < (x + 1) * NREAD / NM; ++y) read_one(Fn, as, bs, ks, y);
      fence();
    }
    if (refill) __builtin_amdgcn_s_setprio(0);
  };

  // fp8: one k-step per stage on single-buffered fragments (F0).  Two
  // fragment sets of the 16x16x128 step do not fit beside the accumulators, so
  // the reads of stage t+1 go into the registers the MFMAs of stage t free, in
  // the order F8Sched lays out: phase 1 runs the blocks (i, j < FN/2) while
  // the B blocks j >= FN/2 of stage t are read; MFMA (0, FN/2) runs across
  // the stage change (all of this wave's reads of stage t landed, its DMA of
  // stage t+1 landed, one barrier for every wave); phase 2 runs the blocks
  // (i, j >= FN/2) with the refill of stage t's slot (stage t+NS) and the
  // reads of B blocks j < FN/2 and of every A block of stage t+1 in between.
  // Every memory instruction sits between two MFMAs, and each wait is for
  // exactly the reads the next MFMA needs, so one wave per SIMD can keep its
  // matrix unit fed.
  auto f8_stage = [&](int t) {
    if constexpr (F8S) {
      using S = F8Sched<FM, FN, RA8, RB8, DPW>;
      static_assert(RA8 * FM == NRA && RB8 * FN == NRB && S::H * 2 == FN, "fragment reads");
      static_assert(S::verified(), "fp8 read schedule");
      constexpr int H = S::H;
      lgkm_wait(std::integral_constant<int, S::wait_start()>{});
      const int bs = b_slot(t);
      static_for<0, S::NP>([&](auto P) {
        constexpr int p = decltype(P)::value;
        constexpr int i = p / H, j = p % H;
        if constexpr (j == 0 && i > 0 && S::wait_row(i) >= 0)
          lgkm_wait(std::integral_constant<int, S::wait_row(i)>{});
        mfma_x(F0, i * FN + j);
        static_for<S::late_lo(p), S::late_hi(p)>([&](auto L) {
          f8_read_b(std::integral_constant<int, H * RB8 + decltype(L)::value>{}, bs);
        });
        fence();
      });
      lgkm_wait(std::integral_constant<int, S::wait_mid()>{});
      mfma_x(F0, H);
      lds_wait();
      stage_change();
      StageSrc q;
      if constexpr (PER_TILE)
        q = next_src();
      else
        q = stage_src(t + NS);
      const int as1 = a_slot(t + 1), bs1 = b_slot(t + 1);
      __builtin_amdgcn_s_setprio(3);
      static_for<0, S::NP>([&](auto Sl) {
        constexpr int s = decltype(Sl)::value;
        static_for<S::dma_lo(s), S::dma_hi(s)>([&](auto Y) { dma_one(q, t + NS, decltype(Y)::value); });
        static_for<S::early_lo(s), S::early_hi(s)>([&](auto E) { f8_read_b(E, bs1); });
        if constexpr (S::a_at(s)) f8_read_a(std::integral_constant<int, s / H>{}, as1);
        fence();
        if constexpr (s + 1 < S::NP) {
          constexpr int c = s + 1;
          mfma_x(F0, (c / H) * FN + H + c % H);
          fence();
        }
      });
      __builtin_amdgcn_s_setprio(0);
    }
  };

  // 16-bit inputs: the two k-steps of a stage in the order M16Sched lays out:
  // k-step 0 on F0 while k-step 1 of the stage is read into F1 (B blocks
  // first, front-loaded); MFMA 0 of k-step 1 runs across the stage change;
  // the rest of k-step 1 carries the refill of stage t's slot (stage t+NS)
  // and the reads of k-step 0 of stage t+1 into F0.
  auto m16_stage = [&](int t) {
    if constexpr (M16S) {
      using S = M16Sched<FM, FN, RA16, RB16, DPW>;
      static_assert(KS == 2 && RA16 * FM == NRA && RB16 * FN == NRB, "16-bit k-steps");
      static_assert(S::verified(), "16-bit read schedule");
      const int as = a_slot(t), bs = b_slot(t);
      lgkm_wait(std::integral_constant<int, S::wait_start()>{});
      static_for<0, S::NM>([&](auto P) {
        constexpr int p = decltype(P)::value;
        constexpr int i = p / FN;
        if constexpr (p % FN == 0 && i > 0) lgkm_wait(std::integral_constant<int, S::wait_row(i)>{});
        mfma_x(F0, p);
        static_for<S::lo0(p), S::lo0(p + 1)>([&](auto X) {
          m16_read(std::integral_constant<int, 1>{}, X, F1, as, bs);
        });
        fence();
      });
      lgkm_wait(std::integral_constant<int, S::wait_start()>{});
      mfma_x(F1, 0);
      lds_wait();
      stage_change();
      StageSrc q;
      if constexpr (PER_TILE)
        q = next_src();
      else
        q = stage_src(t + NS);
      const int as1 = a_slot(t + 1), bs1 = b_slot(t + 1);
      __builtin_amdgcn_s_setprio(3);
      static_for<0, S::NM - 1>([&](auto Sl) {
        constexpr int s = decltype(Sl)::value;
        static_for<S::dlo(s), S::dlo(s + 1)>([&](auto Y) { dma_one(q, t + NS, decltype(Y)::value); });
        static_for<S::lo1(s), S::lo1(s + 1)>([&](auto X) {
          m16_read(std::integral_constant<int, 0>{}, X, F0, as1, bs1);
        });
        fence();
        mfma_x(F1, s + 1);
        fence();
      });
      __builtin_amdgcn_s_setprio(0);
    }
  };

  // k-steps alternate between F0 and F1; KS is even, so every stage starts on
  // F0 (fp8: one k-step per stage, on F0 alone)
  OzCursor cur;      // Ozaki mode: the pair and stage being computed
  int chunk_left = 0;
  if constexpr (MODE == MODE_OZAKI) chunk_left = g.chunk_stages;
  int cur_tile = 0, cur_kt = 0;  // MODE_PERSIST: the tile and stage being computed
  int64_t cur_m0 = m0, cur_n0 = n0;
  for (int t = 0; t < nt; ++t) {
    if constexpr (F8S) {
      f8_stage(t);
    } else if constexpr (M16S) {
      m16_stage(t);
    } else {
#pragma unroll
      for (int ks = 0; ks + 1 < KS; ++ks) {
        lds_wait();  // fragments of k-step ks have landed
        if (ks % 2 == 0)
          kstep(false, F0, t, F1, t, ks + 1);
        else
          kstep(false, F1, t, F0, t, ks + 1);
      }
      lds_wait();  // last k-step's fragments landed: this wave has read all of stage t
      stage_change();
      kstep(true, F1, t, F0, t + 1, 0);
    }
    if constexpr (MODE == MODE_OZAKI) {
      const int level = cur.p + cur.q;
      const bool pair_end = cur.step(ntp, g.slices, g.d);
      if (pair_end || --chunk_left == 0) {
        oz_flush(level);
        chunk_left = g.chunk_stages;
      }
    }
    if constexpr (PER_TILE) {
      // End of a tile: store it while the next tile's first stages load, and
      // start the next one from +0.
      if (++cur_kt == ntp) {
        cur_kt = 0;
        // the next stage's first fragment reads land before the epilogue,
        // which may copy their registers (the compiler takes them as written)
        lds_wait();
        store_tile(cur_m0, cur_n0);
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j) acc[i][j] = AccT{};
        if (++cur_tile < ntiles) tile_origin(cur_tile, &cur_m0, &cur_n0);
      }
    }
  }
  // No LDS transfer or read may still be in flight when the workgroup ends.
  // The last stage issued the fragment reads of a stage that does not exist;
  // their results are never used, but the hardware still writes their
  // registers when the data arrives.  The fences keep the epilogue below the
  // waits, and keep_live holds the registers of those reads until here, so that no register copy or epilogue value (on any path the
  // compiler lays out, the loop peeled or not) is given a register a read
  // will still write.
  fence();
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  __builtin_amdgcn_s_waitcnt(lgkmcnt_imm(0));
  fence();
  // (Those reads all go to F0: every path reads the next stage's first
  // k-step into F0, and F1's reads land within their own stage.  The
  // persistent mode stores its tiles inside the loop, where F0 is live, and
  // has no epilogue here.)
  if constexpr (!PER_TILE) {
    if (nt > 0) {
      constexpr int FD = sizeof(F0.a[0]) / 4;  // dwords per fragment
#pragma unroll
      for (int i = 0; i < FM; ++i) keep_live<FD>(F0.a[i]);
#pragma unroll
      for (int j = 0; j < FN; ++j) keep_live<FD>(F0.b[j]);
    }
  }
  fence();
  if constexpr (!PER_TILE) store_tile(m0, n0);
}

template <int IN, int TBM, int TBN, int WM, int WN, int NS, bool BT>
hipError_t launch_cfg(const gemm_plan_s& p, const GemmArgs& a, bool slice, hipStream_t s) {
  const dim3 grid((unsigned)a.grid), block(WM * WN * 64);
  if (slice)
    hipLaunchKernelGGL((gemm_dma_kernel<IN, GEMM_F32, MODE_SLICE, TBM, TBN, WM, WN, NS, BT, GemmArgs>),
                       grid, block, 0, s, a);
  else if (p.out == GEMM_F32)
    hipLaunchKernelGGL((gemm_dma_kernel<IN, GEMM_F32, MODE_STORE, TBM, TBN, WM, WN, NS, BT, GemmArgs>),
                       grid, block, 0, s, a);
  else if (p.out == GEMM_F16)
    hipLaunchKernelGGL((gemm_dma_kernel<IN, GEMM_F16, MODE_STORE, TBM, TBN, WM, WN, NS, BT, GemmArgs>),
                       grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((gemm_dma_kernel<IN, GEMM_BF16, MODE_STORE, TBM, TBN, WM, WN, NS, BT, GemmArgs>),
                       grid, block, 0, s, a);
  return hipGetLastError();
}

// Persistent single pass on the 256 x 256 tile.
template <int IN, bool BT>
hipError_t launch_persist_in(const gemm_plan_s& p, const PersistArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)a.wgs), block(512);
  if (p.out == GEMM_F32)
    hipLaunchKernelGGL((gemm_dma_kernel<IN, GEMM_F32, MODE_PERSIST, 256, WIDE_TBN, 2, 4, 2, BT,
                                        PersistArgs>), grid, block, 0, s, a);
  else if (p.out == GEMM_F16)
    hipLaunchKernelGGL((gemm_dma_kernel<IN, GEMM_F16, MODE_PERSIST, 256, WIDE_TBN, 2, 4, 2, BT,
                                        PersistArgs>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((gemm_dma_kernel<IN, GEMM_BF16, MODE_PERSIST, 256, WIDE_TBN, 2, 4, 2, BT,
                                        PersistArgs>), grid, block, 0, s, a);
  return hipGetLastError();
}

template <int IN>
hipError_t launch_persist_bt(const gemm_plan_s& p, const PersistArgs& a, hipStream_t s) {
  return p.b_trans ? launch_persist_in<IN, true>(p, a, s) : launch_persist_in<IN, false>(p, a, s);
}

template <int IN, bool BT>
hipError_t launch_tiles(const gemm_plan_s& p, int tile, const GemmArgs& a, bool slice, hipStream_t s) {
  switch (tile) {
    case GEMM_TILE_256x256: return launch_cfg<IN, 256, 256, 2, 4, 2, BT>(p, a, slice, s);
    case GEMM_TILE_128x256: return launch_cfg<IN, 128, 256, 2, 4, 3, BT>(p, a, slice, s);
    case GEMM_TILE_64x256: return launch_cfg<IN, 64, 256, 1, 4, 4, BT>(p, a, slice, s);
    case GEMM_TILE_32x256: return launch_cfg<IN, 32, 256, 1, 4, 4, BT>(p, a, slice, s);
    default: break;
  }
  if constexpr (InT<IN>::EB == 2) {  // the narrow tiles take 16-bit inputs only
    switch (tile) {
      case GEMM_TILE_64x64: return launch_cfg<IN, 64, 64, 2, 1, 2, BT>(p, a, slice, s);
      case GEMM_TILE_32x64: return launch_cfg<IN, 32, 64, 2, 1, 3, BT>(p, a, slice, s);
      case GEMM_TILE_32x32: return launch_cfg<IN, 32, 32, 2, 1, 3, BT>(p, a, slice, s);
      default: break;
    }
  }
  return hipErrorInvalidValue;
}

template <int IN>
hipError_t launch_in(const gemm_plan_s& p, int tile, const GemmArgs& a, bool slice, hipStream_t s) {
  return p.b_trans ? launch_tiles<IN, true>(p, tile, a, slice, s)
                   : launch_tiles<IN, false>(p, tile, a, slice, s);
}

}  // namespace

hipError_t launch_ozaki_gemm(int type2, const OzGemmArgs& a, hipStream_t s) {
  static_assert(kOzTileN == WIDE_TBN, "Ozaki tile");
  // The fp64 sums (two registers per element) must sit in architectural
  // VGPRs, at most 256 per wave.  bf16: a 128 x 256 tile of 8 waves (two per
  // SIMD) of 64 x 64, 253 VGPRs, 3-stage ring (144 KB).  fp8 fragments are
  // twice as wide and spill there, so e4m3 runs a 64 x 256 tile of 4 waves
  // (one per SIMD) of 64 x 64, with its fp32 accumulators in AGPRs and a
  // 4-stage ring (160 KB).  The small tiles are fill-bound: the deeper rings
  // measured 7-10 % faster than 2 and 3 stages.
  const dim3 grid((unsigned)a.grid);
  if (type2 == GEMM_BF16)
    hipLaunchKernelGGL((gemm_dma_kernel<GEMM_BF16, GEMM_F32, MODE_OZAKI, 128, WIDE_TBN, 2, 4, 3, false,
                                        OzGemmArgs>), grid, dim3(512), 0, s, a);
  else if (type2 == GEMM_F8_E4M3)
    hipLaunchKernelGGL((gemm_dma_kernel<GEMM_F8_E4M3, GEMM_F32, MODE_OZAKI, 64, WIDE_TBN, 1, 4, 4, false,
                                        OzGemmArgs>), grid, dim3(256), 0, s, a);
  else if (type2 == GEMM_I8)
    hipLaunchKernelGGL((gemm_dma_kernel<GEMM_I8, GEMM_F32, MODE_OZAKI, 128, WIDE_TBN, 2, 4, 3, false,
                                        OzGemmArgs>), grid, dim3(512), 0, s, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_gemm_persist(const gemm_plan_s& p, const PersistArgs& a, hipStream_t s) {
  switch (p.in) {
    case GEMM_F16: return launch_persist_bt<GEMM_F16>(p, a, s);
    case GEMM_BF16: return launch_persist_bt<GEMM_BF16>(p, a, s);
    case GEMM_F8_E4M3:
      return p.f8_fp32 ? launch_persist_bt<kInE4M3W>(p, a, s) : launch_persist_bt<GEMM_F8_E4M3>(p, a, s);
    case GEMM_F8_E5M2:
      return p.f8_fp32 ? launch_persist_bt<kInE5M2W>(p, a, s) : launch_persist_bt<GEMM_F8_E5M2>(p, a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_gemm_dma(const gemm_plan_s& p, int tile, const GemmArgs& a, bool slice_mode,
                           hipStream_t s) {
  switch (p.in) {
    case GEMM_F16: return launch_in<GEMM_F16>(p, tile, a, slice_mode, s);
    case GEMM_BF16: return launch_in<GEMM_BF16>(p, tile, a, slice_mode, s);
    case GEMM_F8_E4M3:
      return p.f8_fp32 ? launch_in<kInE4M3W>(p, tile, a, slice_mode, s)
                       : launch_in<GEMM_F8_E4M3>(p, tile, a, slice_mode, s);
    case GEMM_F8_E5M2:
      return p.f8_fp32 ? launch_in<kInE5M2W>(p, tile, a, slice_mode, s)
                       : launch_in<GEMM_F8_E5M2>(p, tile, a, slice_mode, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace imm
