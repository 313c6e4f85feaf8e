/*
 * CPU oracle for C = A * B with fp16 / bf16 / fp8 (OCP e4m3fn, e5m2) inputs.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link
 * or call this file: it is used by the test-suite, by the smoke check and by
 * the benchmark's CPU-baseline leg, and by nothing else.  It shares no code,
 * header, table or constant with the HIP library.
 *
 * Citations (page title, section):
 *   [TDI] Tencent engineer article on deterministic LLM inference
 *         ("AI インフラの深化：大規模モデルに確定的な出力を実現する方法").
 *   [GKM] "GEMM kernels" memo on GPU matrix multiply basics (qsysarch).
 *   [CTB] Insight Edge blog on cuTile Python and the Ozaki scheme.
 *
 * What it computes is the plain definition of the product: every output
 * element is the dot product of row i of A with column j of B, summed over
 * k = 0 .. K-1 ([TDI] "Batch Invariance の由来", the C_ij formula; [TDI]
 * "GEMM の最適化戦略", the i/j/k triple loop).  The sum is carried in fp64,
 * in ascending k, starting from +0.0.  Each product of two decoded inputs is
 * exact in fp64 (at most 11 + 11 significand bits), so the only rounding is
 * the fp64 addition; no GPU summation order is emulated.
 *
 * Input decoding follows the format definitions: IEEE-754 binary16 (1/5/10,
 * bias 15), bfloat16 (1/8/7, bias 127), OCP FP8 E4M3FN (1/4/3, bias 7, no
 * infinities, only S.1111.111 is NaN, largest finite 448) and OCP FP8 E5M2
 * (1/5/2, bias 15, IEEE-like).  [TDI] "背景" states the binary16 layout and
 * the unit in the last place ULP(x) = 2^(E - M) for a value with unbiased
 * exponent E and M stored significand bits.
 *
 * Rounding to a narrower format is round-to-nearest, ties-to-even, as [TDI]
 * "背景" describes for 2048 + 1 in binary16 (the exact 2049 sits halfway
 * between 2048 and 2050 and goes to the even significand, 2048).
 *
 * Build: gcc -O2 -fPIC -shared -fopenmp -ffp-contract=off oracle.c -lm
 * (no fast-math: the fp64 sums must be evaluated exactly as written).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Format codes used by the ctypes wrapper. */
enum { ORC_F16 = 0, ORC_BF16 = 1, ORC_E4M3 = 2, ORC_E5M2 = 3, ORC_F32 = 4 };

typedef struct {
  int exp_bits;  /* width of the biased-exponent field */
  int man_bits;  /* stored significand bits (M in ULP = 2^(E-M)) */
  int bias;
  int ieee_special; /* 1: all-ones exponent encodes inf/NaN; 0: e4m3fn rule */
  int bytes;
} orc_fmt;

static int orc_format(int code, orc_fmt* f) {
  switch (code) {
    case ORC_F16:  *f = (orc_fmt){5, 10, 15, 1, 2}; return 0;
    case ORC_BF16: *f = (orc_fmt){8, 7, 127, 1, 2}; return 0;
    case ORC_E4M3: *f = (orc_fmt){4, 3, 7, 0, 1}; return 0;
    case ORC_E5M2: *f = (orc_fmt){5, 2, 15, 1, 1}; return 0;
    case ORC_F32:  *f = (orc_fmt){8, 23, 127, 1, 4}; return 0;
    default: return -1;
  }
}

/* ---- decoding -------------------------------------------------------- */

static double decode_bits(const orc_fmt* f, uint32_t bits) {
  const uint32_t emask = (1u << f->exp_bits) - 1u;
  const uint32_t mmask = (1u << f->man_bits) - 1u;
  const int negative = (bits >> (f->exp_bits + f->man_bits)) & 1u;
  const uint32_t e = (bits >> f->man_bits) & emask;
  const uint32_t m = bits & mmask;
  double v;
  if (e == 0) {
    /* subnormal (or zero): m * 2^(1 - bias - man_bits) */
    v = ldexp((double)m, 1 - f->bias - f->man_bits);
  } else if (f->ieee_special && e == emask) {
    v = (m == 0) ? INFINITY : NAN;
  } else if (!f->ieee_special && e == emask && m == mmask) {
    v = NAN; /* e4m3fn: only the all-ones pattern is NaN */
  } else {
    /* normal: (2^man_bits + m) * 2^(e - bias - man_bits) */
    v = ldexp((double)((1u << f->man_bits) + m), (int)e - f->bias - f->man_bits);
  }
  return negative ? -v : v;
}

static uint32_t load_bits(const void* p, int64_t idx, int bytes) {
  if (bytes == 1) return ((const uint8_t*)p)[idx];
  if (bytes == 2) return ((const uint16_t*)p)[idx];
  return ((const uint32_t*)p)[idx];
}

/* Decode n values of format `code` to fp64. Returns 0, or -1 for a bad code. */
int orc_decode(int code, const void* bits, int64_t n, double* out) {
  orc_fmt f;
  if (orc_format(code, &f)) return -1;
  for (int64_t i = 0; i < n; ++i) out[i] = decode_bits(&f, load_bits(bits, i, f.bytes));
  return 0;
}

/* ---- rounding (fp64 -> narrower binary format, RNE) ------------------- */

/* Round x to the nearest value of format f with ties to even and return its
 * bit pattern.  NaN maps to a quiet NaN; overflow goes to infinity, or to
 * NaN in OCP e4m3fn, which has no infinity (OCP FP8 conversion without
 * saturation). */
static uint32_t round_bits(const orc_fmt* f, double x) {
  const int sign_shift = f->exp_bits + f->man_bits;
  const uint32_t emask = (1u << f->exp_bits) - 1u;
  uint32_t sign = signbit(x) ? (1u << sign_shift) : 0u;
  if (isnan(x)) {
    return f->ieee_special ? (sign | (emask << f->man_bits) | (1u << (f->man_bits - 1)))
                           : (sign | (emask << f->man_bits) | ((1u << f->man_bits) - 1u));
  }
  double a = fabs(x);
  if (isinf(a)) {
    return f->ieee_special ? (sign | (emask << f->man_bits))
                           : (sign | (emask << f->man_bits) | ((1u << f->man_bits) - 1u));
  }
  if (a == 0.0) return sign;
  const int emin = 1 - f->bias;           /* smallest normal exponent */
  /* largest finite exponent: the all-ones field is reserved in IEEE-like
   * formats; e4m3fn uses it for finite values (only S.1111.111 is NaN) */
  const int emax = (int)emask - (f->ieee_special ? 1 : 0) - f->bias;
  int ex;
  (void)frexp(a, &ex);                    /* a = fr * 2^ex, fr in [0.5, 1) */
  int E = ex - 1;                         /* a in [2^E, 2^(E+1)) */
  if (E < emin) E = emin;                 /* subnormal range: fixed quantum */
  /* Quantum (ULP) at this exponent: 2^(E - man_bits). */
  const double q = ldexp(1.0, E - f->man_bits);
  const double n = a / q;                 /* exact: q is a power of two */
  double r = floor(n);
  const double frac = n - r;              /* exact */
  if (frac > 0.5 || (frac == 0.5 && fmod(r, 2.0) != 0.0)) r += 1.0;
  const double v = r * q;                 /* exact */
  /* largest finite significand: all ones, or all ones but the last bit for
   * e4m3fn (1.110b * 2^8 = 448) */
  const double maxfin = ldexp((double)((2u << f->man_bits) - (f->ieee_special ? 1u : 2u)),
                              emax - f->man_bits);
  if (v > maxfin) {
    /* overflow: infinity, or NaN in e4m3fn, which has no infinity */
    return f->ieee_special ? (sign | (emask << f->man_bits))
                           : (sign | (emask << f->man_bits) | ((1u << f->man_bits) - 1u));
  }
  if (v < ldexp(1.0, emin)) {
    /* subnormal: biased exponent 0, significand = v / 2^(emin - man_bits) */
    return sign | (uint32_t)(v / ldexp(1.0, emin - f->man_bits));
  }
  int vex;
  (void)frexp(v, &vex);
  const int Ev = vex - 1;
  const uint32_t mant = (uint32_t)(v / ldexp(1.0, Ev - f->man_bits)) - (1u << f->man_bits);
  return sign | ((uint32_t)(Ev + f->bias) << f->man_bits) | mant;
}

/* Round n doubles to format `code`; out holds 1-, 2- or 4-byte patterns. */
int orc_round(int code, const double* x, int64_t n, void* out) {
  orc_fmt f;
  if (orc_format(code, &f)) return -1;
  for (int64_t i = 0; i < n; ++i) {
    uint32_t b = round_bits(&f, x[i]);
    if (f.bytes == 1) ((uint8_t*)out)[i] = (uint8_t)b;
    else if (f.bytes == 2) ((uint16_t*)out)[i] = (uint16_t)b;
    else ((uint32_t*)out)[i] = b;
  }
  return 0;
}

/* ---- the product ------------------------------------------------------ */

static int set_threads(int nthreads) {
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
  return omp_get_max_threads();
#else
  (void)nthreads;
  return 1;
#endif
}

/*
 * Rows `rows[0..nrows)` of C = scale * (A * B) and of |A| * |B|, where A is
 * M x K and B is K x N, both row-major with leading dimensions K and N.
 * C64 and Cabs are nrows x N (row r of the output is row rows[r] of C).
 * For each row: decode the row of A, then for k ascending add a_ik * b_kj
 * into every c_j (the i-k-j order of the textbook loop; per element the k
 * order is ascending, which is all that matters for the result).  Rows are
 * independent, so the thread count does not change any bit.
 */
int orc_gemm_rows(int64_t M, int64_t N, int64_t K, int code, const void* A,
                  const void* B, double scale, const int64_t* rows,
                  int64_t nrows, double* C64, double* Cabs, int nthreads) {
  orc_fmt f;
  if (orc_format(code, &f) || M < 0 || N < 0 || K < 0) return -1;
  for (int64_t r = 0; r < nrows; ++r)
    if (rows[r] < 0 || rows[r] >= M) return -2;
  double* Bd = (double*)malloc(sizeof(double) * (size_t)(K * N > 0 ? K * N : 1));
  if (!Bd) return -3;
  orc_decode(code, B, K * N, Bd);
  set_threads(nthreads);
  int fail = 0;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t r = 0; r < nrows; ++r) {
    const int64_t i = rows[r];
    double* c = C64 + r * N;
    double* ca = Cabs + r * N;
    double* arow = (double*)malloc(sizeof(double) * (size_t)(K > 0 ? K : 1));
    if (!arow) { fail = 1; continue; }
    for (int64_t k = 0; k < K; ++k) arow[k] = decode_bits(&f, load_bits(A, i * K + k, f.bytes));
    for (int64_t j = 0; j < N; ++j) { c[j] = 0.0; ca[j] = 0.0; }
    for (int64_t k = 0; k < K; ++k) {
      const double a = arow[k];
      const double* b = Bd + k * N;
      for (int64_t j = 0; j < N; ++j) {
        const double p = a * b[j]; /* exact product */
        c[j] += p;
        ca[j] += fabs(p);
      }
    }
    for (int64_t j = 0; j < N; ++j) c[j] *= scale;
    for (int64_t j = 0; j < N; ++j) ca[j] *= fabs(scale);
    free(arow);
  }
  free(Bd);
  return fail ? -3 : 0;
}

/* All M rows. */
int orc_gemm(int64_t M, int64_t N, int64_t K, int code, const void* A,
             const void* B, double scale, double* C64, double* Cabs, int nthreads) {
  int64_t* rows = (int64_t*)malloc(sizeof(int64_t) * (size_t)(M > 0 ? M : 1));
  if (!rows) return -3;
  for (int64_t i = 0; i < M; ++i) rows[i] = i;
  int rc = orc_gemm_rows(M, N, K, code, A, B, scale, rows, M, C64, Cabs, nthreads);
  free(rows);
  return rc;
}

/*
 * Single elements (ii[t], jj[t]) of C and |A||B|, each the ascending-k fp64
 * dot product of row ii[t] of A and column jj[t] of B.  Used to check
 * sampled outputs of products too large to evaluate in full.
 */
int orc_gemm_elems(int64_t M, int64_t N, int64_t K, int code, const void* A,
                   const void* B, double scale, const int64_t* ii,
                   const int64_t* jj, int64_t n, double* c64, double* cabs,
                   int nthreads) {
  orc_fmt f;
  if (orc_format(code, &f) || M < 0 || N < 0 || K < 0) return -1;
  for (int64_t t = 0; t < n; ++t)
    if (ii[t] < 0 || ii[t] >= M || jj[t] < 0 || jj[t] >= N) return -2;
  set_threads(nthreads);
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < n; ++t) {
    double s = 0.0, sa = 0.0;
    for (int64_t k = 0; k < K; ++k) {
      const double p = decode_bits(&f, load_bits(A, ii[t] * K + k, f.bytes)) *
                       decode_bits(&f, load_bits(B, k * N + jj[t], f.bytes));
      s += p;
      sa += fabs(p);
    }
    c64[t] = s * scale;
    cabs[t] = sa * fabs(scale);
  }
  return 0;
}

/*
 * Integer twin: C = A * B over int64 for integer-valued inputs given as
 * int32, by the plain triple loop.  It shares nothing with the fp64 path and
 * pins it on inputs where every product and partial sum is exact.
 */
int orc_gemm_i64(int64_t M, int64_t N, int64_t K, const int32_t* A,
                 const int32_t* B, int64_t* C) {
  if (M < 0 || N < 0 || K < 0) return -1;
  for (int64_t i = 0; i < M; ++i)
    for (int64_t j = 0; j < N; ++j) {
      int64_t s = 0;
      for (int64_t k = 0; k < K; ++k) s += (int64_t)A[i * K + k] * (int64_t)B[k * N + j];
      C[i * N + j] = s;
    }
  return 0;
}

int orc_max_threads(void) { return set_threads(0); }
