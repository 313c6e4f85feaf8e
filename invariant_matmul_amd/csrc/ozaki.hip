// Ozaki-scheme split kernels for gfx950: fp64 matrices -> Type2 slices.
//
// Source: Insight Edge blog on cuTile Python, section "倍精度行列積エミュレー
// ション", subsections "分解(Split)" (equations (1)-(5)) and "Fused Split
// Kernel（分割の融合）" (one maximum, then every slice in a single pass with
// sigma and 2^-c known up front).
//
// Each row of A and each column of B (the vectors of the inner products) has
// its own exponent c0 = ceil(log2 max|x|), 0 for a zero vector, so that a row
// of C depends on its own row of A only.  Slice p of an element uses
// c_p = c0 - p * delta:
//     sigma = 0.75 * 2^(rho + c_p);  v = (x + sigma) - sigma;  x = x - v;
//     slice_p = Type2(v * 2^-c_p)
// With |x| <= 2^c_p the sum x + sigma lies in [2^(rho+c_p-1), 2^(rho+c_p)),
// so v is x rounded to nearest even on the grid 2^(c_p - b), b = 53 - rho,
// the subtraction is exact, and |x - v| <= 2^(c_p - b - 1): with
// delta = b + 1 the next slice again has |x| <= 2^c.  v * 2^-c_p is a
// multiple of 2^-b in [-1, 1], exactly representable in the Type2 format
// (b <= 8 for bf16, b <= 4 for e4m3), so the conversions below are exact bit
// extractions; int8 slices store the integer n = v * 2^(b - c_p), |n| <= 2^b
// with b <= 6.  All fp64 arithmetic is IEEE add/sub/ldexp, no contraction.
//
// Layouts: x is fp64 row-major [R, C]; the slices are [s, Ro, Co] row-major
// with Ro >= R, Co >= C, Co a multiple of 8 (padding entries are zero).
#include "imm_internal.h"

namespace imm {
namespace {

// ceil(log2 m) exactly (0 for m == 0): m = f * 2^e with f in [0.5, 1).
__device__ __forceinline__ int ceil_log2_exact(double m) {
  if (m == 0.0) return 0;
  int e;
  const double f = frexp(m, &e);
  return f == 0.5 ? e - 1 : e;
}

// |x| for the maxima, with a NaN, an infinity or a magnitude above the
// domain's bound turned into +inf (fmax would drop a NaN; +inf survives it).
__device__ __forceinline__ double dom_abs(double x) {
  const double a = fabs(x);
  return a <= kOzMaxMag ? a : __builtin_inf();
}

// The exponent c0 of a vector from the maximum of dom_abs over it, or
// kOzBadExp outside the domain.
__device__ __forceinline__ int exp_of_max(double m) {
  if (m > kOzMaxMag || (m != 0.0 && m < kOzMinMax)) return kOzBadExp;
  return ceil_log2_exact(m);
}

// Exponent of each row of x [R, C] from the maximum of dom_abs over it: one
// workgroup per row.
__global__ __launch_bounds__(256) void oz_row_exp_kernel(const double* x, int64_t C, int32_t* e) {
  const double* row = x + (int64_t)blockIdx.x * C;
  double m = 0.0;
  for (int64_t k = threadIdx.x; k < C; k += 256) m = fmax(m, dom_abs(row[k]));
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m = fmax(m, __shfl_xor(m, off));
  __shared__ double red[4];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) e[blockIdx.x] = exp_of_max(fmax(fmax(red[0], red[1]), fmax(red[2], red[3])));
}

// Maximum of dom_abs over rows [y*rc, (y+1)*rc) of each column of x [R, C].
__global__ __launch_bounds__(256) void oz_col_max_kernel(const double* x, int64_t R, int64_t C,
                                                         int64_t rc, double* part) {
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (c >= C) return;
  const int64_t r0 = (int64_t)blockIdx.y * rc;
  const int64_t r1 = R < r0 + rc ? R : r0 + rc;
  double m = 0.0;
  for (int64_t r = r0; r < r1; ++r) m = fmax(m, dom_abs(x[r * C + c]));
  part[(int64_t)blockIdx.y * C + c] = m;
}

// Column exponents from the chunk maxima (chunks may be 0: all exponents 0).
__global__ __launch_bounds__(256) void oz_col_exp_kernel(const double* part, int64_t chunks,
                                                         int64_t C, int32_t* e) {
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (c >= C) return;
  double m = 0.0;
  for (int64_t y = 0; y < chunks; ++y) m = fmax(m, part[y * C + c]);
  e[c] = exp_of_max(m);
}

// Exact Type2 encodings of a float that holds a slice value.
__device__ __forceinline__ unsigned enc_bf16(float y) { return __float_as_uint(y) >> 16; }
// OCP e4m3fn: sign, 4-bit exponent (bias 7), 3 significand bits.  Slice
// values are 0 or have |y| in [2^-4, 1] with at most 4 significant bits, so
// they are normal e4m3 numbers.
__device__ __forceinline__ unsigned enc_e4m3(float y) {
  const unsigned u = __float_as_uint(y);
  const unsigned sign = (u >> 24) & 0x80u;
  if ((u & 0x7fffffffu) == 0) return sign;
  const int E = (int)((u >> 23) & 255u) - 127;
  return sign | ((unsigned)(E + 7) << 3) | ((u >> 20) & 7u);
}

// One thread per 8 consecutive output columns of one output row; all s
// slices of them.
template <int T2, bool PER_ROW>
__global__ __launch_bounds__(256) void oz_split_kernel(const double* x, int64_t R, int64_t C,
                                                       int64_t Ro, int64_t Co, const int32_t* e,
                                                       int s, int rho, int delta, void* out) {
  const int64_t groups_per_row = Co / 8;
  const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (g >= Ro * groups_per_row) return;
  const int64_t r = g / groups_per_row;
  const int64_t c0 = (g - r * groups_per_row) * 8;
  double xr[8];
  int ex[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int64_t c = c0 + u;
    xr[u] = (r < R && c < C) ? x[r * C + c] : 0.0;
    ex[u] = PER_ROW ? (r < R ? e[r] : 0) : (c < C ? e[c] : 0);
    if (ex[u] == kOzBadExp) {  // outside the domain: zero slices (C is NaN there)
      ex[u] = 0;
      xr[u] = 0.0;
    }
  }
  const int64_t plane = Ro * Co;
  for (int p = 0; p < s; ++p) {
    unsigned enc[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int cp = ex[u] - p * delta;
      const double sigma = ldexp(0.75, rho + cp);  // (2)
      const double v = (xr[u] + sigma) - sigma;   // (3)
      xr[u] = xr[u] - v;                          // (4)
      if constexpr (T2 == GEMM_I8) {
        enc[u] = (unsigned)(int)ldexp(v, 53 - rho - cp) & 0xffu;  // (5) as the integer n
      } else {
        const float y = (float)ldexp(v, -cp);       // (5), exact
        enc[u] = T2 == GEMM_BF16 ? enc_bf16(y) : enc_e4m3(y);
      }
    }
    const int64_t idx = p * plane + r * Co + c0;
    if constexpr (T2 == GEMM_BF16) {
      uint4 w;
      w.x = enc[0] | (enc[1] << 16);
      w.y = enc[2] | (enc[3] << 16);
      w.z = enc[4] | (enc[5] << 16);
      w.w = enc[6] | (enc[7] << 16);
      *reinterpret_cast<uint4*>(static_cast<unsigned short*>(out) + idx) = w;
    } else {
      uint2 w;
      w.x = enc[0] | (enc[1] << 8) | (enc[2] << 16) | (enc[3] << 24);
      w.y = enc[4] | (enc[5] << 8) | (enc[6] << 16) | (enc[7] << 24);
      *reinterpret_cast<uint2*>(static_cast<unsigned char*>(out) + idx) = w;
    }
  }
}

int64_t blocks_of(int64_t n) { return (n + 255) / 256; }

}  // namespace

hipError_t launch_oz_row_exp(const double* x, int64_t R, int64_t C, int32_t* e, hipStream_t s) {
  if (R == 0) return hipSuccess;
  hipLaunchKernelGGL(oz_row_exp_kernel, dim3((unsigned)R), dim3(256), 0, s, x, C, e);
  return hipGetLastError();
}

hipError_t launch_oz_col_exp(const double* x, int64_t R, int64_t C, int64_t rc, double* part,
                             int32_t* e, hipStream_t s) {
  if (C == 0) return hipSuccess;
  const int64_t chunks = (R + rc - 1) / rc;
  if (chunks > 0) {
    hipLaunchKernelGGL(oz_col_max_kernel, dim3((unsigned)blocks_of(C), (unsigned)chunks), dim3(256),
                       0, s, x, R, C, rc, part);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  hipLaunchKernelGGL(oz_col_exp_kernel, dim3((unsigned)blocks_of(C)), dim3(256), 0, s, part, chunks,
                     C, e);
  return hipGetLastError();
}

hipError_t launch_oz_split(int type2, bool per_row, const double* x, int64_t R, int64_t C,
                           int64_t Ro, int64_t Co, const int32_t* e, int slices, int rho, int delta,
                           void* out, hipStream_t s) {
  const int64_t groups = Ro * (Co / 8);
  if (groups == 0) return hipSuccess;
  const dim3 grid((unsigned)blocks_of(groups)), block(256);
  if (type2 == GEMM_BF16) {
    if (per_row)
      hipLaunchKernelGGL((oz_split_kernel<GEMM_BF16, true>), grid, block, 0, s, x, R, C, Ro, Co, e,
                         slices, rho, delta, out);
    else
      hipLaunchKernelGGL((oz_split_kernel<GEMM_BF16, false>), grid, block, 0, s, x, R, C, Ro, Co, e,
                         slices, rho, delta, out);
  } else if (type2 == GEMM_F8_E4M3) {
    if (per_row)
      hipLaunchKernelGGL((oz_split_kernel<GEMM_F8_E4M3, true>), grid, block, 0, s, x, R, C, Ro, Co,
                         e, slices, rho, delta, out);
    else
      hipLaunchKernelGGL((oz_split_kernel<GEMM_F8_E4M3, false>), grid, block, 0, s, x, R, C, Ro, Co,
                         e, slices, rho, delta, out);
  } else if (type2 == GEMM_I8) {
    if (per_row)
      hipLaunchKernelGGL((oz_split_kernel<GEMM_I8, true>), grid, block, 0, s, x, R, C, Ro, Co, e,
                         slices, rho, delta, out);
    else
      hipLaunchKernelGGL((oz_split_kernel<GEMM_I8, false>), grid, block, 0, s, x, R, C, Ro, Co, e,
                         slices, rho, delta, out);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace imm
