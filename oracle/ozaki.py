"""CPU oracle for the Ozaki-scheme fp64 matrix product (FP64 emulation on
low-precision matrix units).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import this module.  The HIP library
never imports it and shares no code with it.

Source: Insight Edge blog on cuTile Python, sections "倍精度行列積エミュレーション"
("Ozaki Schemeについて", "分解(Split)", "行列積の計算", "Fast Mode（GEMMの削減）",
"Fused Split Kernel（分割の融合）").  Notation follows the page: Type1 is the
fp64 input (53 significand bits), Type2 the narrow slice format (bf16: 8,
fp8 e4m3: 4 significand bits, hidden bit included), Type3 the fp32 accumulator
of the matrix unit (24 bits).  A third Type2, int8, is the matrix unit's
integer format: its Type3 is the int32 accumulator (31 bits), and a slice
entry n * 2^-b with |n| <= 2^b fits int8 for b <= 6, so m_Type2 = 6.

What is computed, in the page's order:

1. Parameters.  rho = max(gamma, xi) with gamma = ceil(53 - (24 - log2 k)/2)
   and xi = 53 - m_Type2 ("分解(Split)", the precision parameter).  k is the
   number of products one fp32 accumulation chain sums: min(K, kc), with K
   cut into chunks of kc.  A slice then carries b = 53 - rho bits: its
   entries are integer multiples of 2^-b in [-1, 1], so a product of two
   slice entries is a multiple of 2^-2b of magnitude <= 1 and any fp32 sum of
   k of them is exact (k 2^2b <= 2^24): equation (11) holds exactly for every
   chunk.  The page argues exactly this way for one K tile (a bf16 product
   has 16 bits, and 128 of them sum exactly in fp32's 24).  The default kc
   is the longest chain that keeps all of Type2's bits: 2^(24 - 2 m_Type2),
   256 for bf16 and 65536 for e4m3.
2. Split (equations (1)-(5)) of each row of A and each column of B (the
   vectors x and y of the inner product x^T y in equation (10)):
   c0 = ceil(log2 max_i |x_i|) (equation (1); 0 for a zero vector), then for
   p = 0 .. s-1 with c_p = c0 - p*delta:
       sigma = 0.75 * 2^(rho + c_p)                       (2)
       v     = fl((x + sigma) - sigma)                    (3)
       x     = fl(x - v)                                  (4)
       slice_p = cvt_Type2(fl(2^-c_p * v))                (5)
   The exponents c_p are fixed from the first maximum, as in the page's fused
   split kernel (one max, then sigma and 2^-c for every slice computed up
   front).  The page states no rule for c_p with p > 0; the one used is the
   residual bound: (3) rounds x to a multiple of 2^(c_p - b), so
   |x - v| <= 2^(c_p - b - 1) and c_{p+1} = c_p - delta with delta = b + 1
   keeps |x| <= 2^c for every slice.
3. Products (equations (10), (11)): for every slice pair (p, q) in ascending
   p, then ascending q, skipping p + q >= d (Fast Mode), and for every K
   chunk in ascending order, the exact chunk product
   S = slice_p(A)[:, chunk] @ slice_q(B)[chunk, :] is scaled by
   2^(c_p(A row) + c_q(B column)) and added to an fp64 accumulator that
   starts at +0.0.

Readings where the page is open (each listed in the design notes):
  * per-row / per-column exponents: the page's listing takes one maximum per
    matrix; the equations are written for the vectors of an inner product.
    One exponent per row of A makes row i of C depend on row i of A only,
    the batch-invariance the rest of this library is built on.
  * k in gamma is the length of one exact fp32 chain (a K chunk), whose
    exact sums join the fp64 accumulator one by one; with the default chunks
    every size keeps the page's 7 bf16 / 14 e4m3 slices, as its tables show
    for all sizes up to 16384.
  * default slice count s = ceil(53 / b), the page's "ceil(m_Type1 / m_Type2)"
    with m_Type2 replaced by the bits a slice actually carries, at most 20
    (the limit of the page's split routine); default
    d = s + 2, which reproduces the page's tables (7 bf16 slices with d = 9
    giving 39 products; 14 e4m3 slices with d = 16 giving 130).

The chunk products are evaluated with numpy's fp64 matmul on the integer
slice values n = slice * 2^b: every product and every partial sum is an
integer below 2^53, so any summation order gives the exact result.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

from . import decode, round_rne

TYPE2_BITS = {"bf16": 8, "e4m3": 4, "i8": 6}   # bits of a slice entry's magnitude
TYPE3_BITS = {"bf16": 24, "e4m3": 24, "i8": 31}  # fp32 / int32 accumulator
M_TYPE1 = 53
M_TYPE3 = 24
MAX_SLICES = 20   # the page's split routine stops after at most 20 slices


@dataclass(frozen=True)
class OzakiParams:
    type2: str
    K: int
    rho: int
    b: int        # bits per slice: entries are multiples of 2^-b in [-1, 1]
    delta: int    # exponent step between consecutive slices
    s: int        # slices per operand
    d: int        # Fast Mode: pairs with p + q >= d are skipped
    kc: int       # K chunk: products per exact fp32 chain

    @property
    def pairs(self):
        return pair_list(self.s, self.d)


def gamma_of(K: int, m3: int = M_TYPE3) -> int:
    """gamma = ceil(53 - (m3 - log2 K) / 2), evaluated exactly: the smallest
    integer g with K * 4^(53 - g) <= 2^m3 (m3 = 24 for fp32 accumulation)."""
    if K < 1:
        raise ValueError("K must be positive")
    g = 0
    while K * 4 ** (M_TYPE1 - g) > 2 ** m3:
        g += 1
    return g


def default_chunk(type2: str) -> int:
    """Longest exact chain at full Type2 precision: 2^(m_Type3 - 2 m_Type2)."""
    return 2 ** (TYPE3_BITS[type2] - 2 * TYPE2_BITS[type2])


def params(K: int, type2: str = "bf16", s: int = 0, d: int = 0, kc: int = 0) -> OzakiParams:
    """Precision parameter and slice layout for an inner dimension K cut into
    exact chains of kc products (0: the default chunk)."""
    if type2 not in TYPE2_BITS:
        raise ValueError(f"unsupported Type2 {type2!r}")
    kc = kc or default_chunk(type2)
    xi = M_TYPE1 - TYPE2_BITS[type2]
    rho = max(gamma_of(max(1, min(K, kc)), TYPE3_BITS[type2]), xi)
    b = M_TYPE1 - rho
    if b < 1:
        raise ValueError(f"K = {K} leaves no bits per slice")
    s = s or min(-(-M_TYPE1 // b), MAX_SLICES)
    d = d or s + 2
    return OzakiParams(type2, int(K), rho, b, b + 1, int(s), int(d), int(kc))


def pair_list(s: int, d: int):
    """Slice pairs (p, q), 0-based, in the order they are accumulated: p
    ascending, then q ascending, without the pairs with p + q >= d."""
    return [(p, q) for p in range(s) for q in range(s) if p + q < d]


def ceil_log2(m: np.ndarray) -> np.ndarray:
    """Exact ceil(log2 m) for positive m (0 where m == 0)."""
    mant, e = np.frexp(m)
    c = np.where(mant == 0.5, e - 1, e)
    return np.where(m == 0, 0, c).astype(np.int64)


def split(x: np.ndarray, axis: int, P: OzakiParams):
    """Split x (fp64, 2-D) into P.s Type2 slices.

    axis = 1: one exponent per row (the rows of A); axis = 0: one per column
    (the columns of B).  Returns (slice bits [s, *x.shape], c0) with c0 the
    int64 exponent of each row / column.
    """
    x = np.asarray(x, dtype=np.float64)
    if x.ndim != 2:
        raise ValueError("x must be 2-D")
    c0 = ceil_log2(np.max(np.abs(x), axis=axis)) if x.size else np.zeros(x.shape[1 - axis], np.int64)
    shape = (-1, 1) if axis == 1 else (1, -1)
    r = x.copy()
    out = []
    for p in range(P.s):
        cp = (c0 - p * P.delta).reshape(shape)
        sigma = np.ldexp(0.75, P.rho + cp)             # (2)
        v = (r + sigma) - sigma                         # (3)
        r = r - v                                       # (4)
        if P.type2 == "i8":                             # (5), as the integer n
            n = np.ldexp(v, P.b - cp)
            if not (np.all(n == np.round(n)) and np.all(np.abs(n) <= 2 ** P.b)):
                raise ValueError("an int8 slice entry is not an integer in [-2^b, 2^b]")
            out.append(n.astype(np.int8))
        else:
            out.append(round_rne(P.type2, np.ldexp(v, -cp)))  # (5)
    return np.stack(out), c0


def slice_ints(slices_bits: np.ndarray, P: OzakiParams) -> np.ndarray:
    """Integer values n = slice * 2^b of the slices (as fp64)."""
    if P.type2 == "i8":
        return slices_bits.astype(np.float64)
    return np.ldexp(decode(P.type2, slices_bits), P.b)


def gemm(A: np.ndarray, B: np.ndarray, type2: str = "bf16", s: int = 0, d: int = 0,
         kc: int = 0):
    """C = A @ B by the Ozaki scheme (fp64 in, fp64 out)."""
    A = np.asarray(A, dtype=np.float64)
    B = np.asarray(B, dtype=np.float64)
    if A.ndim != 2 or B.ndim != 2 or A.shape[1] != B.shape[0]:
        raise ValueError(f"shape mismatch {A.shape} @ {B.shape}")
    K = A.shape[1]
    P = params(K, type2, s, d, kc)
    sa, ca = split(A, 1, P)
    sb, cb = split(B, 0, P)
    na, nb = slice_ints(sa, P), slice_ints(sb, P)
    C = np.zeros((A.shape[0], B.shape[1]), dtype=np.float64)
    for p, q in P.pairs:
        scale = (ca - p * P.delta)[:, None] + (cb - q * P.delta)[None, :]
        for k0 in range(0, K, P.kc):
            S = np.ldexp(na[p][:, k0:k0 + P.kc] @ nb[q][k0:k0 + P.kc, :], -2 * P.b)  # (11)
            C = C + np.ldexp(S, scale)                                             # (10)
    return C


def gemm_elems(A: np.ndarray, B: np.ndarray, ii, jj, type2: str = "bf16", s: int = 0,
               d: int = 0, kc: int = 0) -> np.ndarray:
    """C[ii[t], jj[t]] of ``gemm`` for listed positions: each needs only row
    ii[t] of A and column jj[t] of B (their exponents are their own)."""
    ii = np.asarray(ii, dtype=np.int64)
    jj = np.asarray(jj, dtype=np.int64)
    out = np.empty(ii.size, dtype=np.float64)
    for t in range(ii.size):
        out[t] = gemm(A[ii[t]:ii[t] + 1, :], B[:, jj[t]:jj[t] + 1], type2, s, d, kc)[0, 0]
    return out


def fast_mode_error_target(A: np.ndarray, B: np.ndarray) -> np.ndarray:
    """The probabilistic bound the page's Fast Mode section states as its
    accuracy target: 2 sqrt(k) u_fp64 (|A||B|)_ij, u_fp64 = 2^-53."""
    K = A.shape[1]
    return 2.0 * math.sqrt(K) * 2.0 ** -53 * (np.abs(A) @ np.abs(B))
