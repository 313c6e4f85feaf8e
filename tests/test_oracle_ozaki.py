"""Pins of the Ozaki-scheme oracle (oracle/ozaki.py) to facts that do not come
from the oracle itself: the page's product counts, exact rational arithmetic,
integer brute force, closed forms (identity, powers of two, sign) and the
page's stated accuracy target.

Source: Insight Edge blog on cuTile Python, sections "分解(Split)",
"行列積の計算", "Fast Mode（GEMMの削減）", "最適化後の結果" and
"dによる精度/速度トレードオフ".

Every pin takes the oracle module as an argument so that
test_mutants_are_caught can run the same pins against copies of the oracle
with a planted mistake.
"""
from __future__ import annotations

import importlib.util
import math
import os
import sys
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import ozaki as OZ

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "ozaki_gemm_counts.txt")
TORCH_T2 = {"bf16": torch.bfloat16, "e4m3": torch.float8_e4m3fn}


def _rng(seed):
    return np.random.default_rng(seed)


def _exact_product(A, B):
    """A @ B in exact rational arithmetic."""
    M, K = A.shape
    N = B.shape[1]
    Af = [[Fraction(float(v)) for v in row] for row in A]
    Bf = [[Fraction(float(B[k, j])) for k in range(K)] for j in range(N)]
    return [[sum((a * b for a, b in zip(Af[i], Bf[j])), Fraction(0)) for j in range(N)]
            for i in range(M)]


# ---------------------------------------------------------------- pins

def pin_pair_counts(oz=OZ):
    for line in open(GOLDEN, encoding="utf-8"):
        if line.startswith("#") or not line.strip():
            continue
        t2, s, d, n = line.split()
        s, d, n = int(s), int(d), int(n)
        assert len(oz.pair_list(s, d if d else 2 * s)) == n, line
    # the defaults reproduce the page's optimised configurations
    P = oz.params(256, "bf16")
    assert (P.s, P.d, len(P.pairs)) == (7, 9, 39)
    for K in (64, 4096, 65536):
        P = oz.params(K, "e4m3")
        assert (P.s, len(P.pairs)) == (14, 130)
    # ... at every size of the page's tables (1024 .. 16384: 7 x 7 bf16 slices)
    for K in (1024, 2048, 4096, 8192, 16384):
        P = oz.params(K, "bf16")
        assert (P.s, P.d, len(P.pairs)) == (7, 9, 39)
    # int8 slices: 6 bits each, exact in int32 up to chains of 2^19 products
    P = oz.params(16384, "i8")
    assert (P.b, P.kc, P.s, P.d, len(P.pairs)) == (6, 2 ** 19, 9, 11, 60)


def pin_gamma_formula(oz=OZ):
    # gamma = ceil(53 - (24 - log2 k) / 2) as printed, evaluated in floating
    # point away from its integer boundaries
    for K in [1, 2, 3, 7, 64, 100, 255, 256, 257, 1000, 4096, 5000, 16384, 65536, 131072]:
        want = math.ceil(53 - (24 - math.log2(K)) / 2)
        assert oz.gamma_of(K) == want, K
    # rho = max(gamma, xi), xi = 53 - m_Type2
    assert oz.params(256, "bf16").rho == 45 and oz.params(256, "e4m3").rho == 49
    # k is the length of one exact chain: the whole K when it is one chunk
    assert oz.params(16384, "bf16", kc=16384).rho == 48
    assert oz.params(16384, "bf16").rho == 45 and oz.params(1000, "bf16", kc=4096).rho == 46
    # int32 accumulation: gamma = ceil(53 - (31 - log2 k) / 2)
    for K in (1, 1000, 2 ** 19, 2 ** 21):
        assert oz.gamma_of(K, 31) == math.ceil(53 - (31 - math.log2(K)) / 2)


def pin_slices_are_type2_on_grid(oz=OZ):
    x = _rng(1).standard_normal((9, 70)) * np.ldexp(1.0, _rng(2).integers(-30, 30, (9, 1)))
    for t2 in ("bf16", "e4m3", "i8"):
        P = oz.params(70, t2)
        sl, c0 = oz.split(x, 1, P)
        if t2 == "i8":
            assert sl.dtype == np.int8 and np.all(np.abs(sl.astype(int)) <= 2 ** P.b)
            continue
        vals = oracle.decode(t2, sl)
        n = np.ldexp(vals, P.b)
        assert np.all(n == np.round(n)) and np.all(np.abs(n) <= 2 ** P.b)
        # the values are Type2 numbers: torch's own cast leaves them unchanged
        rt = torch.from_numpy(vals).to(TORCH_T2[t2]).to(torch.float64).numpy()
        assert np.array_equal(rt, vals)
        # equation (1): 2^(c0-1) < max|x| <= 2^c0 per row
        m = np.abs(x).max(axis=1)
        assert np.all(m <= np.ldexp(1.0, c0)) and np.all(m > np.ldexp(1.0, c0 - 1))


def pin_split_reconstructs(oz=OZ):
    """Equation (9): x = sum_p 2^c_p slice_p, exactly, when every element lies
    within a few binades of its row maximum (all of its bits are captured)."""
    r = _rng(3)
    x = r.uniform(0.25, 1.0, (6, 40)) * r.choice([-1.0, 1.0], (6, 40))
    x *= np.ldexp(1.0, r.integers(-40, 40, (6, 1)))
    for t2 in ("bf16", "e4m3", "i8"):
        P = oz.params(40, t2)
        sl, c0 = oz.split(x, 1, P)
        vals = np.ldexp(oz.slice_ints(sl, P), -P.b)
        for i in range(x.shape[0]):
            for k in range(x.shape[1]):
                terms = [math.ldexp(vals[p, i, k], int(c0[i]) - p * P.delta) for p in range(P.s)]
                assert math.fsum(terms) == x[i, k]
    # column split of the transpose gives the transposed slices
    P = oz.params(40, "bf16")
    slr, cr = oz.split(x, 1, P)
    slc, cc = oz.split(np.ascontiguousarray(x.T), 0, P)
    assert np.array_equal(cr, cc) and np.array_equal(slr, slc.transpose(0, 2, 1))


def pin_split_residual_bound(oz=OZ):
    """In general |x - sum_p 2^c_p slice_p| <= 2^(c0 - s*delta) (exact check)."""
    r = _rng(4)
    x = r.standard_normal((4, 33)) * np.ldexp(1.0, r.integers(-60, 0, (4, 33)))
    P = oz.params(33, "bf16", s=4)
    sl, c0 = oz.split(x, 1, P)
    vals = oracle.decode("bf16", sl)
    for i in range(4):
        bound = Fraction(2) ** (int(c0[i]) - P.s * P.delta)
        for k in range(33):
            rec = sum(Fraction(float(vals[p, i, k])) * Fraction(2) ** (int(c0[i]) - p * P.delta)
                      for p in range(P.s))
            assert abs(Fraction(float(x[i, k])) - rec) <= bound


def pin_integer_inputs_exact(oz=OZ):
    r = _rng(5)
    A = r.integers(-2 ** 20, 2 ** 20, (7, 64))
    B = r.integers(-2 ** 20, 2 ** 20, (64, 5))
    want = A.astype(object) @ B.astype(object)
    for t2, kc in (("bf16", 0), ("e4m3", 0), ("i8", 0), ("bf16", 16), ("e4m3", 24), ("bf16", 64),
                   ("i8", 40)):
        C = oz.gemm(A.astype(np.float64), B.astype(np.float64), t2, kc=kc)
        assert C.shape == (7, 5)
        assert all(int(C[i, j]) == want[i, j] and C[i, j] == float(want[i, j])
                   for i in range(7) for j in range(5)), (t2, kc)


def pin_identity(oz=OZ):
    r = _rng(6)
    A = r.uniform(0.5, 1.0, (5, 48)) * r.choice([-1.0, 1.0], (5, 48)) * 4.0
    eye = np.eye(48)
    for t2 in ("bf16", "e4m3", "i8"):
        assert np.array_equal(oz.gemm(A, eye, t2).view(np.uint64), A.view(np.uint64))
        assert np.array_equal(oz.gemm(eye, A.T.copy(), t2), A.T)


def pin_powers_of_two_and_sign(oz=OZ):
    r = _rng(7)
    A = r.standard_normal((6, 50))
    B = r.standard_normal((50, 4))
    C = oz.gemm(A, B, "bf16")
    assert np.array_equal(oz.gemm(A * 128.0, B, "bf16"), C * 128.0)
    assert np.array_equal(oz.gemm(A, B / 1024.0, "bf16"), C / 1024.0)
    assert np.array_equal(oz.gemm(-A, B, "bf16"), -C)


def pin_rows_independent(oz=OZ):
    r = _rng(8)
    A = r.standard_normal((9, 40)) * np.ldexp(1.0, r.integers(-8, 8, (9, 1)))
    B = r.standard_normal((40, 6))
    C = oz.gemm(A, B, "e4m3")
    assert np.array_equal(oz.gemm(A[3:5], B, "e4m3"), C[3:5])
    Ci = oz.gemm(A, B, "i8")
    assert np.array_equal(oz.gemm(A[[8, 2]], B, "i8"), Ci[[8, 2]])
    assert np.array_equal(oz.gemm(A[[7, 0]], B, "e4m3"), C[[7, 0]])
    assert np.array_equal(oz.gemm(A, B[:, 2:5], "e4m3"), C[:, 2:5])


def _rigorous_bound(oz, A, B, P, chunks=1):
    """Truncation of both operands, the skipped pairs and the fp64 sums, from
    the residual bound of the split (|x^(p)| <= 2^c_p) -- not from the
    oracle's code."""
    K = A.shape[1]
    ca = oz.ceil_log2(np.abs(A).max(axis=1)).astype(float)
    cb = oz.ceil_log2(np.abs(B).max(axis=0)).astype(float)
    ea = np.exp2(ca - P.s * P.delta)[:, None]          # |residual of A| per row
    eb = np.exp2(cb - P.s * P.delta)[None, :]
    trunc = ea * np.abs(B).sum(axis=0)[None, :] + np.abs(A).sum(axis=1)[:, None] * eb + K * ea * eb
    skipped = sum(2.0 ** (-(p + q) * P.delta) for p in range(P.s) for q in range(P.s)
                  if p + q >= P.d)
    dropped = K * np.exp2(ca[:, None] + cb[None, :]) * skipped
    # every slice term is at most 2^c_p in magnitude
    sa = (np.abs(A) + np.exp2(ca - P.delta + 1)[:, None])
    sb = (np.abs(B) + np.exp2(cb - P.delta + 1)[None, :])
    rounding = len(P.pairs) * chunks * 2.0 ** -53 * (sa @ sb)
    return trunc + dropped + rounding


def pin_random_vs_exact(oz=OZ):
    r = _rng(9)
    for t2, (M, K, N), kc in (("bf16", (4, 96, 3), 0), ("e4m3", (3, 70, 4), 0),
                              ("bf16", (3, 100, 3), 32), ("i8", (3, 90, 3), 0)):
        A = r.uniform(-1.0, 1.0, (M, K))
        B = r.uniform(-1.0, 1.0, (K, N))
        C = oz.gemm(A, B, t2, kc=kc)
        ex = _exact_product(A, B)
        err = np.array([[abs(Fraction(float(C[i, j])) - ex[i][j]) for j in range(N)]
                        for i in range(M)], dtype=float)
        # the page's Fast Mode accuracy target ...
        assert np.all(err <= OZ.fast_mode_error_target(A, B)), t2
        # ... and with one chunk the result is the exact product to a few ulps
        # (several chunks round against partial sums, which may exceed |C|)
        if not kc:
            assert np.all(err <= 4 * 2.0 ** -53 * np.abs(C)), t2
    # wide dynamic range, fewer slices and pairs: the derived bound
    A = r.standard_normal((3, 64)) * np.ldexp(1.0, r.integers(-20, 20, (3, 64)))
    B = r.standard_normal((64, 3)) * np.ldexp(1.0, r.integers(-20, 20, (64, 3)))
    for s, d, kc in ((5, 5, 0), (4, 3, 0), (9, 0, 0), (6, 6, 16)):
        P = oz.params(64, "bf16", s, d, kc)
        C = oz.gemm(A, B, "bf16", s, d, kc)
        ex = _exact_product(A, B)
        err = np.array([[abs(Fraction(float(C[i, j])) - ex[i][j]) for j in range(3)]
                        for i in range(3)], dtype=float)
        assert np.all(err <= _rigorous_bound(oz, A, B, P, -(-64 // P.kc))), (s, d, kc)


def pin_vs_numpy(oz=OZ):
    r = _rng(10)
    A = r.uniform(-1.0, 1.0, (33, 300))
    B = r.uniform(-1.0, 1.0, (300, 17))
    C = oz.gemm(A, B, "bf16")
    ab = np.abs(A) @ np.abs(B)
    assert np.all(np.abs(C - A @ B) <= OZ.fast_mode_error_target(A, B) + 300 * 2.0 ** -53 * ab)


def pin_elems_match_full(oz=OZ):
    r = _rng(11)
    A = r.standard_normal((12, 80))
    B = r.standard_normal((80, 9))
    C = oz.gemm(A, B, "e4m3")
    ii, jj = [0, 11, 5, 5], [8, 0, 3, 4]
    assert np.array_equal(oz.gemm_elems(A, B, ii, jj, "e4m3"), C[ii, jj])


def pin_chunking_only_moves_roundings(oz=OZ):
    """Chunks change which fp64 additions round, never the exact value: on
    inputs where every partial sum is exact, any chunk length gives the same
    bits; on random inputs the results agree to a few ulps."""
    r = _rng(13)
    A = r.integers(-1000, 1000, (5, 200)).astype(np.float64) / 64
    B = r.integers(-1000, 1000, (200, 4)).astype(np.float64) / 128
    base = oz.gemm(A, B, "bf16", kc=200)
    for kc in (16, 48, 64, 128):
        assert np.array_equal(oz.gemm(A, B, "bf16", kc=kc), base), kc
    A = r.standard_normal((5, 300))
    B = r.standard_normal((300, 4))
    ab = np.abs(A) @ np.abs(B)
    c1, c2 = oz.gemm(A, B, "bf16", kc=256), oz.gemm(A, B, "bf16", kc=32)
    assert np.all(np.abs(c1 - c2) <= 64 * 2.0 ** -53 * ab)


def nesting_case(K, kc):
    """One row x and one column y whose exact chunk products are known by hand
    (row and column maxima 1, so c0 = 0 on both sides):
      chunk 0: x_0 y_0 = 1 at slice pair (0, 0); x_1 y_1 = 2^-35 2^-35 = 2^-70,
               whose only nonzero slices are at a depth p with p delta = 35 or
               more, so it is a term of a deeper pair than (0, 0);
      chunk 1 (k = kc): x_kc y_kc = -1 at slice pair (0, 0).
    Every other term is zero."""
    x = np.zeros((1, K))
    y = np.zeros((K, 1))
    x[0, 0], y[0, 0] = 1.0, 1.0
    x[0, 1], y[1, 0] = 2.0 ** -35, 2.0 ** -35
    x[0, kc], y[kc, 0] = -1.0, 1.0
    return x, y


def pin_pair_outer_chunk_inner_order(oz=OZ):
    """The page's fused kernel ("行列積の計算") runs the K loop inside the loop
    over slice pairs and adds each pair's product to the fp64 result; with K
    cut into exact chunks, the chunk loop sits inside the pair loop.  Written
    out in that order for nesting_case, the fp64 additions are
        pair (0, 0): 0 + 1 = 1, then 1 + (-1) = 0;
        the pairs in between add +0;
        the deeper pair holding x_1 y_1: 0 + 2^-70 = 2^-70,
    which is also the exact product.  Chunk-outer order would add 2^-70 to 1
    (lost: 1 + 2^-70 rounds to 1) before the -1 of chunk 1, and give 0."""
    for t2 in ("bf16", "e4m3", "i8"):
        for K, kc in ((32, 16), (256, 128)):
            x, y = nesting_case(K, kc)
            C = oz.gemm(x, y, t2, kc=kc)
            assert C.shape == (1, 1) and C[0, 0] == 2.0 ** -70, (t2, K, kc, C[0, 0])


def pin_zero_rows(oz=OZ):
    A = np.zeros((3, 32))
    A[1] = np.arange(32) - 7.5
    B = _rng(12).standard_normal((32, 4))
    C = oz.gemm(A, B, "bf16")
    assert np.all(C[[0, 2]] == 0) and not np.any(np.signbit(C[[0, 2]]))


PINS = [pin_pair_counts, pin_gamma_formula, pin_slices_are_type2_on_grid,
        pin_split_reconstructs, pin_split_residual_bound, pin_integer_inputs_exact,
        pin_identity, pin_powers_of_two_and_sign, pin_rows_independent,
        pin_random_vs_exact, pin_vs_numpy, pin_elems_match_full, pin_chunking_only_moves_roundings,
        pin_pair_outer_chunk_inner_order, pin_zero_rows]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin()


# ------------------------------------------------------------- mutants

MUTANTS = [
    ("skip_rule_off_by_one", "if p + q < d]", "if p + q <= d]"),
    ("sigma_not_subtracted", "v = (r + sigma) - sigma ", "v = (r + sigma) - 2 * sigma "),
    ("residual_not_updated", "r = r - v  ", "r = r  "),
    ("scale_sign", "scale = (ca - p * P.delta)[:, None] + (cb - q * P.delta)[None, :]",
     "scale = (ca + p * P.delta)[:, None] + (cb - q * P.delta)[None, :]"),
    ("B_rows_reversed", "@ nb[q][k0:k0 + P.kc, :], -2 * P.b)",
     "@ nb[q][k0:k0 + P.kc, :][::-1], -2 * P.b)"),
    ("chunk_scale_missing", "C = C + np.ldexp(S, scale)", "C = C + S"),
    ("one_max_per_matrix", "c0 = ceil_log2(np.max(np.abs(x), axis=axis))",
     "c0 = ceil_log2(np.max(np.abs(x)) + 0 * np.max(np.abs(x), axis=axis))"),
    ("delta_too_small", "return OzakiParams(type2, int(K), rho, b, b + 1, int(s), int(d), int(kc))",
     "return OzakiParams(type2, int(K), rho, b, b - 1, int(s), int(d), int(kc))"),
    ("gamma_without_log", "while K * 4 ** (M_TYPE1 - g) > 2 ** m3:",
     "while 4 ** (M_TYPE1 - g) > 2 ** m3:"),
    ("int8_accumulates_in_fp32", "rho = max(gamma_of(max(1, min(K, kc)), TYPE3_BITS[type2]), xi)",
     "rho = max(gamma_of(max(1, min(K, kc))), xi)"),
    ("ceil_log2_floor", "c = np.where(mant == 0.5, e - 1, e)", "c = e - 1"),
    ("first_chunk_dropped", "for k0 in range(0, K, P.kc):", "for k0 in range(P.kc, K, P.kc):"),
    ("chunk_rho_from_K", "rho = max(gamma_of(max(1, min(K, kc)), TYPE3_BITS[type2]), xi)",
     "rho = max(gamma_of(max(1, kc), TYPE3_BITS[type2]), xi)"),
    ("first_slice_dropped", "for p in range(P.s):\n        cp =",
     "for p in range(P.s):\n        if p == 0: r = r - ((r + np.ldexp(0.75, P.rho + c0.reshape(shape))) - np.ldexp(0.75, P.rho + c0.reshape(shape)))\n        cp ="),
    # the chunk loop outside the pair loop: the same terms, other fp64 roundings
    ("chunk_outer_pair_inner",
     "    for p, q in P.pairs:\n        scale = (ca - p * P.delta)[:, None] + (cb - q * P.delta)[None, :]\n"
     "        for k0 in range(0, K, P.kc):\n",
     "    for k0 in range(0, K, P.kc):\n      for p, q in P.pairs:\n"
     "        scale = (ca - p * P.delta)[:, None] + (cb - q * P.delta)[None, :]\n        if True:\n"),
]


def _mutant_module(tmp_path, name, old, new):
    src = open(OZ.__file__, encoding="utf-8").read()
    assert src.count(old) == 1, f"mutation site for {name} not unique/found"
    src = src.replace(old, new).replace("from . import decode, round_rne",
                                        "from oracle import decode, round_rne")
    path = tmp_path / f"oz_{name}.py"
    path.write_text(src, encoding="utf-8")
    spec = importlib.util.spec_from_file_location(f"oz_{name}", path)
    mod = importlib.util.module_from_spec(spec)
    sys.modules[spec.name] = mod
    spec.loader.exec_module(mod)
    return mod


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, old, new):
    mod = _mutant_module(tmp_path, name, old, new)
    for pin in PINS:
        try:
            pin(mod)
        except (AssertionError, ValueError, OverflowError, IndexError):
            return
    pytest.fail(f"no pin failed for the planted mistake {name!r}")
