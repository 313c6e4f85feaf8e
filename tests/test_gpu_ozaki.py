"""GPU parity of the Ozaki-scheme fp64 product against the CPU oracle.

Source: Insight Edge blog on cuTile Python, section "倍精度行列積エミュレーション"
(split equations (1)-(5), product equations (10)-(11), Fast Mode, the fused
split kernel).  Every slice product is exact (rho from the inner dimension),
so the library and oracle/ozaki.py must agree BIT FOR BIT: the slices, the
exponents and the fp64 result.  Shapes span several output tiles with ragged
edges in M, N and K; the bench-size cases compare sampled elements, which
the oracle computes one by one from their own row and column.
"""
import numpy as np
import pytest
import torch

import invariant_matmul_amd as imm
import workloads as wl
from oracle import ozaki as OZ
from tests.helpers import dev, log

pytestmark = pytest.mark.gpu

T2_VIEW = {"bf16": (torch.int16, np.uint16), "e4m3": (torch.uint8, np.uint8),
           "i8": (torch.int8, np.int8)}


def _inputs(M, N, K, kind, seed):
    g = wl.gen(seed)
    if kind == "uniform":
        return wl.uniform64((M, K), g), wl.uniform64((K, N), g)
    if kind == "wide":
        return wl.wide64((M, K), g), wl.wide64((K, N), g)
    if kind == "int":
        A = torch.randint(-2 ** 20, 2 ** 20, (M, K), generator=g, dtype=torch.int64)
        B = torch.randint(-2 ** 20, 2 ** 20, (K, N), generator=g, dtype=torch.int64)
        return A.to(torch.float64), B.to(torch.float64)
    raise ValueError(kind)


def _run(plan, A, B):
    i = plan.info
    ws = torch.empty(max(1, imm.ozaki_workspace_size(plan)), dtype=torch.uint8, device=dev())
    C = torch.empty((i["M"], i["N"]), dtype=torch.float64, device=dev())
    imm.ozaki_run(plan, A, B, C, ws)
    torch.cuda.synchronize()
    return C, ws


def _bits64(x) -> np.ndarray:
    a = x.cpu().numpy() if isinstance(x, torch.Tensor) else np.asarray(x)
    return np.ascontiguousarray(a, dtype=np.float64).view(np.uint64)


def _slices(ws, off, shape, t2):
    eb = 2 if t2 == "bf16" else 1
    n = int(np.prod(shape))
    raw = ws[off:off + n * eb].cpu().numpy()
    return raw.view(T2_VIEW[t2][1]).reshape(shape)


@pytest.mark.parametrize("t2", ["bf16", "e4m3", "i8"])
def test_split_matches_oracle(t2):
    M, N, K = 70, 90, 150          # ragged: K and N padded to 16
    A, B = _inputs(M, N, K, "wide", 7100)
    plan = imm.ozaki_plan(M, N, K, t2)
    i = plan.info
    P = OZ.params(K, t2)
    C, ws = _run(plan, A.to(dev()), B.to(dev()))
    sa, ca = OZ.split(A.numpy(), 1, P)
    sb, cb = OZ.split(B.numpy(), 0, P)
    kp, np_ = i["k_pad"], i["n_pad"]
    ga = _slices(ws, i["a_slices_offset"], (P.s, M, kp), t2)
    gb = _slices(ws, i["b_slices_offset"], (P.s, kp, np_), t2)
    assert np.array_equal(ga[:, :, :K], sa) and not ga[:, :, K:].any()
    assert np.array_equal(gb[:, :K, :N], sb) and not gb[:, K:, :].any() and not gb[:, :, N:].any()
    ea = ws[i["a_exp_offset"]:i["a_exp_offset"] + 4 * M].cpu().numpy().view(np.int32)
    eb = ws[i["b_exp_offset"]:i["b_exp_offset"] + 4 * N].cpu().numpy().view(np.int32)
    assert np.array_equal(ea, ca) and np.array_equal(eb, cb)


CASES = [
    # (type2, M, N, K, kind, slices, d[, chunk])
    ("bf16", 300, 600, 1000, "uniform", 0, 0),
    ("bf16", 200, 300, 1000, "uniform", 0, 0, 1024),
    ("bf16", 130, 260, 1300, "wide", 0, 0, 384),
    ("e4m3", 70, 260, 700, "uniform", 0, 0, 256),
    ("e4m3", 300, 600, 1000, "uniform", 0, 0),
    ("bf16", 129, 257, 200, "wide", 0, 0),
    ("e4m3", 65, 520, 333, "wide", 0, 0),
    ("bf16", 200, 300, 256, "int", 0, 0),
    ("e4m3", 100, 100, 64, "int", 0, 0),
    ("bf16", 130, 270, 500, "uniform", 4, 3),
    ("e4m3", 70, 300, 260, "uniform", 5, 99),
    ("bf16", 1, 16, 4096, "uniform", 0, 0),
    ("e4m3", 2, 1, 1, "wide", 0, 0),
    ("i8", 300, 600, 1000, "uniform", 0, 0),
    ("i8", 129, 257, 200, "wide", 0, 0),
    ("i8", 200, 300, 256, "int", 0, 0),
    ("i8", 130, 270, 700, "uniform", 5, 4, 256),
    ("i8", 1, 16, 4096, "wide", 0, 0),
]


@pytest.mark.parametrize("case", CASES,
                         ids=[f"{c[0]}-{c[1]}x{c[2]}x{c[3]}-{c[4]}-s{c[5]}d{c[6]}"
                              + (f"c{c[7]}" if len(c) > 7 else "") for c in CASES])
def test_product_bit_exact(case):
    t2, M, N, K, kind, s, d = case[:7]
    kc = case[7] if len(case) > 7 else 0
    A, B = _inputs(M, N, K, kind, 7200 + M + N + K)
    plan = imm.ozaki_plan(M, N, K, t2, s, d, kc)
    log(f"ozaki {t2} {M}x{N}x{K} {kind}: {plan.info['slices']} slices, {plan.info['pairs']} "
        f"pairs, chunk {plan.info['chunk']}")
    C, _ = _run(plan, A.to(dev()), B.to(dev()))
    want = OZ.gemm(A.numpy(), B.numpy(), t2, s, d, kc)
    got = _bits64(C)
    bad = got != _bits64(want)
    assert not bad.any(), (f"{int(bad.sum())} of {bad.size} differ; first {np.argwhere(bad)[:3]}")
    if kind == "int":
        assert np.array_equal(C.cpu().numpy(), (A @ B).numpy())


@pytest.mark.parametrize("t2", ["bf16", "e4m3", "i8"])
def test_rows_invariant_and_repeatable(t2):
    M, N, K = 257, 300, 700
    A, B = _inputs(M, N, K, "wide", 7300)
    Ad, Bd = A.to(dev()), B.to(dev())
    full, _ = _run(imm.ozaki_plan(M, N, K, t2), Ad, Bd)
    full = _bits64(full)
    for m in (1, 7, 64, 129):
        part, _ = _run(imm.ozaki_plan(m, N, K, t2), Ad[:m].contiguous(), Bd)
        assert np.array_equal(_bits64(part), full[:m]), m
    perm = torch.randperm(M, generator=wl.gen(7301))
    pc, _ = _run(imm.ozaki_plan(M, N, K, t2), Ad[perm.to(dev())].contiguous(), Bd)
    assert np.array_equal(_bits64(pc), full[perm.numpy()])
    again, _ = _run(imm.ozaki_plan(M, N, K, t2), Ad, Bd)
    assert np.array_equal(_bits64(again), full)


def test_split_then_multiply_equals_run():
    M, N, K = 90, 130, 300
    A, B = _inputs(M, N, K, "uniform", 7400)
    Ad, Bd = A.to(dev()), B.to(dev())
    plan = imm.ozaki_plan(M, N, K, "bf16")
    C1, _ = _run(plan, Ad, Bd)
    ws = torch.zeros(imm.ozaki_workspace_size(plan), dtype=torch.uint8, device=dev())
    imm.ozaki_split(plan, 1, Bd, ws)
    imm.ozaki_split(plan, 0, Ad, ws)
    C2 = torch.empty_like(C1)
    imm.ozaki_multiply(plan, ws, C2)
    torch.cuda.synchronize()
    assert np.array_equal(_bits64(C1), _bits64(C2))


def test_edge_cases():
    # K = 0 gives +0; zero rows give +0; empty M or N enqueue nothing
    plan = imm.ozaki_plan(5, 7, 0, "bf16")
    C, _ = _run(plan, torch.empty((5, 0), dtype=torch.float64, device=dev()),
                torch.empty((0, 7), dtype=torch.float64, device=dev()))
    assert np.array_equal(_bits64(C), np.zeros((5, 7), np.uint64))
    A, B = _inputs(4, 33, 40, "uniform", 7500)
    A[1] = 0.0
    A[3] = -0.0
    C, _ = _run(imm.ozaki_plan(4, 33, 40, "e4m3"), A.to(dev()), B.to(dev()))
    assert np.array_equal(_bits64(C[[1, 3]]), np.zeros((2, 33), np.uint64))
    assert np.array_equal(_bits64(C), _bits64(OZ.gemm(A.numpy(), B.numpy(), "e4m3")))
    for M, N in ((0, 5), (5, 0)):
        plan = imm.ozaki_plan(M, N, 8, "bf16")
        ws = torch.empty(max(1, imm.ozaki_workspace_size(plan)), dtype=torch.uint8, device=dev())
        imm.ozaki_run(plan, torch.zeros((M, 8), dtype=torch.float64, device=dev()),
                      torch.zeros((8, N), dtype=torch.float64, device=dev()),
                      torch.zeros((M, N), dtype=torch.float64, device=dev()), ws)
    torch.cuda.synchronize()


@pytest.mark.parametrize("name", ["ozaki_bf16_8192", "ozaki_e4m3_8192", "ozaki_i8_8192"])
def test_bench_size_sampled(name):
    """The configuration the benchmark times, checked on sampled elements."""
    w = wl.OZAKI_WORKLOADS[name]
    A, B = w.make()
    plan = imm.ozaki_plan(w.n, w.n, w.n, w.type2)
    C, _ = _run(plan, A.to(dev()), B.to(dev()))
    r = np.random.default_rng(7600)
    ii = np.concatenate([r.integers(0, w.n, 40), [0, w.n - 1, w.n - 1]])
    jj = np.concatenate([r.integers(0, w.n, 40), [w.n - 1, 0, w.n - 1]])
    want = OZ.gemm_elems(A.numpy(), B.numpy(), ii, jj, w.type2)
    got = C.cpu().numpy()[ii, jj]
    assert np.array_equal(_bits64(got), _bits64(want))
    # and it is an fp64-accurate product: within the page's Fast Mode target
    ab = np.abs(A.numpy()[ii]) * np.abs(B.numpy()[:, jj]).T
    exact = np.array([np.sum(A.numpy()[i] * B.numpy()[:, j]) for i, j in zip(ii, jj)])
    assert np.all(np.abs(got - exact) <= 2 * np.sqrt(w.n) * 2.0 ** -53 * ab.sum(axis=1)
                  + w.n * 2.0 ** -53 * ab.sum(axis=1))


def _fuzz_cases(n=16, seed=7700):
    r = np.random.default_rng(seed)
    out = []
    for i in range(n):
        t2 = ["bf16", "e4m3", "i8"][i % 3]
        M, N, K = int(r.integers(1, 300)), int(r.integers(1, 600)), int(r.integers(1, 1500))
        s = int(r.integers(1, 13)) if r.random() < 0.5 else 0
        d = int(r.integers(1, 2 * max(s, 7))) if r.random() < 0.5 else 0
        kc = 128 * int(r.integers(1, 9)) if r.random() < 0.4 else 0
        kind = ["uniform", "wide", "int"][int(r.integers(0, 3))]
        out.append((t2, M, N, K, kind, s, d, kc, 7800 + i))
    return out


@pytest.mark.parametrize("case", _fuzz_cases(), ids=lambda c: f"{c[0]}-{c[1]}x{c[2]}x{c[3]}-{c[4]}-s{c[5]}d{c[6]}c{c[7]}")
def test_seeded_sweep_bit_exact(case):
    """Random shapes, slice formats, slice counts, Fast Mode thresholds and
    chunk lengths: every one bit-exact against the oracle."""
    t2, M, N, K, kind, s, d, kc, seed = case
    A, B = _inputs(M, N, K, kind, seed)
    plan = imm.ozaki_plan(M, N, K, t2, s, d, kc)
    log(f"sweep {case}: {plan.info['slices']} slices, {plan.info['pairs']} pairs, "
        f"chunk {plan.info['chunk']}")
    C, _ = _run(plan, A.to(dev()), B.to(dev()))
    want = OZ.gemm(A.numpy(), B.numpy(), t2, s, d, kc)
    bad = _bits64(C) != _bits64(want)
    assert not bad.any(), f"{int(bad.sum())} of {bad.size} differ; first {np.argwhere(bad)[:3]}"


def test_long_K_wider_column_chunks():
    """K beyond 16384 x 256: the column maxima of B use wider chunks."""
    M, N, K = 1, 2, 16384 * 256 + 1000
    A, B = _inputs(M, N, K, "wide", 7900)
    plan = imm.ozaki_plan(M, N, K, "i8")
    C, _ = _run(plan, A.to(dev()), B.to(dev()))
    want = OZ.gemm(A.numpy(), B.numpy(), "i8")
    assert np.array_equal(_bits64(C), _bits64(want))


@pytest.mark.parametrize("t2", ["bf16", "e4m3", "i8"])
def test_rows_and_columns_outside_the_domain_give_nan(t2):
    """A row of A or a column of B holding a NaN, an infinity, a magnitude
    above 2^300 or a nonzero maximum below 2^-300 is outside the domain: its
    exponent is the marker -2^30, its slices are zero, and its whole row or
    column of C is NaN.  Every other entry keeps the oracle's bits (rows and
    columns are split independently)."""
    M, N, K = 70, 90, 200
    A, B = _inputs(M, N, K, "uniform", 7700)
    A, B = A.clone(), B.clone()
    A[3, 5] = float("nan")
    A[5, 0] = float("inf")
    A[7, 10] = 2.0 ** 301
    A[9, :] = A[9, :] * 2.0 ** -330           # nonzero maximum below 2^-300
    B[7, 2] = float("-inf")
    B[150, 4] = float("nan")
    B[0, 60] = -(2.0 ** 302)
    bad_rows, bad_cols = [3, 5, 7, 9], [2, 4, 60]
    plan = imm.ozaki_plan(M, N, K, t2)
    i = plan.info
    C, ws = _run(plan, A.to(dev()), B.to(dev()))
    got = C.cpu().numpy()
    assert np.isnan(got[bad_rows, :]).all() and np.isnan(got[:, bad_cols]).all()
    ea = ws[i["a_exp_offset"]:i["a_exp_offset"] + 4 * M].cpu().numpy().view(np.int32)
    eb = ws[i["b_exp_offset"]:i["b_exp_offset"] + 4 * N].cpu().numpy().view(np.int32)
    assert (ea[bad_rows] == -(1 << 30)).all() and (eb[bad_cols] == -(1 << 30)).all()
    # the rest: the oracle on the same data with the bad vectors cleared
    Ac, Bc = A.clone(), B.clone()
    Ac[bad_rows, :] = 0.0
    Bc[:, bad_cols] = 0.0
    want = OZ.gemm(Ac.numpy(), Bc.numpy(), t2)
    good_r = [r for r in range(M) if r not in bad_rows]
    good_c = [c for c in range(N) if c not in bad_cols]
    assert np.array_equal(_bits64(got[np.ix_(good_r, good_c)]), _bits64(want[np.ix_(good_r, good_c)]))
    assert not np.isnan(got[np.ix_(good_r, good_c)]).any()


@pytest.mark.parametrize("t2", ["bf16", "e4m3", "i8"])
def test_pair_outer_chunk_inner_order(t2):
    """The kernel adds the exact chunk products to the fp64 sum pair by pair,
    chunks inside each pair (the page's fused kernel, "行列積の計算": the K loop
    inside the slice-pair loops).  On the hand-traced case of the oracle's
    nesting pin that order gives exactly 2^-70; chunks outside the pairs would
    give 0.  Rows 1.. and the other columns are zero-padded copies."""
    from tests.test_oracle_ozaki import nesting_case
    K, kc = 256, 128
    x, y = nesting_case(K, kc)
    A = np.zeros((5, K))
    A[0] = x[0]
    A[3] = -x[0]
    B = np.zeros((K, 20))
    B[:, 0] = y[:, 0]
    B[:, 17] = y[:, 0]
    plan = imm.ozaki_plan(5, 20, K, t2, chunk=kc)
    C, _ = _run(plan, torch.from_numpy(A).to(dev()), torch.from_numpy(B).to(dev()))
    want = OZ.gemm(A, B, t2, kc=kc)
    assert want[0, 0] == 2.0 ** -70 and want[3, 17] == -(2.0 ** -70)
    assert np.array_equal(_bits64(C), _bits64(want))
