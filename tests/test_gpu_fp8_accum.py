"""fp8 through the fp16 step (GEMM_PLAN_FP8_FP32_ACCUM) against the oracle.

The mode widens every fp8 value to fp16 in registers and accumulates with the
16x16x32 fp16 matrix-core step, so its result obeys the fp32 accumulation
bound K 2^-24 (|A||B|)_ij (the Tencent deterministic-inference article,
"背景": fp32 accumulation) at every K, with no allowance for the fp8 step's
window.  Checked here: the widening of every fp8 code, the plain bound at
short K on every DMA tile and both B layouts, products the fp8 step drops,
bit-exact integer products up to a full-size square, and the invariance
rules (tile, M, split entry point, persistent launch, B layout).
"""
import numpy as np
import pytest
import torch

import invariant_matmul_amd as imm
import oracle
import workloads as wl
from tests.helpers import (FP8, bits_of, check_bound, dev, expected_bits, log, run, values_of)

pytestmark = pytest.mark.gpu

ACC = imm.PLAN_FP8_FP32_ACCUM
DMA_TILES = ["256x256", "128x256", "64x256", "32x256"]
TORCH_F8 = {"e4m3": torch.float8_e4m3fn, "e5m2": torch.float8_e5m2}
ONE = {"e4m3": 0x38, "e5m2": 0x3C}   # the code of 1.0


def _plan(M, N, K, dt, out="f32", tile="default", split=0, flags=0):
    return imm.gemm_plan_ex2(M, N, K, dt, out, split_k=split, tile=tile, flags=ACC | flags)


def _f8(codes: np.ndarray, dt: str) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).view(TORCH_F8[dt])


def _finite_codes(dt):
    c = np.arange(256, dtype=np.uint8)
    v = oracle.decode(dt, c)
    return c[np.isfinite(v)]


@pytest.mark.parametrize("dt", FP8)
def test_every_finite_code_widens_exactly(dt):
    # C = A x I puts every code of A's rows in C, C = I x B every code of B's
    # columns: the widened value must be the code's value, bit for bit.
    codes = _finite_codes(dt)
    K = 256
    row = np.zeros(K, dtype=np.uint8)
    row[:codes.size] = codes
    eye = np.where(np.eye(K, dtype=bool), ONE[dt], 0).astype(np.uint8)
    a = np.tile(row, (16, 1))
    c64 = oracle.gemm(a, eye, dt)[0]
    nz = row != 0x80  # -0 times 1 plus +0 products is +0
    assert np.array_equal(c64[0][nz], oracle.decode(dt, row)[nz])
    want = expected_bits(c64, "f32")
    p = _plan(16, K, K, dt, tile="32x256")
    assert np.array_equal(bits_of(run(p, _f8(a, dt).to(dev()), _f8(eye, dt).to(dev()), False)), want)
    b = np.tile(row[:, None], (1, 32))
    want_b = expected_bits(oracle.gemm(eye, b, dt)[0], "f32")
    p = _plan(K, 32, K, dt, tile="32x256")
    assert np.array_equal(bits_of(run(p, _f8(eye, dt).to(dev()), _f8(b, dt).to(dev()), False)), want_b)


@pytest.mark.parametrize("dt", FP8)
def test_nan_and_infinity_propagate(dt):
    K = 64
    g = wl.gen(13000)
    A = wl.integers((32, K), dt, g)
    B = wl.integers((K, 32), dt, g)
    a = wl.bits(A).copy()
    nan = 0x7F if dt == "e4m3" else 0x7E
    a[3, 5] = nan
    if dt == "e5m2":
        a[7, 9] = 0x7C  # +inf
    Cd = run(_plan(32, 32, K, dt), _f8(a, dt).to(dev()), B.to(dev()), False)
    C, got = values_of(Cd), bits_of(Cd)
    C64, _ = oracle.gemm(a, wl.bits(B), dt)
    assert np.isnan(C64).any()
    assert np.array_equal(np.isnan(C), np.isnan(C64))
    inf = np.isinf(C64)
    assert np.array_equal(C[inf], C64[inf])
    fin = np.isfinite(C64)
    assert np.array_equal(got[fin], expected_bits(C64[fin], "f32"))


@pytest.mark.parametrize("dt", FP8)
@pytest.mark.parametrize("bt", [False, True])
def test_short_k_plain_bound_every_tile(dt, bt):
    # the K range where the fp8 step needs its window allowance; ragged M, N
    g = wl.gen(13100 + FP8.index(dt) + 2 * bt)
    M, N = 75, 272
    for K in (16, 32, 48, 64, 96, 128, 256):
        A = wl.normal((M, K), dt, g)
        B = wl.normal((K, N), dt, g)
        C64, Ca = oracle.gemm(wl.bits(A), wl.bits(B), dt)
        Ad = A.to(dev())
        Bd = (B.t().contiguous() if bt else B).to(dev())
        for out in ("f32", "bf16"):
            for tile in DMA_TILES:
                p = _plan(M, N, K, dt, out, tile, flags=imm.PLAN_B_TRANSPOSED if bt else 0)
                r = check_bound(values_of(run(p, Ad, Bd, False)), C64, Ca, K, out)
                r2 = check_bound(values_of(run(p, Ad, Bd, True)), C64, Ca, K, out)
                log(f"{dt} bt={bt} K={K} {out} {tile}: max err/bound {max(r, r2):.3g}")


@pytest.mark.parametrize("dt", FP8)
def test_products_the_fp8_step_drops_are_kept(dt):
    # One product 1 and seven of 2^-14 in one group of 8 K positions: exactly
    # 1 + 7 2^-14 in fp32.  The fp8 step's window ends 13 binades below the
    # group's largest product and drops the seven; this mode keeps them.
    K = 32
    a = np.zeros((16, K))
    b = np.zeros((K, 16))
    a[:, 0] = 1.0
    b[0, :] = 1.0
    a[:, 1:8] = 2.0 ** -7
    b[1:8, :] = 2.0 ** -7
    A = torch.from_numpy(a.astype(np.float32)).to(TORCH_F8[dt])
    B = torch.from_numpy(b.astype(np.float32)).to(TORCH_F8[dt])
    assert np.array_equal(oracle.decode(dt, wl.bits(A)), a)
    exact = 1.0 + 7 * 2.0 ** -14
    fast = values_of(run(imm.gemm_plan_ex2(16, 16, K, dt, "f32"), A.to(dev()), B.to(dev()), False))
    acc = values_of(run(_plan(16, 16, K, dt), A.to(dev()), B.to(dev()), False))
    log(f"{dt}: fp8 step {fast[0, 0]!r}, fp16 step {acc[0, 0]!r}, exact {exact!r}")
    assert np.all(acc == exact)
    assert np.all(fast < exact)  # the default mode's fp8 step drops some of them


@pytest.mark.parametrize("dt", FP8)
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_integer_inputs_bit_exact_ragged(dt, out):
    M, N, K = 300, 272, 384
    g = wl.gen(13200 + FP8.index(dt))
    A = wl.integers((M, K), dt, g)
    B = wl.integers((K, N), dt, g)
    want = expected_bits(oracle.gemm(wl.bits(A), wl.bits(B), dt)[0], out)
    Ad, Bd, Btd = A.to(dev()), B.to(dev()), B.t().contiguous().to(dev())
    for tile in DMA_TILES:
        for split in (1, 3):
            p = _plan(M, N, K, dt, out, tile, split)
            assert np.array_equal(bits_of(run(p, Ad, Bd, False)), want), (tile, "run")
            assert np.array_equal(bits_of(run(p, Ad, Bd, True)), want), (tile, split)
            pt = _plan(M, N, K, dt, out, tile, split, flags=imm.PLAN_B_TRANSPOSED)
            assert np.array_equal(bits_of(run(pt, Ad, Btd, False)), want), (tile, "bt")


@pytest.mark.parametrize("dt", FP8)
def test_bits_invariant_across_tiles_m_entry_points_and_layouts(dt):
    g = wl.gen(13300 + FP8.index(dt))
    M, N, K = 512, 512, 1024
    A = wl.normal((M, K), dt, g).to(dev())
    B = wl.normal((K, N), dt, g).to(dev())
    Bt = B.t().contiguous()
    ref = bits_of(run(_plan(M, N, K, dt), A, B, False))
    for tile in DMA_TILES:
        for flags, Bx in ((0, B), (imm.PLAN_B_TRANSPOSED, Bt), (imm.PLAN_PERSISTENT, B)):
            p = _plan(M, N, K, dt, "f32", tile, flags=flags)
            assert np.array_equal(bits_of(run(p, A, Bx, False)), ref), (tile, flags)
        # the split-K entry point with one slice gives gemm_run's bits
        p1 = _plan(M, N, K, dt, "f32", tile, 1)
        assert np.array_equal(bits_of(run(p1, A, B, True)), ref), (tile, "split 1")
    # rows computed in a smaller batch are the same rows
    for m in (1, 7, 200):
        got = bits_of(run(_plan(m, N, K, dt), A[:m].contiguous(), B, False))
        assert np.array_equal(got, ref[:m]), m
    # a split of K is its own, M-independent result
    s4 = bits_of(run(_plan(M, N, K, dt, split=4), A, B, True))
    s4m = bits_of(run(_plan(9, N, K, dt, split=4), A[:9].contiguous(), B, True))
    assert np.array_equal(s4m, s4[:9])


def test_full_size_square_e5m2_8192():
    w = wl.WORKLOADS["square_e5m2_8192"]
    A, B = w.make()
    p = _plan(w.M, w.N, w.K, w.dtype, w.out)
    assert p.info["mfma_k"] == 32
    log(f"{w.name} with the fp16 step: tile {p.info['run_block_m']}x{p.info['run_block_n']}")
    C = run(p, A.to(dev()), B.to(dev()), False)
    rng = np.random.default_rng(13400)
    ii = rng.integers(0, w.M, 4096)
    jj = rng.integers(0, w.N, 4096)
    got = C[torch.from_numpy(ii).to(dev()), torch.from_numpy(jj).to(dev())]
    c64, ca = oracle.gemm_elems(wl.bits(A), wl.bits(B), w.dtype, ii, jj)
    r = check_bound(got.cpu().to(torch.float64).numpy(), c64, ca, w.K, w.out)
    log(f"{w.name}: max err/bound {r:.3g} (plain bound)")


def test_full_size_integers_e4m3_4096():
    n = 4096
    g = wl.gen(13500)
    A = wl.integers((n, n), "e4m3", g)
    B = wl.integers((n, n), "e4m3", g)
    C = run(_plan(n, n, n, "e4m3", "bf16"), A.to(dev()), B.to(dev()), False)
    got = bits_of(C)
    Ai = A.to(torch.float32).to(torch.int32).numpy()
    Bi = B.to(torch.float32).to(torch.int32).numpy()
    rows = [0, 1234, n - 1]
    want_rows = oracle.round_rne("bf16", oracle.gemm_i64(Ai[rows], Bi).astype(np.float64))
    assert np.array_equal(got[rows], want_rows)
    cols = [0, 777, n - 1]
    want_cols = oracle.round_rne("bf16", oracle.gemm_i64(Ai, np.ascontiguousarray(Bi[:, cols]))
                                 .astype(np.float64))
    assert np.array_equal(got[:, cols], want_cols)
