"""GPU parity: the HIP library against the CPU oracle, through the C ABI.

Bar: bit-exact where every summation order is exact (small-integer inputs,
"grid" inputs with full 8-bit significands), and within
|C - C_ref| <= K 2^-24 (|A||B|)_ij (fp32 output; plus the bf16 rounding for
bf16 output) on random inputs.  Small cases are compared element by element
over several tiles with ragged edges; the full-size workloads, in the launch
configuration the benchmark times, are compared on sampled elements and rows.
"""
import numpy as np
import pytest
import torch

import invariant_matmul_amd as imm
import oracle
import workloads as wl
from tests.helpers import (FP8, FP8_PLAIN_BOUND_MIN_K, bits_of, check_bound, dev, expected_bits,
                           fp8_check_bound, log, run, tiles_for, values_of)

pytestmark = pytest.mark.gpu

TILES = ["256x256", "128x128", "32x128", "256x256_rs", "32x256", "64x256", "128x256", "32x64",
         "64x64", "32x32"]
IN_DTYPES = ["f16", "bf16", "e4m3", "e5m2"]


def _to_dev(*ts):
    return [t.to(dev()) for t in ts]


# ------------------------------------------------------------- exact inputs


def test_exact256_bit_exact_every_path():
    w = wl.WORKLOADS["exact256"]
    A, B = w.make()
    C64, _ = oracle.gemm(wl.bits(A), wl.bits(B), "f16")
    want = expected_bits(C64, "f32")
    Ad, Bd = _to_dev(A, B)
    log("exact256: default plan")
    assert np.array_equal(bits_of(run(imm.gemm_plan(256, 256, 256, "f16"), Ad, Bd, False)), want)
    for tile in TILES:
        for split in (1, 4):
            log(f"exact256: tile {tile} split {split}")
            p = imm.gemm_plan_ex(256, 256, 256, "f16", "f32", split_k=split, tile=tile)
            assert np.array_equal(bits_of(run(p, Ad, Bd, False)), want)
            assert np.array_equal(bits_of(run(p, Ad, Bd, True)), want)


@pytest.mark.parametrize("dt", IN_DTYPES)
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_integer_inputs_bit_exact_ragged(dt, out):
    # 300 x 272 x 384: several tiles in M and N with ragged edges in M and N,
    # and a K tail that is not a multiple of the 128-byte K step for 16-bit.
    M, N, K = 300, 272, 400 if dt in ("f16", "bf16") else 384
    g = wl.gen(7000 + IN_DTYPES.index(dt))
    A = wl.integers((M, K), dt, g)
    B = wl.integers((K, N), dt, g)
    C64, _ = oracle.gemm(wl.bits(A), wl.bits(B), dt)
    want = expected_bits(C64, out)
    Ad, Bd = _to_dev(A, B)
    for tile in tiles_for(dt, TILES):
        for split in (1, 3):
            log(f"int {dt}->{out}: tile {tile} split {split}")
            p = imm.gemm_plan_ex(M, N, K, dt, out, split_k=split, tile=tile)
            assert np.array_equal(bits_of(run(p, Ad, Bd, False)), want), (tile, "run")
            assert np.array_equal(bits_of(run(p, Ad, Bd, True)), want), (tile, split)


@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_grid_inputs_bit_exact(dt):
    # n / 64 with |n| <= 255 and K = 256: every partial sum is exact in fp32.
    g = wl.gen(7100)
    M, N, K = 160, 288, 256
    A = wl.grid((M, K), dt, g)
    B = wl.grid((K, N), dt, g)
    C64, _ = oracle.gemm(wl.bits(A), wl.bits(B), dt)
    want = expected_bits(C64, "f32")
    Ad, Bd = _to_dev(A, B)
    for tile in TILES:
        log(f"grid {dt}: tile {tile}")
        p = imm.gemm_plan_ex(M, N, K, dt, "f32", split_k=2, tile=tile)
        assert np.array_equal(bits_of(run(p, Ad, Bd, False)), want)
        assert np.array_equal(bits_of(run(p, Ad, Bd, True)), want)


def test_power_of_two_scales_exact():
    g = wl.gen(7200)
    M, N, K = 70, 144, 256
    A = wl.integers((M, K), "e4m3", g)
    B = wl.integers((K, N), "e4m3", g)
    C64, _ = oracle.gemm(wl.bits(A), wl.bits(B), "e4m3", scale=0.5)
    Ad, Bd = _to_dev(A, B)
    for out in ("f32", "bf16"):
        p = imm.gemm_plan_ex(M, N, K, "e4m3", out, split_k=2, scale_a=2.0, scale_b=0.25)
        want = expected_bits(C64, out)
        assert np.array_equal(bits_of(run(p, Ad, Bd, False)), want)
        assert np.array_equal(bits_of(run(p, Ad, Bd, True)), want)


# ------------------------------------------------------------ random inputs


@pytest.mark.parametrize("dt", IN_DTYPES)
def test_random_inputs_within_bound_ragged(dt):
    M, N, K = 333, 400, 1040 if dt in ("f16", "bf16") else 1024
    g = wl.gen(7300 + IN_DTYPES.index(dt))
    A = wl.uniform((M, K), dt, g) if dt in ("f16", "bf16") else wl.normal((M, K), dt, g)
    B = wl.uniform((K, N), dt, g) if dt in ("f16", "bf16") else wl.normal((K, N), dt, g)
    a_bits, b_bits = wl.bits(A), wl.bits(B)
    C64, Ca = oracle.gemm(a_bits, b_bits, dt)
    Ad, Bd = _to_dev(A, B)
    for out in ("f32", "bf16"):
        for tile in tiles_for(dt, TILES):
            for split in (1, 5):
                p = imm.gemm_plan_ex(M, N, K, dt, out, split_k=split, tile=tile)
                r1 = fp8_check_bound(values_of(run(p, Ad, Bd, False)), C64, Ca, K, out, dt,
                                     a_bits, b_bits)
                r2 = fp8_check_bound(values_of(run(p, Ad, Bd, True)), C64, Ca, K, out, dt,
                                     a_bits, b_bits)
                log(f"random {dt}->{out} tile {tile} split {split}: max err/bound {r1:.3g} {r2:.3g}")


# --------------------------------------------------------------- edge cases


def test_k_zero_gives_zeros_and_empty_m_is_noop():
    Ad = torch.empty((64, 0), dtype=torch.float16, device=dev())
    Bd = torch.empty((0, 64), dtype=torch.float16, device=dev())
    p = imm.gemm_plan(64, 64, 0, "f16")
    C = torch.full((64, 64), 7.0, dtype=torch.float32, device=dev())
    imm.gemm_run(p, Ad.data_ptr() or 0, Bd.data_ptr() or 0, C)
    torch.cuda.synchronize()
    assert torch.all(C == 0) and not torch.any(torch.signbit(C))
    C.fill_(7.0)
    p2 = imm.gemm_plan_ex(64, 64, 0, "f16", "f32", split_k=3)
    ws = torch.empty(imm.gemm_workspace_size(p2) // 4, dtype=torch.float32, device=dev())
    imm.gemm_splitk_run(p2, 0, 0, C, ws)
    torch.cuda.synchronize()
    assert torch.all(C == 0)
    pe = imm.gemm_plan(0, 64, 64, "f16")
    imm.gemm_run(pe, 0, 0, 0)
    imm.gemm_splitk_run(pe, 0, 0, 0, 0)


@pytest.mark.parametrize("M,N,K", [(1, 8, 8), (1, 16, 16), (33, 8, 1024), (5, 1040, 16)])
def test_tiny_and_narrow_shapes(M, N, K):
    g = wl.gen(7400 + M + N + K)
    A = wl.integers((M, K), "bf16", g)
    B = wl.integers((K, N), "bf16", g)
    C64, _ = oracle.gemm(wl.bits(A), wl.bits(B), "bf16")
    want = expected_bits(C64, "f32")
    Ad, Bd = _to_dev(A, B)
    for tile in TILES:
        p = imm.gemm_plan_ex(M, N, K, "bf16", "f32", split_k=2, tile=tile)
        assert np.array_equal(bits_of(run(p, Ad, Bd, False)), want)
        assert np.array_equal(bits_of(run(p, Ad, Bd, True)), want)


def test_bf16_output_conversion_matches_torch():
    # The epilogue's fp32 -> bf16 rounding (ties to even) against torch's.
    g = wl.gen(7500)
    M, N, K = 64, 256, 512
    A = wl.normal((M, K), "e5m2", g)
    B = wl.normal((K, N), "e5m2", g)
    Ad, Bd = _to_dev(A, B)
    c32 = run(imm.gemm_plan_ex(M, N, K, "e5m2", "f32"), Ad, Bd, False)
    c16 = run(imm.gemm_plan_ex(M, N, K, "e5m2", "bf16"), Ad, Bd, False)
    torch.cuda.synchronize()
    assert torch.equal(c16.view(torch.int16), c32.to(torch.bfloat16).view(torch.int16))


# ------------------------------------------------------ full-size workloads


def _sample_positions(M, N, n, seed):
    rng = np.random.default_rng(seed)
    ii = np.concatenate([rng.integers(0, M, n), [0, M - 1, 0, M - 1]])
    jj = np.concatenate([rng.integers(0, N, n), [0, N - 1, N - 1, 0]])
    return ii, jj


def _check_sampled(w, plan, split, n=2048):
    A, B = w.make()
    Ad, Bd = _to_dev(A, B)
    log(f"{w.name}: running {plan.info['tile']} split {plan.info['split_k'] if split else 1}")
    C = run(plan, Ad, Bd, split)
    ii, jj = _sample_positions(w.M, w.N, n, w.seed)
    got = C[torch.from_numpy(ii).to(dev()), torch.from_numpy(jj).to(dev())]
    got = got.cpu().to(torch.float64).numpy()
    a_bits, b_bits = wl.bits(A), wl.bits(B)
    c64, ca = oracle.gemm_elems(a_bits, b_bits, w.dtype, ii, jj)
    # fp8 at these sizes (K >= FP8_PLAIN_BOUND_MIN_K) gets the plain bound
    chk = lambda got_, c_, ca_, i_, j_: fp8_check_bound(got_, c_, ca_, w.K, w.out, w.dtype,
                                                        a_bits, b_bits, i_, j_)
    r = chk(got, c64, ca, ii, jj)
    # a full row and a full column as well (element by element: the row form
    # of the oracle decodes all of B)
    row = w.M // 2
    jr = np.arange(w.N)
    cr, car = oracle.gemm_elems(a_bits, b_bits, w.dtype, np.full(w.N, row), jr)
    r = max(r, chk(C[row].cpu().to(torch.float64).numpy(), cr, car, np.full(w.N, row), jr))
    col = w.N // 3
    ic = np.arange(w.M)
    cc, cac = oracle.gemm_elems(a_bits, b_bits, w.dtype, ic, np.full(w.M, col))
    r = max(r, chk(C[:, col].cpu().to(torch.float64).numpy(), cc, cac, ic, np.full(w.M, col)))
    log(f"{w.name}: max err/bound {r:.3g}")
    return C


@pytest.mark.parametrize("name", ["square_f16_1024", "square_f16_4096", "square_f16_8192",
                                  "square_e5m2_4096", "square_e5m2_8192", "square_e5m2_16384"])
def test_full_size_square(name):
    w = wl.WORKLOADS[name]
    assert w.dtype not in FP8 or w.K >= FP8_PLAIN_BOUND_MIN_K  # fp8 sizes: plain bound
    plan = imm.gemm_plan(w.M, w.N, w.K, w.dtype)
    assert imm.DTYPE[w.out] == plan.info["out_dtype"]
    _check_sampled(w, plan, split=False)


def test_full_size_square_1024_every_element():
    w = wl.WORKLOADS["square_f16_1024"]
    A, B = w.make()
    C64, Ca = oracle.gemm(wl.bits(A), wl.bits(B), "f16")
    Ad, Bd = _to_dev(A, B)
    r = check_bound(values_of(run(imm.gemm_plan(1024, 1024, 1024, "f16"), Ad, Bd, False)),
                    C64, Ca, 1024, "f32")
    log(f"square_f16_1024 full: max err/bound {r:.3g}")


@pytest.mark.parametrize("split", [1, 8, 32, 128])
def test_full_size_hugek(split):
    w = wl.WORKLOADS["hugek_f16"]
    plan = imm.gemm_plan_ex(w.M, w.N, w.K, "f16", "f32", split_k=split)
    _check_sampled(w, plan, split=True, n=512)


def test_full_size_decode_rows():
    w = wl.WORKLOADS["decode_bf16_m128"]
    A, B = w.make()
    Ad, Bd = _to_dev(A, B)
    plan = imm.gemm_plan(w.M, w.N, w.K, "bf16")
    log(f"decode m128: split {plan.info['split_k']}")
    C = run(plan, Ad, Bd, True)
    rows = [0, 1, 7, 31, 127]
    C64, Ca = oracle.gemm(wl.bits(A), wl.bits(B), "bf16", rows=rows)
    r = check_bound(C[rows].cpu().to(torch.float64).numpy(), C64, Ca, w.K, "f32")
    log(f"decode m128 rows {rows}: max err/bound {r:.3g}")
