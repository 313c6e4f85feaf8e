"""Pins for the oracle's product C = A * B (fp64, ascending k).

What pins it, besides itself: closed forms (identity, all-ones giving K,
unit selectors, zeros), an int64 triple-loop twin on small-integer inputs
(itself pinned to numpy's integer matmul and a hand-worked example),
exactly representable "grid" inputs (full 8-bit significands on a common
2^-6 grid, after the exact-accumulation argument of the Insight Edge cuTile
blog, section "最適化後の結果": a bf16 x bf16 product needs 16 significant
bits and 128 of them fit fp32's 24), and numpy's fp64 matmul within the
fp64 error bound.  Non-square shapes make a transposed operand, a wrong
index or a dropped term fail.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl


def _dec(fmt, t):
    return oracle.decode(fmt, wl.bits(t))


# ------------------------------------------------------------ int64 twin


def test_i64_twin_hand_example():
    A = np.array([[1, 2, 3], [4, 5, 6]])
    B = np.array([[7, 8], [9, 10], [11, 12]])
    assert oracle.gemm_i64(A, B).tolist() == [[58, 64], [139, 154]]


def test_i64_twin_vs_numpy():
    rng = np.random.default_rng(3)
    A = rng.integers(-100, 100, size=(17, 23))
    B = rng.integers(-100, 100, size=(23, 11))
    assert np.array_equal(oracle.gemm_i64(A, B), A.astype(np.int64) @ B.astype(np.int64))


# -------------------------------------------------------- closed forms


@pytest.mark.parametrize("fmt", ["f16", "bf16", "e5m2", "e4m3"])
def test_identity(fmt):
    g = wl.gen(1)
    K = 48
    B = wl.uniform((K, 20), fmt, g)
    A = torch.eye(K, dtype=torch.float32).to(wl.DTYPES[fmt])
    C, Ca = oracle.gemm(wl.bits(A), wl.bits(B), fmt)
    Bd = _dec(fmt, B)
    assert np.array_equal(C, Bd)
    assert np.array_equal(Ca, np.abs(Bd))


@pytest.mark.parametrize("fmt,K", [("f16", 256), ("bf16", 14336), ("f16", 131072),
                                    ("bf16", 16384), ("e5m2", 4096)])
def test_all_ones_gives_K(fmt, K):
    A = torch.ones((3, K), dtype=wl.DTYPES[fmt])
    B = torch.ones((K, 5), dtype=wl.DTYPES[fmt])
    C, Ca = oracle.gemm(wl.bits(A), wl.bits(B), fmt)
    assert np.all(C == K) and np.all(Ca == K)
    # K is exact in fp32 (and in bf16 for these K), so the rounded value is K too.
    assert np.all(oracle.decode("f32", oracle.round_rne("f32", C)) == K)


def test_unit_selector_picks_row_of_B():
    g = wl.gen(2)
    M, K, N = 9, 31, 13
    B = wl.uniform((K, N), "f16", g)
    A = torch.zeros((M, K), dtype=torch.float16)
    A[4, 17] = 1.0
    C, _ = oracle.gemm(wl.bits(A), wl.bits(B), "f16")
    assert np.array_equal(C[4], _dec("f16", B)[17])
    others = np.delete(C, 4, axis=0)
    assert np.all(others == 0.0) and not np.any(np.signbit(others))


def test_zero_B_gives_positive_zero():
    g = wl.gen(3)
    A = wl.uniform((7, 19), "f16", g)
    B = torch.zeros((19, 5), dtype=torch.float16)
    C, Ca = oracle.gemm(wl.bits(A), wl.bits(B), "f16")
    assert np.all(C == 0.0) and not np.any(np.signbit(C)) and np.all(Ca == 0.0)


def test_negative_zero_inputs_sum_to_positive_zero():
    A = torch.tensor([[-0.0, -0.0]], dtype=torch.float16)
    B = torch.tensor([[1.0], [1.0]], dtype=torch.float16)
    C, _ = oracle.gemm(wl.bits(A), wl.bits(B), "f16")
    assert C[0, 0] == 0.0 and not np.signbit(C[0, 0])


# ------------------------------------------------- brute force, integers


@pytest.mark.parametrize("fmt", ["f16", "bf16", "e5m2", "e4m3"])
@pytest.mark.parametrize("shape", [(37, 29, 53), (1, 64, 300), (64, 1, 7), (5, 3, 1)])
def test_integer_inputs_match_int64_twin(fmt, shape):
    M, N, K = shape
    g = wl.gen(100 + M)
    A = wl.integers((M, K), fmt, g)
    B = wl.integers((K, N), fmt, g)
    C, _ = oracle.gemm(wl.bits(A), wl.bits(B), fmt)
    Ci = oracle.gemm_i64(A.to(torch.int32).numpy(), B.to(torch.int32).numpy())
    assert np.array_equal(C, Ci.astype(np.float64))


def test_exact256_workload_matches_int64_twin():
    w = wl.WORKLOADS["exact256"]
    A, B = w.make()
    C, _ = oracle.gemm(wl.bits(A), wl.bits(B), w.dtype)
    Ci = oracle.gemm_i64(A.to(torch.int32).numpy(), B.to(torch.int32).numpy())
    assert np.array_equal(C, Ci.astype(np.float64))
    # Every fp32 rounding of an exact small integer is the integer itself.
    assert np.array_equal(oracle.decode("f32", oracle.round_rne("f32", C)), C)


def test_integer_rows_at_decode_and_hugek_shapes():
    # Row subsets at the large shapes: N=4096, K=14336 and N=256, K=131072.
    for (N, K, rows) in [(4096, 14336, [0, 5]), (256, 131072, [3])]:
        g = wl.gen(N + K)
        A = wl.integers((8, K), "bf16", g)
        B = wl.integers((K, N), "bf16", g)
        C, _ = oracle.gemm(wl.bits(A), wl.bits(B), "bf16", rows=rows)
        Ai = A.to(torch.int64)[rows]
        Ci = (Ai @ B.to(torch.int64)).numpy()  # torch int64 matmul: independent of the oracle
        assert np.array_equal(C, Ci.astype(np.float64))


# ------------------------------------------------ exact grid inputs


@pytest.mark.parametrize("fmt", ["bf16", "f16"])
def test_grid_inputs_exact(fmt):
    # n / 64 with |n| <= 255: every product is a multiple of 2^-12 and every
    # partial sum of K = 256 of them is below 2^12 in magnitude, so all of
    # them are exact in fp32 and the fp64 sum times 4096 is the integer sum.
    g = wl.gen(5)
    A = wl.grid((40, 256), fmt, g)
    B = wl.grid((256, 24), fmt, g)
    nA = (_dec(fmt, A) * 64).astype(np.int64)
    nB = (_dec(fmt, B) * 64).astype(np.int64)
    assert np.array_equal(nA / 64.0, _dec(fmt, A))  # the grid values are exact
    C, _ = oracle.gemm(wl.bits(A), wl.bits(B), fmt)
    assert np.array_equal(C * 4096.0, oracle.gemm_i64(nA, nB).astype(np.float64))
    assert np.max(np.abs(C)) < 2.0 ** 12


# ------------------------------------------- library cross-check, bounds


@pytest.mark.parametrize("fmt", ["f16", "bf16", "e5m2"])
def test_random_vs_numpy_fp64(fmt):
    g = wl.gen(6)
    M, N, K = 33, 47, 1000
    A = wl.uniform((M, K), fmt, g)
    B = wl.uniform((K, N), fmt, g)
    C, Ca = oracle.gemm(wl.bits(A), wl.bits(B), fmt)
    Ad, Bd = _dec(fmt, A), _dec(fmt, B)
    ref = Ad @ Bd
    assert np.all(np.abs(C - ref) <= 2 * K * 2.0 ** -53 * Ca)
    assert np.allclose(Ca, np.abs(Ad) @ np.abs(Bd), rtol=4 * K * 2.0 ** -53, atol=0)


def test_scale_is_applied():
    g = wl.gen(8)
    A = wl.normal((6, 64), "e5m2", g)
    B = wl.normal((64, 9), "e5m2", g)
    C1, Ca1 = oracle.gemm(wl.bits(A), wl.bits(B), "e5m2", scale=1.0)
    C2, Ca2 = oracle.gemm(wl.bits(A), wl.bits(B), "e5m2", scale=0.5)
    assert np.array_equal(C2, C1 * 0.5) and np.array_equal(Ca2, Ca1 * 0.5)
    C3, _ = oracle.gemm(wl.bits(A), wl.bits(B), "e5m2", scale=-2.0)
    assert np.array_equal(C3, -2.0 * C1)


# --------------------------------------------- consistency of the entry points


def test_rows_and_elems_agree_with_full():
    g = wl.gen(9)
    M, N, K = 21, 17, 333
    A = wl.uniform((M, K), "f16", g)
    B = wl.uniform((K, N), "f16", g)
    C, Ca = oracle.gemm(wl.bits(A), wl.bits(B), "f16")
    rows = [20, 0, 7, 7]
    Cr, Car = oracle.gemm(wl.bits(A), wl.bits(B), "f16", rows=rows)
    assert np.array_equal(Cr, C[rows]) and np.array_equal(Car, Ca[rows])
    ii = np.array([0, 20, 5, 13])
    jj = np.array([16, 0, 9, 3])
    ce, cae = oracle.gemm_elems(wl.bits(A), wl.bits(B), "f16", ii, jj)
    assert np.array_equal(ce, C[ii, jj]) and np.array_equal(cae, Ca[ii, jj])


def test_thread_count_does_not_change_bits():
    g = wl.gen(10)
    A = wl.uniform((64, 513), "bf16", g)
    B = wl.uniform((513, 40), "bf16", g)
    C1, _ = oracle.gemm(wl.bits(A), wl.bits(B), "bf16", nthreads=1)
    C4, _ = oracle.gemm(wl.bits(A), wl.bits(B), "bf16", nthreads=4)
    assert np.array_equal(C1, C4)
    oracle.gemm(wl.bits(A[:1]), wl.bits(B[:, :1]), "bf16", nthreads=0)


def test_bad_arguments_raise():
    A = np.zeros((2, 3), dtype=np.uint16)
    B = np.zeros((4, 2), dtype=np.uint16)
    with pytest.raises(ValueError):
        oracle.gemm(A, B, "f16")
    with pytest.raises(ValueError):
        oracle.gemm(A, np.zeros((3, 2), dtype=np.uint16), "f16", rows=[5])
    with pytest.raises(TypeError):
        oracle.gemm(A, np.zeros((3, 2), dtype=np.uint8), "f16")
