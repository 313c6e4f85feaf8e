"""Bit-exact oracle checks at the workloads' full sizes, on integer inputs.

With integers in [-4, 4] every product is at most 16 and every partial sum at
most 16 K <= 2^21 (K <= 131072) in magnitude, so every fp32 summation order
is exact: the GPU result must equal the exact product rounded once to the
output format, bit for bit, whatever the tile, the split of K or the matrix
step (the Tencent deterministic-inference article, "背景": results differ only
through rounding; the Insight Edge cuTile blog's exact-accumulation argument).
For fp8 the matrix step adds its products in a window 13 binades deep below
the step's largest product; integer products of magnitude 1 .. 16 all lie
inside it, so the step is exact here too.

Each shape runs in the launch configuration the benchmark times: the square
fp16 8192^3 and e5m2 16384^3 products through gemm_run, the decode product
128 x 4096 x 14336 bf16 through the split-K path at its default split, the
huge-K product 256 x 256 x 131072 fp16 through the split-K path at 8, 32 and
128 slices.  The oracle evaluates full columns with its int64 twin, and full
rows and 2048 random elements with its fp64 loop; the GPU must match all of
them exactly.
"""
import numpy as np
import pytest
import torch

import invariant_matmul_amd as imm
import oracle
import workloads as wl
from tests.helpers import dev, log, out_torch_dtype

pytestmark = pytest.mark.gpu


def _int_inputs(M, N, K, dt, seed):
    g = wl.gen(seed)
    A = wl.integers((M, K), dt, g)
    B = wl.integers((K, N), dt, g)
    return A, B


def _as_i32(t):
    return t.to(torch.float32).to(torch.int32).numpy()


def _check_exact(C, A, B, dt, out, seed, n_elems=2048):
    """C (device) against the exact product at sampled rows, columns and elements."""
    M, K = A.shape
    N = B.shape[1]
    torch.cuda.synchronize()
    got = wl.bits(C.cpu())
    Ai, Bi = _as_i32(A), _as_i32(B)
    rng = np.random.default_rng(seed)
    rows = sorted({0, M - 1, M // 2, int(rng.integers(0, M))})
    cols = sorted({0, N - 1, N // 3, int(rng.integers(0, N))})
    # full rows, element by element (the row form would decode all of B)
    ri = np.repeat(np.array(rows, dtype=np.int64), N)
    rj = np.tile(np.arange(N, dtype=np.int64), len(rows))
    c_rows, _ = oracle.gemm_elems(wl.bits(A), wl.bits(B), dt, ri, rj)
    want_rows = oracle.round_rne(out, c_rows).reshape(len(rows), N)
    assert np.array_equal(got[rows], want_rows), "rows"
    want_cols = oracle.round_rne(out, oracle.gemm_i64(Ai, np.ascontiguousarray(Bi[:, cols]))
                                 .astype(np.float64))
    assert np.array_equal(got[:, cols], want_cols), "columns"
    ii = rng.integers(0, M, n_elems)
    jj = rng.integers(0, N, n_elems)
    c64, _ = oracle.gemm_elems(wl.bits(A), wl.bits(B), dt, ii, jj)
    assert np.array_equal(got[ii, jj], oracle.round_rne(out, c64)), "elements"
    log(f"  exact: rows {rows}, columns {cols}, {n_elems} elements")


def _run(plan, Ad, Bd, split):
    info = plan.info
    C = torch.empty((info["M"], info["N"]), dtype=out_torch_dtype(info["out_dtype"]), device=dev())
    if split:
        ws = torch.empty(max(1, imm.gemm_workspace_size(plan) // 4), dtype=torch.float32,
                         device=dev())
        imm.gemm_splitk_run(plan, Ad, Bd, C, ws)
    else:
        imm.gemm_run(plan, Ad, Bd, C)
    return C


def test_square_f16_8192_integers():
    n = 8192
    A, B = _int_inputs(n, n, n, "f16", 12000)
    plan = imm.gemm_plan(n, n, n, "f16")
    log(f"square f16 8192^3 integers: tile {plan.info['run_block_m']}x{plan.info['run_block_n']}")
    C = _run(plan, A.to(dev()), B.to(dev()), False)
    _check_exact(C, A, B, "f16", "f32", 12000)


def test_square_e5m2_16384_integers():
    n = 16384
    A, B = _int_inputs(n, n, n, "e5m2", 12001)
    plan = imm.gemm_plan(n, n, n, "e5m2")
    assert plan.info["out_dtype"] == imm.DTYPE["bf16"]
    log(f"square e5m2 16384^3 integers, bf16 out")
    C = _run(plan, A.to(dev()), B.to(dev()), False)
    _check_exact(C, A, B, "e5m2", "bf16", 12001)


def test_decode_bf16_integers_default_split():
    M, N, K = 128, 4096, 14336
    A, B = _int_inputs(M, N, K, "bf16", 12002)
    Ad, Bd = A.to(dev()), B.to(dev())
    for m in (128, 1):
        plan = imm.gemm_plan(m, N, K, "bf16")
        log(f"decode {m}x{N}x{K} bf16 integers: split {plan.info['split_k']}")
        assert plan.info["split_k"] > 1
        C = _run(plan, Ad[:m].contiguous(), Bd, True)
        _check_exact(C, A[:m], B, "bf16", "f32", 12002 + m)


@pytest.mark.parametrize("split", [8, 32, 128])
def test_hugek_f16_integers(split):
    M, N, K = 256, 256, 131072
    A, B = _int_inputs(M, N, K, "f16", 12003)
    plan = imm.gemm_plan_ex(M, N, K, "f16", "f32", split_k=split)
    log(f"huge-K 256x256x131072 f16 integers: split {plan.info['split_k']}")
    assert plan.info["split_k"] == split
    C = _run(plan, A.to(dev()), B.to(dev()), True)
    _check_exact(C, A, B, "f16", "f32", 12003 + split)
