"""The persistent single pass (GEMM_PLAN_PERSISTENT) against the one-tile-per-
workgroup single pass, bit for bit, and against the CPU oracle: bit-exact on
integer inputs, within the error bound on random ones.

The Tencent deterministic-inference article's closing section lists a
persistent matmul as the batch-invariant GEMM.  Here it is the same kernel
with at most one workgroup per compute unit walking the tiles of the
one-tile-per-workgroup grid; every element keeps its instruction chain and K
order, so C must be identical in every bit, for every input and output type,
both B layouts, a bias, ragged edges, fewer tiles than compute units and
several tiles per workgroup -- and rows must not depend on M.
"""
import numpy as np
import pytest
import torch

import invariant_matmul_amd as imm
import oracle
import workloads as wl
from tests.helpers import bits_of, dev, log, out_torch_dtype

pytestmark = pytest.mark.gpu


def _inputs(M, N, K, dt, seed, bt=False):
    g = wl.gen(seed)
    if dt in ("e4m3", "e5m2"):
        A, B = wl.normal((M, K), dt, g), wl.normal((K, N), dt, g)
    else:
        A, B = wl.uniform((M, K), dt, g), wl.uniform((K, N), dt, g)
    if bt:
        B = B.float().t().contiguous().to(B.dtype)   # W = B^T, [N, K]
    return A.to(dev()), B.to(dev())


def _run(M, N, K, dt, out, A, B, flags, bias=None):
    plan = imm.gemm_plan_ex2(M, N, K, dt, out, flags=flags)
    C = torch.empty((M, N), dtype=out_torch_dtype(imm.DTYPE[out]), device=dev())
    imm.gemm_run(plan, A, B, C, bias=bias)
    return bits_of(C), plan.info


CASES = [
    # (M, N, K, dtype, out, B transposed)
    (8192, 8192, 8192, "f16", "f32", False),    # 1024 tiles: 4 per workgroup
    (4100, 4200, 512, "f16", "f32", False),     # 289 tiles, ragged M and N
    (3000, 4096, 1000, "bf16", "bf16", False),  # ragged K
    (2304, 5120, 768, "f16", "f16", True),      # transposed B (weight layout)
    (4096, 4608, 1024, "e4m3", "bf16", False),
    (4352, 4096, 1280, "e5m2", "f32", True),
    (700, 1304, 2048, "bf16", "f32", False),    # fewer tiles than compute units
]


@pytest.mark.parametrize("M,N,K,dt,out,bt", CASES,
                         ids=[f"{c[0]}x{c[1]}x{c[2]}-{c[3]}-{c[4]}" + ("-bt" if c[5] else "")
                              for c in CASES])
def test_persistent_equals_single_pass(M, N, K, dt, out, bt):
    A, B = _inputs(M, N, K, dt, 8100 + M % 97, bt)
    fl = imm.PLAN_B_TRANSPOSED if bt else 0
    want, info = _run(M, N, K, dt, out, A, B, fl)
    if info["run_tile"] != imm.TILE["256x256"]:
        pytest.skip("the plan's single pass uses another tile")
    got, _ = _run(M, N, K, dt, out, A, B, fl | imm.PLAN_PERSISTENT)
    log(f"{M}x{N}x{K} {dt}->{out} bt={bt}: {info['run_tiles_m'] * info['run_tiles_n']} tiles")
    assert np.array_equal(got, want)


def test_persistent_with_bias_and_repeats():
    M, N, K = 2500, 4096, 1536
    A, B = _inputs(M, N, K, "bf16", 8200)
    bias = torch.randn(N, generator=wl.gen(8201), dtype=torch.float32).to(dev())
    want, _ = _run(M, N, K, "bf16", "bf16", A, B, 0, bias)
    for _ in range(3):
        got, _ = _run(M, N, K, "bf16", "bf16", A, B, imm.PLAN_PERSISTENT, bias)
        assert np.array_equal(got, want)


def test_persistent_rows_independent_of_M():
    N, K = 4096, 2048
    A, B = _inputs(3000, N, K, "f16", 8300)
    full, _ = _run(3000, N, K, "f16", "f32", A, B, imm.PLAN_PERSISTENT)
    for m in (1, 255, 257, 1024, 2999):
        part, _ = _run(m, N, K, "f16", "f32", A[:m].contiguous(), B, imm.PLAN_PERSISTENT)
        assert np.array_equal(part, full[:m]), m


# ------------------------------------------------------ against the oracle

ORACLE_CASES = [c for c in CASES if c[0] * c[1] <= 8192 * 8192]


@pytest.mark.parametrize("M,N,K,dt,out,bt", ORACLE_CASES,
                         ids=[f"{c[0]}x{c[1]}x{c[2]}-{c[3]}-{c[4]}" + ("-bt" if c[5] else "")
                              for c in ORACLE_CASES])
def test_persistent_integers_bit_exact_vs_oracle(M, N, K, dt, out, bt):
    """Integer inputs in [-4, 4]: every order is exact, so the persistent pass
    must equal the exact product rounded once (full rows and columns from the
    oracle's int64 twin and fp64 loop, 2048 random elements)."""
    from tests.test_gpu_fullsize_exact import _check_exact
    g = wl.gen(8400 + M % 89)
    A, B = wl.integers((M, K), dt, g), wl.integers((K, N), dt, g)
    Bx = B.float().t().contiguous().to(B.dtype) if bt else B
    fl = (imm.PLAN_B_TRANSPOSED if bt else 0) | imm.PLAN_PERSISTENT
    plan = imm.gemm_plan_ex2(M, N, K, dt, out, flags=fl)
    if plan.info["run_tile"] != imm.TILE["256x256"]:
        pytest.skip("the plan's single pass uses another tile")
    C = torch.empty((M, N), dtype=out_torch_dtype(imm.DTYPE[out]), device=dev())
    imm.gemm_run(plan, A.to(dev()), Bx.to(dev()), C)
    log(f"persistent {M}x{N}x{K} {dt}->{out} bt={bt}: integers")
    _check_exact(C, A, B, dt, out, 8400 + M)


@pytest.mark.parametrize("M,N,K,dt,out,bt", ORACLE_CASES,
                         ids=[f"{c[0]}x{c[1]}x{c[2]}-{c[3]}-{c[4]}" + ("-bt" if c[5] else "")
                              for c in ORACLE_CASES])
def test_persistent_random_within_bound_vs_oracle(M, N, K, dt, out, bt):
    """Random inputs (uniform[-1, 1) for 16-bit inputs, N(0, 1) for fp8): 4096
    sampled elements and one full row within the oracle's error bound."""
    from tests.helpers import fp8_check_bound
    A, B = _inputs(M, N, K, dt, 8500 + M % 83)
    Bx = B.float().t().contiguous().to(B.dtype) if bt else B
    fl = (imm.PLAN_B_TRANSPOSED if bt else 0) | imm.PLAN_PERSISTENT
    plan = imm.gemm_plan_ex2(M, N, K, dt, out, flags=fl)
    if plan.info["run_tile"] != imm.TILE["256x256"]:
        pytest.skip("the plan's single pass uses another tile")
    C = torch.empty((M, N), dtype=out_torch_dtype(imm.DTYPE[out]), device=dev())
    imm.gemm_run(plan, A.to(dev()), Bx.to(dev()), C)
    torch.cuda.synchronize()
    Ch = C.cpu().to(torch.float64).numpy()
    rng = np.random.default_rng(8500 + M)
    ii = np.concatenate([rng.integers(0, M, 4096), np.full(N, M // 2)])
    jj = np.concatenate([rng.integers(0, N, 4096), np.arange(N)])
    a_bits, b_bits = wl.bits(A), wl.bits(B)
    c64, ca = oracle.gemm_elems(a_bits, b_bits, dt, ii, jj)
    r = fp8_check_bound(Ch[ii, jj], c64, ca, K, out, dt, a_bits, b_bits, ii, jj)
    log(f"persistent {M}x{N}x{K} {dt}->{out} bt={bt}: max err/bound {r:.3g}")
