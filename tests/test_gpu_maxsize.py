"""Maximum sizes: products so long or so wide that the DMA tiles' 32-bit
buffer offsets would overflow, where the plan falls back to the
register-staged tiles (64-bit addressing, same instruction and K order).

Inputs are ternary integers ({-1, 0, 1}), so every partial sum is an integer
of magnitude at most K < 2^24 and exact in fp32 in any order: the GPU result
must equal the exact product bit for bit.  The exact product is computed on
the host for sampled rows.
"""
import numpy as np
import pytest
import torch

import invariant_matmul_amd as imm
import workloads as wl
from tests.helpers import dev, log

pytestmark = pytest.mark.gpu


def _cuda_gen(seed):
    g = torch.Generator(device=dev())
    g.manual_seed(seed)
    return g


def _exact_rows(A, B, rows):
    """Exact product of the given rows of A with B (integers below 2^24)."""
    a = A[rows].float().cpu().numpy().astype(np.float64)
    b = B.float().cpu().numpy().astype(np.float64)
    return a @ b


def _run(plan, A, B, split):
    info = plan.info
    C = torch.full((info["M"], info["N"]), float("nan"), dtype=torch.float32, device=dev())
    if split:
        ws = torch.empty(max(1, imm.gemm_workspace_size(plan) // 4), dtype=torch.float32,
                         device=dev())
        imm.gemm_splitk_run(plan, A, B, C, ws)
    else:
        imm.gemm_run(plan, A, B, C)
    torch.cuda.synchronize()
    return C


def test_k_past_the_large_tiles_offset_limit():
    """K = 2^23 + 96 bf16: the A offsets of a 128- or 256-row tile pass 2^31,
    so explicit 256x256 and 128x256 plans run the register-staged tiles; the
    default plan (reduction-dominated, N = 40) steps down from its 128x256
    split-path tile to the 64x256 DMA tile, whose offsets still fit.  All
    give the default's bits."""
    M, N, K = 300, 40, 2 ** 23 + 96
    g = _cuda_gen(9100)
    A = wl.integers((M, K), "bf16", g, -1, 1)
    B = wl.integers((K, N), "bf16", g, -1, 1)
    rows = [0, 137, 299]
    want = _exact_rows(A, B, rows)
    default = imm.gemm_plan(M, N, K, "bf16")
    log(f"max-K default: tile {default.info['tile']} split {default.info['split_k']}")
    assert default.info["tile"] == imm.TILE["64x256"]
    ref = _run(default, A, B, True)
    assert not torch.isnan(ref).any()
    np.testing.assert_array_equal(ref[rows].cpu().numpy().astype(np.float64), want)
    for tile, fallback in (("256x256", "256x256_rs"), ("128x256", "128x128")):
        p = imm.gemm_plan_ex(M, N, K, "bf16", "f32", tile=tile)
        assert p.info["tile"] == imm.TILE[fallback] and p.info["run_tile"] == imm.TILE[fallback]
        assert p.info["split_k"] == default.info["split_k"]
        got = _run(p, A, B, True)
        assert torch.equal(got.view(torch.int32), ref.view(torch.int32)), tile
        one = _run(p, A, B, False)            # single pass over the whole K
        np.testing.assert_array_equal(one[rows].cpu().numpy().astype(np.float64), want)


def test_n_past_the_b_stage_offset_limit():
    """N = 2^24 + 64 fp16: 128 bytes of K rows of B pass 2^31, so the DMA
    tiles give way to the register-staged ones; C is exact."""
    M, N, K = 3, 2 ** 24 + 64, 64
    g = _cuda_gen(9200)
    A = wl.integers((M, K), "f16", g, -1, 1)
    B = wl.integers((K, N), "f16", g, -1, 1)
    plan = imm.gemm_plan(M, N, K, "f16")
    log(f"max-N: run tile {plan.info['run_tile']} tile {plan.info['tile']}")
    assert plan.info["run_tile"] == imm.TILE["256x256_rs"]
    C = _run(plan, A, B, False)
    assert not torch.isnan(C).any()
    cols = torch.randint(0, N, (2048,), generator=_cuda_gen(9201), device=dev())
    cols = torch.cat([cols, torch.tensor([0, N - 1], device=dev())])
    a = A.float().cpu().numpy().astype(np.float64)
    b = B[:, cols].float().cpu().numpy().astype(np.float64)
    np.testing.assert_array_equal(C[:, cols].cpu().numpy().astype(np.float64), a @ b)
