"""GPU tests of the linear-layer form: B given as a [N, K] weight, a bias, fp16 output.

The vLLM batch-invariant operators that the Tencent deterministic-inference
article lists in its closing section include ``linear`` (y = x W^T + b, with
the weight stored [N, K]) and ``mm``/``addmm`` on fp16 tensors.  Checked here:
- B given transposed gives exactly the bits of B given as [K, N] (same values,
  same K order), on every DMA tile, with and without a split of K;
- integer inputs with an integer bias are exact, for fp32, bf16 and fp16
  outputs, in one pass and through the split-K reduction;
- random inputs with a bias stay within the bound (one extra fp32 rounding);
- fp16 output is the round-to-nearest-even of the fp32 result;
- rows of a linear layer do not depend on the other rows of the batch.
"""
import numpy as np
import pytest
import torch

import invariant_matmul_amd as imm
import oracle
import workloads as wl
from tests.helpers import (bits_of, check_bound, dev, expected_bits, log, out_torch_dtype,
                           tiles_for, values_of)

pytestmark = pytest.mark.gpu

DMA_TILES = ["default", "256x256", "128x256", "64x256", "32x256", "32x64", "64x64", "32x32"]
BT = imm.PLAN_B_TRANSPOSED


def _run(plan, A, B, split, bias=None):
    info = plan.info
    C = torch.empty((info["M"], info["N"]), dtype=out_torch_dtype(info["out_dtype"]), device=dev())
    if split:
        ws = torch.empty(max(1, imm.gemm_workspace_size(plan) // 4), dtype=torch.float32,
                         device=dev())
        imm.gemm_splitk_run(plan, A, B, C, ws, bias=bias)
    else:
        imm.gemm_run(plan, A, B, C, bias=bias)
    return C


@pytest.mark.parametrize("dt", ["f16", "bf16", "e4m3"])
@pytest.mark.parametrize("M,N,K", [(300, 272, 320), (7, 528, 1024), (64, 256, 2048)])
def test_transposed_b_gives_the_same_bits(dt, M, N, K):
    g = wl.gen(7000 + M)
    if dt == "e4m3":
        A, B = wl.normal((M, K), dt, g), wl.normal((K, N), dt, g)
    else:
        A, B = wl.uniform((M, K), dt, g), wl.uniform((K, N), dt, g)
    Ad, Bd, Wd = A.to(dev()), B.to(dev()), B.t().contiguous().to(dev())
    for tile in tiles_for(dt, DMA_TILES):
        for split in (0, 3):
            p = imm.gemm_plan_ex2(M, N, K, dt, "f32", split_k=split, tile=tile)
            pt = imm.gemm_plan_ex2(M, N, K, dt, "f32", split_k=split, tile=tile, flags=BT)
            for use_split in (False, True):
                log(f"{dt} {M}x{N}x{K} tile {tile} split {split} splitk_run {use_split}")
                ref = bits_of(_run(p, Ad, Bd, use_split))
                got = bits_of(_run(pt, Ad, Wd, use_split))
                assert np.array_equal(got, ref), (tile, split, use_split)


@pytest.mark.parametrize("out", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_integer_linear_with_bias_is_exact(dt, out):
    M, N, K = 130, 264, 520
    g = wl.gen(7100)
    x = wl.integers((M, K), dt, g)
    W = wl.integers((N, K), dt, g)
    b = torch.randint(-40, 41, (N,), generator=g).to(torch.float32)
    Y64, _ = oracle.linear(wl.bits(x), wl.bits(W), dt, bias=b.double().numpy())
    # |Y| <= 16 * 520 + 40 = 8360: exact in fp32; bf16 and fp16 round it once
    want = expected_bits(Y64, out)
    xd, Wd, bd = x.to(dev()), W.to(dev()), b.to(dev())
    for split in (1, 4):
        for use_split in (False, True):
            p = imm.gemm_plan_ex2(M, N, K, dt, out, split_k=split, flags=BT)
            log(f"{dt}->{out} split {split} splitk_run {use_split} tile {p.info['tile']}")
            got = bits_of(_run(p, xd, Wd, use_split, bias=bd))
            assert np.array_equal(got, want), (split, use_split)


@pytest.mark.parametrize("out", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_random_linear_with_bias_within_bound(dt, out):
    M, N, K = 97, 400, 1536
    g = wl.gen(7200)
    x = wl.uniform((M, K), dt, g)
    W = wl.normal((N, K), dt, g, std=K ** -0.5)
    b = torch.randn((N,), generator=g, dtype=torch.float32)
    Y64, Yabs = oracle.linear(wl.bits(x), wl.bits(W), dt, bias=b.double().numpy())
    xd, Wd, bd = x.to(dev()), W.to(dev()), b.to(dev())
    for use_split in (False, True):
        p = imm.gemm_plan_ex2(M, N, K, dt, out, split_k=0 if not use_split else 5, flags=BT)
        got = values_of(_run(p, xd, Wd, use_split, bias=bd))
        r = check_bound(got, Y64, Yabs, K, out, bias=True)
        log(f"{dt}->{out} splitk_run {use_split}: max err / bound = {r:.3g}")


@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_f16_output_rounds_the_fp32_result(dt):
    M, N, K = 200, 272, 640
    g = wl.gen(7300)
    A, B = wl.uniform((M, K), dt, g), wl.uniform((K, N), dt, g, lo=-8.0, hi=8.0)
    Ad, Bd = A.to(dev()), B.to(dev())
    for split in (1, 3):
        p32 = imm.gemm_plan_ex(M, N, K, dt, "f32", split_k=split)
        p16 = imm.gemm_plan_ex(M, N, K, dt, "f16", split_k=split)
        for use_split in (False, True):
            c32 = _run(p32, Ad, Bd, use_split)
            c16 = _run(p16, Ad, Bd, use_split)
            v32 = values_of(c32)
            assert np.array_equal(bits_of(c16), oracle.round_rne("f16", v32)), (split, use_split)
            assert np.array_equal(bits_of(c16), wl.bits(c32.cpu().to(torch.float16)))


def test_linear_rows_do_not_depend_on_the_batch():
    N, K = 1024, 4096
    g = wl.gen(7400)
    x = wl.uniform((256, K), "bf16", g).to(dev())
    W = wl.normal((N, K), "bf16", g, std=K ** -0.5).to(dev())
    b = torch.randn((N,), generator=g).to(dev())
    full = None
    for m in (256, 129, 64, 7, 1):
        p = imm.gemm_plan_ex2(m, N, K, "bf16", "bf16", flags=BT)
        got = bits_of(_run(p, x[:m].contiguous(), W, p.info["split_k"] > 1, bias=b))
        if full is None:
            full = got
        log(f"linear M={m}: split {p.info['split_k']}, tile {p.info['tile']}")
        assert np.array_equal(got, full[:m]), m
