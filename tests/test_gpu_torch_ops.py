"""GPU tests of the batch-invariant torch operators (invariant_matmul_amd.torch_ops).

The operators are the ones vLLM's batch-invariant mode replaces (listed in the
closing section of the Tencent deterministic-inference article): linear, mm,
addmm, matmul.  Checked: results against the CPU oracle within the bound
(one fp32 sum, an fp32 bias add, one rounding to the input dtype); bitwise
row invariance of a stack of nn.Linear layers run under the mode, at batch
sizes 1 .. 256; and that the mode hands the transposed weight view to the
transposed-B plans without copying it (same bits as an explicit [K, N] copy).
"""
import numpy as np
import pytest
import torch

import invariant_matmul_amd as imm
import oracle
import workloads as wl
from invariant_matmul_amd import torch_ops
from tests.helpers import bits_of, check_bound, dev, log, values_of

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_linear_matches_the_oracle(dt):
    M, N, K = 77, 520, 1024
    g = wl.gen(8000)
    x = wl.uniform((M, K), dt, g)
    W = wl.normal((N, K), dt, g, std=K ** -0.5)
    b = wl.normal((N,), dt, g)
    Y64, Yabs = oracle.linear(wl.bits(x), wl.bits(W), dt, bias=b.double().numpy())
    y = torch_ops.linear(x.to(dev()), W.to(dev()), b.to(dev()))
    assert y.dtype == x.dtype and y.shape == (M, N)
    r = check_bound(values_of(y), Y64, Yabs, K, dt, bias=True)
    log(f"linear {dt}: max err / bound = {r:.3g}")


def test_mm_addmm_matmul_agree_with_the_library():
    M, N, K = 64, 256, 512
    g = wl.gen(8100)
    a = wl.uniform((M, K), "f16", g).to(dev())
    b = wl.uniform((K, N), "f16", g).to(dev())
    bias = wl.uniform((N,), "f16", g).to(dev())
    plan = imm.gemm_plan_ex2(M, N, K, "f16", "f16")
    # K >= 2N: the plan splits K, and the operators take the split-K path
    assert plan.info["split_k"] > 1
    C = torch.empty((M, N), dtype=torch.float16, device=dev())
    ws = torch.empty(imm.gemm_workspace_size(plan) // 4, dtype=torch.float32, device=dev())
    imm.gemm_splitk_run(plan, a, b, C, ws)
    ref = bits_of(C)
    assert np.array_equal(bits_of(torch_ops.mm(a, b)), ref)
    assert np.array_equal(bits_of(torch_ops.matmul(a, b)), ref)
    assert np.array_equal(bits_of(torch_ops.matmul(a.reshape(4, 16, K), b).reshape(M, N)), ref)
    imm.gemm_splitk_run(plan, a, b, C, ws, bias=bias.float())
    assert np.array_equal(bits_of(torch_ops.addmm(bias, a, b)), bits_of(C))
    # a shape without a split goes through the single pass
    p2 = imm.gemm_plan_ex2(M, 512, K, "f16", "f16")
    assert p2.info["split_k"] == 1
    b2 = wl.uniform((K, 512), "f16", g).to(dev())
    C2 = torch.empty((M, 512), dtype=torch.float16, device=dev())
    imm.gemm_run(p2, a, b2, C2)
    assert np.array_equal(bits_of(torch_ops.mm(a, b2)), bits_of(C2))


def test_transposed_weight_view_is_read_in_place():
    M, N, K = 33, 384, 768
    g = wl.gen(8200)
    x = wl.uniform((M, K), "bf16", g).to(dev())
    W = wl.normal((N, K), "bf16", g, std=K ** -0.5).to(dev())
    via_view = torch_ops.mm(x, W.t())             # B given as the [N, K] weight
    via_copy = torch_ops.mm(x, W.t().contiguous())  # B copied to [K, N]
    assert np.array_equal(bits_of(via_view), bits_of(via_copy))


@pytest.mark.parametrize("dt", [torch.float16, torch.bfloat16])
def test_nn_linear_stack_is_batch_invariant_under_the_mode(dt):
    torch.manual_seed(0)
    layers = torch.nn.Sequential(
        torch.nn.Linear(1024, 2048), torch.nn.GELU(), torch.nn.Linear(2048, 512)).to(dev(), dt)
    g = torch.Generator(device="cpu").manual_seed(1)
    x = torch.randn((256, 1024), generator=g).to(dev(), dt)
    with torch.no_grad(), torch_ops.batch_invariant_mode():
        y_full = layers(x)
        full = bits_of(y_full)
        for m in (1, 3, 64, 129):
            part = bits_of(layers(x[:m]))
            log(f"nn.Linear stack {dt} batch {m}")
            assert np.array_equal(part, full[:m]), m
        # rows computed in another order equal the same rows of the first batch
        perm = torch.randperm(256, generator=g).to(dev())
        shuffled = bits_of(layers(x[perm]))
        assert np.array_equal(shuffled, full[perm.cpu().numpy()])
    with torch.no_grad():
        plain = layers(x)
    # outside the mode torch computes the same layers its own way: close, not bitwise
    assert torch.allclose(plain.float(), y_full.float(), rtol=5e-2, atol=5e-2)


def test_fp64_products_go_through_the_ozaki_scheme():
    """fp64 operators: the library's Ozaki product with int8 slices, bit for
    bit against the oracle, any N and K, with a bias added in fp64."""
    from oracle import ozaki
    M, N, K = 45, 123, 301
    g = wl.gen(8500)
    a, b = wl.wide64((M, K), g), wl.wide64((K, N), g)
    bias = wl.uniform64((N,), g)
    want = ozaki.gemm(a.numpy(), b.numpy(), "i8")
    ad, bd = a.to(dev()), b.to(dev())
    got = torch_ops.mm(ad, bd).cpu().numpy()
    assert np.array_equal(got.view(np.uint64), want.view(np.uint64))
    assert np.array_equal(torch_ops.matmul(ad, bd).cpu().numpy(), got)
    lin = torch_ops.linear(ad, bd.t(), bias.to(dev())).cpu().numpy()
    assert np.array_equal(lin, want + bias.numpy()[None, :])
    # rows do not depend on the rest of the batch, under the mode too
    with torch_ops.batch_invariant_mode():
        part = (ad[:7] @ bd).cpu().numpy()
    assert np.array_equal(part, got[:7])


def test_mode_routes_every_entry_point_through_the_library():
    """Under the mode, aten::mm and aten::addmm are the library's: torch.mm,
    the Tensor.mm and Tensor.matmul methods, @, F.linear on 2-D and 3-D input
    and nn.Linear give the direct functions' bits."""
    M, N, K = 48, 384, 256
    g = wl.gen(8600)
    x = wl.uniform((M, K), "f16", g).to(dev())
    W = wl.normal((N, K), "f16", g, std=K ** -0.5).to(dev())
    bias = wl.normal((N,), "f16", g).to(dev())
    want_mm = bits_of(torch_ops.mm(x, W.t().contiguous()))
    want_lin = bits_of(torch_ops.linear(x, W, bias))
    lin = torch.nn.Linear(K, N).to(dev(), torch.float16)
    with torch.no_grad():
        lin.weight.copy_(W)
        lin.bias.copy_(bias)
    Wt = W.t().contiguous()
    with torch.no_grad(), torch_ops.batch_invariant_mode():
        for got in (torch.mm(x, Wt), x.mm(Wt), x.matmul(Wt), x @ Wt, torch.matmul(x, Wt)):
            assert np.array_equal(bits_of(got), want_mm)
        for got in (torch.nn.functional.linear(x, W, bias), lin(x),
                    torch.nn.functional.linear(x.reshape(4, 12, K), W, bias).reshape(M, N)):
            assert np.array_equal(bits_of(got), want_lin)


def test_mode_falls_back_to_torch_for_other_products():
    """fp32 CUDA products and addmm with alpha / beta or a full-matrix bias run
    on torch's batched GEMM under the mode: the values torch gives outside it."""
    g = torch.Generator().manual_seed(8700)
    a = torch.randn((40, 96), generator=g).to(dev())
    b = torch.randn((96, 72), generator=g).to(dev())
    full = torch.randn((40, 72), generator=g).to(dev())
    ah, bh = a.half(), b.half()
    ref = (a @ b, torch.addmm(full, a, b), torch.addmm(full.half(), ah, bh, beta=0.5, alpha=2.0))
    with torch_ops.batch_invariant_mode():
        got = (a @ b, torch.addmm(full, a, b), torch.addmm(full.half(), ah, bh, beta=0.5, alpha=2.0))
    for r, x in zip(ref, got):
        assert x.dtype == r.dtype and x.shape == r.shape
        assert torch.allclose(x.float(), r.float(), rtol=2e-2, atol=2e-2)


def test_backward_under_the_mode_is_batch_invariant():
    """Autograd's backward products are aten::mm calls too: under the mode the
    input gradient of each row depends only on that row."""
    torch.manual_seed(0)
    layer = torch.nn.Linear(512, 256).to(dev(), torch.float16)
    g = torch.Generator().manual_seed(8800)
    x = torch.randn((64, 512), generator=g).to(dev(), torch.float16)
    gy = torch.randn((64, 256), generator=g).to(dev(), torch.float16)

    def input_grad(rows):
        xi = x[:rows].clone().requires_grad_(True)
        with torch_ops.batch_invariant_mode():
            layer(xi).backward(gy[:rows])
        return bits_of(xi.grad)

    full = input_grad(64)
    for m in (1, 5, 33):
        assert np.array_equal(input_grad(m), full[:m]), m
