"""The entry points under HIP graph capture.

The library allocates nothing, never synchronises and records no memset, so
its launches can be captured into a graph (torch.cuda.CUDAGraph on ROCm is a
hipGraph) and replayed.  Each graph here is replayed several times, with
unrelated eager work and synchronisations between the replays, and every
replay must give the bits of the eager call.
"""
import numpy as np
import pytest
import torch

import invariant_matmul_amd as imm
import workloads as wl
from tests.helpers import bits_of, dev, log

pytestmark = pytest.mark.gpu

REPLAYS = 4


def _capture(fn):
    """Warm up on a side stream, then capture fn() into a graph."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def _bits(C):
    if C.dtype == torch.float64:
        torch.cuda.synchronize()
        return C.cpu().contiguous().view(torch.int64).numpy()
    return bits_of(C)


def _replays_match(g, out, ref, other):
    for r in range(REPLAYS):
        out.fill_(float("nan"))       # the replay must rewrite every element
        other()                       # unrelated eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = _bits(out)
        assert np.array_equal(got, ref), f"replay {r}"


@pytest.mark.parametrize("name,split", [("decode_bf16_m128", True), ("square_f16_1024", False),
                                        ("hugek_f16", True)])
def test_gemm_graph_replays_equal_eager(name, split):
    w = wl.WORKLOADS[name]
    A, B = w.make()
    M = 8 if name == "decode_bf16_m128" else w.M
    Ad, Bd = A[:M].contiguous().to(dev()), B.to(dev())
    plan = imm.gemm_plan_ex(M, w.N, w.K, w.dtype, w.out)
    C = torch.empty((M, w.N), dtype=torch.float32, device=dev())
    ws = torch.empty(max(1, imm.gemm_workspace_size(plan) // 4), dtype=torch.float32, device=dev())

    def call():
        if split:
            imm.gemm_splitk_run(plan, Ad, Bd, C, ws)
        else:
            imm.gemm_run(plan, Ad, Bd, C)

    call()
    ref = _bits(C)
    log(f"graph {name}: M={M} split_k={plan.info['split_k'] if split else 1}")
    g = _capture(call)
    # other eager work: a different product into other buffers
    X = torch.randn((256, 256), device=dev()).half()
    Y = torch.empty((256, 256), dtype=torch.float32, device=dev())
    p2 = imm.gemm_plan(256, 256, 256, "f16")
    _replays_match(g, C, ref, lambda: imm.gemm_run(p2, X, X, Y))


def test_ozaki_graph_replays_equal_eager():
    n = 300
    g0 = torch.Generator().manual_seed(77)
    A = (torch.rand((n, n + 40), generator=g0, dtype=torch.float64) * 2 - 1).to(dev())
    B = (torch.rand((n + 40, n - 20), generator=g0, dtype=torch.float64) * 2 - 1).to(dev())
    plan = imm.ozaki_plan(n, n - 20, n + 40, "i8")
    ws = torch.empty(imm.ozaki_workspace_size(plan), dtype=torch.uint8, device=dev())
    C = torch.empty((n, n - 20), dtype=torch.float64, device=dev())

    def call():
        imm.ozaki_run(plan, A, B, C, ws)

    call()
    ref = _bits(C)
    g = _capture(call)
    Z = torch.empty_like(C)
    _replays_match(g, C, ref, lambda: Z.copy_(A[:, :n - 20] * 2.0))
