"""The allocation-free split-K entry point against the split-K entry point
with a caller-owned workspace, bit for bit, through the C ABI.

gemm_splitk_run_noalloc takes its [split_k, M, N] workspace from an array
inside the library (for callers that cannot allocate device memory).  Two
calls in a row share that array, the second with a smaller input, so the
second finds the first one's partial sums in it; both must equal
gemm_splitk_run on the same plan.  The shapes are the decode product
(N = 4096, K = 14336, bf16, the default split of 16 slices) and the huge-K
product (256 x 256 x 131072 fp16, 128 slices: 32 MiB of workspace).
"""
import numpy as np
import pytest
import torch

import invariant_matmul_amd as imm
import workloads as wl
from tests.helpers import bits_of, dev, log, out_torch_dtype

pytestmark = pytest.mark.gpu


def _both(plan, A, B):
    info = plan.info
    ws = torch.empty(max(1, imm.gemm_workspace_size(plan) // 4), dtype=torch.float32,
                     device=dev())
    want = torch.empty((info["M"], info["N"]), dtype=out_torch_dtype(info["out_dtype"]),
                       device=dev())
    imm.gemm_splitk_run(plan, A, B, want, ws)
    got = torch.full_like(want, float("nan"))
    imm.gemm_splitk_run_noalloc(plan, A, B, got)
    return bits_of(got), bits_of(want)


def test_noalloc_decode_two_calls_second_smaller():
    w = wl.WORKLOADS["decode_bf16_m128"]
    A, B = w.make()
    Ad, Bd = A.to(dev()), B.to(dev())
    for m in (128, 8):
        plan = imm.gemm_plan(m, w.N, w.K, "bf16")
        log(f"noalloc decode M={m}: split {plan.info['split_k']}, "
            f"workspace {imm.gemm_workspace_size(plan)} bytes")
        got, want = _both(plan, Ad[:m].contiguous(), Bd)
        assert np.array_equal(got, want), m


def test_noalloc_hugek_then_ragged_smaller():
    w = wl.WORKLOADS["hugek_f16"]
    A, B = w.make()
    Ad, Bd = A.to(dev()), B.to(dev())
    plan = imm.gemm_plan(w.M, w.N, w.K, "f16")
    log(f"noalloc huge-K: split {plan.info['split_k']}, "
        f"workspace {imm.gemm_workspace_size(plan)} bytes")
    got, want = _both(plan, Ad, Bd)
    assert np.array_equal(got, want)
    # a smaller, ragged product right after: M = 37, N = 136, K = 3000 (bf16 out)
    g = wl.gen(9900)
    A2, B2 = wl.uniform((37, 3000), "f16", g).to(dev()), wl.uniform((3000, 136), "f16", g).to(dev())
    plan2 = imm.gemm_plan_ex(37, 136, 3000, "f16", "bf16", split_k=5)
    log(f"noalloc ragged: split {plan2.info['split_k']}")
    got2, want2 = _both(plan2, A2, B2)
    assert np.array_equal(got2, want2)


def test_noalloc_rejects_a_workspace_past_the_limit():
    plan = imm.gemm_plan(512, 4096, 14336, "bf16")
    assert imm.gemm_workspace_size(plan) > imm.NOALLOC_WORKSPACE_BYTES
    A = torch.zeros((512, 14336), dtype=torch.bfloat16, device=dev())
    B = torch.zeros((14336, 4096), dtype=torch.bfloat16, device=dev())
    C = torch.zeros((512, 4096), dtype=torch.float32, device=dev())
    st = imm.lib().gemm_splitk_run_noalloc(plan.handle, A.data_ptr(), B.data_ptr(),
                                           C.data_ptr(), None)
    assert st == 3
