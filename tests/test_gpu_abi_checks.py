"""The C ABI's device-memory checks on a GPU.

Every run call checks, before it enqueues anything, that each operand lies
wholly inside one device allocation of the current device.  The cases here
are chosen so that a kernel would not fault even if a check were missing:
pinned host memory is reachable from the GPU, and the short buffer is short of
an allocation size that the runtime rounds up to whole pages anyway.  (Host
tensors are refused by the Python binding before any HIP call; that is
tested on the CPU.)
"""
import ctypes

import numpy as np
import pytest
import torch

import invariant_matmul_amd as imm
import oracle
import workloads as wl
from tests.helpers import bits_of, dev, expected_bits

pytestmark = pytest.mark.gpu


def _hip():
    h = ctypes.CDLL("libamdhip64.so")
    h.hipMalloc.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_size_t]
    h.hipFree.argtypes = [ctypes.c_void_p]
    h.hipMemGetAddressRange.argtypes = [ctypes.POINTER(ctypes.c_void_p),
                                        ctypes.POINTER(ctypes.c_size_t), ctypes.c_void_p]
    return h


def test_pinned_host_operands_are_rejected():
    M, N, K = 64, 256, 512
    plan = imm.gemm_plan(M, N, K, "f16")
    A = torch.zeros((M, K), dtype=torch.float16, device=dev())
    B = torch.zeros((K, N), dtype=torch.float16, device=dev())
    C = torch.zeros((M, N), dtype=torch.float32, device=dev())
    Ah = torch.zeros((M, K), dtype=torch.float16).pin_memory()
    Ch = torch.zeros((M, N), dtype=torch.float32).pin_memory()
    L = imm.lib()
    assert L.gemm_run(plan.handle, Ah.data_ptr(), B.data_ptr(), C.data_ptr(), None) == 1
    assert L.gemm_run(plan.handle, A.data_ptr(), B.data_ptr(), Ch.data_ptr(), None) == 1
    p4 = imm.gemm_plan_ex(M, N, K, "f16", "f32", split_k=4)
    nws = imm.gemm_workspace_size(p4)
    wsh = torch.zeros(nws // 4, dtype=torch.float32).pin_memory()
    ws = torch.zeros(nws // 4, dtype=torch.float32, device=dev())
    assert L.gemm_splitk_run(p4.handle, A.data_ptr(), B.data_ptr(), C.data_ptr(),
                             wsh.data_ptr(), nws, None) == 1
    assert L.gemm_splitk_run(p4.handle, A.data_ptr(), B.data_ptr(), C.data_ptr(),
                             ws.data_ptr(), nws, None) == 0
    torch.cuda.synchronize()


def test_short_and_exact_raw_allocations():
    M, N, K = 64, 256, 512
    need = M * N * 4                       # 64 KiB of fp32 C: a whole number of pages
    hip = _hip()
    g = wl.gen(9950)
    A, B = wl.integers((M, K), "f16", g), wl.integers((K, N), "f16", g)
    Ad, Bd = A.to(dev()), B.to(dev())
    plan = imm.gemm_plan(M, N, K, "f16")
    ptrs = []
    try:
        for size in (need - 256, need):
            p = ctypes.c_void_p()
            assert hip.hipMalloc(ctypes.byref(p), size) == 0
            ptrs.append(p)
            base, rng = ctypes.c_void_p(), ctypes.c_size_t()
            assert hip.hipMemGetAddressRange(ctypes.byref(base), ctypes.byref(rng), p) == 0
            st = imm.lib().gemm_run(plan.handle, Ad.data_ptr(), Bd.data_ptr(), p.value, None)
            torch.cuda.synchronize()
            if rng.value < need:
                assert st == 1, (size, rng.value)
            else:
                assert st == 0, (size, rng.value)
                C = torch.empty((M, N), dtype=torch.float32, device=dev())
                assert hip.hipMemcpy is not None
                imm.gemm_run(plan, Ad, Bd, C)
                got = np.empty(M * N, dtype=np.uint32)
                hip.hipMemcpy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                          ctypes.c_int]
                assert hip.hipMemcpy(got.ctypes.data, p.value, need, 2) == 0  # device to host
                C64, _ = oracle.gemm(wl.bits(A), wl.bits(B), "f16")
                assert np.array_equal(got.reshape(M, N), expected_bits(C64, "f32"))
                assert np.array_equal(bits_of(C), expected_bits(C64, "f32"))
    finally:
        torch.cuda.synchronize()
        for p in ptrs:
            hip.hipFree(p)
