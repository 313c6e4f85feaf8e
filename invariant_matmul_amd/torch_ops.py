"""Batch-invariant torch operators on top of the library.

The Tencent deterministic-inference article closes with vLLM's
batch-invariant mode, which replaces ``mm``, ``addmm``, ``matmul`` and
``linear`` with a GEMM whose configuration never depends on the batch size.
This module gives the same four operators on this library, and a context
manager that installs the library as torch's CUDA kernels of ``aten::mm`` and
``aten::addmm`` (through ``torch.library``, the mechanism of that mode), so
every CUDA product that reaches them takes the library's path:

    from invariant_matmul_amd import torch_ops
    y = torch_ops.linear(x, weight, bias)          # x [..., K], weight [N, K]
    with torch_ops.batch_invariant_mode():
        y = model(x)                               # nn.Linear, torch.mm, x.mm, @ ...

The split of K is planned from (N, K, dtype) alone (the library's rule) and
the single pass takes its output tile from M (GEMM_PLAN_TILE_BY_M), which
moves work between workgroups but never changes a bit, so row i of a result
depends only on row i of the input, on the weight and on K: never on how many
rows share the call.  A weight given as a transposed
view (``W.t()`` of a contiguous [N, K] tensor, which is how ``linear`` hands
it over) is read in place through the library's transposed-B plans.  Inputs
are fp16 or bf16 CUDA tensors; the result has the input dtype (fp32 sums,
one rounding at the end); a bias is added in fp32 before that rounding.

fp64 CUDA tensors go through the library's Ozaki-scheme product (int8
slices, default slice count and Fast Mode threshold: the Insight Edge cuTile
blog's FP64 emulation, here with one exponent per row, so it is batch-
invariant too); a bias is then added with one fp64 addition.  Any N and K.
Its domain: a row of the first operand or a column of the second that holds
a NaN or an infinity, a magnitude above 2^300, or only nonzero magnitudes
below 2^-300 gives NaN in its whole row or column of the result.

The direct functions raise for anything else.  Under the context manager the
library computes what it supports (2-D weights; fp16 / bf16 with N and K
multiples of 8, or fp64; alpha = beta = 1; a bias of N values); other CUDA
calls of aten::mm / aten::addmm (fp32 tensors, a full-matrix bias, other
alpha and beta) run on torch's own batched GEMM (aten::bmm, batch of one),
since the registration replaces torch's mm kernel while it is active.  CPU
tensors and batched products (aten::bmm) are not affected.  Autograd's
backward products go through aten::mm too, so they take the same path.
"""
from __future__ import annotations

import contextlib
import functools
import threading
import warnings

import torch

from . import (PLAN_B_TRANSPOSED, PLAN_TILE_BY_M, gemm_plan_ex2, gemm_run, gemm_splitk_run,
               gemm_workspace_size, ozaki_plan, ozaki_run, ozaki_workspace_size)

__all__ = ["mm", "addmm", "linear", "matmul", "batch_invariant_mode", "supported"]

_DT = {torch.float16: "f16", torch.bfloat16: "bf16"}


@functools.lru_cache(maxsize=512)
def _plan(M: int, N: int, K: int, dt: str, flags: int):
    return gemm_plan_ex2(M, N, K, dt, dt, flags=flags)


def supported(a: torch.Tensor, b: torch.Tensor) -> bool:
    """True if a @ b (a [..., K], b [K, N]) is a product this module computes."""
    if not (a.is_cuda and b.is_cuda and b.dtype == a.dtype and b.dim() == 2 and a.dim() >= 1
            and a.shape[-1] == b.shape[0]):
        return False
    if a.dtype == torch.float64:
        return True
    return a.dtype in _DT and b.shape[0] % 8 == 0 and b.shape[1] % 8 == 0


@functools.lru_cache(maxsize=512)
def _ozaki_plan(M: int, N: int, K: int):
    return ozaki_plan(M, N, K, "i8")


def _product64(a2: torch.Tensor, b: torch.Tensor, bias) -> torch.Tensor:
    """a2 [M, K] @ b [K, N] (+ bias [N]) in fp64 by the Ozaki scheme."""
    M, K = a2.shape
    N = b.shape[1]
    out = torch.empty((M, N), dtype=torch.float64, device=a2.device)
    if M == 0 or N == 0:
        return out
    plan = _ozaki_plan(M, N, K)
    ws = torch.empty(max(1, ozaki_workspace_size(plan)), dtype=torch.uint8, device=a2.device)
    ozaki_run(plan, a2.contiguous(), b.contiguous(), out, ws)
    if bias is not None:
        out += bias.reshape(1, N).to(device=a2.device, dtype=torch.float64)
    return out


def _product(a2: torch.Tensor, b: torch.Tensor, bias) -> torch.Tensor:
    """a2 [M, K] @ b [K, N] (+ bias [N]) in the dtype of a2."""
    if a2.dtype == torch.float64:
        return _product64(a2, b, bias)
    M, K = a2.shape
    N = b.shape[1]
    dt = _DT[a2.dtype]
    a2 = a2.contiguous()
    flags = PLAN_TILE_BY_M
    if b.is_contiguous():
        bm = b
    elif b.t().is_contiguous():
        bm, flags = b.t(), flags | PLAN_B_TRANSPOSED  # the [N, K] weight itself
    else:
        bm = b.contiguous()
    out = torch.empty((M, N), dtype=a2.dtype, device=a2.device)
    if M == 0 or N == 0:
        return out
    bias32 = None
    if bias is not None:
        bias32 = bias.reshape(N).to(device=a2.device, dtype=torch.float32).contiguous()
    plan = _plan(M, N, K, dt, flags)
    if plan.info["split_k"] > 1:
        ws = torch.empty(max(1, gemm_workspace_size(plan) // 4), dtype=torch.float32,
                         device=a2.device)
        gemm_splitk_run(plan, a2, bm, out, ws, bias=bias32)
    else:
        gemm_run(plan, a2, bm, out, bias=bias32)
    return out


def _require(a, b):
    if not supported(a, b):
        raise ValueError(
            "invariant_matmul_amd.torch_ops: needs fp16/bf16 (K, N multiples of 8) or fp64 CUDA "
            "tensors, a [..., K] and a 2-D [K, N] second operand; got "
            f"{tuple(a.shape)} {a.dtype} @ "
            f"{tuple(b.shape)} {b.dtype}")


def mm(a: torch.Tensor, b: torch.Tensor) -> torch.Tensor:
    """a [M, K] @ b [K, N]."""
    if a.dim() != 2:
        raise ValueError("mm: a must be 2-D")
    _require(a, b)
    return _product(a, b, None)


def addmm(bias: torch.Tensor, a: torch.Tensor, b: torch.Tensor, *, beta=1, alpha=1) -> torch.Tensor:
    """bias + a @ b with a bias of N values (broadcast over rows); beta = alpha = 1."""
    if beta != 1 or alpha != 1:
        raise ValueError("addmm: only beta = alpha = 1")
    if a.dim() != 2:
        raise ValueError("addmm: a must be 2-D")
    _require(a, b)
    if bias.numel() != b.shape[1]:
        raise ValueError("addmm: the bias must hold N values")
    return _product(a, b, bias)


def linear(x: torch.Tensor, weight: torch.Tensor, bias=None) -> torch.Tensor:
    """x [..., K] @ weight[N, K]^T + bias."""
    wt = weight.t()
    _require(x, wt)
    lead = x.shape[:-1]
    y = _product(x.reshape(-1, x.shape[-1]), wt, bias)
    return y.reshape(*lead, weight.shape[0])


def matmul(a: torch.Tensor, b: torch.Tensor) -> torch.Tensor:
    """a [..., K] @ b [K, N] (leading dimensions of a are rows)."""
    _require(a, b)
    if a.dim() == 1:
        return _product(a.reshape(1, -1), b, None).reshape(b.shape[1])
    lead = a.shape[:-1]
    return _product(a.reshape(-1, a.shape[-1]), b, None).reshape(*lead, b.shape[1])


def _torch_mm(a: torch.Tensor, b: torch.Tensor) -> torch.Tensor:
    """a @ b on torch's batched GEMM (a batch of one); both operands contiguous."""
    return torch.bmm(a.unsqueeze(0).contiguous(), b.unsqueeze(0).contiguous()).squeeze(0)


def _row_bias(bias: torch.Tensor, N: int) -> bool:
    """True if bias holds N values broadcast over the rows."""
    return bias.numel() == N and (bias.dim() == 1 or (bias.dim() == 2 and bias.shape[0] == 1))


def _mode_mm(a, b):
    if a.dim() == 2 and supported(a, b):
        return _product(a, b, None)
    return _torch_mm(a, b)


def _mode_addmm(bias, a, b, *, beta=1, alpha=1):
    if (beta == 1 and alpha == 1 and a.dim() == 2 and supported(a, b)
            and _row_bias(bias, b.shape[1])):
        return _product(a, b, bias)
    r = _torch_mm(a, b)
    if alpha != 1:
        r = r * alpha
    if beta == 0:
        return r
    return r + (bias if beta == 1 else bias * beta)


_mode_lock = threading.Lock()
_mode_depth = 0
_mode_lib = None


@contextlib.contextmanager
def batch_invariant_mode():
    """Install this module's products as the CUDA kernels of aten::mm and
    aten::addmm while the context is active (nested contexts share one
    registration; the last exit removes it and torch's kernels return).  The
    registration is process-wide: products issued by other threads while it
    is active take the same path."""
    global _mode_depth, _mode_lib
    with _mode_lock:
        if _mode_depth == 0:
            lib = torch.library.Library("aten", "IMPL")
            with warnings.catch_warnings():
                # replacing a registered kernel is what this mode is for
                warnings.simplefilter("ignore")
                lib.impl("mm", _mode_mm, "CUDA")
                lib.impl("addmm", _mode_addmm, "CUDA")
            _mode_lib = lib
        _mode_depth += 1
    try:
        yield
    finally:
        with _mode_lock:
            _mode_depth -= 1
            if _mode_depth == 0:
                _mode_lib._destroy()
                _mode_lib = None
