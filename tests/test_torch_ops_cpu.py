"""Host-side checks of the torch operator module (no GPU needed)."""
import torch
import torch.nn.functional as F

from invariant_matmul_amd import torch_ops


def _cuda_kernels(op):
    """The dispatcher's CUDA-key registrations of an aten operator."""
    return [ln for ln in torch._C._dispatch_dump(op).splitlines() if ln.startswith("CUDA")]


def test_mode_registers_and_removes_the_cuda_kernels():
    before = {op: _cuda_kernels(op) for op in ("aten::mm", "aten::addmm", "aten::bmm")}
    assert all(len(v) == 1 for v in before.values())
    with torch_ops.batch_invariant_mode():
        with torch_ops.batch_invariant_mode():      # nested: one registration
            inner = {op: _cuda_kernels(op) for op in before}
        outer = {op: _cuda_kernels(op) for op in before}
        for op in ("aten::mm", "aten::addmm"):
            # this module's kernel in front, torch's own one inactive behind it
            assert len(inner[op]) == 2 and "(inactive)" in inner[op][1], inner[op]
            assert "torch_ops.py" in inner[op][0], inner[op]
            assert outer[op] == inner[op]
        assert inner["aten::bmm"] == before["aten::bmm"]   # the fallback stays torch's
    after = {op: _cuda_kernels(op) for op in before}
    assert after == before


def test_mode_leaves_cpu_and_fp32_products_to_torch():
    g = torch.Generator().manual_seed(3)
    a = torch.randn(5, 16, generator=g)
    b = torch.randn(16, 8, generator=g)
    w = torch.randn(8, 16, generator=g)
    ref = (a @ b, torch.mm(a, b), torch.matmul(a, b), F.linear(a, w), torch.addmm(b[0], a, b))
    with torch_ops.batch_invariant_mode():
        got = (a @ b, torch.mm(a, b), torch.matmul(a, b), F.linear(a, w), torch.addmm(b[0], a, b))
    for r, x in zip(ref, got):
        assert torch.equal(r, x)


def test_supported_rules():
    a = torch.empty(4, 64, dtype=torch.float16)
    b = torch.empty(64, 32, dtype=torch.float16)
    assert not torch_ops.supported(a, b)  # CPU tensors
