"""Host-side checks of the torch operator module (no GPU needed)."""
import torch
import torch.nn.functional as F

from invariant_matmul_amd import torch_ops


def test_mode_restores_torch_entry_points():
    before = (F.linear, torch.mm, torch.addmm, torch.matmul, torch.Tensor.__matmul__)
    with torch_ops.batch_invariant_mode():
        inside = (F.linear, torch.mm, torch.addmm, torch.matmul, torch.Tensor.__matmul__)
        assert all(a is not b for a, b in zip(before, inside))
    after = (F.linear, torch.mm, torch.addmm, torch.matmul, torch.Tensor.__matmul__)
    assert all(a is b for a, b in zip(before, after))


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
