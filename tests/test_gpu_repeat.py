"""Repeated runs give the same bits and write every element.

A batch-invariant product must also be run-to-run deterministic ([TDI]
"背景": the same input gives the same output).  Every DMA-tile
configuration (tile, input dtype, B layout, single pass or split-K partial)
runs the same product REPS times into outputs and workspaces filled with NaN
beforehand: any element a kernel fails to write, or writes to the wrong
place, shows up as a NaN or as a difference between runs.  The shapes have a
single K stage (where the last stage's fragment reads are still in flight
when the loop ends) and three.
"""
import numpy as np
import pytest
import torch

import invariant_matmul_amd as imm
import workloads as wl
from tests.helpers import dev, log, out_torch_dtype, tiles_for

pytestmark = pytest.mark.gpu

REPS = 12
DMA_TILES = ["256x256", "128x256", "64x256", "32x256", "64x64", "32x64", "32x32"]


def _once(plan, A, B, split):
    info = plan.info
    C = torch.full((info["M"], info["N"]), float("nan"), dtype=out_torch_dtype(info["out_dtype"]),
                   device=dev())
    if split:
        ws = torch.full((max(1, imm.gemm_workspace_size(plan) // 4),), float("nan"),
                        dtype=torch.float32, device=dev())
        imm.gemm_splitk_run(plan, A, B, C, ws)
    else:
        imm.gemm_run(plan, A, B, C)
    torch.cuda.synchronize()
    return C.cpu()


@pytest.mark.parametrize("dt,flags", [("f16", 0), ("bf16", 0), ("e4m3", 0), ("e5m2", 0),
                                      ("e4m3", imm.PLAN_FP8_FP32_ACCUM)])
@pytest.mark.parametrize("K", [128, 384])
def test_every_dma_configuration_repeats_bitwise(dt, flags, K):
    M, N = 300, 272
    g = wl.gen(14000 + K)
    A = wl.normal((M, K), dt, g).to(dev())
    B = wl.normal((K, N), dt, g)
    Bkn, Bt = B.to(dev()), B.t().contiguous().to(dev())
    for tile in tiles_for(dt, DMA_TILES):
        for fl, Bx in ((0, Bkn), (imm.PLAN_B_TRANSPOSED, Bt)):
            for split in (1, 3):
                p = imm.gemm_plan_ex2(M, N, K, dt, "bf16", split_k=split, tile=tile, flags=flags | fl)
                for use_split in ((False, True) if split == 1 else (True,)):
                    first = _once(p, A, Bx, use_split)
                    assert not torch.isnan(first).any(), (tile, fl, split, use_split, "unwritten")
                    ref = wl.bits(first)
                    for r in range(1, REPS):
                        got = wl.bits(_once(p, A, Bx, use_split))
                        assert np.array_equal(got, ref), (tile, fl, split, use_split, r)
        log(f"{dt} flags {flags} K={K} {tile}: {REPS} runs identical")


def test_other_paths_repeat_bitwise():
    """The persistent launch, the register-staged tiles, the bias epilogue and
    the Ozaki product: same bits on every run, every element written."""
    g = wl.gen(14100)
    M, N, K = 520, 528, 640
    A = wl.normal((M, K), "bf16", g).to(dev())
    B = wl.normal((K, N), "bf16", g).to(dev())
    bias = torch.randn(N, generator=g).to(torch.float32).to(dev())
    cases = [("persistent", imm.gemm_plan_ex2(M, N, K, "bf16", "f32", tile="256x256",
                                              flags=imm.PLAN_PERSISTENT), False, None)]
    for tile in ("128x128", "32x128", "256x256_rs"):
        for split in (1, 3):
            cases.append((f"{tile} split {split}",
                          imm.gemm_plan_ex2(M, N, K, "bf16", "f32", split_k=split, tile=tile),
                          split > 1, None))
    cases.append(("bias 256x256", imm.gemm_plan_ex2(M, N, K, "bf16", "bf16"), False, bias))
    cases.append(("bias split", imm.gemm_plan_ex2(M, N, K, "bf16", "f32", split_k=3), True, bias))
    for name, p, split, b in cases:
        runs = []
        for _ in range(REPS // 2):
            C = torch.full((M, N), float("nan"), dtype=out_torch_dtype(p.info["out_dtype"]),
                           device=dev())
            if split:
                ws = torch.full((imm.gemm_workspace_size(p) // 4,), float("nan"),
                                dtype=torch.float32, device=dev())
                imm.gemm_splitk_run(p, A, B, C, ws, bias=b)
            else:
                imm.gemm_run(p, A, B, C, bias=b)
            torch.cuda.synchronize()
            c = C.cpu()
            assert not torch.isnan(c).any(), (name, "unwritten")
            runs.append(wl.bits(c))
        assert all(np.array_equal(r, runs[0]) for r in runs), name
        log(f"{name}: {len(runs)} runs identical")
    # Ozaki: the slice-pair kernel is a DMA kernel with its own epilogue
    Ad = torch.randn((192, 320), dtype=torch.float64, generator=g).to(dev())
    Bd = torch.randn((320, 200), dtype=torch.float64, generator=g).to(dev())
    for t2 in ("bf16", "e4m3", "i8"):
        outs = [imm.ozaki_mm(Ad, Bd, t2).cpu() for _ in range(REPS // 2)]
        assert not any(torch.isnan(o).any() for o in outs), t2
        assert all(torch.equal(o.view(torch.int64), outs[0].view(torch.int64)) for o in outs), t2
        log(f"ozaki {t2}: {len(outs)} runs identical")
