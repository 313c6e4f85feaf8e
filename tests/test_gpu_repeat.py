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
DMA_TILES = ["256x256", "128x256", "64x256", "32x256", "64x64", "32x64"]


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
