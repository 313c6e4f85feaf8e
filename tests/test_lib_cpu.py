"""Host-side tests of the C ABI (no GPU needed).

- the shared library loads and exports every function include/invariant_matmul.h declares;
- plans are a pure function of (N, K, dtypes, options): nothing but the grid
  and the workspace size changes with M (the Tencent deterministic-inference
  article, section "Batch Invariance の由来", names M-driven choices of the K
  step and of split-K as the cause of batch variance);
- the tile raster (XCD remap + GROUP_M) is a bijection onto the tiles x slices;
- every invalid argument is rejected with its status before any HIP call, and
  a valid call on a machine without a GPU returns GEMM_ERR_HIP.
"""
import ctypes
import itertools
import os
import re

import pytest

import invariant_matmul_amd as imm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "invariant_matmul.h")

M_INDEPENDENT = ("N", "K", "in_dtype", "out_dtype", "tile", "block_m", "block_n", "block_k",
                 "mfma_m", "mfma_n", "mfma_k", "waves", "group_m", "split_k", "k_per_split",
                 "tiles_n", "scale_a", "scale_b", "run_tile", "run_block_m", "run_block_n",
                 "run_waves", "run_tiles_n")

SHAPES = [  # (N, K, dtype) of every workload family, plus a few others
    (256, 256, "f16"), (1024, 1024, "f16"), (4096, 4096, "f16"), (8192, 8192, "f16"),
    (4096, 14336, "bf16"), (256, 131072, "f16"), (4096, 4096, "e5m2"), (8192, 8192, "e5m2"),
    (16384, 16384, "e5m2"), (6144, 4096, "bf16"), (4096, 4096, "e4m3"), (136, 200, "f16"),
]


def _declared_functions():
    text = open(HEADER, encoding="utf-8").read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b((?:gemm|ozaki)_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    names = _declared_functions()
    assert set(names) == set(imm.EXPORTED_SYMBOLS), names
    L = imm.lib()
    for n in names:
        assert hasattr(L, n), n


def test_status_strings():
    for code, name in imm.STATUS.items():
        assert imm.gemm_status_string(code) == name


@pytest.mark.parametrize("N,K,dt", SHAPES)
def test_plan_is_independent_of_M(N, K, dt):
    ref = None
    for M in (1, 2, 7, 8, 31, 32, 33, 64, 127, 128, 1000, 4096, 8192):
        info = imm.gemm_plan(M, N, K, dt).info
        key = {k: info[k] for k in M_INDEPENDENT}
        if ref is None:
            ref = key
        assert key == ref, (M, key, ref)
        assert info["workspace_bytes"] == info["split_k"] * M * N * 4
        assert info["tiles_m"] == -(-M // info["block_m"])
        assert info["run_tiles_m"] == -(-M // info["run_block_m"])
        assert info["grid_splitk"] == info["tiles_m"] * info["tiles_n"] * info["split_k"]
        assert info["grid_run"] == info["run_tiles_m"] * info["run_tiles_n"]


@pytest.mark.parametrize("N,K,dt", SHAPES)
def test_plan_ex_options_are_independent_of_M(N, K, dt):
    for split, gm, tile in [(1, 1, "128x128"), (8, 4, "32x128"), (3, 0, "256x256")]:
        infos = [imm.gemm_plan_ex(M, N, K, dt, "f32", split, gm, tile).info for M in (1, 77, 4096)]
        keys = [{k: i[k] for k in M_INDEPENDENT} for i in infos]
        assert keys[0] == keys[1] == keys[2]


@pytest.mark.parametrize("N,K,dt", SHAPES)
def test_split_covers_K_in_block_multiples(N, K, dt):
    for split in (0, 1, 2, 7, 8, 32, 128, 4096):
        i = imm.gemm_plan_ex(64, N, K, dt, "f32", split_k=split).info
        assert i["k_per_split"] % i["block_k"] == 0
        assert i["k_per_split"] * i["split_k"] >= K
        assert i["k_per_split"] * (i["split_k"] - 1) < K  # no empty slice
        if split:
            assert i["split_k"] <= split


def test_default_plans_of_the_workloads():
    sq = imm.gemm_plan(8192, 8192, 8192, "f16").info
    assert (sq["block_m"], sq["block_n"], sq["split_k"]) == (256, 256, 1)
    assert (sq["mfma_m"], sq["mfma_n"], sq["mfma_k"]) == (16, 16, 32)
    fp8 = imm.gemm_plan(8192, 8192, 8192, "e5m2").info
    assert (fp8["mfma_m"], fp8["mfma_n"], fp8["mfma_k"]) == (16, 16, 128)
    assert fp8["out_dtype"] == imm.DTYPE["bf16"]
    dec = imm.gemm_plan(1, 4096, 14336, "bf16").info
    assert dec["split_k"] > 1 and dec["block_m"] == 32
    # without a split the single pass keeps the large tile (the plan cannot
    # know that M is small)
    assert (dec["run_block_m"], dec["run_block_n"]) == (256, 256)
    hk = imm.gemm_plan(256, 256, 131072, "f16").info
    assert (hk["block_m"], hk["block_n"], hk["split_k"]) == (128, 256, 128)
    # fp8 slices of 2048 elements are 16 steps: no extra doubling
    hk8 = imm.gemm_plan(256, 256, 131072, "e5m2").info
    assert (hk8["block_m"], hk8["split_k"]) == (128, 64)
    # small B: the 64 x 64 tile for 16-bit inputs, 128 x 256 for fp8, for the
    # single pass and the (unsplit) split path
    for dt, tile in (("f16", (64, 64)), ("e5m2", (128, 256)), ("bf16", (64, 64))):
        small = imm.gemm_plan(1024, 1024, 1024, dt).info
        assert (small["run_block_m"], small["run_block_n"]) == tile
        assert (small["block_m"], small["block_n"], small["split_k"]) == (*tile, 1)
        bt = imm.gemm_plan_ex2(1024, 1024, 1024, dt, "f32", flags=imm.PLAN_B_TRANSPOSED).info
        assert (bt["run_block_m"], bt["run_block_n"]) == tile
    # a reduction-dominated small B keeps its split path (and bits); the single pass
    # takes the small-B tile too
    rd = imm.gemm_plan(16, 1024, 2048, "f16").info
    assert (rd["block_m"], rd["block_n"]) == (32, 128) and rd["split_k"] > 1
    assert (rd["run_block_m"], rd["run_block_n"]) == (64, 64)


@pytest.mark.parametrize("M,N,K,dt,split,gm", [
    (8192, 8192, 8192, "f16", 1, 8), (1000, 1000, 512, "f16", 1, 8), (256, 256, 131072, "f16", 128, 8),
    (128, 4096, 14336, "bf16", 0, 8), (300, 136, 200, "bf16", 3, 3), (77, 272, 64, "e5m2", 1, 1),
    (4096, 4096, 4096, "e5m2", 2, 5),
])
def test_raster_is_a_bijection(M, N, K, dt, split, gm):
    p = imm.gemm_plan_ex(M, N, K, dt, "f32", split_k=split, group_m=gm)
    i = p.info
    G = i["grid_splitk"]
    seen = set()
    for w in range(G):
        s, pm, pn = imm.gemm_plan_tile_of(p, w)
        assert 0 <= s < i["split_k"] and 0 <= pm < i["tiles_m"] and 0 <= pn < i["tiles_n"]
        seen.add((s, pm, pn))
    assert len(seen) == G == i["split_k"] * i["tiles_m"] * i["tiles_n"]
    with pytest.raises(imm.GemmError):
        imm.gemm_plan_tile_of(p, G)


def test_raster_groups_rows_within_an_xcd():
    # Consecutive workgroups on one XCD (w, w+8, w+16, ...) sweep GROUP_M rows of
    # tiles before moving to the next column.
    p = imm.gemm_plan_ex(8192, 8192, 8192, "f16", "f32", group_m=8)
    coords = [imm.gemm_plan_tile_of(p, w) for w in range(0, 8 * 16, 8)]
    assert [c[1] for c in coords[:8]] == list(range(8))
    assert all(c[2] == 0 for c in coords[:8]) and all(c[2] == 1 for c in coords[8:16])


# ------------------------------------------------------------ error statuses


def _plan_status(*args):
    # (M, N, K, in, out, split_k, group_m, tile, scale_a, scale_b) through
    # gemm_plan_ex2 without flags; with the default tile also through
    # gemm_plan_ex, which must agree
    L = imm.lib()
    h = ctypes.c_void_p()
    st = L.gemm_plan_ex2(*args, 0, ctypes.byref(h))
    L.gemm_plan_destroy(h)
    if args[7] == 0:
        h1 = ctypes.c_void_p()
        st1 = L.gemm_plan_ex(*args[:7], *args[8:], ctypes.byref(h1))
        L.gemm_plan_destroy(h1)
        assert st1 == st, (args, st1, st)
    return st


@pytest.mark.parametrize("args,status", [
    ((-1, 8, 8, 0, 4, 0, 0, 0, 1.0, 1.0), 1),
    ((8, -8, 8, 0, 4, 0, 0, 0, 1.0, 1.0), 1),
    ((8, 8, -8, 0, 4, 0, 0, 0, 1.0, 1.0), 1),
    ((8, 8, 8, 4, 4, 0, 0, 0, 1.0, 1.0), 2),      # fp32 input unsupported
    ((8, 8, 8, 0, 3, 0, 0, 0, 1.0, 1.0), 2),      # fp8 output unsupported
    ((8, 8, 8, 0, 0, 0, 0, 0, 1.0, 1.0), 0),      # fp16 output
    ((8, 8, 8, 7, 4, 0, 0, 0, 1.0, 1.0), 2),      # unknown dtype
    ((8, 12, 8, 0, 4, 0, 0, 0, 1.0, 1.0), 2),     # N not a multiple of 8
    ((8, 8, 12, 0, 4, 0, 0, 0, 1.0, 1.0), 2),     # K not a multiple of 8
    ((8, 16, 8, 3, 4, 0, 0, 0, 1.0, 1.0), 2),     # fp8 needs K % 16 == 0
    ((8, 8, 8, 0, 4, -1, 0, 0, 1.0, 1.0), 2),     # split_k < 0
    ((8, 8, 8, 0, 4, 4097, 0, 0, 1.0, 1.0), 2),   # split_k too large
    ((8, 8, 8, 0, 4, 0, -1, 0, 1.0, 1.0), 2),     # group_m < 0
    ((8, 8, 8, 0, 4, 0, 0, 11, 1.0, 1.0), 2),     # unknown tile
    ((8, 8, 8, 0, 4, 0, 0, 0, float("inf"), 1.0), 2),
    ((8, 8, 8, 0, 4, 0, 0, 0, 1.0, float("nan")), 2),
    ((2 ** 31, 8, 8, 0, 4, 0, 0, 0, 1.0, 1.0), 2),
    ((8, 8, 8, 0, 4, 0, 0, 0, 1.0, 1.0), 0),
    ((0, 8, 8, 0, 4, 0, 0, 0, 1.0, 1.0), 0),
    ((8, 8, 0, 0, 4, 0, 0, 0, 1.0, 1.0), 0),
])
def test_plan_validation(args, status):
    assert _plan_status(*args) == status


def _plan2_status(*args):
    h = ctypes.c_void_p()
    return imm.lib().gemm_plan_ex2(*args, ctypes.byref(h))


@pytest.mark.parametrize("args,status", [
    ((8, 8, 8, 0, 4, 0, 0, 0, 1.0, 1.0, 0), 0),
    ((8, 8, 8, 0, 4, 0, 0, 0, 1.0, 1.0, 1), 0),            # B given as [N, K]
    ((8, 8, 8, 0, 4, 0, 0, 0, 1.0, 1.0, 2), 0),            # persistent single pass
    ((8, 8, 8, 0, 4, 0, 0, 0, 1.0, 1.0, 3), 0),
    ((8, 8, 8, 0, 4, 0, 0, 0, 1.0, 1.0, 4), 0),            # tile from M (single pass)
    ((8, 8, 8, 0, 4, 0, 0, 0, 1.0, 1.0, 7), 0),
    ((8, 8, 8, 0, 4, 0, 0, 0, 1.0, 1.0, 16), 2),           # unknown flag bit
    ((8, 8, 8, 0, 4, 0, 0, 0, 1.0, 1.0, 8), 2),            # fp16 step for fp8: fp16 input
    ((16, 16, 16, 1, 4, 0, 0, 0, 1.0, 1.0, 8), 2),         # ... bf16 input
    ((16, 16, 16, 2, 1, 0, 0, 0, 1.0, 1.0, 8), 0),         # ... e4m3
    ((16, 16, 16, 3, 4, 0, 0, 0, 1.0, 1.0, 15), 0),        # ... e5m2 with every flag
    ((16, 16, 16, 2, 1, 0, 0, 3, 1.0, 1.0, 8), 2),         # ... needs a DMA tile
    ((16, 16, 16, 2, 1, 0, 0, 5, 1.0, 1.0, 8), 0),
    ((16, 16, 2 ** 26, 2, 1, 0, 0, 0, 1.0, 1.0, 8), 2),    # ... DMA offsets would overflow
    ((16, 16, 2 ** 26, 2, 1, 0, 0, 0, 1.0, 1.0, 0), 0),    # register-staged fallback
    ((8, 8, 8, 0, 4, 0, 0, 3, 1.0, 1.0, 1), 2),            # transposed B needs a DMA tile
    ((8, 8, 8, 0, 4, 0, 0, 5, 1.0, 1.0, 1), 0),
    ((8, 8, 2 ** 24, 0, 4, 0, 0, 0, 1.0, 1.0, 1), 2),      # DMA offsets would overflow
    ((8, 8, 2 ** 24, 0, 4, 0, 0, 0, 1.0, 1.0, 0), 0),      # register-staged fallback
])
def test_plan_flags_validation(args, status):
    assert _plan2_status(*args) == status


def test_transposed_b_plans_use_dma_tiles_and_the_same_split():
    dma = {imm.TILE[t] for t in ("256x256", "128x256", "32x256", "64x256", "64x64", "32x64", "32x32")}
    for N, K, dt in SHAPES:
        a = imm.gemm_plan_ex2(64, N, K, dt, "f32").info
        b = imm.gemm_plan_ex2(64, N, K, dt, "f32", flags=imm.PLAN_B_TRANSPOSED).info
        assert b["tile"] in dma and b["run_tile"] in dma, (N, K, dt)
        # the split (which decides the bits) does not depend on the layout
        assert (a["split_k"], a["k_per_split"]) == (b["split_k"], b["k_per_split"]), (N, K, dt)


def test_fp8_fp16_step_plans_use_dma_tiles_the_same_split_and_report_the_step():
    dma = {imm.TILE[t] for t in ("256x256", "128x256", "32x256", "64x256")}
    for M, N, K in ((1, 4096, 14336), (64, 4096, 14336), (8192, 8192, 8192), (256, 256, 131072),
                    (1024, 1024, 1024), (300, 272, 384), (1, 16, 16)):
        for dt in ("e4m3", "e5m2"):
            a = imm.gemm_plan_ex2(M, N, K, dt, "bf16").info
            for fl in (0, imm.PLAN_B_TRANSPOSED, imm.PLAN_TILE_BY_M):
                b = imm.gemm_plan_ex2(M, N, K, dt, "bf16", flags=fl | imm.PLAN_FP8_FP32_ACCUM).info
                assert b["tile"] in dma and b["run_tile"] in dma, (M, N, K, dt, fl)
                # the split of K does not depend on the step
                assert (a["split_k"], a["k_per_split"]) == (b["split_k"], b["k_per_split"])
                assert (b["mfma_m"], b["mfma_n"], b["mfma_k"]) == (16, 16, 32)
                assert b["block_k"] == a["block_k"] == 128 and b["in_dtype"] == imm.DTYPE[dt]
            assert a["mfma_k"] == 128


def test_null_plan_handles():
    L = imm.lib()
    assert L.gemm_plan(8, 8, 8, 0, None) == 1
    assert L.gemm_plan_info(None, None) == 1
    assert L.gemm_workspace_size(None) == 0
    assert L.gemm_run(None, 16, 16, 16, None) == 1
    assert L.gemm_splitk_run(None, 16, 16, 16, 16, 1 << 20, None) == 1
    L.gemm_plan_destroy(None)


FAKE = 1 << 40  # a 16-byte aligned address; never dereferenced by these tests


def test_run_validation_before_any_hip_call():
    L = imm.lib()
    p = imm.gemm_plan(64, 64, 64, "f16")
    h = p.handle
    assert L.gemm_run(h, 0, FAKE, FAKE, None) == 1          # NULL A
    assert L.gemm_run(h, FAKE, 0, FAKE, None) == 1          # NULL B
    assert L.gemm_run(h, FAKE, FAKE, 0, None) == 1          # NULL C
    assert L.gemm_run(h, FAKE + 2, FAKE, FAKE, None) == 1   # misaligned A
    assert L.gemm_run(h, FAKE, FAKE + 8, FAKE, None) == 1   # misaligned B
    assert L.gemm_run(h, FAKE, FAKE, FAKE + 4, None) == 1   # misaligned C
    ws = imm.gemm_workspace_size(p)
    assert L.gemm_splitk_run(h, FAKE, FAKE, FAKE, 0, ws, None) == 3        # NULL workspace
    assert L.gemm_splitk_run(h, FAKE, FAKE, FAKE, FAKE, ws - 4, None) == 3  # too small
    assert L.gemm_splitk_run(h, FAKE, FAKE, FAKE, FAKE + 4, ws, None) == 1  # misaligned ws


def test_empty_products_are_noops_without_a_gpu():
    L = imm.lib()
    for M, N in ((0, 64), (64, 0)):
        p = imm.gemm_plan(M, N, 64, "f16")
        assert L.gemm_run(p.handle, 0, 0, 0, None) == 0
        assert L.gemm_splitk_run(p.handle, 0, 0, 0, 0, 0, None) == 0


def _have_gpu():
    import torch
    return torch.cuda.is_available()


@pytest.mark.skipif(_have_gpu(), reason="checks the no-GPU error path")
def test_valid_call_without_gpu_returns_hip_error():
    L = imm.lib()
    p = imm.gemm_plan(64, 64, 64, "f16")
    assert L.gemm_run(p.handle, FAKE, FAKE, FAKE, None) == 4
    assert imm.gemm_last_hip_error() != 0
    ws = imm.gemm_workspace_size(p)
    assert L.gemm_splitk_run(p.handle, FAKE, FAKE, FAKE, FAKE, ws, None) == 4
    with pytest.raises(imm.GemmError) as e:
        imm.gemm_run(p, FAKE, FAKE, FAKE)
    assert e.value.status == 4


def test_binding_checks_tensor_shapes_and_dtypes():
    import torch
    p = imm.gemm_plan(4, 8, 16, "f16")
    A = torch.zeros((4, 16), dtype=torch.float16)
    B = torch.zeros((16, 8), dtype=torch.float16)
    C = torch.zeros((4, 8), dtype=torch.float32)
    with pytest.raises(ValueError):
        imm.gemm_run(p, A.to(torch.bfloat16), B, C)
    with pytest.raises(ValueError):
        imm.gemm_run(p, A, B[:8], C)
    with pytest.raises(ValueError):
        imm.gemm_run(p, A, B, C.to(torch.bfloat16))
    with pytest.raises(ValueError):
        imm.gemm_run(p, A.t(), B, C)


def test_binding_rejects_host_tensors_before_any_hip_call():
    # Host tensors of the right shape and dtype: the kernels would read and
    # write host addresses, so the binding refuses them before calling the
    # library (on a machine with or without a GPU).
    import torch
    p = imm.gemm_plan(4, 8, 16, "f16")
    A = torch.zeros((4, 16), dtype=torch.float16)
    B = torch.zeros((16, 8), dtype=torch.float16)
    C = torch.zeros((4, 8), dtype=torch.float32)
    for call in (lambda: imm.gemm_run(p, A, B, C),
                 lambda: imm.gemm_run(p, FAKE, FAKE, C),
                 lambda: imm.gemm_splitk_run(p, A, B, C, torch.zeros(4 * 8 * 4)),
                 lambda: imm.gemm_splitk_run(p, FAKE, FAKE, FAKE, torch.zeros(1024)),
                 lambda: imm.mm(A, B),
                 lambda: imm.mm(A, B, out_dtype="f16", split_k=0)):
        with pytest.raises(ValueError, match="CUDA"):
            call()
    q = imm.ozaki_plan(4, 8, 16, "bf16")
    A64, B64, C64 = torch.zeros((4, 16), dtype=torch.float64), torch.zeros(
        (16, 8), dtype=torch.float64), torch.zeros((4, 8), dtype=torch.float64)
    ws = torch.zeros(imm.ozaki_workspace_size(q), dtype=torch.uint8)
    for call in (lambda: imm.ozaki_run(q, A64, B64, C64, FAKE),
                 lambda: imm.ozaki_run(q, FAKE, FAKE, FAKE, ws),
                 lambda: imm.ozaki_split(q, 0, A64, FAKE),
                 lambda: imm.ozaki_multiply(q, FAKE, C64),
                 lambda: imm.ozaki_mm(A64, B64)):
        with pytest.raises(ValueError, match="CUDA"):
            call()


def test_output_dtype_of_each_plan():
    # mm() allocates C in the plan's output dtype: fp32, bf16 or fp16
    import torch
    assert imm.out_torch_dtype(imm.DTYPE["f32"]) is torch.float32
    assert imm.out_torch_dtype(imm.DTYPE["bf16"]) is torch.bfloat16
    assert imm.out_torch_dtype(imm.DTYPE["f16"]) is torch.float16
    for od in ("f32", "bf16", "f16"):
        info = imm.gemm_plan_ex(4, 8, 16, "f16", od).info
        assert imm.out_torch_dtype(info["out_dtype"]) is {
            "f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[od]
    with pytest.raises(ValueError):
        imm.out_torch_dtype(imm.DTYPE["e5m2"])


# ---- Ozaki-scheme fp64 product: host logic ----------------------------------

def _oz_status(*args):
    h = ctypes.c_void_p()
    st = imm.lib().ozaki_plan(*args, ctypes.byref(h))
    if h.value:
        imm.lib().ozaki_plan_destroy(h)
    return st


@pytest.mark.parametrize("args,status", [
    ((8, 8, 8, 1, 0, 0, 0), 0),              # bf16 slices
    ((8, 8, 8, 2, 0, 0, 0), 0),              # e4m3 slices
    ((8, 8, 8, 5, 0, 0, 0), 0),              # int8 slices
    ((8, 8, 8, 0, 0, 0, 0), 2),              # fp16 is not a slice format here
    ((8, 8, 8, 3, 0, 0, 0), 2),
    ((-1, 8, 8, 1, 0, 0, 0), 1),
    ((8, 8, 8, 1, 20, 0, 0), 0),
    ((8, 8, 8, 1, 21, 0, 0), 2),             # at most 20 slices
    ((8, 8, 8, 1, -1, 0, 0), 2),
    ((8, 8, 8, 1, 0, -2, 0), 2),
    ((8, 8, 8, 1, 0, 0, 128), 0),
    ((8, 8, 8, 1, 0, 0, 100), 2),            # chunks are multiples of 128
    ((8, 8, 8, 1, 0, 0, -128), 2),
    ((8, 8, 8, 1, 0, 0, 2 ** 22), 0),        # one bit per slice left
    ((8, 8, 8, 1, 0, 0, 2 ** 22 + 128), 2),
    ((8, 8, 2 ** 22 - 16, 1, 0, 0, 0), 0),   # chunks keep the chain short for any K ...
    ((8, 8, 2 ** 24 - 16, 2, 0, 0, 0), 0),
    ((8, 8, 2 ** 23, 1, 0, 0, 0), 2),        # ... up to the tile's 32-bit offsets
    ((8, 2 ** 23, 8, 1, 0, 0, 0), 2),
    ((0, 0, 0, 1, 0, 0, 0), 0),
])
def test_ozaki_plan_validation(args, status):
    assert _oz_status(*args) == status


@pytest.mark.parametrize("K", [1, 15, 256, 257, 1000, 4096, 16384, 131072, 2 ** 22])
@pytest.mark.parametrize("t2,kc", [("bf16", 0), ("e4m3", 0), ("bf16", 1024), ("bf16", K_ALL := 2 ** 22),
                                   ("e4m3", 128), ("i8", 0), ("i8", 4096)])
def test_ozaki_plan_matches_oracle_parameters_for_any_M(K, t2, kc):
    from oracle import ozaki as OZ
    P = OZ.params(K, t2, kc=kc)
    ref = None
    for M in (1, 100, 4097):
        i = imm.ozaki_plan(M, 200, K, t2, chunk=kc).info
        got = (i["rho"], i["bits"], i["delta"], i["slices"], i["d"], i["pairs"], i["chunk"],
               i["k_pad"], i["n_pad"], i["tile_m"], i["tile_n"])
        assert got[:7] == (P.rho, P.b, P.delta, P.s, P.d, len(P.pairs), P.kc)
        assert got[7] % 16 == 0 and K <= got[7] < K + 16 and got[8] == 208
        ref = ref or got
        assert got == ref                    # nothing but the grid depends on M


def test_ozaki_explicit_slices_and_d():
    from oracle import ozaki as OZ
    for s, d in ((4, 3), (7, 5), (20, 40), (1, 1)):
        i = imm.ozaki_plan(10, 10, 500, "bf16", s, d).info
        assert (i["slices"], i["d"], i["pairs"]) == (s, d, len(OZ.pair_list(s, d)))


def test_ozaki_workspace_layout():
    i = imm.ozaki_plan(100, 300, 1000, "bf16").info
    s, kp, np_ = i["slices"], i["k_pad"], i["n_pad"]
    assert i["a_slices_offset"] == 0
    assert i["b_slices_offset"] >= s * 100 * kp * 2
    assert i["a_exp_offset"] >= i["b_slices_offset"] + s * kp * np_ * 2
    assert i["b_exp_offset"] >= i["a_exp_offset"] + 100 * 4
    assert i["scratch_offset"] >= i["b_exp_offset"] + np_ * 4
    assert i["workspace_bytes"] >= i["scratch_offset"] + 4 * 300 * 8
    for k in ("b_slices_offset", "a_exp_offset", "b_exp_offset", "scratch_offset"):
        assert i[k] % 256 == 0


def test_ozaki_validation_before_any_hip_call():
    L = imm.lib()
    p = imm.ozaki_plan(64, 64, 64, "bf16")
    h, ws = p.handle, imm.ozaki_workspace_size(p)
    assert L.ozaki_run(None, FAKE, FAKE, FAKE, FAKE, ws, None) == 1
    assert L.ozaki_run(h, 0, FAKE, FAKE, FAKE, ws, None) == 1        # NULL A
    assert L.ozaki_run(h, FAKE, FAKE + 4, FAKE, FAKE, ws, None) == 1  # misaligned B
    assert L.ozaki_run(h, FAKE, FAKE, 0, FAKE, ws, None) == 1        # NULL C
    assert L.ozaki_run(h, FAKE, FAKE, FAKE, 0, ws, None) == 3        # NULL workspace
    assert L.ozaki_run(h, FAKE, FAKE, FAKE, FAKE, ws - 1, None) == 3
    assert L.ozaki_run(h, FAKE, FAKE, FAKE, FAKE + 8, ws, None) == 1  # misaligned workspace
    assert L.ozaki_split(h, 2, FAKE, FAKE, ws, None) == 1             # no such operand
    assert L.ozaki_multiply(h, FAKE, ws, FAKE + 1, None) == 1
    e = imm.ozaki_plan(0, 64, 64, "bf16")
    assert L.ozaki_run(e.handle, 0, 0, 0, 0, 0, None) == 0            # empty: nothing to do


@pytest.mark.skipif(_have_gpu(), reason="checks the no-GPU error path")
def test_ozaki_without_gpu_returns_hip_error():
    L = imm.lib()
    p = imm.ozaki_plan(64, 64, 64, "e4m3")
    ws = imm.ozaki_workspace_size(p)
    assert L.ozaki_run(p.handle, FAKE, FAKE, FAKE, FAKE, ws, None) == 4
    assert L.ozaki_split(p.handle, 0, FAKE, FAKE, ws, None) == 4
    assert L.ozaki_multiply(p.handle, FAKE, ws, FAKE, None) == 4


def test_ozaki_column_maxima_chunks_are_capped():
    # the column maxima of B run over at most 16384 chunks of K (the second
    # grid dimension), wider chunks beyond that
    for K, N in ((1000, 300), (2 ** 22, 64), (2 ** 24 + 16, 8)):
        i = imm.ozaki_plan(8, N, K, "e4m3").info
        scratch = i["workspace_bytes"] - i["scratch_offset"]
        rows = 256 if -(-K // 256) <= 16384 else -(-K // 16384)
        chunks = -(-K // rows)
        assert chunks <= 16384
        assert chunks * N * 8 <= scratch <= -(-(16384 * N * 8) // 256) * 256


@pytest.mark.parametrize("M,N,K,tile,tile8", [
    (1, 6144, 4096, "32x32", "32x256"), (64, 6144, 4096, "32x64", "32x256"),
    (96, 6144, 4096, "32x64", "32x256"), (128, 6144, 4096, "32x64", "32x256"),
    (192, 6144, 4096, "64x64", "32x256"), (256, 6144, 4096, "64x64", "32x256"),
    (512, 6144, 4096, "128x256", "128x256"), (768, 6144, 4096, "128x256", "128x256"),
    (1024, 6144, 4096, "128x256", "128x256"), (1536, 6144, 4096, "256x256", "256x256"),
    (2048, 6144, 4096, "256x256", "256x256"), (3072, 6144, 4096, "128x256", "128x256"),
    (512, 1024, 4096, "32x64", "32x256"), (1024, 1024, 4096, "32x64", "32x256"),
    (2048, 1024, 4096, "64x64", "32x256"), (48, 14336, 4096, "32x64", "32x256"),
    (2048, 2048, 2048, "128x256", "128x256"), (4096, 4096, 4096, "256x256", "256x256"),
    (8192, 8192, 8192, "256x256", "256x256"),
])
def test_tile_by_m_rule(M, N, K, tile, tile8):
    """GEMM_PLAN_TILE_BY_M: the DMA tile with the least estimated time (rounds
    of 256 workgroups x the tile's units per round), the measured fastest at
    each of these shapes (fp8 inputs skip the 64-column tiles); split-K path
    and the default plan unchanged."""
    for dt, want in (("f16", tile), ("bf16", tile), ("e5m2", tile8)):
        flagged = imm.gemm_plan_ex2(M, N, K, dt, "f32", flags=imm.PLAN_TILE_BY_M).info
        plain = imm.gemm_plan_ex2(M, N, K, dt, "f32").info
        assert flagged["run_tile"] == imm.TILE[want], dt
        # the split (which decides bits) never moves; the split-path tile moves
        # only for wide reduction-dominated shapes (K >= 2N, N > 512)
        same = ("split_k", "k_per_split") if K >= 2 * N and N > 512 else (
            "tile", "split_k", "k_per_split", "block_m", "block_n")
        for k in same:
            assert flagged[k] == plain[k], (dt, k)


@pytest.mark.parametrize("M,N,tile", [
    (1, 6144, "32x32"), (64, 6144, "32x32"), (128, 6144, "32x32"), (192, 6144, "64x64"),
    (512, 6144, "64x256"), (512, 1024, "32x32"), (1024, 1024, "32x64"), (48, 14336, "32x64"),
    (1024, 6144, "128x256"),
])
def test_tile_by_m_rule_with_b_transposed(M, N, tile):
    """With B transposed the narrow tiles' rows stream faster (K-contiguous),
    so the 32 x 32 tile covers more of the small-M range than with B as
    [K, N]."""
    for dt in ("f16", "bf16"):
        i = imm.gemm_plan_ex2(M, N, 4096, dt, "f32",
                              flags=imm.PLAN_TILE_BY_M | imm.PLAN_B_TRANSPOSED).info
        assert i["run_tile"] == imm.TILE[tile], dt
    i = imm.gemm_plan_ex2(M, N, 4096, "e5m2", "f32",
                          flags=imm.PLAN_TILE_BY_M | imm.PLAN_B_TRANSPOSED).info
    assert i["run_tile"] not in {imm.TILE[t] for t in ("32x32", "32x64", "64x64")}


@pytest.mark.parametrize("M,tile", [(1, "32x128"), (8, "32x128"), (32, "32x128"), (64, "64x256"),
                                    (128, "128x256"), (256, "256x256"), (512, "256x256")])
def test_tile_by_m_on_the_split_path_of_decode_shapes(M, tile):
    """GEMM_PLAN_TILE_BY_M: the split-K path of a wide reduction-dominated shape
    takes the tile with the fewest row tiles; the split itself (which decides
    the bits) is the plain plan's."""
    N, K = 4096, 14336
    flagged = imm.gemm_plan_ex2(M, N, K, "bf16", "f32", flags=imm.PLAN_TILE_BY_M).info
    plain = imm.gemm_plan_ex2(M, N, K, "bf16", "f32").info
    assert flagged["tile"] == imm.TILE[tile]
    assert plain["tile"] == imm.TILE["32x128"]
    assert (flagged["split_k"], flagged["k_per_split"]) == (plain["split_k"], plain["k_per_split"])
    bt = imm.gemm_plan_ex2(M, N, K, "bf16", "f32",
                           flags=imm.PLAN_TILE_BY_M | imm.PLAN_B_TRANSPOSED).info
    assert bt["tile"] == imm.TILE["32x256" if tile == "32x128" else tile]
    assert (bt["split_k"], bt["k_per_split"]) == (plain["split_k"], plain["k_per_split"])


def test_tile_by_m_leaves_the_split_path_of_narrow_shapes():
    """N <= 512 (the huge-K case) keeps its split-path tile under the flag."""
    for M in (1, 256, 1024):
        flagged = imm.gemm_plan_ex2(M, 256, 131072, "f16", "f32", flags=imm.PLAN_TILE_BY_M).info
        plain = imm.gemm_plan_ex2(M, 256, 131072, "f16", "f32").info
        assert flagged["tile"] == plain["tile"] == imm.TILE["128x256"]


def test_narrow_default_steps_down_to_64_rows_past_the_offset_limit():
    """N <= 512: the 128x256 split-path tile while its 32-bit A offsets fit
    (K < 2^23 for 16-bit inputs), then the 64x256 DMA tile; the split is the
    one any tile gets at that K."""
    for K, tile in ((2 ** 23 - 64, "128x256"), (2 ** 23 + 64, "64x256")):
        d = imm.gemm_plan(300, 40, K, "bf16").info
        assert d["tile"] == imm.TILE[tile], K
        for other in ("128x256", "32x128"):
            e = imm.gemm_plan_ex(300, 40, K, "bf16", "f32", tile=other).info
            assert (e["split_k"], e["k_per_split"]) == (d["split_k"], d["k_per_split"])


def test_tile_by_m_never_makes_a_split_plan_fail():
    """Near and past the K where the DMA tiles' 32-bit offsets overflow: where
    the plain plan exists, the flagged one exists too, with the same split."""
    N = 1024
    for K in (2 ** 21, 2 ** 22 - 64, 2 ** 22 + 64, 2 ** 23):
        for fl in (0, imm.PLAN_B_TRANSPOSED):
            for M in (1, 300):
                try:
                    plain = imm.gemm_plan_ex2(M, N, K, "bf16", "f32", flags=fl).info
                except imm.GemmError:
                    continue
                flagged = imm.gemm_plan_ex2(M, N, K, "bf16", "f32",
                                            flags=fl | imm.PLAN_TILE_BY_M).info
                assert (flagged["split_k"], flagged["k_per_split"]) == (
                    plain["split_k"], plain["k_per_split"]), (K, fl, M)


def test_noalloc_entry_point_host_checks():
    # gemm_splitk_run_noalloc: argument checks, then the workspace limit, both
    # before any HIP call; a valid call without a GPU returns GEMM_ERR_HIP.
    L = imm.lib()
    small = imm.gemm_plan(8, 4096, 14336, "bf16")          # 16 slices: 2 MiB
    assert imm.gemm_workspace_size(small) <= imm.NOALLOC_WORKSPACE_BYTES
    big = imm.gemm_plan(512, 4096, 14336, "bf16")          # 128 MiB
    assert imm.gemm_workspace_size(big) > imm.NOALLOC_WORKSPACE_BYTES
    assert L.gemm_splitk_run_noalloc(None, FAKE, FAKE, FAKE, None) == 1
    assert L.gemm_splitk_run_noalloc(small.handle, 0, FAKE, FAKE, None) == 1
    assert L.gemm_splitk_run_noalloc(small.handle, FAKE, FAKE, FAKE + 4, None) == 1
    assert L.gemm_splitk_run_noalloc(big.handle, FAKE, FAKE, FAKE, None) == 3
    assert L.gemm_splitk_run_noalloc(imm.gemm_plan(0, 64, 64, "f16").handle, 0, 0, 0, None) == 0
    if not _have_gpu():
        assert L.gemm_splitk_run_noalloc(small.handle, FAKE, FAKE, FAKE, None) == 4
    with pytest.raises(imm.GemmError) as e:
        imm.gemm_splitk_run_noalloc(big, FAKE, FAKE, FAKE)
    assert e.value.status == 3 and str(imm.NOALLOC_WORKSPACE_BYTES) in str(e.value)


def test_narrow_tiles_take_16_bit_inputs_only():
    for tile in ("32x64", "64x64", "32x32"):
        for dt in ("f16", "bf16"):
            for fl in (0, imm.PLAN_B_TRANSPOSED):
                i = imm.gemm_plan_ex2(100, 6144, 4096, dt, "f32", tile=tile, flags=fl).info
                assert i["run_tile"] == i["tile"] == imm.TILE[tile]
                assert (i["run_block_m"], i["run_block_n"]) == tuple(map(int, tile.split("x")))
                assert i["run_tiles_n"] == 6144 // int(tile.split("x")[1])
        for dt in ("e4m3", "e5m2"):
            assert _plan2_status(100, 6144, 4096, imm.DTYPE[dt], 4, 0, 0, imm.TILE[tile],
                                 1.0, 1.0, 0) == 2
