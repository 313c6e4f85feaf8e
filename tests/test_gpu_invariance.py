"""GPU batch invariance and run-to-run determinism, bit for bit.

The Tencent deterministic-inference article (sections "背景" and "Batch
Invariance の由来") separates run-to-run determinism (the same request alone,
repeated) from batch invariance (the same request while other rows share the
batch), and shows which GEMM parameters may change bits: BLOCK_M/BLOCK_N,
GROUP_M, num_warps and pipelining may not; the K step and the split of K do.
These tests pin each of those statements on the hardware:

- rows are identical across M (row prefixes), under row permutations, and
  when other rows hold different data;
- repeats, other streams and concurrently running work change nothing;
- GROUP_M and the tile shape change nothing (same instruction, same K order);
- gemm_splitk_run with one slice equals gemm_run;
- a different split of K may change bits on random inputs, never on exact ones.
"""
import numpy as np
import pytest
import torch

import invariant_matmul_amd as imm
import workloads as wl
from tests.helpers import bits_of, dev, log, run, tiles_for

pytestmark = pytest.mark.gpu

TILES = ["256x256", "128x128", "32x128", "256x256_rs", "32x256", "64x256", "128x256", "32x64",
         "64x64", "32x32"]


def _to_dev(*ts):
    return [t.to(dev()) for t in ts]


def _rand(M, N, K, dt, seed):
    g = wl.gen(seed)
    if dt in ("e4m3", "e5m2"):
        return wl.normal((M, K), dt, g), wl.normal((K, N), dt, g)
    return wl.uniform((M, K), dt, g), wl.uniform((K, N), dt, g)


def test_decode_rows_identical_across_M():
    w = wl.WORKLOADS["decode_bf16_m128"]
    A, B = w.make()
    Ad, Bd = _to_dev(A, B)
    full = None
    for m in (128, 32, 8, 1):
        plan = imm.gemm_plan(m, w.N, w.K, "bf16")
        C = bits_of(run(plan, Ad[:m].contiguous(), Bd, True))
        if full is None:
            full = C
        log(f"decode M={m}: split {plan.info['split_k']}")
        assert np.array_equal(C, full[:m]), m


def test_exact256_slices():
    w = wl.WORKLOADS["exact256"]
    A, B = w.make()
    Ad, Bd = _to_dev(A, B)
    full = bits_of(run(imm.gemm_plan(256, 256, 256, "f16"), Ad, Bd, False))
    for m in w.m_slices:
        C = bits_of(run(imm.gemm_plan(m, 256, 256, "f16"), Ad[:m].contiguous(), Bd, False))
        assert np.array_equal(C, full[:m]), m


@pytest.mark.parametrize("dt", ["f16", "bf16", "e4m3", "e5m2"])
@pytest.mark.parametrize("split", [None, 4])
def test_random_rows_identical_across_M(dt, split):
    N, K = 512, 2048
    A, B = _rand(1000, N, K, dt, 8000)
    Ad, Bd = _to_dev(A, B)
    plan = lambda m: imm.gemm_plan_ex(m, N, K, dt, "f32", split_k=split or 0)
    full = bits_of(run(plan(1000), Ad, Bd, split is not None))
    for m in (1, 2, 31, 33, 255, 257, 999):
        C = bits_of(run(plan(m), Ad[:m].contiguous(), Bd, split is not None))
        assert np.array_equal(C, full[:m]), (dt, split, m)


def test_narrow_long_k_rows_identical_across_M():
    """The default plan of a narrow reduction-dominated shape with long slices
    (N = 128, K = 131072: the 128x256 tile and 128 slices of 1024): rows of C
    keep their bits at every M, on the default tile and on an explicit one."""
    N, K = 128, 131072
    A, B = _rand(300, N, K, "bf16", 8050)
    Ad, Bd = _to_dev(A, B)
    p = imm.gemm_plan(300, N, K, "bf16")
    assert (p.info["block_m"], p.info["split_k"]) == (128, 128)
    full = bits_of(run(p, Ad, Bd, True))
    for m in (1, 33, 129, 299):
        for tile in ("default", "32x128"):
            pm = imm.gemm_plan_ex(m, N, K, "bf16", "f32", tile=tile)
            C = bits_of(run(pm, Ad[:m].contiguous(), Bd, True))
            assert np.array_equal(C, full[:m]), (m, tile)


def test_row_depends_only_on_its_own_row():
    # Permute rows and replace every other row with fresh data: the surviving
    # rows must come out with the same bits wherever they land.
    N, K, M = 384, 1024, 700
    A, B = _rand(M, N, K, "bf16", 8100)
    Ad, Bd = _to_dev(A, B)
    for tile in TILES:
        plan = imm.gemm_plan_ex(M, N, K, "bf16", "f32", tile=tile, split_k=2)
        for split in (False, True):
            base = bits_of(run(plan, Ad, Bd, split))
            perm = torch.randperm(M, generator=wl.gen(8101))
            noise = wl.uniform((M, K), "bf16", wl.gen(8102))
            keep = torch.arange(M) % 2 == 0
            A2 = torch.where(keep[:, None], A[perm], noise)
            C2 = bits_of(run(plan, A2.to(dev()), Bd, split))
            pk = perm.numpy()[keep.numpy()]
            assert np.array_equal(C2[keep.numpy()], base[pk]), (tile, split)


def test_repeated_runs_identical():
    w = wl.WORKLOADS["square_f16_1024"]
    A, B = w.make()
    Ad, Bd = _to_dev(A, B)
    plan = imm.gemm_plan(1024, 1024, 1024, "f16")
    ref = run(plan, Ad, Bd, False)
    outs = [run(plan, Ad, Bd, False) for _ in range(100)]
    torch.cuda.synchronize()
    for C in outs:
        assert torch.equal(C.view(torch.int32), ref.view(torch.int32))
    hp = imm.gemm_plan(256, 256, 131072, "f16")
    Ah, Bh = _to_dev(*wl.WORKLOADS["hugek_f16"].make())
    refh = run(hp, Ah, Bh, True)
    for _ in range(50):
        assert torch.equal(run(hp, Ah, Bh, True).view(torch.int32), refh.view(torch.int32))


def test_group_m_and_tile_shape_do_not_change_bits():
    N, K, M = 768, 1536, 640
    for dt in ("f16", "e5m2"):
        A, B = _rand(M, N, K, dt, 8200)
        Ad, Bd = _to_dev(A, B)
        for split in (False, True):
            ref = None
            for tile in tiles_for(dt, TILES):
                for gm in (1, 3, 8):
                    p = imm.gemm_plan_ex(M, N, K, dt, "f32", split_k=3, group_m=gm, tile=tile)
                    C = bits_of(run(p, Ad, Bd, split))
                    if ref is None:
                        ref = C
                    assert np.array_equal(C, ref), (dt, split, tile, gm)
            log(f"{dt} split={split}: 3 tiles x 3 GROUP_M identical")


def test_splitk_one_slice_equals_run():
    for name in ("square_f16_1024", "decode_bf16_m32", "hugek_f16"):
        w = wl.WORKLOADS[name]
        A, B = w.make()
        Ad, Bd = _to_dev(A, B)
        p = imm.gemm_plan_ex(w.M, w.N, w.K, w.dtype, w.out, split_k=1)
        assert np.array_equal(bits_of(run(p, Ad, Bd, False)), bits_of(run(p, Ad, Bd, True))), name


def test_other_stream_and_corunning_work():
    w = wl.WORKLOADS["decode_bf16_m32"]
    A, B = w.make()
    Ad, Bd = _to_dev(A, B)
    plan = imm.gemm_plan(w.M, w.N, w.K, "bf16")
    ref = bits_of(run(plan, Ad, Bd, True))
    s1 = torch.cuda.Stream()
    s2 = torch.cuda.Stream()
    X = torch.randn((4096, 4096), device=dev(), dtype=torch.float32)
    outs = []
    for _ in range(10):
        with torch.cuda.stream(s2):
            for _ in range(3):
                X = torch.tanh(X @ X * 1e-3)  # busy work on another stream
        with torch.cuda.stream(s1):
            outs.append(run(plan, Ad, Bd, True, stream=s1))
    torch.cuda.synchronize()
    for C in outs:
        assert np.array_equal(bits_of(C), ref)


def test_split_changes_bits_only_where_rounding_happens():
    # A different split of K is a different summation tree: on random data some
    # bits differ (non-associativity), on integer data nothing may differ.
    w = wl.WORKLOADS["hugek_f16"]
    A, B = w.make()
    Ad, Bd = _to_dev(A, B)
    outs = {}
    for s in (1, 8, 32, 128):
        outs[s] = bits_of(run(imm.gemm_plan_ex(256, 256, w.K, "f16", "f32", split_k=s), Ad, Bd, True))
    diff = sum(int((outs[s] != outs[1]).sum()) for s in (8, 32, 128))
    log(f"hugek random: elements differing from split 1: {diff}")
    assert diff > 0
    g = wl.gen(8300)
    Ai = wl.integers((256, 16384), "f16", g)
    Bi = wl.integers((16384, 256), "f16", g)
    Aid, Bid = _to_dev(Ai, Bi)
    ref = bits_of(run(imm.gemm_plan_ex(256, 256, 16384, "f16", "f32", split_k=1), Aid, Bid, True))
    for s in (8, 32, 128):
        p = imm.gemm_plan_ex(256, 256, 16384, "f16", "f32", split_k=s)
        assert np.array_equal(bits_of(run(p, Aid, Bid, True)), ref), s


@pytest.mark.parametrize("dt,bt", [("f16", False), ("bf16", True)])
def test_tile_by_m_rows_identical_across_M(dt, bt):
    """GEMM_PLAN_TILE_BY_M switches the single pass between the narrow and the
    256-column tiles as M grows; every row must keep its bits."""
    N, K = 6144, 4096
    g = wl.gen(8400)
    A = wl.uniform((2048, K), dt, g).to(dev())
    B = wl.uniform((K, N), dt, g)
    Bd = (B.float().t().contiguous().to(B.dtype) if bt else B).to(dev())
    fl = imm.PLAN_B_TRANSPOSED if bt else 0
    full = imm.gemm_plan_ex2(2048, N, K, dt, "f32", flags=fl)
    ref = bits_of(run(full, A, Bd, False))
    seen = set()
    for m in (1, 64, 100, 256, 512, 1024, 2048):  # every tile the rule picks on this shape
        plan = imm.gemm_plan_ex2(m, N, K, dt, "f32", flags=fl | imm.PLAN_TILE_BY_M)
        seen.add(plan.info["run_tile"])
        got = bits_of(run(plan, A[:m].contiguous(), Bd, False))
        assert np.array_equal(got, ref[:m]), m
    want = ("32x32", "64x64", "64x256", "128x256", "256x256") if bt else \
        ("32x32", "32x64", "64x64", "128x256", "256x256")
    assert seen == {imm.TILE[t] for t in want}, seen


@pytest.mark.parametrize("bt", [False, True])
def test_tile_by_m_split_path_bits_equal_the_plain_plan(bt):
    """GEMM_PLAN_TILE_BY_M on the split-K path of the decode shape walks the
    32-row, 64x256, 128x256 and 256x256 tiles as M grows; the split stays the
    plain plan's, so every row keeps the bits of the plain plan at full M."""
    w = wl.WORKLOADS["decode_bf16_m128"]
    N, K = w.N, w.K
    g = wl.gen(8450)
    A = wl.normal((256, K), "bf16", g, std=K ** -0.5).to(dev())
    B = wl.normal((K, N), "bf16", g).to(torch.bfloat16)
    Bd = (B.float().t().contiguous().to(torch.bfloat16) if bt else B).to(dev())
    fl = imm.PLAN_B_TRANSPOSED if bt else 0
    plain = imm.gemm_plan_ex2(256, N, K, "bf16", "f32", flags=fl)
    ref = bits_of(run(plain, A, Bd, True))
    seen = set()
    for m in (1, 40, 64, 128, 256):
        plan = imm.gemm_plan_ex2(m, N, K, "bf16", "f32", flags=fl | imm.PLAN_TILE_BY_M)
        assert plan.info["split_k"] == plain.info["split_k"]
        seen.add(plan.info["tile"])
        got = bits_of(run(plan, A[:m].contiguous(), Bd, True))
        log(f"split path tile_by_m M={m} tile {plan.info['tile']} bt={bt}")
        assert np.array_equal(got, ref[:m]), m
    assert len(seen) == 4, seen


@pytest.mark.parametrize("split", [False, True])
@pytest.mark.parametrize("tile", ["256x256", "128x256", "32x256", "32x128"])
def test_nan_and_inf_rows_stay_in_their_rows(tile, split):
    """A request whose row of A holds a NaN or an infinity must not touch the
    other rows of the batch: their bits equal a run without it, and the NaN
    row of C is NaN throughout."""
    M, N, K = 300, 512, 1024
    g = wl.gen(8470)
    A = wl.uniform((M, K), "f16", g)
    B = wl.uniform((K, N), "f16", g).to(dev())
    bad = A.clone()
    bad[3, 17] = float("nan")
    bad[200, 900] = float("inf")
    plan = imm.gemm_plan_ex(M, N, K, "f16", "f32", tile=tile)
    clean = bits_of(run(plan, A.to(dev()), B, split))
    C = run(plan, bad.to(dev()), B, split)
    got = bits_of(C)
    rows = [r for r in range(M) if r not in (3, 200)]
    assert np.array_equal(got[rows], clean[rows])
    assert torch.isnan(C[3]).all()
    assert not torch.isfinite(C[200]).any()


def test_host_threads_on_their_own_streams():
    """Plans are immutable and the library keeps no state between calls: four
    host threads, each on its own stream with its own buffers, running the
    single pass and the split-K path at the same time, all get the bits of the
    single-threaded run."""
    import threading
    M, N, K = 512, 1024, 2048
    g = wl.gen(8480)
    A = wl.uniform((M, K), "bf16", g).to(dev())
    B = wl.uniform((K, N), "bf16", g).to(dev())
    plan = imm.gemm_plan_ex(M, N, K, "bf16", "f32", split_k=4)
    ref_run = bits_of(run(plan, A, B, False))
    ref_split = bits_of(run(plan, A, B, True))
    errors = []

    def worker(t):
        try:
            s = torch.cuda.Stream()
            C = torch.empty((M, N), dtype=torch.float32, device=dev())
            ws = torch.empty(imm.gemm_workspace_size(plan) // 4, dtype=torch.float32, device=dev())
            for i in range(12):
                split = (i + t) % 2 == 1
                with torch.cuda.stream(s):
                    if split:
                        imm.gemm_splitk_run(plan, A, B, C, ws, s)
                    else:
                        imm.gemm_run(plan, A, B, C, s)
                s.synchronize()
                got = wl.bits(C.cpu())
                if not np.array_equal(got, ref_split if split else ref_run):
                    errors.append((t, i, split))
        except Exception as e:  # reported below
            errors.append((t, repr(e)))

    torch.cuda.synchronize()
    threads = [threading.Thread(target=worker, args=(t,)) for t in range(4)]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    assert not errors, errors
