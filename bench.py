"""Benchmark of the batch-invariant GEMM library on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

Prints ONE JSON line.  The headline workload is the square fp16 product
M = N = K = 8192 with fp32 output through gemm_run (one step = one product
over one batch of seeded synthetic input already resident in HBM); `value`
is its throughput in TFLOP/s.  The same run also measures, as secondary
results under "extra": the headline product with its inputs rotated over two
copies (no help from the last-level cache), the fp8 e5m2 8192^3 product (bf16 out), the decode
products N=4096 K=14336 at M in {1, 8, 32, 128} through the split-K path
(GB/s, inputs rotated through enough copies to defeat the 256 MB last-level
cache), the huge-K product 256 x 256 x 131072 at split_k in {1, 8, 32, 128},
the fp64 product by the Ozaki scheme (bf16 and e4m3 slices, n = 4096 .. 16384:
split, slice-pair product and whole call, in fp64-equivalent TFLOP/s and as
matrix-core throughput of the slice products), and torch.matmul (hipBLASLt /
the fp64 path) on the same shapes and a 1 GiB device copy (an achievable HBM
rate) as run-only comparators.

Every timed series is preceded by SETTLE_MS of untimed launches of the same
call, then its warm-up launches: the engine clock rises over the first ~50
ms of load after an idle spell (launches in that window ran up to 10 %
longer on MI355X), and the figures are for sustained load.

"roofline" reports the dominant kernel (the DMA-fed 256x256 GEMM kernel) against
the MI355X dense fp16 matrix peak: achieved = 2*M*N*K flop per launch divided
by the kernel's average duration, timed with HIP events on the launch
stream.  "cpu_baseline" times the CPU oracle (test infrastructure, fp64
triple loop) on a bounded sample of rows of the same product.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_TFLOPS = {"f16": 2516.6, "bf16": 2516.6, "e4m3": 5033.2, "e5m2": 5033.2, "i8": 5033.2}
PEAK_HBM_GBS = 8000.0
MALL_BYTES = 256 * 2 ** 20
KERNEL_SOURCES = [os.path.join(ROOT, "invariant_matmul_amd", "csrc", f)
                  for f in ("gemm_dma.hip", "kernel_common.h", "imm_internal.h")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_square_f16_8192.json")
CLOCK_FILE = os.path.join(ROOT, "profiles", "clock_square_f16_8192.json")
STREAM_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_splitk_decode_hugek.json")
CLOCK_COUNTERS = ("GRBM_GUI_ACTIVE", "GRBM_COUNT", "SQ_BUSY_CYCLES", "SQ_VALU_MFMA_BUSY_CYCLES",
                  "SQ_INSTS_VALU_MFMA_MOPS_F16", "SQ_INSTS_MFMA")
# a second run of the clock pass: LDS and L2 behaviour
LDS_COUNTERS = ("GRBM_GUI_ACTIVE", "SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE", "SQ_INSTS_LDS",
                "TCC_HIT_sum", "TCC_MISS_sum")


def kernel_source_hash() -> str:
    """Hash of what decides the headline kernel's launches: the device sources
    it is built from and the plan the library makes for the headline product
    (tile, waves, raster, split, instruction shape)."""
    import invariant_matmul_amd as imm
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p, "rb") as f:
            h.update(f.read())
    info = imm.gemm_plan(8192, 8192, 8192, "f16").info
    h.update(json.dumps(info, sort_keys=True).encode())
    return h.hexdigest()[:16]


COPY_BYTES = 256 * 2 ** 20  # the plain copy of the profile pass: this many bytes read and written


def write_traffic(fetch_csv, write_csv, out_path=TRAFFIC_FILE):
    """Turn two rocprofv3 --pmc runs of `bench.py --profile-pass` (FETCH_SIZE, then
    WRITE_SIZE, KiB per dispatch) into the per-launch HBM traffic of the headline
    kernel.  Each counter is scaled by what it reads for the plain copy of known
    size in the same pass (FETCH_SIZE counts half the bytes a copy reads on this
    part; WRITE_SIZE counts them all)."""
    import csv

    def per_kernel(path, counter):
        copy, gemm = [], []
        with open(path) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] != counter:
                    continue
                v = float(r["Counter_Value"])
                if "copyBuffer" in r["Kernel_Name"]:
                    copy.append(v)
                elif "gemm_dma_kernel" in r["Kernel_Name"]:
                    gemm.append(v)  # the profile pass launches only the headline kernel
        if not copy or not gemm:
            raise SystemExit(f"{path}: no copy or headline-kernel dispatches with {counter}")
        return statistics.mean(copy), statistics.mean(gemm), len(gemm)

    cf, gf, n = per_kernel(fetch_csv, "FETCH_SIZE")
    cw, gw, _ = per_kernel(write_csv, "WRITE_SIZE")
    ff, wf = COPY_BYTES / 1024 / cf, COPY_BYTES / 1024 / cw
    out = {"kernel": "gemm_dma_kernel<f16, f32 out, 256x256 tile>, M=N=K=8192",
           "kernel_source_hash": kernel_source_hash(),
           "fetch_kib_per_launch": gf, "write_kib_per_launch": gw, "launches": n,
           "copy_fetch_kib": cf, "copy_write_kib": cw,
           "fetch_scale": ff, "write_scale": wf,
           "read_bytes_per_launch": gf * ff * 1024, "write_bytes_per_launch": gw * wf * 1024,
           "bytes_per_launch": (gf * ff + gw * wf) * 1024}
    os.makedirs(os.path.dirname(out_path), exist_ok=True)
    with open(out_path, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out))


# The memory-bound cases of the stream pass, in launch order: (workload, rows, launches).
STREAM_CASES = (("decode_bf16_m1", 1, 6), ("decode_bf16_m8", 8, 6), ("decode_bf16_m32", 32, 6),
                ("hugek_f16", 256, 6))


def stream_pass(torch, imm, wl):
    """A plain copy of COPY_BYTES, then each STREAM_CASES product through the
    default split-K plan, inputs rotated so that no launch finds its A or B in
    the last-level cache."""
    src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    del src, dst
    for name, rows, launches in STREAM_CASES:
        w = wl.WORKLOADS[name]
        A, B = w.make()
        Ad, Bd = A[:rows].contiguous().cuda(), B.cuda()
        bytes_in = Ad.numel() * Ad.element_size() + Bd.numel() * Bd.element_size()
        copies = max(1, -(-2 * MALL_BYTES // bytes_in)) + 1
        As = [Ad] + [Ad.clone() for _ in range(copies - 1)]
        Bs = [Bd] + [Bd.clone() for _ in range(copies - 1)]
        plan = imm.gemm_plan(rows, w.N, w.K, w.dtype)
        C = torch.empty((rows, w.N), dtype=torch.float32, device="cuda")
        ws = torch.empty(max(1, imm.gemm_workspace_size(plan) // 4), dtype=torch.float32,
                         device="cuda")
        torch.cuda.synchronize()
        for i in range(launches):
            imm.gemm_splitk_run(plan, As[i % copies], Bs[i % copies], C, ws)
        torch.cuda.synchronize()
        del As, Bs, C, ws
        torch.cuda.empty_cache()


def write_stream_traffic(fetch_csv, write_csv, out_path=STREAM_TRAFFIC_FILE):
    """Turn two rocprofv3 --pmc runs of `bench.py --stream-pass` (FETCH_SIZE,
    then WRITE_SIZE) into bytes per launch of each split-K kernel of each
    STREAM_CASES product, scaled by the copy as in write_traffic, next to the
    kernel's algorithmic bytes: the partial reads A and B once and writes the
    S slices of M x N fp32; the reduction reads those slices and writes C."""
    import csv

    import invariant_matmul_amd as imm
    import workloads as wl

    def rows_of(path, counter):
        out = []
        with open(path) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] == counter:
                    out.append((int(r["Dispatch_Id"]), r["Kernel_Name"], float(r["Counter_Value"])))
        out.sort()
        # the first three copies are the calibration copy (the input rotation's
        # clones come later and have other sizes)
        copy = [v for _, n, v in out if "copyBuffer" in n][:3]
        ours = [(n, v) for _, n, v in out if "gemm_" in n or "splitk_reduce" in n]
        if not copy:
            raise SystemExit(f"{path}: no copy dispatches with {counter}")
        return statistics.mean(copy), ours

    cf, fetch = rows_of(fetch_csv, "FETCH_SIZE")
    cw, write = rows_of(write_csv, "WRITE_SIZE")
    ff, wf = COPY_BYTES / 1024 / cf, COPY_BYTES / 1024 / cw
    want = sum(2 * n for _, _, n in STREAM_CASES)
    if len(fetch) != want or len(write) != want:
        raise SystemExit(f"expected {want} split-K dispatches, got {len(fetch)} / {len(write)}")
    cases, at = [], 0
    for name, rows, launches in STREAM_CASES:
        w = wl.WORKLOADS[name]
        info = imm.gemm_plan(rows, w.N, w.K, w.dtype).info
        eb = 1 if w.dtype in ("e4m3", "e5m2") else 2
        slices = info["split_k"] * rows * w.N * 4
        algo = {"partial": (rows * w.K + w.K * w.N) * eb + slices,
                "reduce": slices + rows * w.N * 4}
        got = {}
        for i in range(2 * launches):
            (kn, fv), (kn2, wv) = fetch[at + i], write[at + i]
            kind = "reduce" if "splitk_reduce" in kn else "partial"
            if kn != kn2:
                raise SystemExit(f"dispatch order differs between the runs: {kn} / {kn2}")
            got.setdefault(kind, {"kernel": kn, "read": [], "write": []})
            got[kind]["read"].append(fv * ff * 1024)
            got[kind]["write"].append(wv * wf * 1024)
        at += 2 * launches
        entry = {"workload": name, "M": rows, "N": w.N, "K": w.K, "split_k": info["split_k"],
                 "tile": f"{info['block_m']}x{info['block_n']}"}
        for kind, g in got.items():
            rd, wr = statistics.mean(g["read"]), statistics.mean(g["write"])
            entry[kind] = {"kernel": g["kernel"], "launches": len(g["read"]),
                           "read_bytes_per_launch": rd, "write_bytes_per_launch": wr,
                           "algorithmic_bytes": algo[kind],
                           "measured_over_algorithmic": (rd + wr) / algo[kind]}
        cases.append(entry)
    out = {"fetch_scale": ff, "write_scale": wf, "copy_fetch_kib": cf, "copy_write_kib": cw,
           "cases": cases}
    os.makedirs(os.path.dirname(out_path), exist_ok=True)
    with open(out_path, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out))


def write_clock(counter_csv, agent_csv, lds_csv=None, out_path=CLOCK_FILE):
    """Turn one rocprofv3 --pmc run of `bench.py --clock-pass` (the CLOCK_COUNTERS)
    into the engine cycles, clock and matrix-core occupancy of the headline
    kernel, of hipBLASLt's kernel for the same product and of a plain copy.

    GRBM_GUI_ACTIVE is the per-dispatch count of busy engine cycles, summed over
    the XCDs: count / XCDs is the cycles one launch takes, and that over the
    dispatch's duration is the clock the part held.  SQ_VALU_MFMA_BUSY_CYCLES,
    summed over SIMDs, over those cycles times the SIMD count is the fraction of
    cycles the matrix units were busy; that is the kernel's fraction of the
    matrix peak at whatever clock it ran.  The fp16 MFMA op counter (512 flop
    per op) checks the flop count against 2*M*N*K.  The optional second run
    (LDS_COUNTERS) adds, per CU and cycle, the LDS bank-conflict and LDS-active
    cycles, and the L2 hit rate."""
    import csv

    with open(agent_csv) as f:
        gpu = next(r for r in csv.DictReader(f) if r["Agent_Type"] == "GPU")
    xcc, simds = int(gpu["Num_Xcc"]), int(gpu["Simd_Count"])
    fmax_ghz = int(gpu["Max_Engine_Clk_Fcompute"]) / 1000.0
    cus = int(gpu["Cu_Count"])

    def dispatches(path):
        disp = {}
        with open(path) as f:
            for r in csv.DictReader(f):
                d = disp.setdefault(r["Dispatch_Id"], {
                    "name": r["Kernel_Name"],
                    "ns": int(r["End_Timestamp"]) - int(r["Start_Timestamp"])})
                d[r["Counter_Name"]] = float(r["Counter_Value"])
        return disp
    disp = dispatches(counter_csv)

    def kind(name):
        if "gemm_dma_kernel" in name:
            return "headline"
        if name.startswith("Cijk"):
            return "hipblaslt"
        if "copyBuffer" in name:
            return "copy"
        return None

    groups = {}
    for d in disp.values():
        k = kind(d["name"])
        if k is None or "GRBM_GUI_ACTIVE" not in d or d["ns"] <= 0:
            continue
        cyc = d["GRBM_GUI_ACTIVE"] / xcc
        groups.setdefault(k, []).append({
            "us": d["ns"] / 1e3, "cycles": cyc, "ghz": cyc / d["ns"],
            "mfma_busy": d.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / (cyc * simds),
            "mfma_tflop": d.get("SQ_INSTS_VALU_MFMA_MOPS_F16", 0.0) * 512 / 1e12,
            "mfma_insts": d.get("SQ_INSTS_MFMA", 0.0), "name": d["name"][:120]})
    if "headline" not in groups:
        raise SystemExit(f"{counter_csv}: no headline-kernel dispatches with the clock counters")
    out = {"kernel": "gemm_dma_kernel<f16, f32 out, 256x256 tile>, M=N=K=8192",
           "kernel_source_hash": kernel_source_hash(), "counters": list(CLOCK_COUNTERS),
           "num_xcc": xcc, "simds": simds, "max_engine_clock_ghz": fmax_ghz}
    for k, g in groups.items():
        mean = {f: statistics.mean(x[f] for x in g)
                for f in ("us", "cycles", "ghz", "mfma_busy", "mfma_tflop", "mfma_insts")}
        out[k] = {"dispatches": len(g), "kernel_name": g[0]["name"],
                  "mean_us": mean["us"], "mean_cycles": mean["cycles"],
                  "min_cycles": min(x["cycles"] for x in g), "max_cycles": max(x["cycles"] for x in g),
                  "mean_clock_ghz": mean["ghz"],
                  "min_clock_ghz": min(x["ghz"] for x in g), "max_clock_ghz": max(x["ghz"] for x in g),
                  "mfma_busy_frac": mean["mfma_busy"], "mfma_tflop_per_launch": mean["mfma_tflop"],
                  "mfma_insts_per_launch": mean["mfma_insts"]}
    if lds_csv:
        out["counters"] += [c for c in LDS_COUNTERS if c not in out["counters"]]
        lds = {}
        for d in dispatches(lds_csv).values():
            k = kind(d["name"])
            if k is None or "GRBM_GUI_ACTIVE" not in d or "SQ_LDS_IDX_ACTIVE" not in d:
                continue
            cyc = d["GRBM_GUI_ACTIVE"] / xcc
            hit, miss = d.get("TCC_HIT_sum", 0.0), d.get("TCC_MISS_sum", 0.0)
            lds.setdefault(k, []).append({
                "conflict": d["SQ_LDS_BANK_CONFLICT"] / (cyc * cus),
                "active": d["SQ_LDS_IDX_ACTIVE"] / (cyc * cus),
                "insts": d.get("SQ_INSTS_LDS", 0.0),
                "l2hit": hit / (hit + miss) if hit + miss > 0 else 0.0})
        for k, g in lds.items():
            if k in out:
                out[k].update({
                    "lds_bank_conflict_per_cu_cycle": statistics.mean(x["conflict"] for x in g),
                    "lds_active_per_cu_cycle": statistics.mean(x["active"] for x in g),
                    "lds_insts_per_launch": statistics.mean(x["insts"] for x in g),
                    "l2_hit_rate": statistics.mean(x["l2hit"] for x in g)})
    with open(out_path, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out))


TRACE_SUMMARY_FILE = os.path.join(ROOT, "profiles", "gemm_dma_square_f16_8192_kernel_trace.md")
HEADLINE_KERNEL = "gemm_dma_kernel<0, 4, 0, 256, 256, 2, 4, 2, false, imm::GemmArgs>"


def write_trace_summary(trace_csv, bench_json, out_path=TRACE_SUMMARY_FILE):
    """Summarise a rocprofv3 --kernel-trace run of the default bench command:
    the headline kernel's dispatches (all, and the timed ones: the last
    `steps` of its 1024-workgroup launches before the next kernel), and every
    kernel by launch shape, next to the same run's event-timed numbers."""
    import csv
    with open(bench_json) as f:
        line = json.loads(f.read().strip().splitlines()[-1])
    rows = []
    with open(trace_csv) as f:
        for r in csv.DictReader(f):
            wg = int(r["Workgroup_Size_X"]) * int(r["Workgroup_Size_Y"]) * int(r["Workgroup_Size_Z"])
            grid = int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"])
            rows.append((int(r["Start_Timestamp"]), r["Kernel_Name"], grid // max(wg, 1), wg,
                         (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3))
    rows.sort()
    head = [x for x in rows if HEADLINE_KERNEL in x[1] and x[2] == 1024]
    if not head:
        raise SystemExit(f"{trace_csv}: no headline dispatches")
    # the headline leg runs its settle launches, then warm-up + steps back to back, first
    ns = line.get("extra", {}).get("settle", {}).get("headline_launches", 0)
    first = [x[4] for x in head[ns: ns + line["warmup"] + line["steps"]]]
    timed = first[line["warmup"]:]
    groups = {}
    for _, name, wgs, wg, us in rows:
        groups.setdefault((name, wgs, wg), []).append(us)

    def short(n):
        n = n.replace("void imm::(anonymous namespace)::", "").replace("imm::", "")
        n = n.split("(")[0] if n.startswith("gemm_") or n.startswith("splitk") else n
        return n if len(n) <= 72 else n[:69] + "..."

    out = ["# Kernel trace of the default bench run (square fp16 8192^3 headline)", "",
           "Commands (repository root, MI355X):", "",
           "    rocprofv3 --kernel-trace --stats --output-format csv -d gpurun_out/prof_bench -o bench "
           "-- python3 bench.py --steps 20 --warmup 5 > gpurun_out/bench_prof.json",
           "    python3 bench.py --write-trace-summary gpurun_out/prof_bench/bench_kernel_trace.csv "
           "gpurun_out/bench_prof.json", "",
           f"The same run printed value = {line['value']:.1f} TFLOP/s and roofline.avg_launch_ms = "
           f"{line['roofline']['avg_launch_ms'] * 1e3:.1f} us (HIP events on the launch stream).", "",
           f"Headline kernel `{HEADLINE_KERNEL}` at M=N=K=8192 (1024 workgroups x 512 threads): "
           f"{len(head)} dispatches in the whole run, average {statistics.mean(x[4] for x in head):.1f} us. "
           f"After its {ns} untimed settle launches, the next {len(first)} ({line['warmup']} warm-up + "
           f"{line['steps']} timed) back to back: "
           f"the timed {len(timed)} average {statistics.mean(timed):.1f} us, median "
           f"{statistics.median(timed):.1f} us, min {min(timed):.1f} us, max {max(timed):.1f} us.", "",
           "## Per kernel and launch shape", "",
           "| kernel | workgroups | threads/WG | calls | avg us | median us | min us |",
           "|---|---:|---:|---:|---:|---:|---:|"]
    order = sorted(groups.items(), key=lambda kv: -sum(kv[1]))
    for (name, wgs, wg), v in order[:60]:
        out.append(f"| `{short(name)}` | {wgs} | {wg} | {len(v)} | {statistics.mean(v):.2f} | "
                   f"{statistics.median(v):.2f} | {min(v):.2f} |")
    if len(order) > 60:
        out.append(f"| ({len(order) - 60} more kernel shapes, each a smaller share of the time) | | | | | | |")
    with open(out_path, "w") as f:
        f.write("\n".join(out) + "\n")
    print(out_path)


QKV_TRACE_FILE = os.path.join(ROOT, "profiles", "qkv_m_sweep_kernel_trace.md")
QKV_PASS_CALLS = 50


def qkv_pass(torch, imm, wl, N=6144, K=4096, ms=(1, 16, 64, 256, 1024)):
    """The fused-QKV M sweep's calls for a kernel trace: for each M, our plan
    with the tile from M (B as [K, N], then W [N, K]) and torch.matmul /
    F.linear on the same operands, each QKV_PASS_CALLS calls back to back
    after warm-up.  A one-element fill separates the cases in the trace.
    Prints the list of cases (one JSON line)."""
    g = wl.gen(6000)
    A = wl.uniform((max(ms), K), "f16", g).cuda()
    B = wl.uniform((K, N), "f16", g).cuda()
    W = B.t().contiguous()
    sep = torch.empty(1, device="cuda")  # filled only as a separator (no kernel here)
    cases = []
    for m in ms:
        a = A[:m].contiguous()
        C = torch.empty((m, N), dtype=torch.float32, device="cuda")
        pk = imm.gemm_plan_ex2(m, N, K, "f16", "f32", flags=imm.PLAN_TILE_BY_M)
        pw = imm.gemm_plan_ex2(m, N, K, "f16", "f32",
                               flags=imm.PLAN_TILE_BY_M | imm.PLAN_B_TRANSPOSED)
        ref = torch.empty((m, N), dtype=torch.float16, device="cuda")
        runs = [("ours, B [K, N]", f"{pk.info['run_block_m']}x{pk.info['run_block_n']}",
                 lambda: imm.gemm_run(pk, a, B, C)),
                ("torch.matmul, B [K, N]", "hipBLASLt", lambda: torch.matmul(a, B, out=ref)),
                ("ours, W [N, K]", f"{pw.info['run_block_m']}x{pw.info['run_block_n']}",
                 lambda: imm.gemm_run(pw, a, W, C)),
                ("F.linear, W [N, K]", "hipBLASLt", lambda: torch.nn.functional.linear(a, W))]
        for name, tile, fn in runs:
            for _ in range(20):
                fn()
            torch.cuda.synchronize()
            sep.fill_(1.0)
            torch.cuda.synchronize()
            for _ in range(QKV_PASS_CALLS):
                fn()
            torch.cuda.synchronize()
            sep.fill_(1.0)
            torch.cuda.synchronize()
            cases.append({"M": m, "N": N, "K": K, "what": name, "tile": tile})
    print(json.dumps({"calls": QKV_PASS_CALLS, "cases": cases}))


def write_qkv_trace_summary(trace_csv, pass_json, out_path=QKV_TRACE_FILE):
    """Summarise a rocprofv3 --kernel-trace run of `bench.py --qkv-pass`:
    kernel time per call of every case (the kernels between the separating
    fills that enclose its timed calls, divided by the calls)."""
    import csv
    with open(pass_json) as f:
        meta = json.loads(f.read().strip().splitlines()[-1])
    rows = []
    with open(trace_csv) as f:
        for r in csv.DictReader(f):
            rows.append((int(r["Start_Timestamp"]), r["Kernel_Name"],
                         (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3))
    rows.sort()
    is_sep = ["FillFunctor" in n for _, n, us in rows]
    # segments between consecutive separators; the timed calls of case i are
    # segment 2i + 1 (warm-up, sep, timed calls, sep; nothing else fills)
    segs, cur = [], []
    for (t, n, us), sp in zip(rows, is_sep):
        if sp:
            segs.append(cur)
            cur = []
        else:
            cur.append((n, us))
    segs.append(cur)
    calls = meta["calls"]
    out = ["# Kernel trace of the fused-QKV M sweep (N = 6144, K = 4096, fp16)", "",
           "Commands (repository root, MI355X):", "",
           "    rocprofv3 --kernel-trace --output-format csv -d gpurun_out/prof_qkv -o qkv "
           "-- python3 bench.py --qkv-pass > gpurun_out/qkv_pass.json",
           "    python3 bench.py --write-qkv-trace-summary gpurun_out/prof_qkv/qkv_kernel_trace.csv "
           "gpurun_out/qkv_pass.json", "",
           f"Each case: {calls} calls back to back after 20 warm-up calls, one B (held by the "
           "last-level cache between calls), our fp32 out against torch's fp16 out. Kernel time "
           "per call is the trace's kernel durations between the separating fills divided by "
           "the calls; it leaves out launch gaps, which the bench's event timings include.", "",
           "| M | call | tile | kernels per call | kernel us per call | main kernel |",
           "|---:|---|---|---:|---:|---|"]
    if len(segs) != 2 * len(meta["cases"]) + 1:
        raise SystemExit(f"{trace_csv}: {len(segs) - 1} separators, expected {2 * len(meta['cases'])}")
    for i, c in enumerate(meta["cases"]):
        seg = segs[2 * i + 1]
        if len(seg) < calls:
            raise SystemExit(f"{trace_csv}: {len(seg)} kernels for case {i} ({c}), expected >= {calls}")
        tot = sum(us for _, us in seg)
        main = max(set(n for n, _ in seg), key=lambda n: sum(us for m_, us in seg if m_ == n))
        main = main.replace("void imm::(anonymous namespace)::", "").split("(")[0]
        main = main if len(main) <= 60 else main[:57] + "..."
        out.append(f"| {c['M']} | {c['what']} | {c['tile']} | {len(seg) / calls:.2f} | "
                   f"{tot / calls:.2f} | `{main}` |")
    with open(out_path, "w") as f:
        f.write("\n".join(out) + "\n")
    print(out_path)


def _smi_power_clocks():
    """Socket power (W) and the XCDs' engine clocks (MHz) from amd-smi."""
    import re
    import subprocess
    r = subprocess.run(["amd-smi", "metric", "-p", "-c", "--json"], capture_output=True,
                       text=True, timeout=60)
    if r.returncode != 0:
        return {"error": r.stderr.strip()[:200]}
    j = json.loads(r.stdout)
    gpu = j["gpu_data"][0] if isinstance(j, dict) else j[0]
    power = gpu["power"]["socket_power"]["value"]
    clocks = [v["clk"]["value"] for k, v in gpu["clock"].items()
              if re.fullmatch(r"gfx_\d+", k) and isinstance(v, dict)]
    return {"socket_power_w": power, "gfx_clocks_mhz": clocks}


def power_sample(torch, imm, wl, seconds=6.0):
    """The headline product in a loop (random inputs, then all-zero ones),
    with amd-smi read half-way through each: the board's power and clocks
    under the same instructions and data movement with different operand
    switching activity."""
    import threading
    out = {"idle": _smi_power_clocks()}
    w = wl.WORKLOADS["square_f16_8192"]
    A, B = w.make()
    Ad, Bd = A.cuda(), B.cuda()
    plan = imm.gemm_plan(w.M, w.N, w.K, w.dtype)
    C = torch.empty((w.M, w.N), dtype=torch.float32, device="cuda")
    for kind in ("random", "zeros"):
        if kind == "zeros":
            Ad.zero_()
            Bd.zero_()
        stop = time.time() + seconds
        launches = [0]

        def loop():
            while time.time() < stop:
                for _ in range(20):
                    imm.gemm_run(plan, Ad, Bd, C)
                torch.cuda.synchronize()
                launches[0] += 20

        th = threading.Thread(target=loop)
        t0 = time.time()
        th.start()
        time.sleep(seconds / 2)
        sample = _smi_power_clocks()
        th.join()
        dt = time.time() - t0
        out[kind] = {**sample, "launches": launches[0],
                     "TFLOPs": launches[0] * w.flops / dt / 1e12}
    return out


def log(msg):
    print(msg, file=sys.stderr, flush=True)


SETTLE_MS = 150.0
# untimed settle launches before each timed series, in order (the headline's first)
SETTLE_LAUNCHES = []


def settle(fn, torch, ms=SETTLE_MS):
    """Launch fn back to back, untimed, until about `ms` of GPU time has
    passed; returns the number of launches."""
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    n = 0
    while True:
        for _ in range(4):
            fn(0)
        n += 4
        e.record()
        e.synchronize()
        if s.elapsed_time(e) >= ms:
            return n


def time_launches(fn, n, warmup, torch, settle_ms=SETTLE_MS, queue_ahead=False):
    """Per-call durations (ms) from HIP events recorded on the current stream,
    after the settle launches and `warmup` untimed calls.

    queue_ahead: for calls of a few tens of us, whose host side (argument
    checks, launches, two event records) takes about as long as the GPU side.
    The timed calls are then enqueued behind a spin kernel of a few ms, so the
    GPU never waits for the host between them; otherwise a call's start event
    can fire while the host is still preparing the launch, and some calls
    measure 1.5-2x their kernel time."""
    SETTLE_LAUNCHES.append(settle(fn, torch, settle_ms) if settle_ms > 0 else 0)
    for _ in range(warmup):
        fn(0)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(n)]
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    if queue_ahead and hasattr(torch.cuda, "_sleep"):
        # about 0.1 ms of engine cycles per timed call, at least 2 ms
        torch.cuda._sleep(int(2.4e5 * max(20, n)))
    t0.record()
    for i in range(n):
        ev[i][0].record()
        fn(i)
        ev[i][1].record()
    t1.record()
    torch.cuda.synchronize()
    per = [a.elapsed_time(b) for a, b in ev]
    return per, t0.elapsed_time(t1)


def summary(per):
    s = sorted(per)
    return {"median_ms": statistics.median(s), "min_ms": s[0],
            "p90_ms": s[min(len(s) - 1, int(0.9 * len(s)))], "n": len(s)}


def oracle_sample(w, A, B, threads, target_s, gpu_ms=None, rows=None):
    """Time the CPU oracle on the first rows of one workload's product.

    One probe call on `threads` rows gives the time per row; then one call on
    about target_s seconds' worth of rows (all of them if that fits) is timed.
    decode_B_s is the oracle's decoder run alone on B (the oracle decodes B
    once per call, on one thread, before its row loop); accumulate_s is the
    rest of the call.  full_product_s_est extrapolates to all M rows."""
    import oracle
    import workloads as wl
    a_bits, b_bits = wl.bits(A), wl.bits(B)
    M, N, K = a_bits.shape[0], b_bits.shape[1], a_bits.shape[1]

    def call(r):
        t = time.perf_counter()
        oracle.gemm(a_bits, b_bits, w.dtype, rows=list(range(r)), nthreads=threads)
        return time.perf_counter() - t

    t = time.perf_counter()
    oracle.decode(w.dtype, b_bits)
    dec = time.perf_counter() - t
    if rows is None:
        r1 = min(M, threads)
        if dec >= target_s / 2:
            rows = r1  # decoding B alone takes most of the budget: one row per thread
        else:
            per_row = max((call(r1) - dec) / r1, 1e-9)
            rows = int(min(M, max(r1, (target_s - dec) / per_row)))
            if threads < rows < M:
                rows -= rows % threads
    total = call(rows)
    acc = max(total - dec, 0.0)
    out = {"workload": w.name, "shape": f"{M}x{N}x{K} {w.dtype}", "rows": rows, "of_rows": M,
           "threads": threads, "total_s": total, "decode_B_s": dec, "accumulate_s": acc,
           "GFLOPs": 2.0 * rows * N * K / total / 1e9,
           "full_product_s_est": dec + acc * M / rows}
    if gpu_ms:
        out["gpu_ms"] = gpu_ms
        out["gpu_speedup_est"] = out["full_product_s_est"] / (gpu_ms * 1e-3)
    return out


def cpu_baseline(samples):
    """The oracle (test infrastructure: fp64 triple loop, OpenMP over rows) on
    the host cores, one bounded sample per workload.  samples: list of
    (workload, A, B, gpu_ms, target_s).  The headline value is the oracle's
    rate on the square fp16 8192^3 sample; per_config holds every workload,
    plus the 256^3 exact product on one core."""
    import oracle
    threads = oracle.max_threads()
    per = []
    for w, A, B, gpu_ms, target in samples:
        per.append(oracle_sample(w, A, B, threads, target, gpu_ms))
        if w.name == "exact256":
            per.append(oracle_sample(w, A, B, 1, target, gpu_ms, rows=w.M))
    head = next(x for x in per if x["workload"] == "square_f16_8192")
    return {"value": head["GFLOPs"] / 1e3, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"rows 0..{head['rows'] - 1} of the 8192x8192x8192 f16 product, one call "
                      f"({head['total_s']:.1f} s wall, of which {head['decode_B_s']:.1f} s decoding "
                      f"B); per_config samples every workload the same way, full where it fits "
                      f"in its budget, and the 256^3 product also on one core",
            "per_config": per}


def bench_square(name, steps, warmup, torch, imm, wl, queue_ahead=False):
    w = wl.WORKLOADS[name]
    A, B = w.make()
    Ad, Bd = A.cuda(), B.cuda()
    plan = imm.gemm_plan(w.M, w.N, w.K, w.dtype)
    out_t = torch.float32 if w.out == "f32" else torch.bfloat16
    C = torch.empty((w.M, w.N), dtype=out_t, device="cuda")
    per, total = time_launches(lambda i: imm.gemm_run(plan, Ad, Bd, C), steps, warmup, torch,
                               queue_ahead=queue_ahead)
    return w, plan, per, total, (A, B, Ad, Bd)


def fp8_comparator(w, plan, host, torch, imm, rounds=3):
    """The fp8 product next to torch._scaled_mm (hipBLASLt) on the same inputs
    and per-tensor scales of 1, bf16 out, in alternating rounds of 20 launches
    (the part's clock follows its recent power draw); best round medians."""
    _, _, Ad, Bd = host
    Bcm = Bd.t().contiguous().t()  # the column-major B that _scaled_mm takes
    one = torch.tensor(1.0, device="cuda")
    C = torch.empty((w.M, w.N), dtype=torch.bfloat16, device="cuda")
    last = [None]
    runs = {"ours": lambda i: imm.gemm_run(plan, Ad, Bd, C),
            "hipblaslt": lambda i: last.__setitem__(0, torch._scaled_mm(
                Ad, Bcm, scale_a=one, scale_b=one, out_dtype=torch.bfloat16))}
    best = {k: [] for k in runs}
    for r in range(rounds):
        for k in (("ours", "hipblaslt") if r % 2 == 0 else ("hipblaslt", "ours")):
            per, _ = time_launches(runs[k], 20, 5, torch)
            best[k].append(statistics.median(per))
    out = {}
    for k, v in best.items():
        ms = min(v)
        out[k] = {"best_round_median_ms": ms, "round_medians_ms": v,
                  "TFLOPs": w.flops / (ms * 1e-3) / 1e12}
    torch.cuda.synchronize()
    C2 = last[0].float()
    out["max_abs_diff_over_max_abs"] = float((C.float() - C2).abs().max() / C2.abs().max())
    return out


def bench_splitk(name, split, torch, imm, wl, n=30, warmup=5, M=None):
    """Split-K path with inputs rotated through enough copies to defeat the MALL."""
    w = wl.WORKLOADS[name]
    A, B = w.make()
    Ad, Bd = A.cuda(), B.cuda()
    Mrows = w.M if M is None else M
    Ad = Ad[:Mrows].contiguous()
    bytes_in = Ad.numel() * Ad.element_size() + Bd.numel() * Bd.element_size()
    copies = max(1, -(-2 * MALL_BYTES // bytes_in)) + 1
    As = [Ad] + [Ad.clone() for _ in range(copies - 1)]
    Bs = [Bd] + [Bd.clone() for _ in range(copies - 1)]
    plan = imm.gemm_plan_ex(Mrows, w.N, w.K, w.dtype, w.out, split_k=split)
    C = torch.empty((Mrows, w.N), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(1, imm.gemm_workspace_size(plan) // 4), dtype=torch.float32,
                     device="cuda")
    per, _ = time_launches(
        lambda i: imm.gemm_splitk_run(plan, As[i % copies], Bs[i % copies], C, ws),
        n, warmup, torch, queue_ahead=True)
    algo = bytes_in + Mrows * w.N * 4
    med = statistics.median(per)
    out = {"M": Mrows, "N": w.N, "K": w.K, "split_k": plan.info["split_k"],
           "tile": f"{plan.info['block_m']}x{plan.info['block_n']}",
           "copies_rotated": copies, **summary(per),
           "algorithmic_bytes": algo, "GBps": algo / (med * 1e-3) / 1e9,
           "pct_hbm_peak": 100.0 * algo / (med * 1e-3) / 1e9 / PEAK_HBM_GBS,
           "TFLOPs": 2.0 * Mrows * w.N * w.K / (med * 1e-3) / 1e12,
           "workspace_traffic_bytes": 2 * plan.info["workspace_bytes"]}
    if split == 0:
        # GEMM_PLAN_TILE_BY_M: the split-path tile from M (same split, same bits)
        pm = imm.gemm_plan_ex2(Mrows, w.N, w.K, w.dtype, w.out, flags=imm.PLAN_TILE_BY_M)
        if pm.info["tile"] != plan.info["tile"]:
            pmm, _ = time_launches(
                lambda i: imm.gemm_splitk_run(pm, As[i % copies], Bs[i % copies], C, ws),
                n, warmup, torch, queue_ahead=True)
            mm_ = statistics.median(pmm)
            out.update({"tile_by_m": f"{pm.info['block_m']}x{pm.info['block_n']}",
                        "tile_by_m_median_us": mm_ * 1e3,
                        "tile_by_m_GBps": algo / (mm_ * 1e-3) / 1e9})
    return out


def _probe_lib():
    """The streaming-read probe library (built next to the GEMM library)."""
    import ctypes

    from invariant_matmul_amd import build as _b
    if not os.path.exists(_b.PROBE_LIB):
        raise RuntimeError(f"{_b.PROBE_LIB} is not built")
    L = ctypes.CDLL(_b.PROBE_LIB)
    L.imm_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int,
                                 ctypes.c_int, ctypes.c_void_p]
    L.imm_probe_read.restype = ctypes.c_int
    return L


def bench_read_probe(torch, nbytes, copies, n=20, warmup=5):
    """Streaming read of nbytes (rotated over `copies` buffers so that with
    copies * nbytes well above the 256 MB last-level cache every read comes
    from HBM), best median over grid sizes and load kinds."""
    L = _probe_lib()
    bufs = [torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
            for _ in range(copies)]
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    best = None

    def launch(i, wgs, nt):
        rc = L.imm_probe_read(bufs[i % copies].data_ptr(), nbytes, sink.data_ptr(), wgs, nt, stream)
        if rc != 0:
            raise RuntimeError(f"imm_probe_read failed: {rc}")

    for wgs in (1024, 2048, 4096, 8192):
        for nt in (0, 1):
            per, _ = time_launches(lambda i: launch(i, wgs, nt), n, warmup, torch)
            med = statistics.median(per)
            if best is None or med < best["median_ms"]:
                best = {"median_ms": med, "workgroups": wgs, "nontemporal": bool(nt)}
    del bufs
    torch.cuda.empty_cache()
    best.update({"bytes": nbytes, "copies_rotated": copies,
                 "GBps": nbytes / (best["median_ms"] * 1e-3) / 1e9})
    best["pct_hbm_peak"] = 100.0 * best["GBps"] / PEAK_HBM_GBS
    return best


def bench_hbm_probes(torch, nbytes=2 ** 30):
    """Achievable HBM rates on this part: a 1 GiB streaming read, a read of the
    decode product's B (14336 x 4096 bf16) rotated over 5 copies, and the
    runtime's 1 GiB device copy (read + write bytes over time)."""
    out = {"read_1GiB": bench_read_probe(torch, nbytes, 1),
           "read_decode_B": bench_read_probe(torch, 14336 * 4096 * 2, 5)}
    x = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    y = torch.empty_like(x)
    tc, _ = time_launches(lambda i: y.copy_(x), 20, 5, torch)
    out["copy_1GiB_GBps"] = 2 * nbytes / (statistics.median(tc) * 1e-3) / 1e9
    del x, y
    torch.cuda.empty_cache()
    return out


def bench_m_sweep(torch, imm, wl, N=6144, K=4096, ms=(1, 16, 64, 256, 1024, 4096, 8192)):
    """The price of one M-independent plan: gemm_run on the fused-QKV projection
    shape at growing M, next to torch.matmul (hipBLASLt, which picks its kernel
    per shape and is not batch-invariant).  Rows are prefixes of one A."""
    g = wl.gen(6000)
    A = wl.uniform((max(ms), K), "f16", g).cuda()
    B = wl.uniform((K, N), "f16", g).cuda()
    W = B.t().contiguous()
    out = []
    for m in ms:
        a = A[:m].contiguous()
        plan = imm.gemm_plan(m, N, K, "f16")
        C = torch.empty((m, N), dtype=torch.float32, device="cuda")
        per, _ = time_launches(lambda i: imm.gemm_run(plan, a, B, C), 20, 5, torch, queue_ahead=True)
        # the same bits with the tile taken from M (GEMM_PLAN_TILE_BY_M)
        mplan = imm.gemm_plan_ex2(m, N, K, "f16", "f32", flags=imm.PLAN_TILE_BY_M)
        mper, _ = time_launches(lambda i: imm.gemm_run(mplan, a, B, C), 20, 5, torch,
                                queue_ahead=True)
        ref = torch.empty((m, N), dtype=torch.float16, device="cuda")
        tper, _ = time_launches(lambda i: torch.matmul(a, B, out=ref), 20, 5, torch,
                                queue_ahead=True)
        # the weight layout of a linear layer: W [N, K] read in place
        # (GEMM_PLAN_B_TRANSPOSED), tile from M, next to F.linear on the same W
        wplan = imm.gemm_plan_ex2(m, N, K, "f16", "f32",
                                  flags=imm.PLAN_TILE_BY_M | imm.PLAN_B_TRANSPOSED)
        wper, _ = time_launches(lambda i: imm.gemm_run(wplan, a, W, C), 20, 5, torch,
                                queue_ahead=True)
        lper, _ = time_launches(lambda i: torch.nn.functional.linear(a, W), 20, 5, torch,
                                queue_ahead=True)
        med, mmed, tmed = statistics.median(per), statistics.median(mper), statistics.median(tper)
        out.append({"M": m, "N": N, "K": K,
                    "tile": f"{plan.info['run_block_m']}x{plan.info['run_block_n']}",
                    "median_us": med * 1e3, "TFLOPs": 2.0 * m * N * K / (med * 1e-3) / 1e12,
                    "tile_by_m": f"{mplan.info['run_block_m']}x{mplan.info['run_block_n']}",
                    "tile_by_m_median_us": mmed * 1e3,
                    "torch_matmul_median_us": tmed * 1e3,
                    "torch_matmul_TFLOPs": 2.0 * m * N * K / (tmed * 1e-3) / 1e12,
                    "weight_nk_tile_by_m": f"{wplan.info['run_block_m']}x{wplan.info['run_block_n']}",
                    "weight_nk_tile_by_m_median_us": statistics.median(wper) * 1e3,
                    "torch_linear_median_us": statistics.median(lper) * 1e3})
    return out


def bench_ozaki(name, torch, imm, wl, n_iter=5, warmup=2):
    """fp64 product by the Ozaki scheme: split, slice-pair product, whole call,
    next to torch.matmul in fp64 (the native fp64 matrix path) as a comparator."""
    w = wl.OZAKI_WORKLOADS[name]
    A, B = w.make()
    Ad, Bd = A.cuda(), B.cuda()
    del A, B
    plan = imm.ozaki_plan(w.n, w.n, w.n, w.type2)
    i = plan.info
    ws = torch.empty(imm.ozaki_workspace_size(plan), dtype=torch.uint8, device="cuda")
    C = torch.empty((w.n, w.n), dtype=torch.float64, device="cuda")
    split, _ = time_launches(lambda k: (imm.ozaki_split(plan, 0, Ad, ws),
                                        imm.ozaki_split(plan, 1, Bd, ws)), n_iter, warmup, torch)
    mult, _ = time_launches(lambda k: imm.ozaki_multiply(plan, ws, C), n_iter, warmup, torch)
    run, _ = time_launches(lambda k: imm.ozaki_run(plan, Ad, Bd, C, ws), n_iter, warmup, torch)
    ts, tm, tr = (statistics.median(x) for x in (split, mult, run))
    mfma_flops = i["pairs"] * w.flops
    out = {"n": w.n, "type2": w.type2, "slices": i["slices"], "d": i["d"], "pairs": i["pairs"],
           "bits_per_slice": i["bits"], "split_ms": ts, "multiply_ms": tm, "total_ms": tr,
           "fp64_TFLOPs": w.flops / (tr * 1e-3) / 1e12,
           "multiply_matrix_TFLOPs": mfma_flops / (tm * 1e-3) / 1e12,
           "multiply_pct_mfma_peak": 100.0 * mfma_flops / (tm * 1e-3) / 1e12 /
           PEAK_TFLOPS[w.type2]}
    torch.cuda.empty_cache()
    try:
        ref = torch.empty((w.n, w.n), dtype=torch.float64, device="cuda")
        tper, _ = time_launches(lambda k: torch.matmul(Ad, Bd, out=ref), n_iter, warmup, torch)
        out["torch_matmul_f64_TFLOPs"] = w.flops / (statistics.median(tper) * 1e-3) / 1e12
        # the page's accuracy figure: relative (Frobenius) error against the
        # fp64 product (itself rounded, so ~1e-15 is the floor)
        out["rel_error_vs_torch_f64"] = float(torch.linalg.norm(C - ref) / torch.linalg.norm(ref))
        del ref
    except Exception as e:  # comparator only
        out["torch_matmul_f64_error"] = str(e)
    del ws, C, Ad, Bd
    torch.cuda.empty_cache()
    return out


def bench_ozaki_d_sweep(torch, imm, wl, n=8192, ds=(11, 9, 8, 7, 6, 5), type2s=("bf16", "i8")):
    """Fast Mode trade-off: skipping the pairs with p + q >= d for smaller d,
    time and relative error against torch's fp64 product (the page's
    "dによる精度/速度トレードオフ" table runs d = 9 .. 5 at n = 16384)."""
    w = wl.OZAKI_WORKLOADS[f"ozaki_bf16_{n}"]
    A, B = w.make()
    Ad, Bd = A.cuda(), B.cuda()
    del A, B
    ref = torch.matmul(Ad, Bd)
    C = torch.empty_like(ref)
    out = []
    for t2 in type2s:
        for d in ds:
            plan = imm.ozaki_plan(n, n, n, t2, 0, d)
            ws = torch.empty(imm.ozaki_workspace_size(plan), dtype=torch.uint8, device="cuda")
            per, _ = time_launches(lambda k: imm.ozaki_run(plan, Ad, Bd, C, ws), 3, 1, torch)
            med = statistics.median(per)
            out.append({"type2": t2, "n": n, "d": plan.info["d"], "pairs": plan.info["pairs"],
                        "total_ms": med, "fp64_TFLOPs": w.flops / (med * 1e-3) / 1e12,
                        "rel_error_vs_torch_f64":
                            float(torch.linalg.norm(C - ref) / torch.linalg.norm(ref))})
            del ws
            torch.cuda.empty_cache()
    del Ad, Bd, ref, C
    torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-extra", action="store_true", help="headline workload only")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline")
    ap.add_argument("--profile-pass", action="store_true",
                    help="a few launches of the headline kernel plus a plain copy of known "
                         "size, for hardware-counter runs; prints nothing else")
    ap.add_argument("--write-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="host only: write the headline kernel's HBM traffic from two "
                         "counter runs of --profile-pass, then exit")
    ap.add_argument("--stream-pass", action="store_true",
                    help="a plain copy of known size, then the decode and huge-K split-K products "
                         "on cold inputs, for HBM-traffic counter runs; prints nothing else")
    ap.add_argument("--write-stream-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="host only: write the split-K kernels' HBM traffic from two counter "
                         "runs of --stream-pass, then exit")
    ap.add_argument("--clock-pass", action="store_true",
                    help="back-to-back launches of the headline kernel, of torch.matmul on "
                         "the same fp16 product and of a plain copy, for the clock counters; "
                         "prints nothing else")
    ap.add_argument("--write-trace-summary", nargs=2, metavar=("TRACE_CSV", "BENCH_JSON"),
                    help="host only: write the kernel-trace summary of a rocprofv3 --kernel-trace run "
                         "of the default bench command, then exit")
    ap.add_argument("--qkv-pass", action="store_true",
                    help="the fused-QKV M sweep's calls, back to back with separators, for a "
                         "kernel trace; prints the list of cases")
    ap.add_argument("--write-qkv-trace-summary", nargs=2, metavar=("TRACE_CSV", "PASS_JSON"),
                    help="host only: write the kernel-trace summary of a --qkv-pass run, then exit")
    ap.add_argument("--power-sample", action="store_true",
                    help="run the headline product in a loop on random, then all-zero inputs "
                         "and read the board's power and engine clocks with amd-smi during "
                         "each; prints one JSON line")
    ap.add_argument("--write-clock", nargs="+", metavar="CSV",
                    help="host only: COUNTER_CSV AGENT_CSV [LDS_CSV]: write the headline kernel's "
                         "engine clock and matrix-core occupancy from a counter run of "
                         "--clock-pass (and LDS / L2 behaviour from a second one), then exit")
    args = ap.parse_args()
    if args.write_traffic:
        write_traffic(*args.write_traffic)
        return
    if args.write_stream_traffic:
        write_stream_traffic(*args.write_stream_traffic)
        return
    if args.write_trace_summary:
        write_trace_summary(*args.write_trace_summary)
        return
    if args.write_qkv_trace_summary:
        write_qkv_trace_summary(*args.write_qkv_trace_summary)
        return
    if args.write_clock:
        if len(args.write_clock) not in (2, 3):
            ap.error("--write-clock takes COUNTER_CSV AGENT_CSV [LDS_CSV]")
        write_clock(*args.write_clock)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (this build has no multi-GPU path); "
              f"--gpus {args.gpus} is not supported", file=sys.stderr)
        sys.exit(2)

    import torch

    import invariant_matmul_amd as imm
    import workloads as wl

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    imm.lib()

    if args.qkv_pass:
        qkv_pass(torch, imm, wl)
        return

    if args.profile_pass:
        w = wl.WORKLOADS["square_f16_8192"]
        A, B = w.make()
        Ad, Bd = A.cuda(), B.cuda()
        plan = imm.gemm_plan(w.M, w.N, w.K, w.dtype)
        C = torch.empty((w.M, w.N), dtype=torch.float32, device="cuda")
        src = torch.empty(256 * 2 ** 20 // 4, dtype=torch.float32, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)   # plain copy: 256 MiB read + 256 MiB written
        for _ in range(3):
            imm.gemm_run(plan, Ad, Bd, C)
        torch.cuda.synchronize()
        print("profile pass done", flush=True)
        return

    if args.power_sample:
        print(json.dumps(power_sample(torch, imm, wl)), flush=True)
        return

    if args.stream_pass:
        stream_pass(torch, imm, wl)
        print("stream pass done", flush=True)
        return

    if args.clock_pass:
        w = wl.WORKLOADS["square_f16_8192"]
        A, B = w.make()
        Ad, Bd = A.cuda(), B.cuda()
        plan = imm.gemm_plan(w.M, w.N, w.K, w.dtype)
        C = torch.empty((w.M, w.N), dtype=torch.float32, device="cuda")
        ref = torch.empty((w.M, w.N), dtype=torch.float16, device="cuda")
        src = torch.empty(2 ** 30 // 4, dtype=torch.float32, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)   # plain copy: 1 GiB read + 1 GiB written
        for _ in range(10):
            imm.gemm_run(plan, Ad, Bd, C)
        for _ in range(10):
            torch.matmul(Ad, Bd, out=ref)
        torch.cuda.synchronize()
        print("clock pass done", flush=True)
        return

    log("headline: square fp16 8192^3, gemm_run")
    w, plan, per, total, host = bench_square("square_f16_8192", args.steps, args.warmup,
                                             torch, imm, wl)
    ms_per_step = total / args.steps
    value = w.flops / (ms_per_step * 1e-3) / 1e12
    kavg = statistics.mean(per)
    achieved = w.flops / (kavg * 1e-3) / 1e12
    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
        if t.get("kernel_source_hash") == kernel_source_hash():
            traffic = t.get("bytes_per_launch")
    clock = None
    if os.path.exists(CLOCK_FILE):
        with open(CLOCK_FILE) as f:
            c = json.load(f)
        if c.get("kernel_source_hash") == kernel_source_hash():
            # the launch's cycle count is stable across runs; the clock is not
            h = c["headline"]
            ghz = h["mean_cycles"] / (kavg * 1e6)
            peak_at = PEAK_TFLOPS["f16"] * ghz / c["max_engine_clock_ghz"]
            clock = {"cycles_per_launch": h["mean_cycles"], "clock_ghz_timed": ghz,
                     "peak_at_clock_tflops": peak_at, "frac_at_clock": achieved / peak_at,
                     "mfma_busy_frac_counters": h["mfma_busy_frac"],
                     "source": os.path.relpath(CLOCK_FILE, ROOT)}
    roofline = {"bound": "mfma", "achieved": achieved, "peak": PEAK_TFLOPS["f16"],
                "unit": "TFLOP/s", "frac": achieved / PEAK_TFLOPS["f16"], "traffic": traffic,
                "frac_at_clock": clock["frac_at_clock"] if clock else None,
                "clock_ghz_timed": clock["clock_ghz_timed"] if clock else None,
                "kernel": "gemm_dma_kernel<f16, f32 out, 256x256 tile>",
                "algorithmic_flop_per_launch": w.flops, "avg_launch_ms": kavg}

    extra = {"headline_kernel": summary(per), "headline_clock": clock,
             "settle": {"ms": SETTLE_MS, "headline_launches": SETTLE_LAUNCHES[0]},
             "plan": {k: plan.info[k] for k in ("run_block_m", "run_block_n", "block_k", "run_waves",
                                                  "group_m", "split_k", "mfma_k")}}
    secondary = {}
    # (workload, host A, host B, GPU median ms, seconds of oracle time) for the CPU baseline
    samples = []
    A, B = host[0], host[1]
    if not args.no_extra:
        Ad, Bd = host[2], host[3]
        try:
            ref = torch.empty((w.M, w.N), dtype=torch.float16, device="cuda")
            tper, _ = time_launches(lambda i: torch.matmul(Ad, Bd, out=ref), 20, 5, torch)
            extra["torch_matmul_f16_8192_TFLOPs"] = w.flops / (statistics.median(tper) * 1e-3) / 1e12
            del ref
        except Exception as e:  # comparator only
            extra["torch_matmul_error"] = str(e)
        # The headline series again after 2 s of idle, with its warm-up but no
        # settle launches: what the first launches after an idle spell get.
        log("headline after an idle spell")
        Ci = torch.empty((w.M, w.N), dtype=torch.float32, device="cuda")
        torch.cuda.synchronize()
        time.sleep(2.0)
        iper, itot = time_launches(lambda i: imm.gemm_run(plan, Ad, Bd, Ci), args.steps, args.warmup,
                                   torch, settle_ms=0)
        del Ci
        extra["headline_after_idle"] = {**summary(iper), "idle_s": 2.0, "settle_ms": 0,
                                        "ms_per_step": itot / args.steps,
                                        "TFLOPs": w.flops / (itot / args.steps * 1e-3) / 1e12}
        secondary["fp16_8192_after_2s_idle_no_settle_TFLOPs"] = round(
            extra["headline_after_idle"]["TFLOPs"], 1)
        # The same product with A and B rotated over two copies (537 MB, twice
        # the 256 MB last-level cache), so that no launch finds its operands
        # left in that cache by the one before.
        log("headline with rotated inputs")
        Cr = torch.empty((w.M, w.N), dtype=torch.float32, device="cuda")
        As, Bs = [Ad, Ad.clone()], [Bd, Bd.clone()]
        rper, _ = time_launches(lambda i: imm.gemm_run(plan, As[i % 2], Bs[i % 2], Cr), 20, 4, torch)
        extra["headline_rotated_inputs"] = {
            **summary(rper), "copies": 2,
            "TFLOPs": w.flops / (statistics.median(rper) * 1e-3) / 1e12,
            "pct_mfma_peak": 100.0 * w.flops / (statistics.median(rper) * 1e-3) / 1e12 / PEAK_TFLOPS["f16"]}
        secondary["fp16_8192_rotated_inputs_TFLOPs"] = round(extra["headline_rotated_inputs"]["TFLOPs"], 1)
        del Ad, Bd, As, Bs, Cr, host
        torch.cuda.empty_cache()
        samples.append((w, A, B, statistics.median(per), 6.0))

        log("exact 256^3 fp16 (integers)")
        we = wl.WORKLOADS["exact256"]
        Ae, Be = we.make()
        pe = imm.gemm_plan(we.M, we.N, we.K, we.dtype)
        Ce = torch.empty((we.M, we.N), dtype=torch.float32, device="cuda")
        Aed, Bed = Ae.cuda(), Be.cuda()
        pere, _ = time_launches(lambda i: imm.gemm_run(pe, Aed, Bed, Ce), 30, 5, torch)
        samples.append((we, Ae, Be, statistics.median(pere), 1.0))
        del Aed, Bed, Ce

        secondary["fp8_e5m2_bf16_out"] = {}
        for n8, steps8 in ((4096, 30), (8192, 30), (16384, 10)):
            log(f"fp8 e5m2 {n8}^3")
            w8, plan8, per8, _, h8 = bench_square(f"square_e5m2_{n8}", steps8, 5, torch, imm, wl,
                                                  queue_ahead=n8 == 4096)
            med8 = statistics.median(per8)
            e8 = {**summary(per8), "TFLOPs": w8.flops / (med8 * 1e-3) / 1e12,
                  "pct_mfma_peak": 100 * w8.flops / (med8 * 1e-3) / 1e12 / PEAK_TFLOPS["e5m2"]}
            sec8 = {"TFLOPs": round(e8["TFLOPs"], 1), "pct_peak": round(e8["pct_mfma_peak"], 2),
                    "median_us": round(med8 * 1e3, 1)}
            if n8 == 8192:
                try:
                    e8["vs_hipblaslt"] = fp8_comparator(w8, plan8, h8, torch, imm)
                    sec8["hipblaslt_TFLOPs"] = round(e8["vs_hipblaslt"]["hipblaslt"]["TFLOPs"], 1)
                    sec8["ours_alternating_TFLOPs"] = round(e8["vs_hipblaslt"]["ours"]["TFLOPs"], 1)
                except Exception as e:  # comparator only
                    e8["hipblaslt_error"] = str(e)
            extra[f"square_e5m2_{n8}"] = e8
            secondary["fp8_e5m2_bf16_out"][str(n8)] = sec8
            samples.append((w8, h8[0], h8[1], med8, {4096: 2.0, 8192: 2.0, 16384: 2.0}[n8]))
            del h8
            torch.cuda.empty_cache()
        for n in ("square_f16_4096", "square_f16_1024"):
            # the default plan and GEMM_PLAN_TILE_BY_M in alternating rounds, so
            # that the part's clock (which follows its recent power draw) treats
            # both alike; each reports its best round's median
            wn, _, pn, _, hn = bench_square(n, 30, 10, torch, imm, wl, queue_ahead=True)
            pd = imm.gemm_plan(wn.M, wn.N, wn.K, wn.dtype)
            mp = imm.gemm_plan_ex2(wn.M, wn.N, wn.K, wn.dtype, wn.out, flags=imm.PLAN_TILE_BY_M)
            Cn = torch.empty((wn.M, wn.N), dtype=torch.float32, device="cuda")
            rounds = {"default": [statistics.median(pn)], "tile_by_m": []}
            for r in range(3):
                for key, pl in (("tile_by_m", mp), ("default", pd)):
                    pr, _ = time_launches(lambda i: imm.gemm_run(pl, hn[2], hn[3], Cn), 30, 5, torch,
                                          queue_ahead=True)
                    rounds[key].append(statistics.median(pr))
                    if key == "default":
                        pn = pr if statistics.median(pr) < statistics.median(pn) else pn
            medn = min(rounds["default"])
            extra[n] = {**summary(pn), "TFLOPs": wn.flops / (medn * 1e-3) / 1e12,
                        "tile": f"{pd.info['run_block_m']}x{pd.info['run_block_n']}",
                        "tile_by_m": f"{mp.info['run_block_m']}x{mp.info['run_block_n']}",
                        "tile_by_m_TFLOPs": wn.flops / (min(rounds["tile_by_m"]) * 1e-3) / 1e12,
                        "round_medians_ms": {k: [round(x, 4) for x in v] for k, v in rounds.items()}}
            secondary[f"fp16_{wn.M}_TFLOPs"] = round(extra[n]["TFLOPs"], 1)
            samples.append((wn, hn[0], hn[1], medn, {4096: 2.0, 1024: 1.0}[wn.M]))
            del hn, Cn
            torch.cuda.empty_cache()
        log("HBM probes (streaming reads, 1 GiB device copy)")
        probes = bench_hbm_probes(torch)
        extra["hbm_probes"] = probes
        secondary["hbm_read_probe_GBps"] = {"1GiB": round(probes["read_1GiB"]["GBps"]),
                                            "decode_B_rotated": round(probes["read_decode_B"]["GBps"])}
        log("decode bf16 N=4096 K=14336, split-K path")
        wd = wl.WORKLOADS["decode_bf16_m128"]
        Adec, Bdec = wd.make()
        extra["decode_bf16"] = [bench_splitk("decode_bf16_m128", 0, torch, imm, wl, M=m)
                                for m in (1, 8, 32, 128)]
        secondary["decode_bf16_N4096_K14336"] = []
        for d in extra["decode_bf16"]:
            d["pct_of_read_probe"] = 100.0 * d["GBps"] / probes["read_decode_B"]["GBps"]
            d["pct_of_copy_probe"] = 100.0 * d["GBps"] / probes["copy_1GiB_GBps"]
            secondary["decode_bf16_N4096_K14336"].append(
                {"M": d["M"], "split": d["split_k"], "us": round(d["median_ms"] * 1e3, 2),
                 "GBps": round(d["GBps"]), "pct_hbm_peak": round(d["pct_hbm_peak"], 1),
                 "pct_read_probe": round(d["pct_of_read_probe"], 1)})
            wm = wl.WORKLOADS[f"decode_bf16_m{d['M']}"]
            samples.append((wm, Adec[:d["M"]].contiguous(), Bdec, d["median_ms"], 2.0))
        torch.cuda.empty_cache()
        log("M sweep on the fused-QKV projection shape N=6144 K=4096, gemm_run")
        extra["qkv_m_sweep_f16"] = bench_m_sweep(torch, imm, wl)
        secondary["qkv_f16_N6144_K4096_us"] = [
            {"M": x["M"], "default": round(x["median_us"], 1),
             "tile_by_m": round(x["tile_by_m_median_us"], 1),
             "torch": round(x["torch_matmul_median_us"], 1),
             "w_nk_tile_by_m": round(x["weight_nk_tile_by_m_median_us"], 1),
             "torch_linear": round(x["torch_linear_median_us"], 1)} for x in extra["qkv_m_sweep_f16"]]
        torch.cuda.empty_cache()
        log("huge-K fp16 256x256x131072, split-K path")
        # split 0 = the plan's default for this shape
        extra["hugek_f16"] = [bench_splitk("hugek_f16", s, torch, imm, wl) for s in (1, 8, 32, 128, 0)]
        secondary["hugek_f16_256x256x131072"] = [
            {"split": x["split_k"], "default": i == 4, "us": round(x["median_ms"] * 1e3, 1),
             "GBps": round(x["GBps"]), "pct_hbm_peak": round(x["pct_hbm_peak"], 1)}
            for i, x in enumerate(extra["hugek_f16"])]
        wh = wl.WORKLOADS["hugek_f16"]
        Ah, Bh = wh.make()
        samples.append((wh, Ah, Bh, extra["hugek_f16"][-1]["median_ms"], 2.0))
        torch.cuda.empty_cache()
        log("fp64 by the Ozaki scheme (bf16, e4m3 and int8 slices)")
        extra["ozaki_f64"] = [bench_ozaki(f"ozaki_{t2}_{n}", torch, imm, wl)
                              for t2 in ("bf16", "e4m3", "i8") for n in (4096, 8192, 16384)]
        secondary["ozaki_f64_TFLOPs"] = {f"{x['type2']}_{x['n']}": round(x["fp64_TFLOPs"], 1)
                                         for x in extra["ozaki_f64"]}
        log("Ozaki Fast Mode d sweep at 8192")
        extra["ozaki_d_sweep"] = bench_ozaki_d_sweep(torch, imm, wl)
    else:
        samples.append((w, A, B, statistics.median(per), 6.0))

    cpu = None
    if not args.no_cpu:
        log("cpu baseline (oracle)")
        cpu = cpu_baseline(samples)

    line = {
        "metric": "GEMM TFLOPS & % MFMA peak (8192^3 fp16, fp8); GB/s at M<=32; batch-invariance",
        "value": value, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f16",
        "data": "synthetic (seeded uniform[-1,1) fp16, resident in HBM)",
        "config": {"workload": "square fp16 GEMM M=N=K=8192, fp32 accumulate, fp32 output, "
                               "gemm_run (no split-K)",
                   "M": w.M, "N": w.N, "K": w.K, "pct_mfma_peak": 100 * value / PEAK_TFLOPS["f16"],
                   "secondary": secondary},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
