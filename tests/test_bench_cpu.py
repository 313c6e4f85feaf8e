"""Host logic of bench.py, on the CPU: the --gpus contract and the two counter
summaries (HBM traffic, clock and matrix-unit occupancy) on synthetic
rocprofv3 CSV files of known content."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

COUNTER_FIELDS = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value",
                  "Start_Timestamp", "End_Timestamp"]
HEADLINE = "void imm::(anonymous namespace)::gemm_dma_kernel<0, 4, 0, 256, 256, 2, 4, 2, false, imm::GemmArgs>(imm::GemmArgs)"
BLAS = "Cijk_Ailk_Bljk_HHS_BH_MT256x256x64_MI16x16x1"
COPY = "__amd_rocclr_copyBuffer"


def write_counters(path, dispatches):
    """dispatches: list of (id, kernel, start_ns, end_ns, {counter: value})."""
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=COUNTER_FIELDS)
        w.writeheader()
        for did, name, t0, t1, counters in dispatches:
            for c, v in counters.items():
                w.writerow({"Dispatch_Id": did, "Kernel_Name": name, "Counter_Name": c,
                            "Counter_Value": v, "Start_Timestamp": t0, "End_Timestamp": t1})


def write_agent(path, xcc=8, simds=1024, cus=256, mhz=2400):
    fields = ["Agent_Type", "Num_Xcc", "Simd_Count", "Cu_Count", "Max_Engine_Clk_Fcompute"]
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=fields)
        w.writeheader()
        w.writerow({"Agent_Type": "CPU", "Num_Xcc": 0, "Simd_Count": 0, "Cu_Count": 0,
                    "Max_Engine_Clk_Fcompute": 0})
        w.writerow({"Agent_Type": "GPU", "Num_Xcc": xcc, "Simd_Count": simds, "Cu_Count": cus,
                    "Max_Engine_Clk_Fcompute": mhz})


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_traffic_scales_each_counter_by_the_copy(tmp_path):
    copy_kib = bench.COPY_BYTES / 1024
    fetch, write = tmp_path / "fetch.csv", tmp_path / "write.csv"
    # FETCH_SIZE reads half a copy's bytes, WRITE_SIZE all of them
    write_counters(fetch, [(1, COPY, 0, 10, {"FETCH_SIZE": copy_kib / 2}),
                           (2, HEADLINE, 20, 30, {"FETCH_SIZE": 1000.0}),
                           (3, HEADLINE, 40, 50, {"FETCH_SIZE": 3000.0})])
    write_counters(write, [(1, COPY, 0, 10, {"WRITE_SIZE": copy_kib}),
                           (2, HEADLINE, 20, 30, {"WRITE_SIZE": 500.0})])
    out = tmp_path / "traffic.json"
    bench.write_traffic(str(fetch), str(write), out_path=str(out))
    t = json.loads(out.read_text())
    assert t["fetch_scale"] == pytest.approx(2.0)
    assert t["write_scale"] == pytest.approx(1.0)
    assert t["launches"] == 2
    assert t["read_bytes_per_launch"] == pytest.approx(2000.0 * 2 * 1024)
    assert t["write_bytes_per_launch"] == pytest.approx(500.0 * 1024)
    assert t["bytes_per_launch"] == pytest.approx((4000.0 + 500.0) * 1024)
    assert t["kernel_source_hash"] == bench.kernel_source_hash()


def test_traffic_without_the_copy_is_an_error(tmp_path):
    fetch = tmp_path / "fetch.csv"
    write_counters(fetch, [(2, HEADLINE, 20, 30, {"FETCH_SIZE": 1000.0})])
    with pytest.raises(SystemExit):
        bench.write_traffic(str(fetch), str(fetch), out_path=str(tmp_path / "t.json"))


def test_clock_cycles_occupancy_lds_and_l2(tmp_path):
    agent, counters, lds = tmp_path / "agent.csv", tmp_path / "c.csv", tmp_path / "lds.csv"
    write_agent(agent)
    cyc = 1.5e6                      # per XCD
    ns = 1.0e6                       # 1 ms: 1.5 GHz
    busy = 0.75 * cyc * 1024         # matrix units busy 75 % of the SIMD-cycles
    head = {"GRBM_GUI_ACTIVE": 8 * cyc, "SQ_VALU_MFMA_BUSY_CYCLES": busy,
            "SQ_INSTS_VALU_MFMA_MOPS_F16": 2.0 ** 40 / 512, "SQ_INSTS_MFMA": 2.0 ** 26}
    write_counters(counters, [
        (1, COPY, 0, 400_000, {"GRBM_GUI_ACTIVE": 8 * 0.96e6}),                 # 2.4 GHz
        (2, HEADLINE, 1_000_000, 1_000_000 + int(ns), head),
        (3, HEADLINE, 3_000_000, 3_000_000 + int(2 * ns), dict(head)),          # same cycles, half clock
        (4, BLAS, 6_000_000, 6_000_000 + int(ns), {"GRBM_GUI_ACTIVE": 8 * 1.6e6,
                                                   "SQ_VALU_MFMA_BUSY_CYCLES": 0.5 * 1.6e6 * 1024}),
        (5, "some_other_kernel", 0, 10, {"GRBM_GUI_ACTIVE": 5.0})])
    write_counters(lds, [(7, HEADLINE, 0, int(ns), {"GRBM_GUI_ACTIVE": 8 * cyc,
                                                     "SQ_LDS_BANK_CONFLICT": 0.0,
                                                     "SQ_LDS_IDX_ACTIVE": 0.25 * cyc * 256,
                                                     "SQ_INSTS_LDS": 123.0,
                                                     "TCC_HIT_sum": 78.0, "TCC_MISS_sum": 22.0})])
    out = tmp_path / "clock.json"
    bench.write_clock(str(counters), str(agent), str(lds), out_path=str(out))
    c = json.loads(out.read_text())
    h = c["headline"]
    assert h["dispatches"] == 2
    assert h["mean_cycles"] == pytest.approx(cyc)
    assert h["min_clock_ghz"] == pytest.approx(0.75)
    assert h["max_clock_ghz"] == pytest.approx(1.5)
    assert h["mfma_busy_frac"] == pytest.approx(0.75)
    assert h["mfma_tflop_per_launch"] == pytest.approx(2.0 ** 40 / 1e12)
    assert h["lds_active_per_cu_cycle"] == pytest.approx(0.25)
    assert h["lds_bank_conflict_per_cu_cycle"] == 0.0
    assert h["l2_hit_rate"] == pytest.approx(0.78)
    assert c["copy"]["mean_clock_ghz"] == pytest.approx(2.4)
    assert c["hipblaslt"]["mfma_busy_frac"] == pytest.approx(0.5)
    assert "some_other_kernel" not in json.dumps(c)
    assert c["max_engine_clock_ghz"] == pytest.approx(2.4)
    assert c["kernel_source_hash"] == bench.kernel_source_hash()


def test_clock_without_the_headline_kernel_is_an_error(tmp_path):
    agent, counters = tmp_path / "agent.csv", tmp_path / "c.csv"
    write_agent(agent)
    write_counters(counters, [(1, COPY, 0, 400_000, {"GRBM_GUI_ACTIVE": 8 * 0.96e6})])
    with pytest.raises(SystemExit):
        bench.write_clock(str(counters), str(agent), out_path=str(tmp_path / "x.json"))


PARTIAL = "void imm::(anonymous namespace)::gemm_tile_kernel<1, 4, 32, 128, 1, 4, true>(imm::GemmArgs)"
REDUCE = "void imm::(anonymous namespace)::splitk_reduce_kernel<4>(imm::ReduceArgs)"
HK_PARTIAL = "void imm::(anonymous namespace)::gemm_dma_kernel<0, 4, 1, 128, 256, 2, 4, 3, false, imm::GemmArgs>(imm::GemmArgs)"


def _stream_dispatches(counter, copy_value, per_case):
    """Calibration copies, a clone of another size, then each case's launches
    (partial, reduction) with the values per_case(case_index, kind)."""
    d, did = [], 1
    for _ in range(3):
        d.append((did, COPY, 0, 10, {counter: copy_value}))
        did += 1
    for ci, (_, _, launches) in enumerate(bench.STREAM_CASES):
        d.append((did, COPY, 0, 10, {counter: 12345.0}))  # input rotation clone
        did += 1
        for _ in range(launches):
            part = HK_PARTIAL if ci == len(bench.STREAM_CASES) - 1 else PARTIAL
            d.append((did, part, 0, 10, {counter: per_case(ci, "partial")}))
            d.append((did + 1, REDUCE, 0, 10, {counter: per_case(ci, "reduce")}))
            did += 2
    return d


def test_stream_traffic_per_case_and_kernel(tmp_path):
    copy_kib = bench.COPY_BYTES / 1024
    fetch, write = tmp_path / "fetch.csv", tmp_path / "write.csv"
    write_counters(fetch, _stream_dispatches("FETCH_SIZE", copy_kib / 2,
                                             lambda c, k: 1000.0 * (c + 1) + (5 if k == "reduce" else 0)))
    write_counters(write, _stream_dispatches("WRITE_SIZE", copy_kib,
                                             lambda c, k: 10.0 * (c + 1)))
    out = tmp_path / "s.json"
    bench.write_stream_traffic(str(fetch), str(write), out_path=str(out))
    t = json.loads(out.read_text())
    assert t["fetch_scale"] == pytest.approx(2.0) and t["write_scale"] == pytest.approx(1.0)
    assert [c["workload"] for c in t["cases"]] == [c[0] for c in bench.STREAM_CASES]
    for ci, c in enumerate(t["cases"]):
        p, r = c["partial"], c["reduce"]
        assert p["launches"] == r["launches"] == bench.STREAM_CASES[ci][2]
        assert p["read_bytes_per_launch"] == pytest.approx(2 * 1000.0 * (ci + 1) * 1024)
        assert r["read_bytes_per_launch"] == pytest.approx(2 * (1000.0 * (ci + 1) + 5) * 1024)
        assert p["write_bytes_per_launch"] == pytest.approx(10.0 * (ci + 1) * 1024)
        # algorithmic bytes: A and B once plus the slices; the slices plus C
        M, N, K, S = c["M"], c["N"], c["K"], c["split_k"]
        assert p["algorithmic_bytes"] == (M * K + K * N) * 2 + S * M * N * 4
        assert r["algorithmic_bytes"] == S * M * N * 4 + M * N * 4
    assert t["cases"][-1]["partial"]["kernel"] == HK_PARTIAL


def test_stream_traffic_rejects_a_missing_launch(tmp_path):
    copy_kib = bench.COPY_BYTES / 1024
    fetch, write = tmp_path / "fetch.csv", tmp_path / "write.csv"
    d = _stream_dispatches("FETCH_SIZE", copy_kib, lambda c, k: 1.0)
    write_counters(fetch, d[:-1])
    write_counters(write, _stream_dispatches("WRITE_SIZE", copy_kib, lambda c, k: 1.0))
    with pytest.raises(SystemExit):
        bench.write_stream_traffic(str(fetch), str(write), out_path=str(tmp_path / "x.json"))


def test_cpu_baseline_samples_every_workload():
    import workloads as wl
    small = wl.Workload("square_f16_8192", 96, 64, 128, "f16", "f32", 2002, "uniform", "run")
    exact = wl.WORKLOADS["exact256"]
    samples = [(small, *small.make(), 0.5, 0.2), (exact, *exact.make(), 0.01, 0.2)]
    cpu = bench.cpu_baseline(samples)
    assert cpu["kind"] == "oracle" and cpu["unit"] == "TFLOP/s" and cpu["cores"] >= 1
    names = [x["workload"] for x in cpu["per_config"]]
    assert names == ["square_f16_8192", "exact256", "exact256"]
    one_core = cpu["per_config"][2]
    assert one_core["threads"] == 1 and one_core["rows"] == 256 == one_core["of_rows"]
    for x in cpu["per_config"]:
        assert x["total_s"] > 0 and x["decode_B_s"] >= 0 and x["accumulate_s"] >= 0
        assert 1 <= x["rows"] <= x["of_rows"]
        assert x["full_product_s_est"] >= x["total_s"] - x["decode_B_s"] - 1e-9
        assert x["gpu_speedup_est"] > 0
    assert cpu["value"] == cpu["per_config"][0]["GFLOPs"] / 1e3


def test_trace_summary_skips_the_settle_launches(tmp_path):
    # 12 settle launches (1100 us), 2 warm-up (1000 us), 3 timed (800, 900, 1000 us),
    # then more headline launches of a later leg (700 us) and another kernel
    fields = ["Kernel_Name", "Start_Timestamp", "End_Timestamp", "Workgroup_Size_X",
              "Workgroup_Size_Y", "Workgroup_Size_Z", "Grid_Size_X", "Grid_Size_Y", "Grid_Size_Z"]
    durs = [1100] * 12 + [1000, 1000] + [800, 900, 1000] + [700] * 4
    rows, t = [], 0
    for d in durs:
        rows.append((HEADLINE, t, t + d * 1000, 512, 1024 * 512))
        t += d * 1000 + 5000
    rows.append((COPY, t, t + 50000, 256, 256 * 100))
    trace = tmp_path / "trace.csv"
    with open(trace, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=fields)
        w.writeheader()
        for name, t0, t1, wg, grid in rows:
            w.writerow({"Kernel_Name": name, "Start_Timestamp": t0, "End_Timestamp": t1,
                        "Workgroup_Size_X": wg, "Workgroup_Size_Y": 1, "Workgroup_Size_Z": 1,
                        "Grid_Size_X": grid, "Grid_Size_Y": 1, "Grid_Size_Z": 1})
    line = {"value": 1.0, "warmup": 2, "steps": 3, "roofline": {"avg_launch_ms": 0.9},
            "extra": {"settle": {"ms": 150.0, "headline_launches": 12}}}
    bj = tmp_path / "bench.json"
    bj.write_text(json.dumps(line) + "\n")
    out = tmp_path / "summary.md"
    bench.write_trace_summary(str(trace), str(bj), out_path=str(out))
    text = out.read_text()
    assert "After its 12 untimed settle launches, the next 5 (2 warm-up + 3 timed)" in text
    assert "the timed 3 average 900.0 us, median 900.0 us, min 800.0 us, max 1000.0 us" in text
    assert f"{len(durs)} dispatches in the whole run" in text
