"""bench.py's contract that runs without a GPU: more than one GPU is refused
with a message before anything touches a device, unknown workloads are
refused, the workloads' algorithmic byte counts are the documented
formulas at the documented sizes, counter traffic is reported only for
the kernel source it was measured on, and the committed counter records add
up."""
import json
import os
import subprocess
import sys

import pytest

from kv_insert_amd import workloads as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def run_bench(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=120, cwd=ROOT)


def test_more_than_one_gpu_is_refused():
    r = run_bench("--gpus", "2")
    assert r.returncode == 2
    assert "exactly one GPU" in r.stderr
    assert r.stdout == ""


def test_front_algorithmic_bytes():
    assert wl.C1.algorithmic_bytes() == 18_893_584
    assert wl.C2.algorithmic_bytes() == 37_922_944
    assert wl.C3.algorithmic_bytes() == 151_292_032
    assert wl.C4.algorithmic_bytes() == 151_589_120


def test_attn2_algorithmic_bytes():
    # one request of 32768 keys, 8 KV heads: every K|V slot once per head,
    # q + gate + out rows, the 2048 block-table entries and seq_lens
    a = wl.A1
    kv = 32768 * 8 * 256
    rows = 3 * 8 * 512 * 8 * 2
    assert a.algorithmic_bytes() == kv + rows + 4 * 2048 + 4
    # a window reads only the union of the rows' windows
    w = wl.Attn2Workload("w", nkv=1, max_model_len=8192, lens=(1000,), window=100)
    lo = 1000 - 8 - 100 + 1
    assert w.algorithmic_bytes() == (1000 - lo) * 256 + 3 * 8 * 512 * 2 + 4 * (63 - lo // 16) + 4


def test_layer_front_and_route_bytes():
    assert wl.LF1.algorithmic_bytes() == 16 * 8192 * (2 + 8 + 2) + 2 * 8192
    assert wl.LF2.algorithmic_bytes() == 8 * 8192 * (4 + 4 + 2) + 2 * 8192
    assert wl.RT1.algorithmic_bytes() == 8 * 256 * 4 + 256 * 4 + 2 * 8 * 8 * 4


def test_traffic_is_reported_only_for_the_kernel_it_was_measured_on(tmp_path):
    """bench.py reports a counter record's HBM bytes only while the kernel
    source still has the hash the record was taken on."""
    src = tmp_path / "kernel.hip"
    src.write_text("// kernel v1\n")
    rec = tmp_path / "counters.json"
    w = wl.C3
    rec.write_text(json.dumps({"kernel_sha256_16": bench.kernel_hash(str(src)),
                               "workloads": {w.name: {"hbm_bytes_per_launch": 123}}}))
    assert bench.measured_traffic(w, str(rec), str(src)) == 123
    assert bench.measured_traffic(wl.C4, str(rec), str(src)) is None      # no entry
    src.write_text("// kernel v2\n")
    assert bench.measured_traffic(w, str(rec), str(src)) is None          # source changed
    assert bench.measured_traffic(w, str(tmp_path / "missing.json"), str(src)) is None


def test_committed_counter_records_have_their_fields():
    """Each record in profiles/ names the hash it was taken on and gives HBM
    bytes per call for workloads bench.py knows."""
    for path, table in ((bench.COUNTERS, wl.WORKLOADS), (bench.ATTN2_COUNTERS, wl.ATTN2_WORKLOADS),
                        (bench.LF_COUNTERS, wl.LAYER_FRONT_WORKLOADS)):
        rec = json.load(open(path))
        assert len(rec["kernel_sha256_16"]) == 16
        assert rec["workloads"]
        for name, entry in rec["workloads"].items():
            assert name in table or (table is wl.WORKLOADS and name.startswith("sweep_m"))
            w = bench.workload_by_name(name) if table is wl.WORKLOADS else table[name]
            b = entry.get("hbm_bytes_per_launch", entry.get("hbm_bytes_per_call"))
            if b is None:   # a workload with a kernel trace only
                assert table is wl.ATTN2_WORKLOADS and "trace_split_avg_us" in entry
                continue
            assert b > w.algorithmic_bytes() * 0.9


def test_committed_counter_records_add_up():
    """Each record's HBM bytes are its own counter readings (KiB per
    dispatch) scaled by its copy calibration: FETCH_SIZE x fetch factor +
    WRITE_SIZE x write factor, summed over the call's kernels."""
    for path in (bench.COUNTERS, bench.LF_COUNTERS):
        rec = json.load(open(path))
        cal = rec["calibration"]
        assert cal["fetch_factor"] == pytest.approx(
            cal["copy_bytes_read"] / 1024 / cal["copy_FETCH_SIZE_KiB"], rel=1e-4)
        assert cal["write_factor"] == pytest.approx(
            cal["copy_bytes_written"] / 1024 / cal["copy_WRITE_SIZE_KiB"], rel=1e-4)
        for entry in rec["workloads"].values():
            b = entry.get("hbm_bytes_per_launch", entry.get("hbm_bytes_per_call"))
            expect = 1024 * (entry["FETCH_SIZE_KiB"] * cal["fetch_factor"]
                             + entry["WRITE_SIZE_KiB"] * cal["write_factor"])
            assert b == pytest.approx(expect, rel=1e-5)   # the factors are stored to 5 places
    rec = json.load(open(bench.ATTN2_COUNTERS))
    for entry in rec["workloads"].values():
        if "split_fetch_kib" not in entry:
            continue
        expect = 1024 * ((entry["split_fetch_kib"] + entry["merge_fetch_kib"]) * rec["fetch_scale"]
                         + (entry["split_write_kib"] + entry["merge_write_kib"]) * rec["write_scale"])
        assert entry["hbm_bytes_per_call"] == pytest.approx(expect, rel=1e-5)


def test_cpu_baseline_reports_all_cores_and_one_core(monkeypatch):
    """The oracle is timed on the host's cores and on one core, each on full
    calls of the workload, with the sample stated: every core the process may
    run on, unless OMP_NUM_THREADS sets a smaller share."""
    monkeypatch.delenv("OMP_NUM_THREADS", raising=False)
    r = bench.cpu_baseline(wl.C1, 0.5)
    host = len(os.sched_getaffinity(0))
    assert r["kind"] == "oracle" and r["cores"] == host and r["host_cores"] == host
    assert r["us_per_call"] > 0 and f"{host} cores" in r["sample"]
    one = r["single_core"]
    assert one["cores"] == 1 and one["us_per_call"] > 0 and "1 thread" in one["sample"]
    assert r["value"] > 0 and one["value"] > 0
    monkeypatch.setenv("OMP_NUM_THREADS", "2")
    assert bench.host_threads() == (min(2, host), host)


def _write_csv(path, header, rows):
    import csv
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as fh:
        w = csv.writer(fh, quoting=csv.QUOTE_NONNUMERIC)
        w.writerow(header)
        w.writerows(rows)


def test_profile_summary_splits_dispatches_by_workload(tmp_path):
    """The summary attributes a profiled run's dispatches to workloads in
    the announced order, drops each workload's warmup, takes medians of the
    counters and scales them by the copy calibration."""
    d = tmp_path
    order = [{"profile_workload": "m8_nkv8_n9216", "M": 8, "num_kv_heads": 8, "N": 9216,
              "front_dispatches": 4, "warmup": 1, "algorithmic_bytes": 151_292_032},
             {"profile_workload": "m1_nkv1_n1152", "M": 1, "num_kv_heads": 1, "N": 1152,
              "front_dispatches": 3, "warmup": 1, "algorithmic_bytes": 18_893_584}]
    (d / "order.jsonl").write_text("noise\n" + "\n".join(json.dumps(o) for o in order) + "\n")
    k8 = "_ZN4qkvf12_GLOBAL__N_111front_fusedILi8EEEvPKDF16b"
    k1 = "_ZN4qkvf12_GLOBAL__N_111front_fusedILi1EEEvPKDF16b"
    names = [k8] * 4 + [k1] * 3
    dur = [99.0, 25.0, 26.0, 27.0, 50.0, 8.0, 9.0]          # us; first of each is warmup
    trace = [["KERNEL_DISPATCH", 7 + i, names[i], 1000, 1000 + int(dur[i] * 1000)]
             for i in range(7)]
    trace.insert(2, ["KERNEL_DISPATCH", 8, "other_kernel", 0, 10])   # not the front
    trace[3][1] = 9
    for i, row in enumerate(trace):
        row[1] = i + 1
    _write_csv(str(d / "trace" / "run_kernel_trace.csv"),
               ["Kind", "Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp"], trace)
    fetch_kib = [1.0, 75000.0, 75010.0, 75020.0, 2.0, 9300.0, 9310.0]
    write_kib = [1.0, 1200.0, 1201.0, 1202.0, 2.0, 40.0, 41.0]
    for sub, cname, vals in (("fetch", "FETCH_SIZE", fetch_kib), ("write", "WRITE_SIZE", write_kib)):
        _write_csv(str(d / sub / "run_counter_collection.csv"),
                   ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"],
                   [[i + 1, names[i], cname, vals[i]] for i in range(7)])
    for sub, cname, v in (("calib_fetch", "FETCH_SIZE", 125000.0),
                          ("calib_write", "WRITE_SIZE", 250000.0)):
        _write_csv(str(d / sub / "run_counter_collection.csv"),
                   ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"],
                   [[1, "__amd_rocclr_copyBuffer", cname, v], [2, "__amd_rocclr_copyBuffer", cname, v]])
    (d / "calibration.json").write_text(json.dumps({"copy_bytes_read": 256_000_000,
                                                    "copy_bytes_written": 256_000_000}))
    (d / "all.jsonl").write_text(json.dumps({"workload": "m8_nkv8_n9216", "us_per_call": 25.5,
                                             "cpu_baseline": {"us_per_call": 1e5, "cores": 16,
                                                              "host_cores": 128}}) + "\n")
    out = tmp_path / "rec.json"
    table = bench.summarize_profiles(str(d), str(out))
    rec = json.load(open(out))
    e8, e1 = rec["workloads"]["m8_nkv8_n9216"], rec["workloads"]["m1_nkv1_n1152"]
    assert e8["trace_avg_us"] == pytest.approx(26.0) and e8["trace_dispatches"] == 3
    assert e1["trace_avg_us"] == pytest.approx(8.5) and e1["trace_min_us"] == pytest.approx(8.0)
    assert e8["FETCH_SIZE_KiB"] == 75010.0 and e1["WRITE_SIZE_KiB"] == 40.5
    ff = 256_000_000 / (125000.0 * 1024)
    assert e8["hbm_bytes_per_launch"] == round(1024 * (75010.0 * ff + 1201.0 * 256_000_000 /
                                                       (250000.0 * 1024)))
    assert "| m8_nkv8_n9216 | 8 | 8 | 9216 | 25.50 |" in table and "(16 / 128)" in table
    # a count that does not match the announcement is refused
    order[1]["front_dispatches"] = 4
    (d / "order.jsonl").write_text("\n".join(json.dumps(o) for o in order) + "\n")
    with pytest.raises(SystemExit):
        bench.summarize_profiles(str(d), str(out))


def test_attn2_profile_summary_drops_warmup_and_scales_counters(tmp_path, monkeypatch):
    """The attn2 summary takes each kernel's trace after the warm-up
    dispatches, the median split and merge counters, scaled by the copy
    calibration, and the --all event line of the workload."""
    d = tmp_path
    name = "attn2_r1_nkv8_L32768"
    monkeypatch.setattr(bench.qf, "attn2_plan", lambda *args: 32)
    split = "void qkvf::(anonymous namespace)::attn2_split<false>(bf16 const*)"
    merge = "void qkvf::(anonymous namespace)::attn2_merge<false, 32>(bf16 const*)"
    rows, t = [], 0
    for i in range(25):   # 20 warm-up calls, then 5 timed
        sd, md = (99.0, 9.0) if i < 20 else (20.0 + i - 20, 4.0)
        rows.append(["KERNEL_DISPATCH", 2 * i + 1, split, t, t + int(sd * 1000)])
        rows.append(["KERNEL_DISPATCH", 2 * i + 2, merge, t + 50_000, t + 50_000 + int(md * 1000)])
        t += 100_000
    base = d / "a2" / name
    _write_csv(str(base / "trace" / "run_kernel_trace.csv"),
               ["Kind", "Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp"], rows)
    for sub, cname, sv, mv in (("fetch", "FETCH_SIZE", 33000.0, 2400.0),
                               ("write", "WRITE_SIZE", 4352.0, 64.0)):
        _write_csv(str(base / sub / "run_counter_collection.csv"),
                   ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"],
                   [[1, split, cname, sv], [2, merge, cname, mv], [3, split, cname, sv + 2],
                    [4, merge, cname, mv], [5, split, cname, sv + 1], [6, merge, cname, mv]])
    for sub, cname, v in (("calib_fetch", "FETCH_SIZE", 125000.0),
                          ("calib_write", "WRITE_SIZE", 250000.0)):
        _write_csv(str(d / sub / "run_counter_collection.csv"),
                   ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"],
                   [[1, "__amd_rocclr_copyBuffer", cname, v]])
    (d / "calibration.json").write_text(json.dumps({"copy_bytes_read": 256_000_000,
                                                    "copy_bytes_written": 256_000_000}))
    (d / "all.jsonl").write_text(json.dumps({"workload": name, "us_per_call": 22.0,
                                             "cpu_baseline": {"us_per_call": 4e5, "cores": 16,
                                                              "host_cores": 16}}) + "\n")
    out = tmp_path / "a2.json"
    table = bench.summarize_attn2_profiles(str(d), str(out))
    e = json.load(open(out))["workloads"][name]
    assert e["trace_dispatches"] == 5 and e["trace_split_avg_us"] == pytest.approx(22.0)
    assert e["trace_split_min_us"] == pytest.approx(20.0) and e["trace_merge_avg_us"] == 4.0
    assert e["split_fetch_kib"] == 33001.0 and e["merge_write_kib"] == 64.0
    ff = 256_000_000 / (125000.0 * 1024)
    assert e["hbm_bytes_per_call"] == round(1024 * ((33001.0 + 2400.0) * ff + (4353.0 + 64.0)))
    assert f"| {name} | 32 | 22.00 | 22.00 (20.00 / 24.00) | 4.00 (4.00 / 4.00) |" in table
