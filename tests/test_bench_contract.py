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
            assert name in table
            b = entry.get("hbm_bytes_per_launch", entry.get("hbm_bytes_per_call"))
            assert b > table[name].algorithmic_bytes() * 0.9


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
            assert b == pytest.approx(expect, abs=1.0)
    rec = json.load(open(bench.ATTN2_COUNTERS))
    for entry in rec["workloads"].values():
        expect = 1024 * ((entry["split_fetch_kib"] + entry["merge_fetch_kib"]) * rec["fetch_scale"]
                         + (entry["split_write_kib"] + entry["merge_write_kib"]) * rec["write_scale"])
        assert entry["hbm_bytes_per_call"] == pytest.approx(expect, abs=1.0)


def test_cpu_baseline_reports_all_cores_and_one_core():
    """The oracle is timed on the host's cores and on one core, each on full
    calls of the workload, with the sample stated."""
    import bench
    from kv_insert_amd import workloads as wl
    r = bench.cpu_baseline(wl.C1, 0.5)
    assert r["kind"] == "oracle" and r["cores"] >= 1 and r["us_per_call"] > 0
    one = r["single_core"]
    assert one["cores"] == 1 and one["us_per_call"] > 0 and "1 thread" in one["sample"]
    assert r["value"] > 0 and one["value"] > 0
