"""bench.py's contract that runs without a GPU: more than one GPU is refused
with a message before anything touches a device, unknown workloads are
refused, and the workloads' algorithmic byte counts are the documented
formulas at the documented sizes."""
import os
import subprocess
import sys

from kv_insert_amd import workloads as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


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
