"""qkvf_run_static, the front's entry point that allocates nothing (its
partials pass through the library's static device array), against
qkvf_run on the same inputs: two calls in a row, the second with a smaller
input, each bit for bit equal to qkvf_run's result and within the oracle's
bar."""
import pytest
import torch

import kv_insert_amd as qf
from kv_insert_amd import workloads as wl

from helpers import Case, check, run_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    qf.lib()
    yield
    torch.cuda.synchronize()


def _static(case, g):
    qf.run_static(g["x"], g["W"], g["positions"], g["slots"], g["cos_sin"], g["y"],
                  g["kv_cache"], case.nkv, M=case.M)


@pytest.mark.parametrize("first,second", [
    (wl.sweep(16, 8), wl.sweep(3, 8)),      # fewer tokens
    (wl.C3, wl.C1),                         # fewer tokens and fewer KV heads
    (wl.sweep(16, 2), wl.C2),               # 2 KV heads: 8 K splits, then 4
], ids=["m16_then_m3", "c3_then_c1", "nkv2_m16_then_m8"])
def test_static_entry_matches_run_twice_in_a_row(first, second):
    a, b = Case(first), Case(second)
    ref_a = run_gpu(a, label=f"qkvf_run {first.name}")
    ref_b = run_gpu(b, label=f"qkvf_run {second.name}")
    ga, gb = a.device(), b.device()
    say(f"qkvf_run_static {first.name} then {second.name}")
    _static(a, ga)
    _static(b, gb)
    torch.cuda.synchronize()
    assert qf.device_fault() == 0
    for ref, g in ((ref_a, ga), (ref_b, gb)):
        assert torch.equal(g["y"].view(torch.int16), ref["y"].view(torch.int16))
        assert torch.equal(g["kv_cache"].view(torch.int16), ref["kv_cache"].view(torch.int16))
    check(a, ga)
    check(b, gb)


def test_static_entry_refuses_shapes_beyond_its_array():
    case = Case(wl.C2)
    g = case.device()
    with pytest.raises(qf.QkvfError) as e:
        qf.run_static(g["x"], g["W"], g["positions"], g["slots"], g["cos_sin"], g["y"],
                      g["kv_cache"], case.nkv, M=17)
    assert e.value.code == "QKVF_ERR_ROWS"
    with pytest.raises(qf.QkvfError) as e:
        qf.run_static(g["x"], g["W"], g["positions"], g["slots"], g["cos_sin"], g["y"],
                      g["kv_cache"], 16)
    assert e.value.code == "QKVF_ERR_SHAPE"
