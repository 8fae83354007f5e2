"""GPU tests of the front's hand-off between blocks: the fault word, the
fault state, a call that gives up, calls beside other work, and workspace
reuse across row counts.  Every failure here is forced from the host (the
fault word written by the host, or a spin limit of one polling round), so
every kernel exits normally."""
import ctypes

import numpy as np
import pytest
import torch

import kv_insert_amd as qf
from kv_insert_amd import workloads as wl

from helpers import CANARY, Case, check, run_gpu, say, to_bits

pytestmark = pytest.mark.gpu

H2D, D2H = 1, 2


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    qf.lib()
    yield
    qf.set_spin_limit(0)
    torch.cuda.synchronize()


def _hip():
    return ctypes.CDLL("libamdhip64.so")


def _write_word(addr: int, value: int) -> None:
    v = ctypes.c_uint(value)
    assert _hip().hipMemcpy(ctypes.c_void_p(addr), ctypes.byref(v), 4, H2D) == 0


def _read_word_on_stream(addr: int, stream) -> int:
    """Copy the word on `stream` and wait for that stream only."""
    host = torch.empty(1, dtype=torch.int32, pin_memory=True)
    hip = _hip()
    assert hip.hipMemcpyAsync(ctypes.c_void_p(host.data_ptr()), ctypes.c_void_p(addr), 4, D2H,
                              ctypes.c_void_p(stream.cuda_stream)) == 0
    assert hip.hipStreamSynchronize(ctypes.c_void_p(stream.cuda_stream)) == 0
    return int(host.item()) & 0xFFFFFFFF


def _call(case, g, stream=None):
    qf.prepare(case.N, case.nkv, case.M)
    qf.run(g["x"], g["W"], g["positions"], g["slots"], g["cos_sin"], g["y"], g["kv_cache"],
           M=case.M, stream=stream)


def test_fault_word_reads_zero_on_the_callers_stream():
    case = Case(wl.C2)
    g = case.device()
    s = torch.cuda.Stream()
    say("fault word on the caller's stream")
    with torch.cuda.stream(s):
        _call(case, g, s)
        _call(case, g, s)
    addr = qf.fault_word_address()
    assert _read_word_on_stream(addr, s) == 0
    torch.cuda.synchronize()
    check(case, g)


def test_fault_state_stores_nothing_until_cleared():
    """With the fault word set (here by the host), a call stores no y and no
    cache entry; qkvf_device_fault reports it, clears it and empties the
    workspace, and the next call is correct again."""
    case = Case(wl.C3)
    g = case.device()
    qf.prepare(case.N, case.nkv, case.M)
    assert qf.device_fault() == 0
    addr = qf.fault_word_address()
    _write_word(addr, 1)
    cache_before = g["kv_cache"].clone()
    say("call in the fault state")
    _call(case, g)
    torch.cuda.synchronize()
    assert torch.all(g["y"].view(torch.int16) == CANARY)
    assert torch.equal(g["kv_cache"].view(torch.int16), cache_before.view(torch.int16))
    assert qf.device_fault() == 12           # QKVF_ERR_TIMEOUT, now cleared
    assert qf.device_fault() == 0
    run_gpu(case, g, label="after clearing the fault")
    check(case, g)


@pytest.mark.parametrize("w", [wl.C3, wl.C1, wl.sweep(16, 2)], ids=lambda w: w.name)
def test_a_call_that_gives_up_stores_only_correct_values(w):
    """With one polling round allowed, readers that find a partial missing
    give up: they must store nothing, while the others store correct values.
    Every y element is then the canary or the correct value, every cache slot
    its old bits or the correct bits, and the fault is reported."""
    case = Case(w)
    good = run_gpu(case, label=f"{w.name} reference call")
    check(case, good)
    g = case.device()
    cache_before = g["kv_cache"].clone()
    try:
        qf.set_spin_limit(1)
        say(f"{w.name} with a spin limit of one round")
        _call(case, g)
        torch.cuda.synchronize()
    finally:
        qf.set_spin_limit(0)
    assert qf.device_fault() == 12, "no reader gave up: the test shows nothing"
    y = g["y"].view(torch.int16)
    ok_y = (y == CANARY) | (y == good["y"].view(torch.int16))
    assert bool(ok_y.all())
    untouched = int((y == CANARY).sum())
    assert untouched > 0
    c = g["kv_cache"].view(torch.int16)
    ok_c = (c == cache_before.view(torch.int16)) | (c == good["kv_cache"].view(torch.int16))
    assert bool(ok_c.all())
    print(f"{untouched} of {y.numel()} y values not stored")
    # the workspace is usable again after the report
    g2 = case.device()
    run_gpu(case, g2, label=f"{w.name} after the fault")
    assert torch.equal(g2["y"].view(torch.int16), good["y"].view(torch.int16))


def test_front_beside_a_large_copy_on_another_stream():
    """Calls on one stream while a copy of several GB runs on another stream
    of the same priority: the copy holds CUs, so some of the front's blocks
    start late; the others wait for them and the result is unchanged."""
    case = Case(wl.C3)
    ref = run_gpu(case, label="C3 alone")
    check(case, ref)
    n = (3 << 30) // 2
    src = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    other = torch.cuda.Stream()
    mine = torch.cuda.Stream()
    g = case.device()
    torch.cuda.synchronize()
    say("C3 beside a 3 GB copy")
    with torch.cuda.stream(other):
        for _ in range(3):
            dst.copy_(src)
    with torch.cuda.stream(mine):
        for _ in range(20):
            _call(case, g, mine)
    torch.cuda.synchronize()
    assert qf.device_fault() == 0
    assert torch.equal(g["y"].view(torch.int16), ref["y"].view(torch.int16))
    assert torch.equal(g["kv_cache"].view(torch.int16), ref["kv_cache"].view(torch.int16))
    del src, dst
    torch.cuda.empty_cache()


@pytest.mark.parametrize("nkv, rows", [(8, [16, 1, 7, 16, 3, 16]),
                                       (2, [16, 1, 11, 12, 7, 16, 3])],
                         ids=["nkv8", "nkv2_split_switch"])
def test_alternating_row_counts_leave_no_stale_partials(nkv, rows):
    """Row counts one after another on one stream: each uses its own
    positions in the workspace (with 2 KV heads also its own split count, 4
    below 12 rows and 8 from 12), so a partial left full by one call would
    be taken by a later one.  Every call must equal the same call made
    alone."""
    w = wl.sweep(16, nkv)
    W = wl.make_weights(w, 0)
    cases = {m: Case(w, M=m, W=W) for m in set(rows)}
    alone = {}
    for m, c in cases.items():
        alone[m] = run_gpu(c, label=f"alone M={m}")["y"].clone()
    qf.prepare(w.N, w.nkv, 16)
    outs = []
    say("alternating row counts")
    for m in rows:
        c = cases[m]
        g = c.device()
        qf.run(g["x"], g["W"], g["positions"], g["slots"], g["cos_sin"], g["y"], g["kv_cache"],
               M=m)
        outs.append((m, g))
    torch.cuda.synchronize()
    assert qf.device_fault() == 0
    for m, g in outs:
        assert torch.equal(g["y"].view(torch.int16), alone[m].view(torch.int16)), m
    check(cases[outs[-1][0]], outs[-1][1])   # the last call against the oracle
