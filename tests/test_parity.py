"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Every case compares every output element (tolerance |gpu - oracle| <=
1.6e-2 |oracle| + 2e-3 with the tie-aware rule of oracle.checker) and the
whole cache bit for bit (untouched slots keep their bits; written slots hold
the result row's k | v columns)."""
import numpy as np
import pytest
import torch

import kv_insert_amd as qf
from kv_insert_amd import workloads as wl
from oracle import checker

from helpers import CANARY, Case, check, run_gpu, say, to_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    qf.lib()  # raises if the library is not built: there is no other path
    yield
    torch.cuda.synchronize()


@pytest.mark.parametrize("w", [wl.C1, wl.C2, wl.C3, wl.C4], ids=lambda w: w.name)
def test_workload_parity_full_size(w):
    case = Case(w)
    g = run_gpu(case)
    rep = check(case, g)
    print(rep)


_W_BY_NKV = {}


def _sweep_weights(nkv):
    if nkv not in _W_BY_NKV:
        _W_BY_NKV.clear()
        _W_BY_NKV[nkv] = wl.make_weights(wl.sweep(16, nkv), 0)
    return _W_BY_NKV[nkv]


# nkv is the inner parameter, so consecutive cases share one weight set.
@pytest.mark.parametrize("M", wl.SWEEP_M)
@pytest.mark.parametrize("nkv", wl.SWEEP_NKV)
def test_sweep_parity(nkv, M):
    w = wl.sweep(M, nkv)
    case = Case(w, W=_sweep_weights(nkv))
    g = run_gpu(case)
    check(case, g)


@pytest.mark.parametrize("M", [6, 7, 9, 10, 11, 13, 14, 15])
@pytest.mark.parametrize("nkv", [1, 2])
def test_balanced_rows_other_token_counts(nkv, M):
    """The row counts the sweep skips, with 1 and 2 KV heads: balanced rows
    per XCD, whose v and gate readers take runs of columns that end inside a
    head; odd M leaves half a reader wave idle; 2 KV heads switch from 4 to
    8 K splits (and x ahead of the weights) between 11 and 12 rows."""
    w = wl.sweep(M, nkv)
    case = Case(w, W=_sweep_weights(nkv))
    g = run_gpu(case)
    check(case, g)


@pytest.mark.parametrize("M", [6, 11, 13, 15])
@pytest.mark.parametrize("nkv", [4, 8])
def test_whole_heads_other_token_counts(nkv, M):
    """The row counts the sweep skips, with 4 and 8 KV heads (whole heads
    per XCD, 16-row tiles): odd M leaves half a reader wave idle, and x
    moves ahead of the weights between 11 and 12 rows."""
    w = wl.sweep(M, nkv)
    case = Case(w, W=_sweep_weights(nkv))
    g = run_gpu(case)
    check(case, g)


@pytest.mark.parametrize("nkv", [1, 8])
def test_edge_positions_and_slots(nkv):
    """First and last table rows, first and last cache slots, page edges."""
    w = wl.sweep(16, nkv)
    case = Case(w)
    last = w.pages * wl.PAGE_SLOTS - 1
    case.positions = torch.tensor([0, 1, w.table_rows - 1, 2, 4095, 4096, 131070, 77,
                                   5, 6, 7, 8, 9, 10, 11, 12], dtype=torch.int64)
    case.slots = torch.tensor([0, 15, 16, last, last - 1, 31, 32, 1000, 1001, 1002, 47,
                               48, 63, 64, 999, 2047], dtype=torch.int64)
    g = run_gpu(case, label=f"edge nkv={nkv}")
    check(case, g)


def test_negative_slot_writes_no_cache_entry():
    case = Case(wl.C2)
    case.slots = case.slots.clone()
    case.slots[3] = -1
    case.slots[7] = -5
    g = run_gpu(case, label="negative slots")
    check(case, g)


def test_layer_without_rope_only_norms():
    case = Case(wl.C2, rope=False)
    g = run_gpu(case, label="no rope")
    check(case, g)


def test_zero_token_rows_give_zero_heads():
    case = Case(wl.C4)
    case.x = case.x.clone()
    case.x[2] = 0
    case.x[9] = 0
    g = run_gpu(case, label="zero rows")
    check(case, g)
    y = g["y"].float().cpu()
    assert torch.all(y[2] == 0) and torch.all(y[9] == 0)
    assert torch.isfinite(y).all()


def test_small_rows_where_eps_matters():
    """Rows scaled by 1e-2 down to 3e-5 put the heads' mean square near the
    norm's eps = 1e-6, the only place where eps changes the normed q and k
    heads (at unit scale it cannot be seen)."""
    case = Case(wl.C2)
    scales = torch.tensor([1e-3, 3e-4, 1e-4, 3e-5, 1.0, 1e-2, 3e-3, 1e-3])
    case.x = (case.x.float() * scales[:, None]).to(torch.bfloat16)
    g = run_gpu(case, label="small rows")
    check(case, g)


def test_exact_integer_inputs_are_bit_exact():
    """x, W in {-1, 0, 1}: every fp32 summation order is exact, so the
    projection (v and gate columns, V in the cache) must match bit for bit."""
    w = wl.sweep(8, 2)
    rng = np.random.default_rng(77)
    case = Case(w)
    case.x = torch.from_numpy(rng.choice([-1.0, 0, 0, 0, 1.0], size=(8, 8192)).astype(np.float32)).to(torch.bfloat16)
    case.W = torch.from_numpy(rng.choice([-1.0, 0, 0, 0, 1.0], size=(w.N, 8192)).astype(np.float32)).to(torch.bfloat16)
    g = run_gpu(case, label="exact integers")
    check(case, g)
    z = case.x.double() @ case.W.double().T
    qk = (8 * w.nkv + w.nkv) * 64
    y = g["y"].double().cpu()
    assert torch.equal(y[:, qk:], z[:, qk:].to(torch.bfloat16).double())


def test_exact_integer_rounding_is_nearest_even_with_ties():
    """x in {0, 1} and W rows of +-{0, 1} at half density: every fp32
    summation order is still exact, but |z| sits around 2048, where bf16's
    spacing is 8 below and 16 above, so most values round and one in eight
    or sixteen is an exact tie.  The v and gate columns must equal the
    exact sums rounded to nearest, ties to even, bit for bit."""
    w = wl.sweep(8, 2)
    rng = np.random.default_rng(78)
    case = Case(w)
    case.x = torch.from_numpy(rng.choice([0.0, 1.0], size=(8, 8192)).astype(np.float32)).to(torch.bfloat16)
    sign = rng.choice([-1.0, 1.0], size=(w.N, 1))
    case.W = torch.from_numpy((rng.choice([0.0, 1.0], size=(w.N, 8192)) * sign).astype(np.float32)).to(torch.bfloat16)
    z = case.x.double() @ case.W.double().T
    qk = (8 * w.nkv + w.nkv) * 64
    zt = z[:, qk:]
    assert zt.abs().min() > 1024 and zt.abs().max() < 4096
    ties = ((zt.abs() - 1024) % 8 == 4) & (zt.abs() < 2048) | ((zt.abs() - 2048) % 16 == 8) & (zt.abs() >= 2048)
    assert int(ties.sum()) > 100
    g = run_gpu(case, label="integer rounding and ties")
    check(case, g)
    y = g["y"].double().cpu()
    assert torch.equal(y[:, qk:], zt.to(torch.bfloat16).double())


def test_rows_past_M_and_neighbours_untouched():
    w = wl.C4
    case = Case(w, M=5)
    g = case.device()
    big = torch.empty(16 + 2, w.N, dtype=torch.bfloat16, device="cuda")
    big.view(torch.int16).fill_(CANARY)
    g["y"] = big[1:1 + case.M]
    run_gpu(case, g, label="canary rows")
    check(case, g)
    rest = torch.cat([big[:1], big[1 + case.M:]]).view(torch.int16)
    assert torch.all(rest == CANARY)


def test_repeat_and_rotation_are_bitwise_deterministic():
    w = wl.C3
    c0 = Case(w, 0)
    c1 = Case(w, 1)
    g0 = run_gpu(c0, label="determinism set0 first")
    y_first = g0["y"].clone()
    cache_first = g0["kv_cache"].clone()
    run_gpu(c1, label="determinism set1")
    g0b = c0.device()
    run_gpu(c0, g0b, label="determinism set0 again")
    assert torch.equal(y_first.view(torch.int16), g0b["y"].view(torch.int16))
    assert torch.equal(cache_first.view(torch.int16), g0b["kv_cache"].view(torch.int16))
    # in place again on the same buffers
    qf.run(g0b["x"], g0b["W"], g0b["positions"], g0b["slots"], g0b["cos_sin"], g0b["y"],
           g0b["kv_cache"])
    torch.cuda.synchronize()
    assert torch.equal(y_first.view(torch.int16), g0b["y"].view(torch.int16))


def test_check_entry_on_device():
    case = Case(wl.C2)
    g = case.device()
    nkv = case.nkv
    say("qkvf_check")
    assert qf.check(g["x"], g["W"], g["positions"], g["slots"], g["cos_sin"], g["y"],
                    g["kv_cache"], nkv) == 0
    dup = g["slots"].clone()
    dup[1] = dup[0]
    assert qf.check(g["x"], g["W"], g["positions"], dup, g["cos_sin"], g["y"],
                    g["kv_cache"], nkv) == 9
    far = g["positions"].clone()
    far[0] = g["cos_sin"].shape[0]
    assert qf.check(g["x"], g["W"], far, g["slots"], g["cos_sin"], g["y"],
                    g["kv_cache"], nkv) == 9
    over = g["kv_cache"].view(-1)[: case.M * case.N].view(case.M, case.N)
    assert qf.check(g["x"], g["W"], g["positions"], g["slots"], g["cos_sin"], over,
                    g["kv_cache"], nkv) == 10
    host_x = case.x.clone()
    assert qf.check(host_x, g["W"], g["positions"], g["slots"], g["cos_sin"], g["y"],
                    g["kv_cache"], nkv) == 11
    assert qf.check(g["x"], g["W"], g["positions"], g["slots"], g["cos_sin"], g["y"],
                    g["kv_cache"], 4) == 2


def test_run_refuses_unprepared_row_count():
    torch.cuda.synchronize()
    qf.release()
    qf.prepare(1152, 1, 4)
    case = Case(wl.sweep(8, 1))
    g = case.device()
    with pytest.raises(qf.QkvfError) as e:
        qf.run(g["x"], g["W"], g["positions"], g["slots"], g["cos_sin"], g["y"], g["kv_cache"])
    assert e.value.code == "QKVF_ERR_NOT_PREPARED"
    qf.prepare(1152, 1, 16)
    run_gpu(case, g, label="after prepare")
    check(case, g)


def test_graph_capture_and_replays():
    """One call captured in a HIP graph and replayed with new inputs copied
    into its buffers, with eager calls and synchronizations in between; every
    replay matches the oracle (the per-call epoch keeps replays apart)."""
    w = wl.C2
    cases = [Case(w, s) for s in range(3)]
    g = cases[0].device()
    qf.prepare(w.N, w.nkv, w.M)
    say("graph capture")
    qf.run(g["x"], g["W"], g["positions"], g["slots"], g["cos_sin"], g["y"], g["kv_cache"])
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        qf.run(g["x"], g["W"], g["positions"], g["slots"], g["cos_sin"], g["y"], g["kv_cache"])
    other = Case(wl.sweep(4, 1))
    go = other.device()
    for rep in range(4):
        c = cases[rep % 3]
        for k in ("x", "W", "positions", "slots"):
            g[k].copy_(getattr(c, k).to("cuda"))
        g["kv_cache"].copy_(c.cache.to("cuda"))
        g["y"].view(torch.int16).fill_(CANARY)
        torch.cuda.synchronize()
        say(f"graph replay {rep}")
        graph.replay()
        torch.cuda.synchronize()
        assert qf.device_fault() == 0
        check(c, g)
        # eager work of another shape between replays
        run_gpu(other, go, label=f"eager between replays {rep}")
        check(other, go)
        qf.prepare(w.N, w.nkv, w.M)


@pytest.mark.parametrize("w", [wl.C2, wl.C3, wl.sweep(16, 1), wl.sweep(5, 2), wl.sweep(16, 4)],
                         ids=lambda w: w.name)
def test_write_through_handoff_is_bitwise_identical(w):
    """Both hand-off modes give the same bits (and match the oracle)."""
    case = Case(w)
    g0 = run_gpu(case, label=f"{w.name} default hand-off")
    y0, c0 = g0["y"].clone(), g0["kv_cache"].clone()
    try:
        qf.set_handoff(1)
        g1 = run_gpu(case, label=f"{w.name} write-through hand-off")
    finally:
        qf.set_handoff(0)
    check(case, g1)
    assert torch.equal(y0.view(torch.int16), g1["y"].view(torch.int16))
    assert torch.equal(c0.view(torch.int16), g1["kv_cache"].view(torch.int16))
