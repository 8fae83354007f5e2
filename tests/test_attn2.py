"""attn2 on the GPU through the C ABI, compared with the oracle on the same
inputs: the full-size workloads in the launch shape the benchmark times, a
sweep over KV heads, context lengths (page and chunk edges), split counts and
windows, the largest request count, needles at split boundaries, cache
entries that must not be read, strided views of the front's output, graph
replays and the front followed by attn2."""
from __future__ import annotations

import dataclasses

import numpy as np
import pytest
import torch

import kv_insert_amd as qf
from kv_insert_amd import workloads as wl
from oracle import checker

from helpers import CANARY, say, to_bits

pytestmark = pytest.mark.gpu

NAN_BITS = 0x7FC1


class Attn2Case:
    """Host inputs of one attn2 call."""

    def __init__(self, a: wl.Attn2Workload, set_index: int = 0):
        self.a = dataclasses.replace(a, sets=max(1, set_index + 1))
        self.nkv = a.nkv
        self.y = wl.make_attn2_y(a, set_index)
        self.cache = wl.make_attn2_cache(self.a)
        self.table = wl.make_attn2_table(self.a, set_index)
        self.lens = wl.make_attn2_lens(a)
        self.window = a.eff_window

    @property
    def R(self) -> int:
        return int(self.lens.shape[0])

    def views(self, y=None):
        return wl.attn2_views(self.y if y is None else y, self.nkv)

    def host_check(self, cache=None, table=None, lens=None) -> None:
        """Everything the kernel indexes is inside its buffer."""
        cache = self.cache if cache is None else cache
        table = self.table if table is None else table
        lens = self.lens if lens is None else lens
        assert cache.dtype == torch.bfloat16 and cache.is_contiguous()
        assert tuple(cache.shape[1:]) == (self.nkv, wl.PAGE_SLOTS, wl.SLOT_WIDTH)
        assert table.dtype == torch.int32 and table.shape[0] == lens.shape[0]
        assert lens.dtype == torch.int32
        for r in range(lens.shape[0]):
            L = int(lens[r])
            assert 8 <= L <= self.a.max_model_len
            need = (L + wl.PAGE_SLOTS - 1) // wl.PAGE_SLOTS
            assert need <= table.shape[1]
            used = table[r, :need]
            assert int(used.min()) >= 0 and int(used.max()) < cache.shape[0]

    def oracle_check(self, out_bits, y=None, cache=None, table=None, lens=None):
        q, g = self.views(self.y if y is None else y)
        return checker.check_attn2(
            out_bits, to_bits(q), to_bits(g), to_bits(self.cache if cache is None else cache),
            self.nkv, (self.table if table is None else table).numpy(),
            (self.lens if lens is None else lens).numpy(), self.window)


def new_out(rows: int, width: int, stride: int | None = None) -> torch.Tensor:
    stride = width if stride is None else stride
    buf = torch.empty(rows, stride, dtype=torch.bfloat16, device="cuda")
    buf.view(torch.int16).fill_(CANARY)
    return buf[:, :width]


def run_attn2(case: Attn2Case, label: str, y=None, cache=None, table=None, lens=None,
              out=None, q=None, gate=None):
    """Launch attn2 once on device copies and return the output tensor."""
    case.host_check(cache, table, lens)
    dev = "cuda"
    yd = (case.y if y is None else y).to(dev)
    qd, gd = wl.attn2_views(yd, case.nkv)
    qd = qd if q is None else q
    gd = gd if gate is None else gate
    cd = (case.cache if cache is None else cache).to(dev)
    td = (case.table if table is None else table).to(dev)
    ld = (case.lens if lens is None else lens).to(dev)
    out = new_out(8 * case.R, 8 * case.nkv * wl.HEAD_DIM) if out is None else out
    say(f"attn2 {label} R={case.R} nkv={case.nkv} lens={list(map(int, ld.cpu()))[:6]} "
        f"mml={case.a.max_model_len} window={case.window} "
        f"splits={qf.attn2_plan(case.nkv, case.a.max_model_len, case.window, case.R)}")
    qf.attn2_prepare(case.nkv, case.a.max_model_len, case.R, case.window)
    qf.attn2_run(qd, gd, cd, td, ld, out)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("name", list(wl.ATTN2_WORKLOADS))
def test_attn2_workloads(name):
    case = Attn2Case(wl.ATTN2_WORKLOADS[name])
    out = run_attn2(case, name)
    stats = case.oracle_check(to_bits(out))
    print(name, stats)


SWEEP = [
    # (nkv, max_model_len, window, lens)
    (1, 2048, 0, (8, 9, 15, 16, 17, 31, 32, 33)),
    (2, 2048, 0, (47, 48, 49, 63, 64, 65, 2048)),
    (4, 8192, 0, (8, 100, 511, 512, 513, 5000)),
    (8, 8192, 0, (33, 8192)),
    (1, 65536, 0, (8, 40, 1000, 20000)),
    (2, 65536, 0, (65536, 17)),
    (8, 131072, 0, (70000,)),
    (4, 8192, 100, (8, 99, 100, 101, 107, 108, 109, 3000)),
    (1, 8192, 1, (8, 9, 24, 4096)),
    (8, 16384, 7, (8, 15, 16, 300)),
    (2, 16384, 8, (16, 17, 1000)),
    (2, 2048, 4096, (8, 500, 2048)),      # window covering every position: none
    # requests sharing the split slots: equal lengths whose first split length
    # does not fit (a bisection), and mixed lengths where short requests take
    # one split (finished by their block) beside long ones (merged)
    (8, 4096, 0, (1600,) * 12),
    (4, 65536, 0, (60000, 8, 100, 3000)),
    (2, 131072, 2000, (131072, 9, 2500, 40000)),
]


@pytest.mark.parametrize("nkv,mml,window,lens", SWEEP)
def test_attn2_sweep(nkv, mml, window, lens):
    a = wl.Attn2Workload(f"sweep_nkv{nkv}_mml{mml}_w{window}", nkv=nkv, max_model_len=mml,
                         lens=lens, window=window, q_scale=2.0, index=20 + nkv)
    case = Attn2Case(a)
    out = run_attn2(case, a.name)
    case.oracle_check(to_bits(out))


def test_attn2_max_requests():
    rng = np.random.default_rng(7)
    lens = tuple(int(v) for v in rng.integers(8, 2049, size=64))
    a = wl.Attn2Workload("max_reqs", nkv=1, max_model_len=2048, lens=lens, index=30)
    case = Attn2Case(a)
    case.oracle_check(to_bits(run_attn2(case, a.name)))
    # the same with splits: a longer max_model_len, the same lengths
    b = dataclasses.replace(a, max_model_len=16384, name="max_reqs_split")
    case = Attn2Case(b)
    case.oracle_check(to_bits(run_attn2(case, b.name)))


@pytest.mark.parametrize("nkv,mml,lens,window", [(2, 2048, (8, 100, 2048), 0),
                                                 (8, 32768, (5000,), 0),
                                                 (4, 8192, (3000, 777), 100)])
def test_attn2_small_values_where_eps_matters(nkv, mml, lens, window):
    """Values of ~2e-3 put mean(o^2) near the o-norm's eps: only there do the
    softmax sums and eps change the output (the weightless RMS norm cancels
    any other scale of o), so this checks the kernel's row sums and the
    merge's weighting of the splits, which unit-scale values cannot."""
    a = wl.Attn2Workload(f"small_v_nkv{nkv}", nkv=nkv, max_model_len=mml, lens=lens,
                         window=window, index=50 + nkv)
    case = Attn2Case(a)
    c = case.cache.float()
    c[..., 64:] *= 2e-3
    case.cache = c.to(torch.bfloat16)
    case.oracle_check(to_bits(run_attn2(case, a.name)))


def shared_page_case(a: wl.Attn2Workload, seed: int) -> Attn2Case:
    """An Attn2Case whose requests all read one set of pages (enough for
    max_model_len), each through its own random permutation of the block
    table: attention only reads the cache, so long contexts over many
    requests need no more than one request's pages."""
    case = Attn2Case.__new__(Attn2Case)
    case.a, case.nkv, case.window = a, a.nkv, a.eff_window
    case.y = wl.make_attn2_y(a, 0)
    pages = a.table_width
    g = torch.Generator().manual_seed(seed)
    case.cache = torch.randn(pages, a.nkv, wl.PAGE_SLOTS, wl.SLOT_WIDTH,
                             generator=g).to(torch.bfloat16)
    case.table = torch.stack([torch.randperm(pages, generator=g) for _ in a.lens]).to(torch.int32)
    case.lens = wl.make_attn2_lens(a)
    return case


@pytest.mark.parametrize("window", [0, 6000])
def test_attn2_multi_segment_splits(window):
    """With one split per (request, KV head) a block walks the request's whole
    context, so lengths past 4096 keys cross the segments in which the kernel
    stages page offsets, at and around the segment edges; with a window the
    walk starts in the middle of a page."""
    lens = (4096, 4097, 4100, 8192, 5000, 8191, 6000, 7777) * 4
    a = wl.Attn2Workload(f"multi_segment_w{window}", nkv=8, max_model_len=8192, lens=lens,
                         window=window, index=41)
    assert qf.attn2_plan(a.nkv, a.max_model_len, a.eff_window, a.R) == 1
    case = shared_page_case(a, seed=41 + window)
    case.oracle_check(to_bits(run_attn2(case, a.name)))


def test_attn2_needles_at_split_and_page_edges():
    """Each (row, head) query is a scaled copy of one key, so its softmax is
    concentrated there: a key lost at a split, chunk or page edge shows."""
    a = dataclasses.replace(wl.A1, sets=1)
    case = Attn2Case(a)
    L = a.lens[0]
    Z = qf.attn2_plan(a.nkv, a.max_model_len, 0, 1)
    per = max((L // 32 + Z - 1) // Z, 8) * 32
    picks = sorted({0, 1, 15, 16, 31, 32, per - 1, per, per + 1, 2 * per - 1, 2 * per,
                    L - 9, L - 8, L - 2, L - 1})
    cache = case.cache.float()
    q, _ = case.views()
    rng = np.random.default_rng(8)
    for row in range(8):
        pos = L - 8 + row
        for h in range(8 * a.nkv):
            k = picks[(row * 7 + h) % len(picks)]
            k = min(k, pos) if rng.random() < 0.8 else int(rng.integers(0, pos + 1))
            page = int(case.table[0, k // 16])
            key = cache[page, h // 8, k % 16, :64]
            q[row, h * 64:(h + 1) * 64] = (4.0 * key).to(torch.bfloat16)
    out = run_attn2(case, "needles")
    case.oracle_check(to_bits(out))


def test_attn2_ignores_entries_it_must_not_read():
    """Poison (NaN) every cache entry outside the attended keys: slots past L
    in the last page, keys before the earliest window start, pages no
    request owns and the filler page.  The output must not change."""
    a = wl.Attn2Workload("poison", nkv=4, max_model_len=8192, lens=(1000, 77, 8, 4100),
                         window=300, q_scale=2.0, index=31)
    case = Attn2Case(a)
    base = run_attn2(case, "poison-clean")
    case.oracle_check(to_bits(base))
    poisoned = case.cache.clone()
    bits = poisoned.view(torch.int16)
    owned = torch.zeros(poisoned.shape[0], dtype=torch.bool)
    for r, L in enumerate(a.lens):
        lo = a.first_key(L)
        for k in range(0, (L + 15) // 16 * 16):
            if k < lo or k >= L:
                bits[int(case.table[r, k // 16]), :, k % 16, :] = NAN_BITS
        owned[case.table[r, :(L + 15) // 16].long()] = True
    bits[~owned] = NAN_BITS
    got = run_attn2(case, "poison", cache=poisoned)
    assert torch.equal(got.view(torch.int16).cpu(), base.view(torch.int16).cpu())


def test_attn2_views_strides_and_determinism():
    """q and gate as views of the front's rows, or as contiguous copies, and
    an output with a wider row stride: identical bits; columns past the
    output width keep their contents; two calls agree bit for bit."""
    a = dataclasses.replace(wl.A2, sets=1, lens=(3000, 901), max_model_len=8192)
    case = Attn2Case(a)
    width = 8 * a.nkv * 64
    base = run_attn2(case, "views")
    case.oracle_check(to_bits(base))
    again = run_attn2(case, "views-again")
    assert torch.equal(again.view(torch.int16), base.view(torch.int16))
    q, g = case.views()
    wide = new_out(8 * case.R, width, stride=width + 72)
    got = run_attn2(case, "contiguous-q-gate", q=q.contiguous().cuda(), gate=g.contiguous().cuda(),
                    out=wide)
    assert torch.equal(got.view(torch.int16), base.view(torch.int16))
    full = wide.as_strided((8 * case.R, width + 72), (width + 72, 1))
    assert bool((full[:, width:].view(torch.int16) == CANARY).all())


def test_attn2_block_table_permutation():
    """Moving the pages of the cache and the table with them changes nothing."""
    a = wl.Attn2Workload("perm", nkv=2, max_model_len=16384, lens=(5000, 333), index=32)
    case = Attn2Case(a)
    base = run_attn2(case, "perm-base")
    g = torch.Generator().manual_seed(9)
    perm = torch.randperm(case.cache.shape[0], generator=g)
    moved = torch.empty_like(case.cache)
    moved[perm] = case.cache
    table = perm[case.table.long()].to(torch.int32)
    got = run_attn2(case, "perm-moved", cache=moved, table=table)
    assert torch.equal(got.view(torch.int16), base.view(torch.int16))


def test_attn2_refusals_on_device():
    a = wl.Attn2Workload("refuse", nkv=2, max_model_len=4096, lens=(64, 64, 64), index=33)
    case = Attn2Case(a)
    qf.attn2_prepare(a.nkv, a.max_model_len, 2, 0)
    yd = case.y.cuda()
    q, g = wl.attn2_views(yd, a.nkv)
    out = new_out(24, 8 * a.nkv * 64)
    args = (q, g, case.cache.cuda(), case.table.cuda(), case.lens.cuda(), out)
    with pytest.raises(qf.QkvfError, match="ROWS"):
        qf.attn2_run(*args)   # three requests after preparing for two
    with pytest.raises(qf.QkvfError, match="ALIGN"):
        qf.attn2_run(q[:16, 1:], g[:16], args[2], args[3], args[4][:2], out[:16])
    assert bool((out.view(torch.int16) == CANARY).all())


GRAPH_CASES = [
    # (first lengths, the lengths of the three replays)
    ((9000,), [(9000,), (8000,), (7000,)]),
    # requests sharing the split slots: each replay's lengths give another
    # split length and another share of the slots, from the same launch
    ((20000, 9000, 300), [(20000, 9000, 300), (300, 8, 20000), (12000, 12000, 12000)]),
]


@pytest.mark.parametrize("first,replays", GRAPH_CASES, ids=["one_request", "shared_slots"])
def test_attn2_graph_replays(first, replays):
    """Captured once, replayed with new inputs copied into the captured
    buffers (eager work between replays); every replay matches eager."""
    a = wl.Attn2Workload("graph", nkv=8, max_model_len=65536, lens=first, index=34)
    case = Attn2Case(a)
    dev = "cuda"
    y = case.y.cuda()
    q, g = wl.attn2_views(y, a.nkv)
    cache, table, lens = case.cache.cuda(), case.table.cuda(), case.lens.cuda()
    out = new_out(8 * a.R, 8 * a.nkv * 64)
    case.host_check()
    say(f"attn2 graph capture R={a.R}")
    qf.attn2_prepare(a.nkv, a.max_model_len, a.R, 0)
    stream = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        qf.attn2_run(q, g, cache, table, lens, out, stream=stream)   # warm-up on the stream
        stream.synchronize()
        with torch.cuda.graph(graph, stream=stream):
            qf.attn2_run(q, g, cache, table, lens, out, stream=stream)
    for i, new_lens in enumerate(replays):
        ys = wl.make_attn2_y(a, set_index=1 + i)
        y.copy_(ys.to(dev))
        # within the pages each request owns (the table's other entries are
        # the filler page)
        assert all(L <= max(first) for L in new_lens)
        lens.copy_(torch.tensor(new_lens, dtype=torch.int32))
        torch.cuda.synchronize()
        say(f"attn2 graph replay {i}")
        graph.replay()
        torch.cuda.synchronize()
        replay = out.clone()
        out.view(torch.int16).fill_(CANARY)
        torch.cuda.synchronize()
        qf.attn2_run(q, g, cache, table, lens, out)
        torch.cuda.synchronize()
        assert torch.equal(replay.view(torch.int16), out.view(torch.int16)), f"replay {i}"
        case.oracle_check(to_bits(out), y=ys, lens=lens.cpu())


def test_front_then_attn2():
    """The front writes the 8 verify-step tokens' K|V into the request's
    pages and its q | gate rows feed attn2; attn2 on the device's own y and
    cache matches the oracle on those same bytes, and the front itself
    matches its oracle."""
    from helpers import Case, check
    nkv, L = 2, 700
    a = wl.Attn2Workload("front_then_attn2", nkv=nkv, max_model_len=4096, lens=(L,), index=35)
    case = Attn2Case(a)
    pages = case.cache.shape[0]
    w = dataclasses.replace(wl.C2, pages=pages, slot_hi=pages * 16 - 7)
    front = Case(w)
    pos = torch.arange(L - 8, L, dtype=torch.int64)
    slots = torch.tensor([int(case.table[0, p // 16]) * 16 + p % 16 for p in pos.tolist()],
                         dtype=torch.int64)
    front.positions, front.slots = pos, slots
    front.cache = case.cache.clone()
    assert front.M == 8 and int(slots.max()) < front.cache.shape[0] * 16
    g = front.device()
    say("front for attn2")
    qf.prepare(front.N, nkv, 8)
    qf.run(g["x"], g["W"], g["positions"], g["slots"], g["cos_sin"], g["y"], g["kv_cache"], M=8)
    torch.cuda.synchronize()
    assert qf.device_fault() == 0
    check(front, g)
    y_gpu = g["y"].cpu()
    cache_gpu = g["kv_cache"].cpu()
    out = run_attn2(case, "after-front", y=y_gpu, cache=cache_gpu)
    case.oracle_check(to_bits(out), y=y_gpu, cache=cache_gpu)


def test_layer_front_then_front_then_attn2():
    """The first layer's decode step, each stage fed the previous stage's
    device output: LayerFront turns 8 embedded rows into x, the front
    projects x and inserts the 8 verify tokens' K|V into the request's pages,
    attn2 attends over the cache.  Every stage matches the oracle on the
    bytes it was given."""
    from helpers import Case, check
    nkv, L = 2, 1000
    a = wl.Attn2Workload("chain", nkv=nkv, max_model_len=4096, lens=(L,), index=36)
    case = Attn2Case(a)
    pages = case.cache.shape[0]
    w = dataclasses.replace(wl.C2, pages=pages, slot_hi=pages * 16 - 7)
    front = Case(w)
    # LayerFront: fp32 embedded rows -> stream, out = the front's x
    g = torch.Generator().manual_seed(36)
    emb = torch.randn(8, wl.HIDDEN, generator=g)
    norm_w = (1.0 + 0.1 * torch.randn(wl.HIDDEN, generator=g)).to(torch.bfloat16)
    emb_d = emb.cuda()
    stream = torch.empty(8, wl.HIDDEN, device="cuda")
    x_d = torch.empty(8, wl.HIDDEN, dtype=torch.bfloat16, device="cuda")
    say("chain: layer_front")
    qf.layer_front(emb_d, stream, x_d, weight=norm_w.cuda(), eps=1e-6)
    torch.cuda.synchronize()
    checker.check_layer_front(emb.numpy(), to_bits(norm_w), 1e-6, stream.cpu().numpy(),
                              to_bits(x_d.cpu()))
    # the front on that x, inserting the verify tokens at positions L-8 .. L-1
    front.x = x_d.cpu()
    front.positions = torch.arange(L - 8, L, dtype=torch.int64)
    front.slots = torch.tensor([int(case.table[0, p // 16]) * 16 + p % 16
                                for p in range(L - 8, L)], dtype=torch.int64)
    front.cache = case.cache.clone()
    gd = front.device()
    say("chain: front")
    qf.prepare(front.N, nkv, 8)
    qf.run(gd["x"], gd["W"], gd["positions"], gd["slots"], gd["cos_sin"], gd["y"], gd["kv_cache"], M=8)
    torch.cuda.synchronize()
    assert qf.device_fault() == 0
    check(front, gd)
    # attn2 on the front's y and cache
    y_gpu, cache_gpu = gd["y"].cpu(), gd["kv_cache"].cpu()
    out = run_attn2(case, "chain", y=y_gpu, cache=cache_gpu)
    case.oracle_check(to_bits(out), y=y_gpu, cache=cache_gpu)
