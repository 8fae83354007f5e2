"""attn2 and the batch a request is in: the same request alone, with one
other request and with three others (and at another position in the
batch).  With batch-invariant splits (qkvf_attn2_prepare_ex(..., 1)) its
output rows must be bit for bit the same in every batch; by default the
requests share the launch's split slots, so a request's split length follows
the lengths of its batch: every result must match the oracle, and the rows
are bit for bit the same when the batch is the same set of lengths in
another order."""
from __future__ import annotations

import pytest
import torch

import kv_insert_amd as qf
from kv_insert_amd import workloads as wl
from oracle import checker

from helpers import CANARY, say, to_bits

pytestmark = pytest.mark.gpu

FULL = wl.Attn2Workload("batch_of_four", nkv=8, max_model_len=32768,
                        lens=(30000, 9001, 2000, 50), index=40)


@pytest.fixture(scope="module")
def full():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    qf.lib()
    a = FULL
    y = wl.make_attn2_y(a, 0)
    cache = wl.make_attn2_cache(a)
    table = wl.make_attn2_table(a, 0)
    lens = wl.make_attn2_lens(a)
    for r, L in enumerate(a.lens):   # every page a request reads is inside the cache
        need = (L + wl.PAGE_SLOTS - 1) // wl.PAGE_SLOTS
        assert need <= table.shape[1]
        assert 0 <= int(table[r, :need].min()) and int(table[r, :need].max()) < cache.shape[0]
    return {"y": y, "cache": cache, "cache_dev": cache.to("cuda"), "table": table, "lens": lens}


def run_batch(full, reqs, invariant: bool):
    """attn2 on the requests `reqs` (indices into FULL, in this order);
    returns the output rows [8 len(reqs), 512 nkv] on the host."""
    nkv = FULL.nkv
    y = torch.cat([full["y"][8 * r:8 * r + 8] for r in reqs]).to("cuda")
    table = torch.stack([full["table"][r] for r in reqs]).contiguous().to("cuda")
    lens = torch.tensor([FULL.lens[r] for r in reqs], dtype=torch.int32, device="cuda")
    q, g = wl.attn2_views(y, nkv)
    out = torch.empty(8 * len(reqs), 8 * nkv * wl.HEAD_DIM, dtype=torch.bfloat16, device="cuda")
    out.view(torch.int16).fill_(CANARY)
    R = len(reqs)
    z = qf.attn2_plan(nkv, FULL.max_model_len, 0, 1 if invariant else R)
    say(f"attn2 batch {list(reqs)} invariant={invariant} splits={z}")
    qf.attn2_prepare(nkv, FULL.max_model_len, R, 0, batch_invariant=invariant)
    qf.attn2_run(q, g, full["cache_dev"], table, lens, out)
    torch.cuda.synchronize()
    host = to_bits(out)
    # every batch is checked against the oracle on its own inputs
    checker.check_attn2(host, to_bits(y.cpu()[:, :8 * nkv * 64]), to_bits(g.cpu()),
                        to_bits(full["cache"]), nkv, table.cpu().numpy(), lens.cpu().numpy())
    return host


BATCHES = [(0,), (0, 1), (0, 1, 2, 3), (2, 3, 0, 1), (1,)]


def test_batch_invariant_splits_give_the_same_bits_in_every_batch(full):
    outs = {b: run_batch(full, b, invariant=True) for b in BATCHES}
    rows = lambda b, r: outs[b][8 * b.index(r):8 * b.index(r) + 8]
    for b in BATCHES[1:]:
        if 0 in b:
            assert (rows(b, 0) == rows((0,), 0)).all(), b
    for b in ((0, 1), (0, 1, 2, 3), (2, 3, 0, 1)):
        assert (rows(b, 1) == rows((1,), 1)).all(), b
    assert (rows((0, 1, 2, 3), 3) == rows((2, 3, 0, 1), 3)).all()


def test_default_splits_follow_the_batch_and_match_the_oracle(full):
    """By default the requests share 32 split slots per KV head: every batch
    matches the oracle (checked in run_batch); a request's rows are the same
    bits in two batches of the same lengths, and may differ in the last bits
    otherwise."""
    outs = {b: run_batch(full, b, invariant=False) for b in BATCHES}
    rows = lambda b, r: outs[b][8 * b.index(r):8 * b.index(r) + 8]
    z = {b: qf.attn2_plan(FULL.nkv, FULL.max_model_len, 0, len(b)) for b in BATCHES}
    assert all(v == 32 for v in z.values())
    # the same lengths in another order: the same split length, the same bits
    assert (rows((0, 1, 2, 3), 0) == rows((2, 3, 0, 1), 0)).all()
    assert (rows((0, 1, 2, 3), 2) == rows((2, 3, 0, 1), 2)).all()
    same = {b: bool((rows(b, 0) == rows((0,), 0)).all()) for b in BATCHES[1:] if 0 in b}
    print("request 0 bit-identical to its one-request result:", same)
