"""Pins of the attn2 oracle (paged decode attention of the 8-token verify
step with the o-norm and sigmoid gate) against closed forms, a float64
torch computation, invariances and a hand-worked fixture.  No GPU."""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
EPS = oracle.ATTN2_EPS
SCALE = oracle.ATTN2_SCALE


def bits(a):
    return (torch.from_numpy(np.asarray(a, dtype=np.float32)).to(torch.bfloat16)
            .view(torch.int16).numpy().view(np.uint16))


def rand_case(rng, R, nkv, Ls, pages=None, scale_q=1.0, scale_v=1.0):
    nq = 8 * nkv
    max_pages = max((L + 15) // 16 for L in Ls)
    pages = pages or R * max_pages + 3
    q = bits(rng.standard_normal((R * 8, nq * 64)) * scale_q)
    gate = bits(rng.standard_normal((R * 8, nq * 64)))
    c = rng.standard_normal((pages, nkv, 16, 128))
    c[..., 64:] *= scale_v
    cache = bits(c)
    perm = rng.permutation(pages)
    bt = np.zeros((R, max_pages), np.int32)
    for r in range(R):
        bt[r] = perm[r * max_pages:(r + 1) * max_pages]
    return q, gate, cache, bt, np.array(Ls, np.int32)


def dense_reference(q, gate, cache, nkv, bt, seq_lens, window):
    """float64 torch: gather K/V by the block table (numpy indexing), masked
    softmax(q K^T * scale) V, then the weightless RMS norm and sigmoid gate."""
    nq = 8 * nkv
    R = len(seq_lens)
    qf = torch.from_numpy(oracle.bf16_to_float(q))
    gf = torch.from_numpy(oracle.bf16_to_float(gate))
    cf = oracle.bf16_to_float(cache)
    out = np.zeros((R * 8, nq * 64))
    for r in range(R):
        L = int(seq_lens[r])
        pos = np.arange(L)
        kv = cf[bt[r][pos // 16], :, pos % 16, :]          # [L, nkv, 128]
        K = torch.from_numpy(kv[:, :, :64])
        V = torch.from_numpy(kv[:, :, 64:])
        for t in range(8):
            p = L - 8 + t
            mask = torch.from_numpy(pos <= p)
            if window > 0:
                mask &= torch.from_numpy(pos > p - window)
            for h in range(nq):
                j = h // 8
                qh = qf[r * 8 + t, h * 64:(h + 1) * 64]
                s = (K[:, j, :] @ qh) * SCALE
                s = torch.where(mask, s, torch.tensor(-math.inf, dtype=torch.float64))
                a = torch.softmax(s, dim=0)
                o = a @ V[:, j, :]
                o = o / torch.sqrt(torch.mean(o * o) + EPS)
                o = o * torch.sigmoid(gf[r * 8 + t, h * 64:(h + 1) * 64])
                out[r * 8 + t, h * 64:(h + 1) * 64] = o.numpy()
    return out


@pytest.mark.parametrize("nkv,Ls,window", [(1, [8], 0), (1, [37, 8, 100], 0), (2, [64, 300], 0),
                                          (1, [200], 40), (2, [50, 129], 16), (4, [33], 1)])
def test_attn2_matches_float64_torch(nkv, Ls, window):
    rng = np.random.default_rng(100 + nkv * 7 + len(Ls) + window)
    q, gate, cache, bt, sl = rand_case(rng, len(Ls), nkv, Ls)
    got = oracle.attn2(q, gate, cache, nkv, bt, sl, window)
    ref = dense_reference(q, gate, cache, nkv, bt, sl, window)
    # both round the same double value to bf16; allow one unit where the
    # double results straddle a rounding midpoint
    g = oracle.bf16_to_float(got)
    assert np.all(np.abs(g - ref) <= np.abs(ref) * 2.0 ** -7 + 1e-30)


@pytest.mark.parametrize("Ls,window", [([8, 37, 100], 0), ([50, 129], 16)])
def test_attn2_small_values_where_eps_matters(Ls, window):
    """Values of ~2e-3 put mean(o^2) near eps = 1e-6: only there do the
    softmax normalisation and eps change the normed output (the weightless
    RMS norm cancels any other scale of o), so a dropped normalisation or a
    dropped eps shows here and nowhere else."""
    rng = np.random.default_rng(300 + len(Ls) + window)
    q, gate, cache, bt, sl = rand_case(rng, len(Ls), 1, Ls, scale_v=2e-3)
    ref = dense_reference(q, gate, cache, 1, bt, sl, window)
    v = oracle.bf16_to_float(cache)[..., 64:]
    assert 1e-8 < float(np.mean(v * v)) < 1e-4
    g = oracle.bf16_to_float(oracle.attn2(q, gate, cache, 1, bt, sl, window))
    assert np.all(np.abs(g - ref) <= np.abs(ref) * 2.0 ** -7 + 1e-30)


def test_first_row_sees_only_key_zero():
    """L = 8: row 0 sits at position 0 and sees key 0 alone, so the
    attention is V_0 exactly."""
    rng = np.random.default_rng(1)
    q, gate, cache, bt, sl = rand_case(rng, 1, 1, [8])
    out = oracle.attn2(q, gate, cache, 1, bt, sl)
    V0 = oracle.bf16_to_float(cache[bt[0, 0], 0, 0, 64:])
    g = oracle.bf16_to_float(gate[0])
    for h in range(8):
        o = V0 / math.sqrt(np.mean(V0 * V0) + EPS) / (1 + np.exp(-g[h * 64:(h + 1) * 64]))
        np.testing.assert_array_equal(out[0, h * 64:(h + 1) * 64], bits(o))


def test_zero_query_averages_visible_values():
    rng = np.random.default_rng(2)
    L, W = 50, 20
    q, gate, cache, bt, sl = rand_case(rng, 1, 1, [L])
    q[:] = 0
    gate[:] = 0  # sigmoid(0) = 1/2
    for window in (0, W):
        out = oracle.attn2(q, gate, cache, 1, bt, sl, window)
        for t in range(8):
            p = L - 8 + t
            lo = max(0, p - window + 1) if window else 0
            ks = np.arange(lo, p + 1)
            V = oracle.bf16_to_float(cache[bt[0, ks // 16], 0, ks % 16, 64:])
            o = V.mean(axis=0)
            o = o / math.sqrt(np.mean(o * o) + EPS) * 0.5
            got = oracle.bf16_to_float(out[t, :64])
            np.testing.assert_allclose(got, o, rtol=2.0 ** -7, atol=0)


def test_keys_after_the_row_and_outside_the_window_do_not_matter():
    rng = np.random.default_rng(3)
    L, W = 90, 30
    q, gate, cache, bt, sl = rand_case(rng, 1, 2, [L])
    base = oracle.attn2(q, gate, cache, 2, bt, sl, W)
    c2 = cache.copy()
    # beyond L in the last page, and before the earliest window start
    last = bt[0, (L - 1) // 16]
    c2[last, :, (L - 1) % 16 + 1:, :] ^= 0x1234
    for k in range(0, L - 8 - W + 1):
        c2[bt[0, k // 16], :, k % 16, :] ^= 0x0F0F
    np.testing.assert_array_equal(oracle.attn2(q, gate, c2, 2, bt, sl, W), base)
    # the last key is seen by row 7 only
    c3 = cache.copy()
    c3[last, :, (L - 1) % 16, 64:] ^= 0x4000
    got = oracle.attn2(q, gate, c3, 2, bt, sl, W)
    np.testing.assert_array_equal(got[:7], base[:7])
    assert not np.array_equal(got[7], base[7])


def test_block_table_indirection():
    rng = np.random.default_rng(4)
    q, gate, cache, bt, sl = rand_case(rng, 2, 1, [70, 45])
    base = oracle.attn2(q, gate, cache, 1, bt, sl)
    perm = rng.permutation(cache.shape[0])
    moved = np.empty_like(cache)
    moved[perm] = cache
    np.testing.assert_array_equal(oracle.attn2(q, gate, moved, 1, perm[bt].astype(np.int32), sl), base)


def test_output_rms_closed_form():
    """out / sigmoid(gate) has RMS sqrt(ms / (ms + eps)) over each head."""
    rng = np.random.default_rng(5)
    q, gate, cache, bt, sl = rand_case(rng, 1, 1, [40])
    gate[:] = bits(np.full(gate.shape, 30.0))  # sigmoid = 1 to double precision
    out = oracle.bf16_to_float(oracle.attn2(q, gate, cache, 1, bt, sl))
    rms = np.sqrt(np.mean(out.reshape(8, 8, 64) ** 2, axis=-1))
    np.testing.assert_allclose(rms, 1.0, atol=1e-2)


def test_golden_two_keys_by_hand():
    g = json.load(open(os.path.join(GOLDEN, "attn2_two_keys.json")))
    q = np.zeros((8, 512), np.float32)
    gate = np.zeros((8, 512), np.float32)
    cache = np.zeros((1, 1, 16, 128), np.float32)
    q[1, 0] = g["q0"]
    cache[0, 0, 0, 0] = g["k0"][0]
    cache[0, 0, 1, 0] = g["k1"][0]
    cache[0, 0, 0, 64:66] = g["v0"]
    cache[0, 0, 1, 64:66] = g["v1"]
    out = oracle.attn2(bits(q), bits(gate), bits(cache), 1, np.zeros((1, 1), np.int32),
                       np.array([8], np.int32))
    np.testing.assert_array_equal(oracle.bf16_to_float(out[1, :2]), g["expected_row1_head0"][:2])
    assert np.all(out[1, 2:64] & 0x7FFF == 0)
