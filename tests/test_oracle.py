"""Pins of the CPU oracle against things other than itself: library routines,
closed forms, invariants, exact arithmetic, brute force and hand-worked
fixtures.  No GPU."""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from kv_insert_amd import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
EPS = 1e-6


def rand_bf16(rng, shape, scale=1.0):
    v = torch.from_numpy(rng.standard_normal(shape).astype(np.float32) * scale)
    return v.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def torch_bits(values_f32):
    return (torch.from_numpy(np.asarray(values_f32, dtype=np.float32))
            .to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16))


# --- bf16 rounding -----------------------------------------------------------

def test_bf16_rounding_matches_torch_random():
    rng = np.random.default_rng(1)
    f = (rng.standard_normal(200_000) * np.exp(rng.uniform(-30, 30, 200_000))).astype(np.float32)
    np.testing.assert_array_equal(oracle.float_to_bf16(f), torch_bits(f))


def test_bf16_rounding_exact_ties_go_to_even():
    rng = np.random.default_rng(2)
    kept = rng.integers(0x0080, 0x7F00, 50_000).astype(np.uint32)  # normal range
    sign = (rng.integers(0, 2, kept.size).astype(np.uint32) << 15)
    hi = (kept | sign) << 16
    cases = []
    for low in (0x8000, 0x7FFF, 0x8001, 0x0000, 0xFFFF):
        cases.append((hi | low).view(np.float32))
    f = np.concatenate(cases)
    got = oracle.float_to_bf16(f)
    np.testing.assert_array_equal(got, torch_bits(f))
    # Exactly half: the kept part must come out even.
    ties = oracle.float_to_bf16((hi | 0x8000).view(np.float32))
    assert np.all(ties & 1 == 0)


def test_bf16_values_round_trip():
    allbits = np.arange(0, 0x10000, dtype=np.uint32)
    finite = allbits[(allbits & 0x7F80) != 0x7F80].astype(np.uint16)
    f = oracle.bf16_to_float(finite).astype(np.float32)
    np.testing.assert_array_equal(oracle.float_to_bf16(f), finite)


# --- projection ----------------------------------------------------------------

def test_project_brute_force_exact_rationals():
    """Tiny case: the exact rational sum, rounded once, is within the double
    accumulation bound of the oracle's value."""
    rng = np.random.default_rng(3)
    M, N = 2, 3
    x = rand_bf16(rng, (M, 8192))
    W = rand_bf16(rng, (N, 8192), 0.011)
    z, a = oracle.project(x, W)
    xf = oracle.bf16_to_float(x)
    Wf = oracle.bf16_to_float(W)
    for m in range(M):
        for n in range(N):
            exact = sum((Fraction(float(xf[m, k])) * Fraction(float(Wf[n, k]))
                         for k in range(8192)), Fraction(0))
            bound = 8192 * 2.0 ** -53 * a[m, n]
            assert abs(float(exact) - z[m, n]) <= bound
            assert a[m, n] == pytest.approx(float(np.abs(xf[m] * Wf[n]).sum()), rel=1e-12)


def test_project_against_torch_float64_matmul():
    rng = np.random.default_rng(4)
    M, N = 5, 96
    x = rand_bf16(rng, (M, 8192))
    W = rand_bf16(rng, (N, 8192), 0.011)
    z, _ = oracle.project(x, W, nthreads=4)
    ref = torch.from_numpy(oracle.bf16_to_float(x)) @ torch.from_numpy(oracle.bf16_to_float(W)).T
    np.testing.assert_allclose(z, ref.numpy(), rtol=0, atol=1e-12)


def test_project_exact_integer_inputs():
    """x, W in {-1, 0, 1}: every order sums exactly; compare with int64."""
    rng = np.random.default_rng(5)
    M, N = 4, 40
    xi = rng.choice([-1, 0, 0, 0, 1], size=(M, 8192)).astype(np.int64)
    Wi = rng.choice([-1, 0, 0, 0, 1], size=(N, 8192)).astype(np.int64)
    x = torch_bits(xi.astype(np.float32))
    W = torch_bits(Wi.astype(np.float32))
    z, _ = oracle.project(x, W)
    np.testing.assert_array_equal(z, (xi @ Wi.T).astype(np.float64))


def test_project_one_hot_selects_a_column():
    rng = np.random.default_rng(6)
    N = 17
    W = rand_bf16(rng, (N, 8192), 0.011)
    for j in (0, 1, 4095, 8191):
        x = np.zeros((1, 8192), dtype=np.uint16)
        x[0, j] = 0x3F80  # 1.0
        z, _ = oracle.project(x, W)
        np.testing.assert_array_equal(z[0], oracle.bf16_to_float(W[:, j]))
        np.testing.assert_array_equal(oracle.round_projection(z)[0], W[:, j])


# --- one head: norm and rotation ---------------------------------------------

def _table_row(pos):
    return wl.rope_table(pos + 1)[pos].numpy()


def test_head_norm_closed_form_at_position_zero():
    """Position 0 is the identity rotation; the normed head has RMS
    sqrt(ms / (ms + eps))."""
    rng = np.random.default_rng(7)
    cs0 = _table_row(0)
    assert np.all(cs0[:32] == 1.0) and np.all(cs0[32:] == 0.0)
    for scale in (1.0, 30.0, 1e-3):
        p = rand_bf16(rng, 64, scale)
        out, out_d = oracle.head(p, cs0, EPS)
        pv = oracle.bf16_to_float(p)
        ms = float(np.mean(pv * pv))
        rms = math.sqrt(float(np.mean(out_d * out_d)))
        assert rms == pytest.approx(math.sqrt(ms / (ms + EPS)), rel=1e-12)
        # identity rotation: same as the norm alone
        out2, out2_d = oracle.head(p, None, EPS)
        np.testing.assert_array_equal(out, out2)
        np.testing.assert_allclose(out_d, out2_d, rtol=0, atol=0)


def test_head_rotation_matches_rotation_matrices():
    """Each pair (2i, 2i+1) of the normed head is turned by the angle
    pos * 10000^(-2i/64) — checked with 2x2 rotation matrices in float64."""
    rng = np.random.default_rng(8)
    for pos in (1, 7, 4095, 131071):
        p = rand_bf16(rng, 64)
        out, out_d = oracle.head(p, _table_row(pos), EPS)
        pv = oracle.bf16_to_float(p)
        n = pv / math.sqrt(float(np.mean(pv * pv)) + EPS)
        for i in range(32):
            th = wl.rope_angle(pos, i)
            R = np.array([[math.cos(th), -math.sin(th)], [math.sin(th), math.cos(th)]])
            expect = R @ n[2 * i:2 * i + 2]
            np.testing.assert_allclose(out_d[2 * i:2 * i + 2], expect, rtol=0, atol=2e-6)
        np.testing.assert_array_equal(out, oracle.float_to_bf16(out_d.astype(np.float32)))


def test_head_rotation_preserves_pair_norms():
    rng = np.random.default_rng(9)
    p = rand_bf16(rng, 64)
    row = _table_row(12345)
    _, o = oracle.head(p, row, EPS)
    _, n = oracle.head(p, None, EPS)
    c = row[:32].astype(np.float64)
    s = row[32:].astype(np.float64)
    lhs = o[0::2] ** 2 + o[1::2] ** 2
    rhs = (n[0::2] ** 2 + n[1::2] ** 2) * (c * c + s * s)
    np.testing.assert_allclose(lhs, rhs, rtol=1e-12, atol=0)
    np.testing.assert_allclose(c * c + s * s, 1.0, atol=3e-7)


def test_head_zero_is_zero():
    out, out_d = oracle.head(np.zeros(64, np.uint16), _table_row(99), EPS)
    assert np.all(out_d == 0.0) and np.all((out & 0x7FFF) == 0)


def test_head_scale_invariance_of_outlier_rows():
    """A x30 outlier head gives the same normed values (within eps effects)."""
    rng = np.random.default_rng(10)
    base = rng.standard_normal(64).astype(np.float32)
    p1 = torch_bits(base)
    p30 = torch_bits(oracle.bf16_to_float(p1).astype(np.float32) * 30)  # exact: x30 may round
    _, o1 = oracle.head(p1, _table_row(5), EPS)
    _, o30 = oracle.head(p30, _table_row(5), EPS)
    np.testing.assert_allclose(o1, o30, rtol=0, atol=1e-2)


def test_golden_hand_worked_head():
    g = json.load(open(os.path.join(GOLDEN, "head_quarter_turn.json")))
    p = np.zeros(64, np.float32)
    p[:len(g["p"])] = g["p"]
    row = np.concatenate([np.ones(32, np.float32), np.zeros(32, np.float32)])
    for i, v in g["cos"].items():
        row[int(i)] = v
    for i, v in g["sin"].items():
        row[32 + int(i)] = v
    out, out_d = oracle.head(torch_bits(p), row, g["eps"])
    k = len(g["expected_bf16"])
    np.testing.assert_array_equal(oracle.bf16_to_float(out[:k]), g["expected_bf16"])
    np.testing.assert_allclose(out_d[:k], g["expected_double"], rtol=1e-12)
    assert np.all(out_d[k:] == 0)


# --- epilogue: layout of the row and the cache --------------------------------

def test_golden_slot_placement():
    g = json.load(open(os.path.join(GOLDEN, "slot_placement.json")))
    nkv, N = g["nkv"], g["N"]
    assert oracle.n_cols(nkv) == N
    M = len(g["slots"])
    rng = np.random.default_rng(11)
    p = rand_bf16(rng, (M, N))
    cache = rng.integers(0, 0x10000, (4, nkv, 16, 128)).astype(np.uint16)
    before = cache.copy()
    y = oracle.epilogue(p, np.arange(M), np.array(g["slots"]), wl.rope_table(8).numpy(),
                        nkv, EPS, cache)
    for m, (page, off) in enumerate(g["expected_page_offset"]):
        for j in range(nkv):
            k0, k1 = g["k_columns"][j]
            v0, v1 = g["v_columns"][j]
            np.testing.assert_array_equal(cache[page, j, off, :64], y[m, k0:k1])
            np.testing.assert_array_equal(cache[page, j, off, 64:], y[m, v0:v1])
            np.testing.assert_array_equal(cache[page, j, off, 64:], p[m, v0:v1])
    changed = np.argwhere(np.any(cache != before, axis=-1))
    assert {tuple(c) for c in changed} <= {(pg, j, o) for pg, o in g["expected_page_offset"]
                                           for j in range(nkv)}


@pytest.mark.parametrize("nkv", [1, 2, 4, 8])
def test_epilogue_row_layout_and_untouched_cache(nkv):
    rng = np.random.default_rng(20 + nkv)
    M = 5
    N = oracle.n_cols(nkv)
    nq = 8 * nkv
    p = rand_bf16(rng, (M, N))
    positions = rng.integers(0, 4096, M)
    slots = rng.permutation(64 * 16)[:M].astype(np.int64)
    slots[2] = -1  # padding token: no insert
    table = wl.rope_table(4096).numpy()
    cache = rng.integers(0, 0x10000, (64, nkv, 16, 128)).astype(np.uint16)
    before = cache.copy()
    y = oracle.epilogue(p, positions, slots, table, nkv, EPS, cache)
    qk = (nq + nkv) * 64
    # v and gate pass through bit for bit
    np.testing.assert_array_equal(y[:, qk:], p[:, qk:])
    # q and k heads: the head function on the token's table row
    for m in range(M):
        for h in range(nq + nkv):
            out, _ = oracle.head(p[m, 64 * h:64 * h + 64], table[positions[m]], EPS)
            np.testing.assert_array_equal(y[m, 64 * h:64 * h + 64], out)
    # cache: written slots hold [k | v] of the row, everything else unchanged
    expect = before.copy()
    for m in range(M):
        if slots[m] < 0:
            continue
        pg, off = divmod(int(slots[m]), 16)
        for j in range(nkv):
            expect[pg, j, off, :64] = y[m, nq * 64 + 64 * j: nq * 64 + 64 * j + 64]
            expect[pg, j, off, 64:] = y[m, (nq + nkv) * 64 + 64 * j:(nq + nkv) * 64 + 64 * j + 64]
    np.testing.assert_array_equal(cache, expect)


def test_no_rope_layer_only_norms():
    rng = np.random.default_rng(30)
    nkv, M = 1, 2
    N = oracle.n_cols(nkv)
    p = rand_bf16(rng, (M, N))
    cache = np.zeros((4, nkv, 16, 128), np.uint16)
    y = oracle.epilogue(p, np.array([3, 9]), np.array([0, 1]), None, nkv, EPS, cache)
    for h in range(9):
        out, _ = oracle.head(p[0, 64 * h:64 * h + 64], None, EPS)
        np.testing.assert_array_equal(y[0, 64 * h:64 * h + 64], out)


def test_front_is_projection_then_epilogue():
    rng = np.random.default_rng(31)
    w = wl.C1
    x = rand_bf16(rng, (1, 8192))
    W = rand_bf16(rng, (w.N, 8192), 0.011)
    table = wl.rope_table(64).numpy()
    c1 = np.zeros((64, 1, 16, 128), np.uint16)
    c2 = c1.copy()
    y, p = oracle.front(x, W, np.array([17]), np.array([100]), table, 1, EPS, c1, nthreads=2)
    z, _ = oracle.project(x, W)
    p2 = oracle.round_projection(z)
    np.testing.assert_array_equal(p, p2)
    y2 = oracle.epilogue(p2, np.array([17]), np.array([100]), table, 1, EPS, c2)
    np.testing.assert_array_equal(y, y2)
    np.testing.assert_array_equal(c1, c2)
