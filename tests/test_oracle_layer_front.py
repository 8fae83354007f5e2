"""Pins of the LayerFront oracle (the first layer's fp32 stream, aux copy
and pre-QKV-projection RMS norm) against closed forms, an independent float64
formula, invariances and a hand-worked fixture.  No GPU."""
import json
import math
import os

import numpy as np
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
H = oracle.HIDDEN
EPS = oracle.LAYER_FRONT_EPS


def bits(a):
    return (torch.from_numpy(np.asarray(a, dtype=np.float32)).to(torch.bfloat16)
            .view(torch.int16).numpy().view(np.uint16))


def reference(x_f32, w=None, eps=EPS):
    """Independent: numpy float64 mean and sqrt, torch's float32 -> bf16."""
    s = x_f32.astype(np.float64)
    r = 1.0 / np.sqrt(np.mean(s * s, axis=1, keepdims=True) + eps)
    v = s * r * (1.0 if w is None else oracle.bf16_to_float(w).astype(np.float64))
    return bits(v.astype(np.float32))


def test_stream_and_aux_are_exact_copies():
    rng = np.random.default_rng(1)
    xb = bits(rng.standard_normal((5, H)))
    s, a, _ = oracle.layer_front(xb, aux=True)
    want = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).float().numpy()
    assert np.array_equal(s.view(np.uint32), want.view(np.uint32))
    assert np.array_equal(a.view(np.uint32), s.view(np.uint32))
    xf = rng.standard_normal((3, H)).astype(np.float32) * 7
    s, a, _ = oracle.layer_front(xf)
    assert a is None and np.array_equal(s.view(np.uint32), xf.view(np.uint32))


def test_matches_independent_float64_formula():
    rng = np.random.default_rng(2)
    for dtype in ("bf16", "f32"):
        x = rng.standard_normal((6, H)).astype(np.float32)
        x[2] *= 30.0                      # an outlier row
        x[4] *= 1e-3                      # a row where eps matters
        w = bits(rng.uniform(0.5, 1.5, H))
        xin = bits(x) if dtype == "bf16" else x
        xf = oracle.bf16_to_float(xin) if dtype == "bf16" else x
        for weight in (None, w):
            _, _, out = oracle.layer_front(xin, weight)
            ref = reference(xf, weight)
            # both round the same real number: equal except where the two
            # float64 evaluations straddle a rounding midpoint (never seen)
            diff = np.count_nonzero(out != ref)
            assert diff <= out.size * 1e-5, (dtype, weight is None, diff)


def test_constant_row_closed_form():
    """A constant row c normalises to c / sqrt(c^2 + eps) exactly."""
    for c in (1.0, 0.5, -3.0, 1e-3, 2e-4):
        x = np.full((1, H), c, np.float32)
        _, _, out = oracle.layer_front(x)
        want = bits(np.float32(c / math.sqrt(c * c + EPS)))
        assert np.all(out == want), c


def test_rms_scale_invariance_and_zero_row():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((3, H)).astype(np.float32)
    x[1] = 0.0
    _, _, out = oracle.layer_front(x)
    o = oracle.bf16_to_float(out).astype(np.float64)
    assert np.all(out[1] == 0)
    ms = np.mean(x[0].astype(np.float64) ** 2)
    assert abs(math.sqrt(np.mean(o[0] ** 2)) - math.sqrt(ms / (ms + EPS))) < 4e-3
    # x30 in fp32 is exact; the normalised row changes only through eps
    _, _, out30 = oracle.layer_front(x * np.float32(30.0))
    assert np.count_nonzero(out30[0] != out[0]) <= H * 1e-3


def test_weight_scales_the_output():
    rng = np.random.default_rng(4)
    x = bits(rng.standard_normal((2, H)))
    _, _, plain = oracle.layer_front(x)
    _, _, one = oracle.layer_front(x, bits(np.ones(H)))
    _, _, two = oracle.layer_front(x, bits(np.full(H, 2.0)))
    assert np.array_equal(one, plain)
    assert np.array_equal(oracle.bf16_to_float(two), 2 * oracle.bf16_to_float(plain))


def test_rows_are_independent():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((7, H)).astype(np.float32)
    _, _, out = oracle.layer_front(x)
    perm = rng.permutation(7)
    _, _, outp = oracle.layer_front(x[perm])
    assert np.array_equal(outp, out[perm])


def test_golden_three_four_by_hand():
    g = json.load(open(os.path.join(GOLDEN, "layer_front_three_four.json")))
    x = np.zeros((1, H), np.float32)
    x[0, 0], x[0, 1] = 3.0, 4.0
    for xin in (x, bits(x)):
        _, _, out = oracle.layer_front(xin)
        assert oracle.bf16_to_float(out[0, :2]).tolist() == g["expected_out_0_1"]
        assert np.all(out[0, 2:] == 0)


def test_checker_accepts_the_oracle_and_rejects_flips():
    from oracle import checker
    rng = np.random.default_rng(6)
    x = bits(rng.standard_normal((2, H)))
    s, a, out = oracle.layer_front(x, aux=True)
    checker.check_layer_front(x, None, EPS, s, out, aux=a)
    bad = out.copy()
    bad[1, 100] ^= 1                       # one unit away, far from a midpoint
    _, _, _, ex = oracle.layer_front(x, exact=True)
    v = ex[1, 100]
    half = 2.0 ** (math.floor(math.log2(abs(v))) - 8)
    if abs(abs(v) - (abs(oracle.bf16_to_float(out[1, 100])) + half)) > 1e-3 * half:
        try:
            checker.check_layer_front(x, None, EPS, s, bad, aux=a)
        except checker.ParityError:
            pass
        else:
            raise AssertionError("a one-unit flip passed")
    s2 = s.copy()
    s2[0, 5] = np.nextafter(s2[0, 5], np.float32(np.inf))
    try:
        checker.check_layer_front(x, None, EPS, s2, out, aux=a)
    except checker.ParityError:
        pass
    else:
        raise AssertionError("a stream difference passed")
