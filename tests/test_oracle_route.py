"""Pins of the MuseRouting oracle (sigmoid scores, bias for the selection
only, top-8 of 256, normalised weights) against torch's sigmoid, an
independent sort, closed forms, ties and a hand-worked fixture.  No GPU."""
import json
import os

import numpy as np
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
E, K = oracle.ROUTE_EXPERTS, oracle.ROUTE_TOP_K


def torch_scores(logits):
    return torch.sigmoid(torch.from_numpy(logits.astype(np.float64))).float().numpy()


def sorted_topk(keys):
    """Independent selection: Python's sort on (-key, id)."""
    return [e for _, e in sorted((-float(k), e) for e, k in enumerate(keys))][:K]


def test_score_matches_torch_sigmoid():
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(20000) * 4, np.linspace(-80, 80, 4001)]).astype(np.float32)
    ours = np.array([oracle.route_score(v) for v in x], np.float32)
    ref = torch_scores(x)
    assert np.count_nonzero(ours.view(np.uint32) != ref.view(np.uint32)) <= 2
    assert np.all(np.abs(ours.view(np.int32).astype(np.int64) - ref.view(np.int32)) <= 1)
    assert oracle.route_score(0.0) == 0.5
    assert np.all(np.diff(ours[-4001:]) >= 0)          # monotone


def test_selection_matches_an_independent_sort():
    rng = np.random.default_rng(2)
    for trial in range(40):
        b = rng.integers(1, 9)
        logits = (rng.standard_normal((b, E)) * rng.choice([0.5, 2.0, 6.0])).astype(np.float32)
        bias = (rng.standard_normal(E) * rng.choice([0.0, 0.05, 0.5])).astype(np.float32)
        ids, _ = oracle.route(logits, bias, 1.0)
        for t in range(b):
            keys = torch_scores(logits[t]) + bias
            assert ids[t].tolist() == sorted_topk(keys), (trial, t)


def test_equal_keys_rank_by_lower_id():
    logits = np.full((1, E), -3.0, np.float32)
    logits[0, [200, 7, 99, 150, 3, 64, 250, 31, 128, 12]] = 1.5   # ten equal scores
    ids, w = oracle.route(logits, np.zeros(E, np.float32), 2.0)
    assert ids[0].tolist() == [3, 7, 12, 31, 64, 99, 128, 150]
    assert np.all(w[0] == np.float32(0.25))                         # 2.0 / 8


def test_bias_steers_selection_not_weights():
    rng = np.random.default_rng(3)
    logits = rng.standard_normal((4, E)).astype(np.float32)
    ids0, w0 = oracle.route(logits, np.zeros(E, np.float32), 1.7)
    # a uniform shift changes no ranking and no weight
    ids1, w1 = oracle.route(logits, np.full(E, 0.25, np.float32), 1.7)
    assert np.array_equal(ids0, ids1) and np.array_equal(w0, w1)
    # a large bias pulls in expert e; its weight still comes from its score
    e = int(np.argmin(logits[0]))
    bias = np.zeros(E, np.float32)
    bias[e] = 10.0
    ids2, w2 = oracle.route(logits, bias, 1.7)
    assert ids2[0, 0] == e
    s = torch_scores(logits[0])
    assert w2[0, 0] < w2[0, 1:].min()          # the smallest score, the smallest weight
    assert abs(float(w2[0, 0]) / float(w2[0, 1]) - s[e] / s[ids2[0, 1]]) < 1e-5


def test_weights_closed_forms():
    rng = np.random.default_rng(4)
    logits = rng.standard_normal((8, E)).astype(np.float32) * 3
    for scale in (1.0, 2.5, 0.125):
        ids, w = oracle.route(logits, np.zeros(E, np.float32), scale)
        np.testing.assert_allclose(w.astype(np.float64).sum(1), scale, rtol=2e-7)
        assert np.all(np.diff(w, axis=1) <= 0)     # best first: with no bias, scores descend
    # equal chosen scores: every weight is scale / 8
    logits = np.full((1, E), -4.0, np.float32)
    logits[0, :K] = 2.0
    _, w = oracle.route(logits, np.zeros(E, np.float32), 2.5)
    assert np.all(w == np.float32(0.3125))


def test_golden_bias_and_tie_by_hand():
    g = json.load(open(os.path.join(GOLDEN, "route_bias_and_tie.json")))
    logits = np.full((1, E), -5.0, np.float32)
    logits[0, 10:18] = 3.0
    logits[0, 5] = 2.0
    bias = np.zeros(E, np.float32)
    bias[5] = 0.5
    ids, w = oracle.route(logits, bias, g["route_scale"])
    assert ids[0].tolist() == g["expected_ids"]
    assert w[0].tolist() == [np.float32(v) for v in g["expected_weights"]]


def test_division_epsilon_dominates_tiny_scores():
    """With every score ~1.8e-35 the 1e-15 term dominates the denominator:
    the weights are ~score * scale / 1e-15, not scale / 8."""
    logits = np.full((1, E), -80.0, np.float32)
    ids, w = oracle.route(logits, np.zeros(E, np.float32), 2.0)
    s = float(torch_scores(np.array([-80.0], np.float32))[0])
    assert ids[0].tolist() == list(range(K))        # all keys equal: lowest ids
    np.testing.assert_allclose(w[0].astype(np.float64), s * 2.0 / 1e-15, rtol=1e-6)
