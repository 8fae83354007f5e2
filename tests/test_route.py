"""MuseRouting on the GPU through the C ABI against the oracle, bit for bit
(ids and fp32 weights): random logits at several scales and biases, 1 to 8
tokens, equal keys, the hand-worked fixture, tiny scores where the division
epsilon dominates, saturated logits, strided rows, refusals and HIP-graph
replays."""
from __future__ import annotations

import json
import os

import numpy as np
import pytest
import torch

import kv_insert_amd as qf
import oracle

from helpers import say

pytestmark = pytest.mark.gpu
E, K = 256, 8
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def gpu_route(logits_np, bias_np, scale, stride=None, label=""):
    b = logits_np.shape[0]
    stride = E if stride is None else stride
    assert 1 <= b <= 8 and stride >= E and stride % 4 == 0
    buf = torch.full((b, stride), float("nan"), dtype=torch.float32, device="cuda")
    buf[:, :E] = torch.from_numpy(logits_np).cuda()
    bias = torch.from_numpy(bias_np).cuda()
    ids = torch.full((b + 1, K), -7, dtype=torch.int32, device="cuda")
    w = torch.full((b + 1, K), -7.0, dtype=torch.float32, device="cuda")
    say(f"route {label} tokens={b} stride={stride} scale={scale}")
    qf.route(buf[:, :E] if stride == E else buf, bias, scale, ids, w)
    torch.cuda.synchronize()
    assert bool((ids[b] == -7).all()) and bool((w[b] == -7.0).all()), "wrote past the last token"
    return ids[:b].cpu().numpy(), w[:b].cpu().numpy()


def check(logits_np, bias_np, scale, stride=None, label=""):
    gi, gw = gpu_route(logits_np, bias_np, scale, stride, label)
    oi, ow = oracle.route(logits_np, bias_np, scale)
    assert np.array_equal(gi, oi), f"{label}: ids differ\n{gi}\n{oi}"
    assert np.array_equal(gw.view(np.uint32), ow.view(np.uint32)), f"{label}: weights differ"


@pytest.mark.parametrize("tokens", [1, 3, 8])
@pytest.mark.parametrize("lscale,bscale", [(1.0, 0.0), (2.0, 0.05), (6.0, 0.5), (0.01, 1e-3)])
def test_route_random(tokens, lscale, bscale):
    rng = np.random.default_rng(tokens * 100 + int(lscale * 10) + int(bscale * 1000))
    for trial in range(4):
        logits = (rng.standard_normal((tokens, E)) * lscale).astype(np.float32)
        bias = (rng.standard_normal(E) * bscale).astype(np.float32)
        scale = float(rng.choice([1.0, 2.5, 0.7, 16.0]))
        check(logits, bias, scale, label=f"random {lscale}/{bscale} #{trial}")


def test_route_ties_and_fixture():
    g = json.load(open(os.path.join(GOLDEN, "route_bias_and_tie.json")))
    logits = np.full((1, E), -5.0, np.float32)
    logits[0, 10:18] = 3.0
    logits[0, 5] = 2.0
    bias = np.zeros(E, np.float32)
    bias[5] = 0.5
    ids, w = gpu_route(logits, bias, g["route_scale"], label="fixture")
    assert ids[0].tolist() == g["expected_ids"]
    assert w[0].tolist() == [np.float32(v) for v in g["expected_weights"]]
    # equal keys everywhere, and equal keys made by the bias
    check(np.zeros((2, E), np.float32), np.zeros(E, np.float32), 1.0, label="all equal")
    rng = np.random.default_rng(7)
    lg = rng.standard_normal((4, E)).astype(np.float32)
    lg[:, 40:60] = 0.25                     # twenty equal scores near the top
    check(lg, np.zeros(E, np.float32), 2.0, label="equal block")
    lg2 = np.zeros((3, E), np.float32)
    bias = np.tile(np.array([0.0, 0.125, 0.0, 0.125], np.float32), 64)
    check(lg2, bias, 1.0, label="bias ties")


def test_route_saturated_and_tiny():
    check(np.full((2, E), -80.0, np.float32), np.zeros(E, np.float32), 2.0, label="eps dominates")
    rng = np.random.default_rng(8)
    lg = (rng.choice([-80.0, 80.0], (8, E)) * rng.uniform(0.5, 1.0, (8, E))).astype(np.float32)
    check(lg, (rng.standard_normal(E) * 0.1).astype(np.float32), 1.0, label="saturated")


def test_route_strided_rows():
    rng = np.random.default_rng(9)
    lg = rng.standard_normal((5, E)).astype(np.float32)
    check(lg, (rng.standard_normal(E) * 0.1).astype(np.float32), 1.5, stride=264, label="stride 264")


def test_route_refusals():
    lg = torch.zeros(9, E, device="cuda")
    bias = torch.zeros(E, device="cuda")
    ids = torch.zeros(9, K, dtype=torch.int32, device="cuda")
    w = torch.zeros(9, K, device="cuda")
    with pytest.raises(qf.QkvfError, match="ROWS"):
        qf.route(lg, bias, 1.0, ids, w)                  # 9 tokens
    with pytest.raises(qf.QkvfError, match="ROWS"):
        qf.route(lg[:0], bias, 1.0, ids, w)
    with pytest.raises(qf.QkvfError, match="ALIGN"):
        flat = torch.zeros(E + 4, device="cuda")
        qf.route(lg[:2], flat[1:E + 1], 1.0, ids, w)
    with pytest.raises(qf.QkvfError, match="SHAPE"):
        qf.route(lg[:2], bias, float("inf"), ids, w)


def test_route_graph_replays():
    tokens = 8
    lg = torch.zeros(tokens, E, device="cuda")
    bias = torch.zeros(E, device="cuda")
    ids = torch.zeros(tokens, K, dtype=torch.int32, device="cuda")
    w = torch.zeros(tokens, K, device="cuda")
    stream = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    say("route graph capture")
    with torch.cuda.stream(stream):
        qf.route(lg, bias, 2.5, ids, w, stream=stream)
        stream.synchronize()
        with torch.cuda.graph(graph, stream=stream):
            qf.route(lg, bias, 2.5, ids, w, stream=stream)
    rng = np.random.default_rng(10)
    for i in range(3):
        ln = (rng.standard_normal((tokens, E)) * 3).astype(np.float32)
        bn = (rng.standard_normal(E) * 0.1).astype(np.float32)
        lg.copy_(torch.from_numpy(ln).cuda())
        bias.copy_(torch.from_numpy(bn).cuda())
        torch.cuda.synchronize()
        say(f"route graph replay {i}")
        graph.replay()
        torch.cuda.synchronize()
        oi, ow = oracle.route(ln, bn, 2.5)
        assert np.array_equal(ids.cpu().numpy(), oi)
        assert np.array_equal(w.cpu().numpy().view(np.uint32), ow.view(np.uint32))
