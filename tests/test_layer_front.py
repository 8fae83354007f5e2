"""LayerFront on the GPU through the C ABI against the oracle: bf16 and fp32
inputs, with and without the norm's weight and the aux copy, one to many
rows, outlier, tiny and zero rows, the fp32 stream updated in place, canaries
around every output, refusals, and HIP-graph replays."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import kv_insert_amd as qf
from kv_insert_amd import workloads as wl
from oracle import checker

from helpers import say, to_bits

pytestmark = pytest.mark.gpu
H = 8192
CANARY_F32 = 0x7F800001   # a signalling-NaN pattern no result can take
CANARY_BF16 = 0x7F7F


def host_x(rows, dtype, seed, scale_rows=None):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(rows, H, generator=g)
    if scale_rows:
        for r, s in scale_rows.items():
            x[r] *= s
    return x.to(torch.bfloat16) if dtype == "bf16" else x


def padded(rows, dtype, fill):
    """A device buffer with one canary row before and after the data."""
    buf = torch.empty(rows + 2, H, dtype=dtype, device="cuda")
    buf.view(torch.int32 if dtype == torch.float32 else torch.int16).fill_(fill)
    return buf, buf[1:rows + 1]


def canaries_intact(buf, fill):
    v = buf.view(torch.int32 if buf.dtype == torch.float32 else torch.int16)
    return bool((v[0] == fill).all()) and bool((v[-1] == fill).all())


def np_x(x):
    return to_bits(x) if x.dtype == torch.bfloat16 else x.numpy()


def run_case(x, weight=None, eps=1e-6, aux=True, label=""):
    rows = x.shape[0]
    xd = x.cuda()
    wd = None if weight is None else weight.cuda()
    sbuf, s = padded(rows, torch.float32, CANARY_F32)
    obuf, o = padded(rows, torch.bfloat16, CANARY_BF16)
    abuf, a = padded(rows, torch.float32, CANARY_F32) if aux else (None, None)
    say(f"layer_front {label} rows={rows} dtype={x.dtype} weight={weight is not None} aux={aux}")
    qf.layer_front(xd, s, o, aux=a, weight=wd, eps=eps)
    torch.cuda.synchronize()
    assert canaries_intact(sbuf, CANARY_F32) and canaries_intact(obuf, CANARY_BF16)
    if aux:
        assert canaries_intact(abuf, CANARY_F32)
    stats = checker.check_layer_front(np_x(x), None if weight is None else to_bits(weight), eps,
                                      s.cpu().numpy(), to_bits(o.cpu()),
                                      None if a is None else a.cpu().numpy())
    return stats


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("rows", [1, 8, 16, 300])
def test_layer_front_rows_and_dtypes(dtype, rows):
    x = host_x(rows, dtype, seed=rows + (7 if dtype == "f32" else 0))
    g = torch.Generator().manual_seed(99)
    w = (1.0 + 0.1 * torch.randn(H, generator=g)).to(torch.bfloat16)
    run_case(x, weight=w, aux=True, label="weighted")
    run_case(x, weight=None, aux=False, label="weightless")


def test_layer_front_outlier_tiny_and_zero_rows():
    x = host_x(16, "f32", seed=3, scale_rows={0: 30.0, 1: 1e-4, 2: 0.0, 3: 1e6})
    run_case(x, label="f32 extremes")
    run_case(x.to(torch.bfloat16), label="bf16 extremes")
    out = torch.empty(16, H, dtype=torch.bfloat16, device="cuda")
    s = torch.empty(16, H, device="cuda")
    qf.layer_front(x.cuda(), s, out)
    torch.cuda.synchronize()
    # the row is +0 and -0 (x times 0.0 keeps the sign); its outputs are zeros
    assert bool((out[2].float() == 0).all()), "a zero row must give zeros"
    assert bool(torch.isfinite(out.float()).all())


def test_layer_front_eps_values():
    x = host_x(4, "bf16", seed=4, scale_rows={1: 1e-3, 2: 1e-2})
    for eps in (0.0, 1e-6, 1e-5, 1e-2):
        run_case(x, eps=eps, aux=False, label=f"eps={eps}")


def test_layer_front_stream_in_place():
    """With an fp32 x, the stream may be x itself."""
    x = host_x(16, "f32", seed=5)
    g = torch.Generator().manual_seed(5)
    w = (1.0 + 0.1 * torch.randn(H, generator=g)).to(torch.bfloat16)
    xd = x.cuda()
    out = torch.empty(16, H, dtype=torch.bfloat16, device="cuda")
    aux = torch.empty(16, H, device="cuda")
    say("layer_front in place")
    qf.layer_front(xd, xd, out, aux=aux, weight=w.cuda())
    torch.cuda.synchronize()
    checker.check_layer_front(x.numpy(), to_bits(w), 1e-6, xd.cpu().numpy(), to_bits(out.cpu()),
                              aux.cpu().numpy())


def test_layer_front_refusals_and_empty():
    x = torch.zeros(4, H, dtype=torch.bfloat16, device="cuda")
    s = torch.empty(4, H, device="cuda")
    o = torch.empty(4, H, dtype=torch.bfloat16, device="cuda")
    qf.layer_front(x[:0], s[:0], o[:0])      # rows == 0: nothing to do
    with pytest.raises(qf.QkvfError, match="ALIGN"):
        flat = torch.empty(4 * H + 8, device="cuda")
        qf.layer_front(x, flat[4:4 + 4 * H].view(4, H), o)
    with pytest.raises(qf.QkvfError, match="SHAPE"):
        qf.layer_front(x, s, o, eps=float("nan"))
    with pytest.raises(qf.QkvfError, match="SHAPE"):
        qf.layer_front(x, s, o, eps=-1.0)


def test_layer_front_graph_replays():
    rows = 16
    x = host_x(rows, "bf16", seed=6)
    xd = x.cuda()
    s = torch.empty(rows, H, device="cuda")
    o = torch.empty(rows, H, dtype=torch.bfloat16, device="cuda")
    a = torch.empty(rows, H, device="cuda")
    stream = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    say("layer_front graph capture")
    with torch.cuda.stream(stream):
        qf.layer_front(xd, s, o, aux=a, stream=stream)
        stream.synchronize()
        with torch.cuda.graph(graph, stream=stream):
            qf.layer_front(xd, s, o, aux=a, stream=stream)
    for i in range(3):
        xn = host_x(rows, "bf16", seed=60 + i)
        xd.copy_(xn.cuda())
        torch.cuda.synchronize()
        say(f"layer_front graph replay {i}")
        graph.replay()
        torch.cuda.synchronize()
        checker.check_layer_front(to_bits(xn), None, 1e-6, s.cpu().numpy(), to_bits(o.cpu()),
                                  a.cpu().numpy())
