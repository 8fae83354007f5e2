"""The streaming-read probe (measurement context, not a step of the method)
reads every byte of its buffer: each thread's XOR of its 16-byte pieces, as
the header defines the split of the buffer, matches the same XOR on the host."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import kv_insert_amd as qf

from helpers import say

pytestmark = pytest.mark.gpu


def host_xor(words: np.ndarray, quanta: int) -> np.ndarray:
    """words: uint32 view of the buffer.  Block b owns pieces
    [b * per * 512, (b + 1) * per * 512) (per = quanta); thread t of it the
    pieces t, t + 512, ...; a piece is 4 words."""
    pieces = words.reshape(256, quanta, 512, 4)          # [block][k][thread][word]
    return np.bitwise_xor.reduce(np.bitwise_xor.reduce(pieces, axis=3), axis=1).reshape(-1)


@pytest.mark.parametrize("quanta", [1, 3, 8, 9, 16, 17, 20, 32])
def test_stream_read_reads_every_byte(quanta):
    n = quanta * qf.STREAM_QUANTUM // 4
    g = torch.Generator().manual_seed(500 + quanta)
    host = torch.randint(-(2 ** 31), 2 ** 31 - 1, (n,), generator=g, dtype=torch.int32)
    src = host.cuda()
    sink = torch.full((256 * 512,), -1, dtype=torch.int32, device="cuda")
    say(f"stream_read {quanta} x 2 MiB")
    qf.stream_read(src, sink)
    torch.cuda.synchronize()
    want = host_xor(host.numpy().view(np.uint32), quanta)
    got = sink.cpu().numpy().view(np.uint32)
    assert np.array_equal(got, want)


def test_stream_read_refuses_a_partial_quantum_on_device():
    src = torch.zeros(qf.STREAM_QUANTUM // 4 + 4, dtype=torch.int32, device="cuda")
    sink = torch.zeros(256 * 512, dtype=torch.int32, device="cuda")
    with pytest.raises(qf.QkvfError):
        qf.stream_read(src, sink)
