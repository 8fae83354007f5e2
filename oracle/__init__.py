"""CPU oracle of the decode-batch attention front (test infrastructure only).

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` use this package; the library under ``kv_insert_amd`` never
imports it, and it imports nothing from there.  The arithmetic lives in
``qkvf_oracle.c`` (plain loops, double precision); this module builds it with
gcc and marshals numpy arrays through ctypes.

bf16 tensors cross this boundary as ``numpy.uint16`` arrays of their bit
patterns.

What it computes: the projection of 1..16 tokens onto the QKV + o-gate
weights, rounded to bf16, then the per-head weightless RMS norm and the
interleaved rotary embedding of the q and k heads, the output row store and
the K|V insert into the paged cache (qkv_front page, module summary;
cute_ops page, split_qkv and the attn2 contract for the cache layout).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "qkvf_oracle.c")
LIB = os.path.join(HERE, "libqkvf_oracle.so")

HIDDEN = 8192
HEAD_DIM = 64
QHEADS_PER_KV = 8
PAGE_SLOTS = 16
SLOT_WIDTH = 128

_lib = None


def build(force: bool = True) -> str:
    """Compile qkvf_oracle.c into libqkvf_oracle.so next to it."""
    if force or not os.path.exists(LIB):
        tmp = LIB + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
             "-o", tmp, SRC, "-lm"])
        os.replace(tmp, LIB)
    return LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    # QKVF_ORACLE_LIB names another build of qkvf_oracle.c (the sanitizer
    # test loads one compiled with -fsanitize=address,undefined).
    other = os.environ.get("QKVF_ORACLE_LIB")
    if other:
        lib = ctypes.CDLL(other)
    else:
        if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
            build()
        lib = ctypes.CDLL(LIB)
    P = ctypes.c_void_p
    lib.qkvfo_float_to_bf16.restype = ctypes.c_uint16
    lib.qkvfo_float_to_bf16.argtypes = [ctypes.c_float]
    lib.qkvfo_double_to_bf16.restype = ctypes.c_uint16
    lib.qkvfo_double_to_bf16.argtypes = [ctypes.c_double]
    lib.qkvfo_bf16_to_double.restype = ctypes.c_double
    lib.qkvfo_bf16_to_double.argtypes = [ctypes.c_uint16]
    lib.qkvfo_round_array.restype = None
    lib.qkvfo_round_array.argtypes = [P, P, ctypes.c_size_t]
    lib.qkvfo_project.restype = None
    lib.qkvfo_project.argtypes = [P, P, ctypes.c_int, ctypes.c_int, P, P, ctypes.c_int]
    lib.qkvfo_head.restype = None
    lib.qkvfo_head.argtypes = [P, P, ctypes.c_double, P, P]
    lib.qkvfo_epilogue.restype = None
    lib.qkvfo_epilogue.argtypes = [P, P, P, P, ctypes.c_int, ctypes.c_int,
                                   ctypes.c_double, P, P]
    lib.qkvfo_front.restype = None
    lib.qkvfo_front.argtypes = [P, P, P, P, P, ctypes.c_int, ctypes.c_int,
                                ctypes.c_double, P, P, P, P, ctypes.c_int]
    lib.qkvfo_layer_front.restype = None
    lib.qkvfo_layer_front.argtypes = [P, ctypes.c_int, ctypes.c_int64, P, ctypes.c_double, P, P, P,
                                      P]
    lib.qkvfo_route_score.restype = ctypes.c_float
    lib.qkvfo_route_score.argtypes = [ctypes.c_float]
    lib.qkvfo_route.restype = None
    lib.qkvfo_route.argtypes = [P, ctypes.c_int64, P, ctypes.c_double, ctypes.c_int, P, P]
    lib.qkvfo_attn2.restype = None
    lib.qkvfo_attn2.argtypes = [P, ctypes.c_int64, P, ctypes.c_int64, P, ctypes.c_int,
                                P, ctypes.c_int64, P, ctypes.c_int, ctypes.c_int,
                                ctypes.c_double, ctypes.c_double, P, ctypes.c_int64]
    _lib = lib
    return lib


def _ptr(a: np.ndarray | None):
    return None if a is None else a.ctypes.data


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def n_cols(nkv: int) -> int:
    """Output width for nkv KV heads: [q | k | v | gate], 64 columns per head,
    8 q heads and 8 gate heads per KV head (cute_ops page, split_qkv)."""
    return 2 * (QHEADS_PER_KV * nkv + nkv) * HEAD_DIM


def float_to_bf16(v) -> np.ndarray:
    """Round binary32 values to bf16 (nearest, ties to even); bit patterns."""
    lib = _load()
    flat = np.ascontiguousarray(np.asarray(v, dtype=np.float32).ravel())
    out = np.empty(flat.size, dtype=np.uint16)
    lib.qkvfo_round_array(_ptr(flat), _ptr(out), flat.size)
    return out.reshape(np.shape(v))


def bf16_to_float(b) -> np.ndarray:
    """Widen bf16 bit patterns to float64 (exact)."""
    b = np.asarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def project(x: np.ndarray, W: np.ndarray, nthreads: int = 1):
    """z[m, n] = sum_k x[m, k] W[n, k] in double, plus sum_k |x W|.

    x: uint16 [M, 8192], W: uint16 [N, 8192] (bf16 bits)."""
    lib = _load()
    x = _c(x, np.uint16)
    W = _c(W, np.uint16)
    M, N = x.shape[0], W.shape[0]
    assert x.shape[1] == HIDDEN and W.shape[1] == HIDDEN
    z = np.empty((M, N), dtype=np.float64)
    a = np.empty((M, N), dtype=np.float64)
    lib.qkvfo_project(_ptr(x), _ptr(W), M, N, _ptr(z), _ptr(a), nthreads)
    return z, a


def round_projection(z: np.ndarray) -> np.ndarray:
    """bf16 of the double projection, through binary32 (uint16 bits)."""
    f = np.asarray(z, dtype=np.float64).astype(np.float32)
    return float_to_bf16(f)


def head(p: np.ndarray, cs_row: np.ndarray | None, eps: float):
    """Norm (+ rotation when cs_row is given) of one 64-wide head.

    Returns (bf16 bits [64], float64 values before rounding [64])."""
    lib = _load()
    p = _c(p, np.uint16)
    assert p.shape == (HEAD_DIM,)
    cs = None if cs_row is None else _c(cs_row, np.float32)
    out = np.empty(HEAD_DIM, dtype=np.uint16)
    out_d = np.empty(HEAD_DIM, dtype=np.float64)
    lib.qkvfo_head(_ptr(p), _ptr(cs), eps, _ptr(out), _ptr(out_d))
    return out, out_d


def epilogue(p, positions, slots, cos_sin, nkv: int, eps: float, kv_cache):
    """Everything after the rounded projection p (uint16 [M, N]).

    kv_cache (uint16 [pages, nkv, 16, 128]) is updated in place; returns y."""
    lib = _load()
    p = _c(p, np.uint16)
    M, N = p.shape
    assert N == n_cols(nkv)
    positions = _c(positions, np.int64)
    slots = _c(slots, np.int64)
    cs = None if cos_sin is None else _c(cos_sin, np.float32)
    assert kv_cache.dtype == np.uint16 and kv_cache.flags.c_contiguous
    assert kv_cache.shape[1:] == (nkv, PAGE_SLOTS, SLOT_WIDTH)
    y = np.empty((M, N), dtype=np.uint16)
    lib.qkvfo_epilogue(_ptr(p), _ptr(positions), _ptr(slots), _ptr(cs), nkv, M,
                       eps, _ptr(y), _ptr(kv_cache))
    return y


def front(x, W, positions, slots, cos_sin, nkv: int, eps: float, kv_cache,
          nthreads: int = 1):
    """The whole front; kv_cache is updated in place.  Returns (y, p)."""
    lib = _load()
    x = _c(x, np.uint16)
    W = _c(W, np.uint16)
    M, N = x.shape[0], W.shape[0]
    assert N == n_cols(nkv) and x.shape[1] == HIDDEN and W.shape[1] == HIDDEN
    positions = _c(positions, np.int64)
    slots = _c(slots, np.int64)
    cs = None if cos_sin is None else _c(cos_sin, np.float32)
    assert kv_cache.dtype == np.uint16 and kv_cache.flags.c_contiguous
    assert kv_cache.shape[1:] == (nkv, PAGE_SLOTS, SLOT_WIDTH)
    z = np.empty((M, N), dtype=np.float64)
    p = np.empty((M, N), dtype=np.uint16)
    y = np.empty((M, N), dtype=np.uint16)
    lib.qkvfo_front(_ptr(x), _ptr(W), _ptr(positions), _ptr(slots), _ptr(cs),
                    nkv, M, eps, _ptr(z), _ptr(p), _ptr(y), _ptr(kv_cache),
                    nthreads)
    return y, p


ATTN2_SCALE = 0.125   # reading: 1 / sqrt(head_dim)
ATTN2_EPS = 1e-6      # reading: the o-norm epsilon


def attn2(q, gate, kv_cache, nkv: int, block_table, seq_lens, window: int = 0,
          scale: float = ATTN2_SCALE, eps: float = ATTN2_EPS):
    """Paged decode attention of 8 query rows per request with the o-norm and
    sigmoid gate.  q, gate: uint16 [R*8, >= nq*64] (rows may be wider: only
    the first nq*64 columns are read); kv_cache: uint16 [pages, nkv, 16,
    128]; block_table: int32 [R, max_pages]; seq_lens: int32 [R].
    Returns uint16 [R*8, nq*64]."""
    lib = _load()
    q = np.ascontiguousarray(q, dtype=np.uint16)
    gate = np.ascontiguousarray(gate, dtype=np.uint16)
    kv = np.ascontiguousarray(kv_cache, dtype=np.uint16)
    bt = np.ascontiguousarray(block_table, dtype=np.int32)
    sl = np.ascontiguousarray(seq_lens, dtype=np.int32)
    R = sl.shape[0]
    nq = QHEADS_PER_KV * nkv
    assert q.shape[0] == R * 8 and gate.shape[0] == R * 8
    assert q.shape[1] >= nq * HEAD_DIM and gate.shape[1] >= nq * HEAD_DIM
    assert kv.shape[1:] == (nkv, PAGE_SLOTS, SLOT_WIDTH)
    assert bt.shape[0] == R and np.all(sl >= 8)
    assert int(sl.max()) <= bt.shape[1] * PAGE_SLOTS
    out = np.empty((R * 8, nq * HEAD_DIM), dtype=np.uint16)
    lib.qkvfo_attn2(_ptr(q), q.shape[1], _ptr(gate), gate.shape[1], _ptr(kv), nkv,
                    _ptr(bt), bt.shape[1], _ptr(sl), R, int(window), scale, eps,
                    _ptr(out), out.shape[1])
    return out


LAYER_FRONT_EPS = 1e-6   # reading: the pre-QKV-projection norm's epsilon


def layer_front(x, weight=None, eps: float = LAYER_FRONT_EPS, aux: bool = False,
                exact: bool = False):
    """LayerFront of rows of 8192: x is uint16 bf16 bits or float32, shape
    [rows, 8192]; weight uint16 bf16 bits [8192] or None (a weightless norm).
    Returns (stream fp32, aux fp32 or None, out uint16 bf16 bits), plus the
    float64 values before rounding when exact=True."""
    lib = _load()
    x = np.asarray(x)
    if x.dtype == np.float32:
        is_fp32 = 1
    elif x.dtype == np.uint16:
        is_fp32 = 0
    else:
        raise TypeError("x must hold bf16 bits (uint16) or float32")
    x = np.ascontiguousarray(x)
    assert x.ndim == 2 and x.shape[1] == HIDDEN
    rows = x.shape[0]
    w = None if weight is None else np.ascontiguousarray(weight, dtype=np.uint16)
    assert w is None or w.shape == (HIDDEN,)
    stream = np.empty((rows, HIDDEN), np.float32)
    a = np.empty((rows, HIDDEN), np.float32) if aux else None
    out = np.empty((rows, HIDDEN), np.uint16)
    ex = np.empty((rows, HIDDEN), np.float64) if exact else None
    lib.qkvfo_layer_front(_ptr(x), is_fp32, rows, _ptr(w), float(eps), _ptr(stream), _ptr(a),
                          _ptr(out), _ptr(ex))
    return (stream, a, out, ex) if exact else (stream, a, out)


ROUTE_EXPERTS = 256
ROUTE_TOP_K = 8
ROUTE_DIVISION_EPS = 1e-15   # the page's division epsilon


def route_score(logit: float) -> float:
    """The fp32 sigmoid score of one logit (the exact sigmoid rounded once)."""
    return float(_load().qkvfo_route_score(float(logit)))


def route(logits, bias, route_scale: float):
    """MuseRouting of fp32 logits [b, >= 256] with an fp32 bias [256]:
    returns (ids int32 [b, 8], weights fp32 [b, 8]), best first."""
    lib = _load()
    lg = np.ascontiguousarray(logits, dtype=np.float32)
    b = np.ascontiguousarray(bias, dtype=np.float32)
    assert lg.ndim == 2 and lg.shape[1] >= ROUTE_EXPERTS and b.shape == (ROUTE_EXPERTS,)
    tokens = lg.shape[0]
    ids = np.empty((tokens, ROUTE_TOP_K), np.int32)
    w = np.empty((tokens, ROUTE_TOP_K), np.float32)
    lib.qkvfo_route(_ptr(lg), lg.shape[1], _ptr(b), float(route_scale), tokens, _ptr(ids), _ptr(w))
    return ids, w
