"""libqkvfront: the decode-batch attention front on MI355X (gfx950).

A thin ctypes binding of the C ABI declared in include/qkvf.h.  Every step
of the front runs in the HIP kernels of libqkvfront.so; this module only
passes device pointers, sizes and the current stream.  It raises if the
library is not built: there is no other code path.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libqkvfront.so")

HIDDEN = 8192
HEAD_DIM = 64
QHEADS_PER_KV = 8
PAGE_SLOTS = 16
SLOT_WIDTH = 128
MAX_ROWS = 16

STATUS = {
    0: "QKVF_OK", 1: "QKVF_ERR_DEVICE", 2: "QKVF_ERR_SHAPE", 3: "QKVF_ERR_ROWS",
    4: "QKVF_ERR_ALIGN", 5: "QKVF_ERR_NULLPTR", 6: "QKVF_ERR_NOT_PREPARED",
    7: "QKVF_ERR_ALLOC", 8: "QKVF_ERR_HIP", 9: "QKVF_ERR_RANGE",
    10: "QKVF_ERR_OVERLAP", 11: "QKVF_ERR_MEMORY", 12: "QKVF_ERR_TIMEOUT",
}
EXPORTS = ("qkvf_prepare", "qkvf_run", "qkvf_run_static", "qkvf_check", "qkvf_strerror", "qkvf_plan",
           "qkvf_workspace_bytes", "qkvf_set_handoff", "qkvf_set_spin_limit",
           "qkvf_device_fault", "qkvf_fault_word",
           "qkvf_release",
           "qkvf_attn2_prepare", "qkvf_attn2_prepare_ex", "qkvf_attn2_run", "qkvf_attn2_plan", "qkvf_layer_front", "qkvf_route",
           "qkvf_stream_read")


class QkvfError(ValueError):
    """A call the library refused; .status is the qkvf_status code."""

    def __init__(self, status: int, what: str):
        self.status = status
        self.code = STATUS.get(status, str(status))
        super().__init__(f"{what}: {self.code}: {strerror(status)}")


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libqkvfront.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built: run `python -m kv_insert_amd.build` "
                           "or __graft_entry__.build()")
    L = ctypes.CDLL(LIB_PATH)
    P, I, I64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
    L.qkvf_prepare.argtypes = [I, I, I]
    L.qkvf_prepare.restype = I
    L.qkvf_run.argtypes = [P, P, P, P, P, P, P, I, P]
    L.qkvf_run.restype = I
    L.qkvf_run_static.argtypes = [I, I, P, P, P, P, P, P, P, I, P]
    L.qkvf_run_static.restype = I
    L.qkvf_check.argtypes = [I, I, I, I64, I64, P, P, P, P, P, P, P, I]
    L.qkvf_check.restype = I
    L.qkvf_strerror.argtypes = [I]
    L.qkvf_strerror.restype = ctypes.c_char_p
    L.qkvf_plan.argtypes = [I, I, P, P, P, P]
    L.qkvf_plan.restype = I
    L.qkvf_workspace_bytes.argtypes = []
    L.qkvf_workspace_bytes.restype = ctypes.c_size_t
    L.qkvf_set_handoff.argtypes = [I]
    L.qkvf_set_handoff.restype = I
    L.qkvf_device_fault.argtypes = []
    L.qkvf_device_fault.restype = I
    L.qkvf_set_spin_limit.argtypes = [ctypes.c_uint]
    L.qkvf_set_spin_limit.restype = I
    L.qkvf_fault_word.argtypes = [P]
    L.qkvf_fault_word.restype = I
    L.qkvf_attn2_prepare.argtypes = [I, I, I, I]
    L.qkvf_attn2_prepare.restype = I
    L.qkvf_attn2_prepare_ex.argtypes = [I, I, I, I, I]
    L.qkvf_attn2_prepare_ex.restype = I
    L.qkvf_attn2_run.argtypes = [P, I64, P, I64, P, P, I64, P, I, P, I64, P]
    L.qkvf_attn2_run.restype = I
    L.qkvf_attn2_plan.argtypes = [I, I, I, I, P]
    L.qkvf_attn2_plan.restype = I
    L.qkvf_layer_front.argtypes = [P, I, I64, P, ctypes.c_float, P, P, P, P]
    L.qkvf_layer_front.restype = I
    L.qkvf_route.argtypes = [P, I64, P, ctypes.c_double, I, P, P, P]
    L.qkvf_route.restype = I
    L.qkvf_stream_read.argtypes = [P, ctypes.c_size_t, P, P]
    L.qkvf_stream_read.restype = I
    L.qkvf_release.argtypes = []
    L.qkvf_release.restype = None
    _lib = L
    return L


def strerror(status: int) -> str:
    return lib().qkvf_strerror(int(status)).decode()


def n_cols(num_kv_heads: int) -> int:
    return 2 * (QHEADS_PER_KV * num_kv_heads + num_kv_heads) * HEAD_DIM


def _raise(status: int, what: str):
    if status != 0:
        raise QkvfError(status, what)


def prepare(N: int, num_kv_heads: int, M: int = MAX_ROWS) -> None:
    """qkvf_prepare: ready (N, num_kv_heads) for row counts 1..M on the
    current device and bind it as this thread's shape."""
    _raise(lib().qkvf_prepare(int(N), int(num_kv_heads), int(M)), "qkvf_prepare")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream_handle(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def run(x, W, positions, slots, cos_sin, y, kv_cache, M: int | None = None, stream=None) -> None:
    """qkvf_run on torch device tensors; enqueues on `stream` (default: the
    current torch stream).  Shapes are the caller's contract (see qkvf_check)."""
    M = x.shape[0] if M is None else int(M)
    st = lib().qkvf_run(_ptr(x), _ptr(W), _ptr(positions), _ptr(slots), _ptr(cos_sin),
                        _ptr(y), _ptr(kv_cache), M, _stream_handle(stream))
    _raise(st, "qkvf_run")


def run_static(x, W, positions, slots, cos_sin, y, kv_cache, num_kv_heads: int,
               M: int | None = None, stream=None) -> None:
    """qkvf_run_static: qkvf_run without qkvf_prepare and without any
    allocation (the partials pass through the library's static array)."""
    M = x.shape[0] if M is None else int(M)
    st = lib().qkvf_run_static(int(W.shape[0]), int(num_kv_heads), _ptr(x), _ptr(W),
                               _ptr(positions), _ptr(slots), _ptr(cos_sin), _ptr(y),
                               _ptr(kv_cache), M, _stream_handle(stream))
    _raise(st, "qkvf_run_static")


def check(x, W, positions, slots, cos_sin, y, kv_cache, num_kv_heads: int,
          M: int | None = None, read_indices: bool = True) -> int:
    """qkvf_check on torch tensors; returns the status code (0 = ok)."""
    M = x.shape[0] if M is None else int(M)
    N = W.shape[0]
    pages = kv_cache.shape[0]
    rows = 0 if cos_sin is None else cos_sin.shape[0]
    return lib().qkvf_check(int(N), int(num_kv_heads), M, int(pages), int(rows), _ptr(x),
                            _ptr(W), _ptr(positions), _ptr(slots), _ptr(cos_sin), _ptr(y),
                            _ptr(kv_cache), 1 if read_indices else 0)


def plan(N: int, M: int) -> dict:
    """qkvf_plan: the launch shape of (N, M)."""
    vals = [ctypes.c_int() for _ in range(4)]
    _raise(lib().qkvf_plan(int(N), int(M), *[ctypes.byref(v) for v in vals]), "qkvf_plan")
    return dict(zip(("grid", "k_splits", "waves_per_block", "tiles_per_block"),
                    (v.value for v in vals)))


def workspace_bytes() -> int:
    return int(lib().qkvf_workspace_bytes())


def set_handoff(mode: int) -> None:
    """qkvf_set_handoff: 0 = partials stay in the producing XCD's L2 where the
    placement allows (default), 1 = always write through (same results)."""
    _raise(lib().qkvf_set_handoff(int(mode)), "qkvf_set_handoff")


def set_spin_limit(rounds: int) -> None:
    """qkvf_set_spin_limit: polling rounds before a block gives up (0 = the
    default); for tests of the failure path."""
    _raise(lib().qkvf_set_spin_limit(int(rounds)), "qkvf_set_spin_limit")


def device_fault() -> int:
    """qkvf_device_fault: synchronize; 0, or QKVF_ERR_TIMEOUT if a call on the
    current device gave up waiting (its outputs are then invalid)."""
    return int(lib().qkvf_device_fault())


def fault_word_address() -> int:
    """qkvf_fault_word: the device address of the current device's fault
    word (nonzero once a call gave up waiting)."""
    p = ctypes.c_void_p()
    _raise(lib().qkvf_fault_word(ctypes.byref(p)), "qkvf_fault_word")
    return int(p.value)


def release() -> None:
    lib().qkvf_release()


def attn2_prepare(num_kv_heads: int, max_model_len: int, max_reqs: int, window: int = 0,
                  batch_invariant: bool = False) -> None:
    """qkvf_attn2_prepare(_ex): bind a layer's attn2 configuration to this
    thread; batch_invariant fixes the split count at one request's, so a
    request's output does not depend on the rest of its batch."""
    _raise(lib().qkvf_attn2_prepare_ex(int(num_kv_heads), int(max_model_len), int(max_reqs),
                                       int(window), 1 if batch_invariant else 0),
           "qkvf_attn2_prepare")


def attn2_run(q, gate, kv_cache, block_table, seq_lens, out, stream=None) -> None:
    """qkvf_attn2_run on torch tensors: q, gate, out are 2-D bf16 views whose
    rows are the 8 query rows of each request (row strides taken from the
    views); block_table int32 [R, pages]; seq_lens int32 [R]."""
    st = lib().qkvf_attn2_run(_ptr(q), q.stride(0), _ptr(gate), gate.stride(0), _ptr(kv_cache),
                              _ptr(block_table), block_table.stride(0), _ptr(seq_lens),
                              int(seq_lens.shape[0]), _ptr(out), out.stride(0),
                              _stream_handle(stream))
    _raise(st, "qkvf_attn2_run")


def attn2_plan(num_kv_heads: int, max_model_len: int, window: int = 0, num_reqs: int = 1) -> int:
    """qkvf_attn2_plan: the split slots per KV head of a launch for num_reqs
    requests, which the requests share in proportion to their lengths (with
    num_reqs = 1: the request's split count; 1: no merge pass)."""
    z = ctypes.c_int()
    _raise(lib().qkvf_attn2_plan(int(num_kv_heads), int(max_model_len), int(window),
                                 int(num_reqs), ctypes.byref(z)), "qkvf_attn2_plan")
    return z.value


DTYPE_BF16, DTYPE_F32 = 0, 1


def layer_front(x, stream_out, out, aux=None, weight=None, eps: float = 1e-6, stream=None) -> None:
    """qkvf_layer_front on torch tensors: x [rows, 8192] bf16 or fp32,
    stream_out fp32 [rows, 8192] (may be x when x is fp32), out bf16, aux fp32
    or None, weight bf16 [8192] or None; enqueued on `stream` (a torch or HIP
    stream, default the current one)."""
    import torch
    if x.dtype == torch.bfloat16:
        dt = DTYPE_BF16
    elif x.dtype == torch.float32:
        dt = DTYPE_F32
    else:
        raise ValueError("x must be bfloat16 or float32")
    st = lib().qkvf_layer_front(_ptr(x), dt, int(x.shape[0]), _ptr(weight), float(eps),
                                _ptr(stream_out), _ptr(aux), _ptr(out), _stream_handle(stream))
    _raise(st, "qkvf_layer_front")


def route(logits, bias, route_scale: float, ids, weights, stream=None) -> None:
    """qkvf_route on torch tensors: logits fp32 [b, >= 256] (rows 16-byte
    aligned), bias fp32 [256], ids int32 [b, 8], weights fp32 [b, 8]."""
    st = lib().qkvf_route(_ptr(logits), logits.stride(0), _ptr(bias), float(route_scale),
                          int(logits.shape[0]), _ptr(ids), _ptr(weights), _stream_handle(stream))
    _raise(st, "qkvf_route")


STREAM_QUANTUM = 256 * 512 * 16   # qkvf_stream_read reads whole multiples of 2 MiB


def stream_read(src, sink, stream=None) -> None:
    """qkvf_stream_read on torch tensors: src any contiguous device tensor of a
    whole number of 2 MiB (16-byte aligned), sink int32/uint32 [256 * 512]."""
    st = lib().qkvf_stream_read(_ptr(src), src.numel() * src.element_size(), _ptr(sink),
                                _stream_handle(stream))
    _raise(st, "qkvf_stream_read")
