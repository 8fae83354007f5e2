"""The C-ABI boundary without a GPU: the library loads, exports what the
header declares, and refuses malformed calls with the documented status
before touching a device."""
import ctypes
import os
import re
import threading

import pytest

import kv_insert_amd as qf
from kv_insert_amd import build as qbuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qkvf.h")


@pytest.fixture(scope="module")
def L():
    if qbuild.is_stale():
        qbuild.build()
    return qf.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qkvf_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_exports():
    assert declared_functions() == sorted(qf.EXPORTS)


def test_library_exports_every_declared_symbol(L):
    for name in declared_functions():
        assert hasattr(L, name), name
    out = os.popen(f"nm -D --defined-only {qf.LIB_PATH}").read()
    for name in declared_functions():
        assert re.search(rf"\bT {name}\b", out), name


def test_status_codes_match_header():
    text = open(HEADER).read()
    pairs = dict((int(v), k) for k, v in re.findall(r"(QKVF_[A-Z_]+)\s*=\s*(\d+)", text))
    assert pairs == qf.STATUS


def test_strerror_is_distinct_text(L):
    texts = [qf.strerror(s) for s in qf.STATUS]
    assert all(texts) and len(set(texts)) == len(texts)
    assert qf.strerror(999) == "unknown qkvf status"


@pytest.mark.parametrize("nkv", [1, 2, 4, 8])
def test_plan_is_a_function_of_shape(L, nkv):
    N = qf.n_cols(nkv)
    for M in (1, 8, 16):
        p = qf.plan(N, M)
        # 2 KV heads below 12 token rows split K 4 ways (fewer, larger tiles)
        S = 4 if nkv == 8 or (nkv == 2 and M < 12) else 8
        H = N // 64
        if nkv >= 4:
            # whole heads per XCD; its 32 blocks share their 16-row tiles
            heads = [(x + 1) * H // 8 - x * H // 8 for x in range(8)]
            tiles = [h * 4 * S // 32 for h in heads]       # per block on XCD x
            assert all(h * 4 * S % 32 == 0 for h in heads)
            # every W row tile and every K split is covered exactly once
            assert sum(32 * t for t in tiles) == (N // 16) * S
        else:
            # N / 8 rows per XCD in 32 / S groups: a short tile, then 16-row tiles
            rows = N // 8 // (32 // S)
            assert rows == 36 * nkv * S // 8 and 8 * (32 // S) * rows == N
            tiles = [-(-rows // 16)]
        assert p == {"grid": 256, "k_splits": S, "waves_per_block": 8,
                     "tiles_per_block": max(tiles)}
        assert max(tiles) == {1: 3, 2: 3 if S == 4 else 5, 4: 9, 8: 9}[nkv]


def test_plan_rejects_bad_shapes(L):
    with pytest.raises(qf.QkvfError) as e:
        qf.plan(1000, 4)
    assert e.value.code == "QKVF_ERR_SHAPE"
    for M in (0, 17, -1):
        with pytest.raises(qf.QkvfError) as e:
            qf.plan(1152, M)
        assert e.value.code == "QKVF_ERR_ROWS"


def test_workspace_size_is_constant(L):
    # 32-bit partials [splits][16 rows][N] with splits * N = 36864 for every
    # nkv, then 64 words (fault word, padding) and 256 scratch words
    assert qf.workspace_bytes() == 36864 * 16 * 4 + 64 * 4 + 256 * 4


def test_fault_word_and_spin_limit_without_a_workspace(L):
    assert L.qkvf_fault_word(None) == 5
    word = ctypes.c_void_p(1)
    res = []

    def fresh():
        res.append(L.qkvf_fault_word(ctypes.byref(word)))

    t = threading.Thread(target=fresh)
    t.start()
    t.join()
    assert res[0] in (1, 6)          # no device here, or nothing prepared on it
    assert word.value is None        # cleared on refusal
    assert L.qkvf_set_spin_limit(1) == 0
    assert L.qkvf_set_spin_limit(0) == 0


@pytest.mark.parametrize("N,nkv,M,code", [
    (1152, 3, 4, 2), (2304, 1, 4, 2), (9216, 8, 0, 3), (9216, 8, 17, 3),
    (1153, 1, 1, 2), (0, 0, 1, 2),
])
def test_prepare_rejects_bad_shapes_before_the_device(L, N, nkv, M, code):
    assert L.qkvf_prepare(N, nkv, M) == code


def test_run_without_prepare_is_refused(L):
    res = []

    def fresh_thread():  # the bound shape is per thread
        res.append(L.qkvf_run(16, 16, 16, 16, 16, 16, 16, 1, None))

    t = threading.Thread(target=fresh_thread)
    t.start()
    t.join()
    assert res == [6]


def test_check_refuses_in_order(L):
    P = 1 << 20  # aligned stand-in addresses; never dereferenced
    good = dict(x=P, W=2 * P, positions=3 * P, slots=4 * P, cos_sin=5 * P, y=6 * P,
                kv_cache=7 * P)

    def chk(N=9216, nkv=8, M=8, pages=16, rows=16, **kw):
        a = dict(good, **kw)
        return L.qkvf_check(N, nkv, M, pages, rows, a["x"], a["W"], a["positions"],
                            a["slots"], a["cos_sin"], a["y"], a["kv_cache"], 0)

    assert chk(N=9215) == 2
    assert chk(M=0) == 3
    for name in ("x", "W", "positions", "slots", "y", "kv_cache"):
        assert chk(**{name: None}) == 5, name
    for name in ("x", "W", "y", "kv_cache", "cos_sin"):
        assert chk(**{name: good[name] + 8}) == 4, name
    for name in ("positions", "slots"):
        assert chk(**{name: good[name] + 4}) == 4, name
    assert chk(pages=0) == 9


def test_set_handoff_modes(L):
    assert L.qkvf_set_handoff(2) == 9
    assert L.qkvf_set_handoff(-1) == 9
    assert L.qkvf_set_handoff(1) == 0
    assert L.qkvf_set_handoff(0) == 0


def test_no_device_here_means_device_error(L):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert L.qkvf_prepare(1152, 1, 1) == 1


@pytest.mark.parametrize("nkv,mml,window,reqs,splits", [
    (8, 131072, 0, 1, 32), (8, 32768, 0, 2, 32), (1, 131072, 0, 1, 64), (2, 4096, 0, 1, 32),
    (4, 8192, 0, 3, 64), (8, 2048, 0, 1, 16), (8, 128, 0, 1, 1), (8, 129, 0, 1, 2),
    (8, 256, 0, 1, 2), (8, 257, 0, 1, 3), (8, 131072, 4096, 2, 32), (8, 131072, 4096, 1, 32),
    (8, 131072, 8192, 1, 32), (2, 2048, 4096, 1, 16),
    (1, 8, 0, 1, 1), (8, 131072, 0, 64, 1), (8, 131072, 0, 40, 1), (8, 131072, 0, 31, 32),
    (1, 2048, 1, 1, 1), (2, 131072, 0, 40, 128), (1, 131072, 0, 64, 256), (1, 256, 0, 64, 128),
    (4, 256, 0, 2, 4), (4, 128, 0, 2, 1), (8, 4096, 0, 32, 1),
])
def test_attn2_plan(L, nkv, mml, window, reqs, splits):
    """Split slots per KV head: ceil(256 / nkv), capped by reqs x the splits
    one request can take (one per 128 keys of the span, max_model_len or
    window + 7, and at most 64); 1 when that is not more than reqs (every
    request one split, no merge)."""
    import ctypes
    z = ctypes.c_int(-1)
    assert L.qkvf_attn2_plan(nkv, mml, window, reqs, ctypes.byref(z)) == 0
    assert z.value == splits
    assert qf.attn2_plan(nkv, mml, window, reqs) == splits
    assert L.qkvf_attn2_plan(nkv, mml, window, 0, None) == 3
    assert L.qkvf_attn2_plan(nkv, mml, window, 65, None) == 3


@pytest.mark.parametrize("nkv,mml,reqs,window,code", [
    (3, 4096, 1, 0, 2), (0, 4096, 1, 0, 2), (8, 7, 1, 0, 2), (8, 4096, 1, -1, 2),
    (8, 4096, 0, 0, 3), (8, 4096, 65, 0, 3),
])
def test_attn2_prepare_rejects_bad_shapes_before_the_device(L, nkv, mml, reqs, window, code):
    assert L.qkvf_attn2_prepare(nkv, mml, reqs, window) == code
    assert L.qkvf_attn2_plan(nkv, mml, max(window, 0), 1, None) in (0, 2)


def test_attn2_prepare_ex_refuses_an_unknown_mode(L):
    assert L.qkvf_attn2_prepare_ex(8, 4096, 1, 0, 2) == 9
    assert L.qkvf_attn2_prepare_ex(8, 4096, 1, 0, -1) == 9
    assert L.qkvf_attn2_prepare_ex(3, 4096, 1, 0, 1) == 2
    assert L.qkvf_attn2_prepare_ex(8, 4096, 65, 0, 1) == 3


def test_attn2_run_without_prepare_is_refused(L):
    res = []

    def fresh_thread():
        res.append(L.qkvf_attn2_run(16, 4096, 16, 4096, 16, 16, 1, 16, 1, 16, 4096, None))

    t = threading.Thread(target=fresh_thread)
    t.start()
    t.join()
    assert res == [6]


def test_route_refusals_before_the_device(L):
    P = 1 << 20
    assert L.qkvf_route(P, 256, P, 1.0, 0, P, P, None) == 3
    assert L.qkvf_route(P, 256, P, 1.0, 9, P, P, None) == 3
    assert L.qkvf_route(P, 255, P, 1.0, 1, P, P, None) == 2
    assert L.qkvf_route(P, 256, P, float("nan"), 1, P, P, None) == 2
    assert L.qkvf_route(None, 256, P, 1.0, 1, P, P, None) == 5
    assert L.qkvf_route(P + 4, 256, P, 1.0, 1, P, P, None) == 4
    assert L.qkvf_route(P, 258, P, 1.0, 1, P, P, None) == 4


def test_layer_front_refusals_before_the_device(L):
    P = 1 << 20
    assert L.qkvf_layer_front(P, 2, 1, None, 1e-6, P, None, P, None) == 2
    assert L.qkvf_layer_front(P, 0, 1, None, -1.0, P, None, P, None) == 2
    assert L.qkvf_layer_front(P, 0, -1, None, 1e-6, P, None, P, None) == 3
    assert L.qkvf_layer_front(P, 0, (1 << 20) + 1, None, 1e-6, P, None, P, None) == 3
    assert L.qkvf_layer_front(P, 0, 0, None, 1e-6, P, None, P, None) == 0
    assert L.qkvf_layer_front(None, 0, 1, None, 1e-6, P, None, P, None) == 5
    assert L.qkvf_layer_front(P + 16, 1, 1, None, 1e-6, P, None, P, None) == 4
    assert L.qkvf_layer_front(P, 0, 1, P + 2, 1e-6, P, None, P, None) == 4


def test_stream_read_refusals_before_the_device(L):
    P, Q = 1 << 21, qf.STREAM_QUANTUM
    assert L.qkvf_stream_read(None, Q, P, None) == 5
    assert L.qkvf_stream_read(P, Q, None, None) == 5
    assert L.qkvf_stream_read(P, 0, P, None) == 2
    assert L.qkvf_stream_read(P, Q + 16, P, None) == 2
    assert L.qkvf_stream_read(P, (1 << 16) * Q + Q, P, None) == 2
    assert L.qkvf_stream_read(P + 8, Q, P, None) == 4
    assert L.qkvf_stream_read(P, Q, P + 2, None) == 4


def test_run_static_refusals_before_the_device(L):
    P = 1 << 20
    args = [P, P, P, P, P, P, P]
    assert L.qkvf_run_static(1152, 3, *args, 1, None) == 2
    assert L.qkvf_run_static(1000, 1, *args, 1, None) == 2
    assert L.qkvf_run_static(1152, 1, *args, 0, None) == 3
    assert L.qkvf_run_static(1152, 1, *args, 17, None) == 3
    assert L.qkvf_run_static(1152, 1, None, P, P, P, P, P, P, 1, None) == 5
    assert L.qkvf_run_static(1152, 1, P + 8, P, P, P, P, P, P, 1, None) == 4
    import torch
    if not torch.cuda.is_available():
        assert L.qkvf_run_static(1152, 1, *args, 1, None) == 1


def test_header_is_c_and_a_c_program_links_the_library(L, tmp_path):
    """include/qkvf.h compiles as C11 with gcc, and a C program linked
    against libqkvfront.so gets the documented launch shapes and refusals
    (tests/c_consumer/consumer.c; no GPU call)."""
    import subprocess
    exe = tmp_path / "consumer"
    src = os.path.join(ROOT, "tests", "c_consumer", "consumer.c")
    build = subprocess.run(
        ["gcc", "-std=c11", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__",
         "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include", src,
         "-L", os.path.dirname(qf.LIB_PATH), "-lqkvfront",
         "-Wl,-rpath," + os.path.dirname(qf.LIB_PATH), "-o", str(exe)],
        capture_output=True, text=True)
    assert build.returncode == 0, build.stderr[-3000:]
    # Diagnostics from HIP's own headers are not ours; none may name these files.
    for name in ("qkvf.h", "consumer.c"):
        assert name + ":" not in build.stderr, build.stderr[-3000:]
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0 and "failures 0" in run.stdout, run.stdout + run.stderr
