"""Tie-aware comparison of a front result against the oracle (test infra).

The qkv_front page (module summary) defines the result only up to the fp32
summation order of the projection.  Any fp32 order gives the exact sum up to
a small error, so the bf16-rounded projection p is unique except where the
exact sum lies within that error of a bf16 rounding midpoint; there both
neighbours are correct.  For v and gate columns a one-unit difference in p
always fits the tolerance below.  For q and k heads it passes through the
norm and the rotation, where a cancelling pair can turn it into an absolute
error above the tolerance; so a q or k head that fails the plain check is
re-derived with the oracle's own head function for every combination of the
alternative roundings of its near-tie elements, and passes if any
combination matches.

Tolerance on every floating-point output (bf16 values widened exactly):
    |gpu - oracle| <= RTOL * |oracle| + ATOL.
The cache is checked bit for bit: every slot the call does not own keeps its
old bits, and the slot of token m holds exactly the k | v columns of the
result row m (K then V for each KV head).
"""
from __future__ import annotations

import itertools

import numpy as np

from . import (HEAD_DIM, PAGE_SLOTS, QHEADS_PER_KV, attn2, bf16_to_float, epilogue,
               head, layer_front, n_cols, project, round_projection)

RTOL = 1.6e-2
ATOL = 2e-3
# Half-width of the window around a bf16 rounding midpoint inside which the
# exact projection may round either way under some fp32 summation order, in
# units of 2^-24 * sum_k |x_k W_nk|.
TIE_WINDOW = 16.0
# Smallest effect on a normed value for which an alternative rounding is
# enumerated; smaller flips cannot break ATOL.
MIN_FLIP_EFFECT = 1e-4
MAX_ENUM = 12


class ParityError(AssertionError):
    pass


def _within(gpu: np.ndarray, ref: np.ndarray) -> np.ndarray:
    return np.abs(gpu - ref) <= RTOL * np.abs(ref) + ATOL


def _other_neighbour(bits: int, z: float) -> int | None:
    """The bf16 neighbour of `bits` on the side of the exact value z."""
    v = float(bf16_to_float(np.uint16(bits)))
    if z == v:
        return None
    up = z > v
    neg = bool(bits & 0x8000)
    mag = bits & 0x7FFF
    if (up and not neg) or (not up and neg):
        return (bits + 1) & 0xFFFF          # away from zero
    if mag == 0:                             # crossing zero
        return 0x8001 if up is False else 0x0001
    return (bits - 1) & 0xFFFF              # toward zero


def _near_ties(z_row, a_row, p_row, cols):
    """Columns of a head whose exact value lies near a rounding midpoint,
    with their alternative bf16 rounding."""
    out = []
    for c in cols:
        z = float(z_row[c])
        b = int(p_row[c])
        alt = _other_neighbour(b, z)
        if alt is None:
            continue
        mid = 0.5 * (float(bf16_to_float(np.uint16(b))) + float(bf16_to_float(np.uint16(alt))))
        window = TIE_WINDOW * 2.0 ** -24 * float(a_row[c]) + 2.0 ** -24 * abs(z)
        if abs(z - mid) <= window:
            out.append((c, alt))
    return out


def check_front(x, W, positions, slots, cos_sin, nkv: int, eps: float,
                cache_before: np.ndarray, y_gpu: np.ndarray,
                cache_gpu: np.ndarray, nthreads: int = 1,
                oracle_state=None) -> dict:
    """Compare one front call's outputs against the oracle.

    All bf16 arrays are uint16 bit patterns: x [M, 8192], W [N, 8192], y_gpu
    [M, N], caches [pages, nkv, 16, 128].  Raises ParityError on a mismatch;
    returns a small report.  oracle_state (optional) is a (z, abs_sum) pair
    from an earlier oracle.project on the same x and W.
    """
    x = np.ascontiguousarray(x, dtype=np.uint16)
    M, N = x.shape[0], n_cols(nkv)
    assert W.shape[0] == N and y_gpu.shape == (M, N)
    if oracle_state is None:
        z, a = project(x, W, nthreads)
    else:
        z, a = oracle_state
    p = round_projection(z)
    cache_ref = np.array(cache_before, copy=True)
    y_ref = epilogue(p, positions, slots, cos_sin, nkv, eps, cache_ref)

    yg = bf16_to_float(y_gpu)
    yr = bf16_to_float(y_ref)
    ok = _within(yg, yr)
    nq = QHEADS_PER_KV * nkv
    qk_cols = (nq + nkv) * HEAD_DIM
    report = {"elements": int(M * N), "plain_fail": int((~ok).sum()),
              "tie_rescued_heads": 0, "max_ratio": 0.0}
    # v and gate columns: the plain check is the whole check.
    bad_vg = np.argwhere(~ok[:, qk_cols:])
    if bad_vg.size:
        m, c = bad_vg[0]
        c += qk_cols
        raise ParityError(
            f"v/gate mismatch at token {m} column {c}: gpu {yg[m, c]!r} "
            f"oracle {yr[m, c]!r} ({len(bad_vg)} elements)")
    # q and k heads: failing heads get the tie-aware retry.
    for m in range(M):
        cs_row = None if cos_sin is None else np.asarray(cos_sin)[int(positions[m])]
        bad_heads = sorted({c // HEAD_DIM for c in np.flatnonzero(~ok[m, :qk_cols])})
        for h in bad_heads:
            cols = range(h * HEAD_DIM, (h + 1) * HEAD_DIM)
            ties = _near_ties(z[m], a[m], p[m], cols)
            pv = bf16_to_float(p[m, h * HEAD_DIM:(h + 1) * HEAD_DIM])
            r = 1.0 / np.sqrt(np.mean(pv * pv) + eps)
            ties = [(c, alt) for c, alt in ties
                    if abs(float(bf16_to_float(np.uint16(alt))) -
                           float(bf16_to_float(p[m, c]))) * r >= MIN_FLIP_EFFECT]
            ties.sort(key=lambda t: -abs(float(bf16_to_float(np.uint16(t[1]))) -
                                         float(bf16_to_float(p[m, t[0]]))))
            ties = ties[:MAX_ENUM]
            gpu_head = yg[m, h * HEAD_DIM:(h + 1) * HEAD_DIM]
            rescued = False
            for choice in itertools.product((0, 1), repeat=len(ties)):
                if not any(choice):
                    continue
                ph = np.array(p[m, h * HEAD_DIM:(h + 1) * HEAD_DIM], copy=True)
                for (c, alt), take in zip(ties, choice):
                    if take:
                        ph[c - h * HEAD_DIM] = alt
                alt_out, _ = head(ph, cs_row, eps)
                if np.all(_within(gpu_head, bf16_to_float(alt_out))):
                    rescued = True
                    break
            if not rescued:
                c = h * HEAD_DIM + int(np.flatnonzero(~ok[m, h * HEAD_DIM:(h + 1) * HEAD_DIM])[0])
                raise ParityError(
                    f"q/k head mismatch at token {m} head {h} column {c}: gpu "
                    f"{yg[m, c]!r} oracle {yr[m, c]!r}; {len(ties)} near-tie "
                    f"elements tried")
            report["tie_rescued_heads"] += 1
    err = np.abs(yg - yr) / (RTOL * np.abs(yr) + ATOL)
    report["max_ratio"] = float(err[ok].max()) if ok.any() else 0.0

    # Cache: placement and untouched slots, bit for bit.
    expect = np.array(cache_before, copy=True)
    k_col = nq * HEAD_DIM
    v_col = k_col + nkv * HEAD_DIM
    for m in range(M):
        s = int(slots[m])
        if s < 0:
            continue
        page, off = divmod(s, PAGE_SLOTS)
        for j in range(nkv):
            expect[page, j, off, :HEAD_DIM] = y_gpu[m, k_col + j * HEAD_DIM:k_col + (j + 1) * HEAD_DIM]
            expect[page, j, off, HEAD_DIM:] = y_gpu[m, v_col + j * HEAD_DIM:v_col + (j + 1) * HEAD_DIM]
    if not np.array_equal(expect, cache_gpu):
        diff = np.argwhere(expect != cache_gpu)
        raise ParityError(f"cache differs from the expected placement at "
                          f"{tuple(diff[0])} ({len(diff)} elements)")
    return report


def check_attn2(out, q, gate, kv_cache, nkv: int, block_table, seq_lens, window: int = 0):
    """Compare an attn2 result (uint16 bf16 bits [8 R, >= 512 nkv]) with the
    oracle on the same inputs, element by element, to RTOL / ATOL.

    The attention output is one fp32-order-dependent real per element before
    its final bf16 rounding, so a correct result differs from the oracle by
    its summation error plus at most one bf16 unit (2^-8 relative), both far
    inside RTOL; no tie enumeration is needed."""
    ref = attn2(q, gate, kv_cache, nkv, block_table, seq_lens, window)
    width = QHEADS_PER_KV * nkv * HEAD_DIM
    got = bf16_to_float(np.ascontiguousarray(out[:, :width]))
    want = bf16_to_float(ref)
    ok = _within(got, want)
    if not ok.all():
        rows, cols = np.nonzero(~ok)
        i = int(np.argmax(np.abs(got - want) * ~ok))
        r, c = divmod(i, width)
        raise ParityError(
            f"attn2: {len(rows)} of {got.size} outputs outside tolerance; worst at row {r} "
            f"(request {r // 8}, token {r % 8}) head {c // HEAD_DIM} dim {c % HEAD_DIM}: "
            f"gpu {got[r, c]!r} oracle {want[r, c]!r}")
    err = np.abs(got - want)
    return {"outputs": int(got.size), "max_abs_err": float(err.max()),
            "max_err_over_tol": float((err / (RTOL * np.abs(want) + ATOL)).max())}


# LayerFront: a bf16 output whose exact value lies within this relative
# distance of a rounding midpoint may round either way under fp32 arithmetic
# (the row's fp32 sum of squares, the root and two products: < 2^-20).
LF_TIE_REL = 2.0 ** -19


def check_layer_front(x, weight, eps, stream, out, aux=None):
    """Compare a LayerFront result with the oracle: stream and aux bit for
    bit; out bit for bit except where the exact value is within LF_TIE_REL of
    a bf16 rounding midpoint, where the other neighbour is also correct.
    x: uint16 bf16 bits or float32 [rows, 8192]; outputs as numpy arrays
    (stream / aux float32, out uint16)."""
    want_s, want_a, want_o, ex = layer_front(x, weight, eps, aux=aux is not None, exact=True)
    if not np.array_equal(np.asarray(stream).view(np.uint32), want_s.view(np.uint32)):
        bad = np.argwhere(np.asarray(stream).view(np.uint32) != want_s.view(np.uint32))
        raise ParityError(f"layer_front stream differs at {len(bad)} places, first {bad[0].tolist()}")
    if aux is not None and not np.array_equal(np.asarray(aux).view(np.uint32),
                                              want_a.view(np.uint32)):
        raise ParityError("layer_front aux differs from the stream")
    out = np.asarray(out, dtype=np.uint16)
    diff = out != want_o
    ties = 0
    if diff.any():
        g = bf16_to_float(out[diff]).astype(np.float64)
        e = ex[diff]
        # half a bf16 unit at e, plus the tie window
        ae = np.abs(e)
        expo = np.floor(np.log2(np.where(ae > 0, ae, 1.0)))
        half = np.ldexp(1.0, (expo - 8).astype(np.int64))
        ok = (ae > 0) & (np.abs(g - e) <= half + LF_TIE_REL * ae)
        if not ok.all():
            idx = np.argwhere(diff)[~ok][0]
            r, k = int(idx[0]), int(idx[1])
            raise ParityError(
                f"layer_front out: {int((~ok).sum())} of {out.size} values wrong; first at row {r} "
                f"column {k}: gpu {bf16_to_float(out[r, k])!r} oracle "
                f"{bf16_to_float(want_o[r, k])!r} exact {ex[r, k]!r}")
        ties = int(diff.sum())
    return {"values": int(out.size), "tie_flips": ties}
