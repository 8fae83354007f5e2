"""Comparison of a front result against the oracle (test infrastructure).

The qkv_front page (module summary) defines the result only up to the fp32
summation order of the projection.  Any fp32 order gives the exact sum up to
a small error, so the bf16-rounded projection p is unique except where the
exact sum lies within that error of a bf16 rounding midpoint; there both
neighbours are correct.  The norm and the rotation run in fp32 on the GPU
and in double in the oracle, so an output o of a q or k head is likewise
unique after its bf16 rounding except where the oracle's exact value lies
within the fp32 error of a midpoint.

check_front therefore compares rounding by rounding, not only to a
tolerance.  A bf16 value is a correct rounding of an exact value e computed
with error at most w when the reals that round to it reach [e - w, e + w]:
that is the oracle's own rounding, its other neighbour near a rounding
midpoint, and, where w exceeds half a unit (a sum that cancels far below its
terms), every value within reach.
  v and gate columns: y must be such a rounding of the exact projection z
      with w = TIE_WINDOW * 2^-24 * sum_k |x_k W_nk| + 2^-24 |z|;
  q and k heads: y must be such a rounding of the oracle's exact output o
      with w = OUT_WINDOW * 2^-24 * (|n_a c| + |n_b s|) + 2 * 2^-24 |o| (n_a,
      n_b the normed pair, c, s its rotation), for the oracle's p or, when
      that fails, for one combination of the other values the head's
      projection elements may take (a different p moves every value of its
      head through the norm, and can move an output of a cancelling pair by
      more than the tolerance); elements whose other values move the normed
      head by less than SMALL_EFFECT widen w by their effect instead;
  the cache bit for bit: every slot the call does not own keeps its old
      bits, and the slot of token m holds exactly the k | v columns of the
      result row m (K then V for each KV head).
Every accepted element also meets the stated tolerance
    |gpu - oracle| <= RTOL * |oracle| + ATOL
against the oracle's value for the rounding it was matched to.
"""
from __future__ import annotations

import itertools

import numpy as np

from . import (HEAD_DIM, PAGE_SLOTS, QHEADS_PER_KV, attn2, bf16_to_float, epilogue,
               head, layer_front, n_cols, project, round_projection)

RTOL = 1.6e-2
ATOL = 2e-3
U = 2.0 ** -24
# Half-width of the window around a bf16 rounding midpoint inside which the
# exact projection may round either way under some fp32 summation order, in
# units of 2^-24 * sum_k |x_k W_nk|.
TIE_WINDOW = 16.0
# The same for an output of a q or k head, in units of
# 2^-24 * (|n_a c| + |n_b s|): the fp32 sum of squares (a 6-level tree),
# its reciprocal square root, the two products and the difference of the
# rotation stay below about 8 of them.
OUT_WINDOW = 16.0
# At most this many near-tie elements of one head are combined (2^12 tries).
MAX_ENUM = 12


class ParityError(AssertionError):
    pass


def _within(gpu: np.ndarray, ref: np.ndarray) -> np.ndarray:
    return np.abs(gpu - ref) <= RTOL * np.abs(ref) + ATOL


def _neighbour_toward(bits, exact):
    """The bf16 neighbour of each `bits` on the side of its exact value
    (bits itself where the exact value equals it).  Vectorised over arrays."""
    bits = np.asarray(bits, dtype=np.uint16).astype(np.int64)
    exact = np.asarray(exact, dtype=np.float64)
    v = bf16_to_float(bits.astype(np.uint16))
    up = exact > v
    down = exact < v
    neg = (bits & 0x8000) != 0
    mag = bits & 0x7FFF
    away = (up & ~neg) | (down & neg)          # larger magnitude, same sign
    toward = (up & neg) | (down & ~neg)        # smaller magnitude
    out = bits.copy()
    out = np.where(away, bits + 1, out)
    out = np.where(toward & (mag != 0), bits - 1, out)
    out = np.where(toward & (mag == 0) & up, 0x0001, out)     # -0 upward
    out = np.where(toward & (mag == 0) & down, 0x8001, out)   # +0 downward
    return (out & 0xFFFF).astype(np.uint16)


def _other_neighbour(bits: int, z: float) -> int | None:
    """The bf16 neighbour of `bits` on the side of the exact value z (None
    when z equals the value of bits)."""
    n = int(_neighbour_toward(np.uint16(bits), z))
    return None if n == int(bits) else n


def _rounding_interval(bits):
    """The reals that round to each bf16 value (to nearest): [lo, hi], the
    midpoints to its neighbours below and above.  Vectorised."""
    bits = np.asarray(bits, dtype=np.uint16)
    v = bf16_to_float(bits)
    up = bf16_to_float(_neighbour_toward(bits, np.full(bits.shape, np.inf)))
    dn = bf16_to_float(_neighbour_toward(bits, np.full(bits.shape, -np.inf)))
    with np.errstate(invalid="ignore", over="ignore"):
        hi = np.where(np.isinf(up), np.inf, 0.5 * (v + up))
        lo = np.where(np.isinf(dn), -np.inf, 0.5 * (v + dn))
    return lo, hi


def _rounding_ok(gpu, exact, window) -> np.ndarray:
    """Per element: gpu is the bf16 rounding of some value within `window`
    of the exact value (its rounding interval reaches [exact - window,
    exact + window]).  The correctly rounded value always passes; where the
    window is below half a unit that allows only the other neighbour of a
    near-tie, where it is larger (a sum that cancels to far below its
    terms) every value within reach."""
    lo, hi = _rounding_interval(gpu)
    exact = np.asarray(exact, dtype=np.float64)
    return (exact >= lo - window) & (exact <= hi + window)


def _p_window(z, a):
    return TIE_WINDOW * U * np.asarray(a, dtype=np.float64) + U * np.abs(z)


def _candidates(p_bits: int, z: float, window: float, cap: int = 64):
    """Every bf16 value a correct projection may take for exact value z:
    the values whose rounding interval reaches z +- window (p_bits first)."""
    out = [int(p_bits)]
    for direction in (np.inf, -np.inf):
        b = int(p_bits)
        for _ in range(cap):
            nb = int(_neighbour_toward(np.uint16(b), direction))
            if nb == b or not _rounding_ok(np.uint16(nb), z, window):
                break
            out.append(nb)
            b = nb
    return out


def _near_ties(z_row, a_row, p_row, cols):
    """Columns of a head whose projection may round to another bf16 value,
    with those values."""
    out = []
    for c in cols:
        cand = _candidates(int(p_row[c]), float(z_row[c]), float(_p_window(z_row[c], a_row[c])))
        for alt in cand[1:]:
            out.append((c, alt))
    return out


# A near-tie whose other values move the head's normed values by less than
# this is not enumerated: its effect is added to the output windows instead.
SMALL_EFFECT = 2.0 ** -14


def _head_matches(gpu_head, ph, cs_row, eps, soft=None):
    """Whether a head's GPU output is the rounding of the oracle's output for
    the projection values ph (bf16 bits [64]), up to the fp32 error of the
    norm and rotation and the spread `soft` [64] of projection values not
    enumerated.  Returns (ok, oracle bits, oracle exact values, number of
    values that differ from the oracle's rounding)."""
    out, od = head(ph, cs_row, eps)
    _, nd = head(ph, None, eps)          # the normed values before the rotation
    half = HEAD_DIM // 2
    if cs_row is None:
        c = np.ones(half)
        s = np.zeros(half)
    else:
        c = np.abs(np.asarray(cs_row[:half], dtype=np.float64))
        s = np.abs(np.asarray(cs_row[half:HEAD_DIM], dtype=np.float64))
    na, nb = np.abs(nd[0::2]), np.abs(nd[1::2])
    mag = np.empty(HEAD_DIM)
    mag[0::2] = na * c + nb * s
    mag[1::2] = nb * c + na * s
    window = OUT_WINDOW * U * mag + 2 * U * np.abs(od)
    if soft is not None and np.any(soft > 0):
        pv = bf16_to_float(ph)
        ss = float(np.sum(pv * pv))
        r = 1.0 / np.sqrt(ss / HEAD_DIM + eps)
        da, db = r * soft[0::2], r * soft[1::2]   # spread of the normed pair values
        spread = np.empty(HEAD_DIM)
        spread[0::2] = da * c + db * s
        spread[1::2] = db * c + da * s
        # the norm's factor moves by at most sum |p| d / sum p^2 (relative)
        rel = float(np.sum(np.abs(pv) * soft)) / ss if ss > 0 else 0.0
        window = window + spread + 2 * rel * np.abs(od)
    ok = _rounding_ok(gpu_head, od, window)
    return bool(ok.all()), out, od, int(np.sum(np.asarray(gpu_head) != out))


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
    y_gpu = np.ascontiguousarray(y_gpu, dtype=np.uint16)
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
    nq = QHEADS_PER_KV * nkv
    qk_cols = (nq + nkv) * HEAD_DIM
    report = {"elements": int(M * N), "plain_fail": int((~_within(yg, yr)).sum()),
              "vg_tie_alternatives": 0, "qk_output_tie_alternatives": 0,
              "tie_rescued_heads": 0, "max_ratio": 0.0}

    # v and gate columns: the rounded projection itself.
    vg = slice(qk_cols, N)
    ok_vg = _rounding_ok(y_gpu[:, vg], z[:, vg], _p_window(z[:, vg], a[:, vg]))
    if not ok_vg.all():
        bad = np.argwhere(~ok_vg)
        m, c = int(bad[0][0]), int(bad[0][1]) + qk_cols
        far = int((~_within(yg[:, vg], yr[:, vg])).sum())
        raise ParityError(
            f"v/gate rounding mismatch at token {m} column {c}: gpu {yg[m, c]!r} oracle "
            f"{yr[m, c]!r} exact {z[m, c]!r} ({len(bad)} elements, {far} of them beyond "
            f"the tolerance)")
    report["vg_tie_alternatives"] = int((y_gpu[:, vg] != p[:, vg]).sum())

    # q and k heads, one at a time.  Elements whose projection may take
    # another value: those with a valid neighbour above or below.
    qk = slice(0, qk_cols)
    wq = _p_window(z[:, qk], a[:, qk])
    up_ok = _rounding_ok(_neighbour_toward(p[:, qk], np.full(p[:, qk].shape, np.inf)), z[:, qk], wq)
    dn_ok = _rounding_ok(_neighbour_toward(p[:, qk], np.full(p[:, qk].shape, -np.inf)), z[:, qk], wq)
    multi = up_ok | dn_ok
    up1 = _neighbour_toward(p[:, qk], np.full(p[:, qk].shape, np.inf))
    dn1 = _neighbour_toward(p[:, qk], np.full(p[:, qk].shape, -np.inf))
    # a second value on either side: only where the sum cancels far below
    # its terms; those elements take the element-by-element search
    deep = (up_ok & _rounding_ok(_neighbour_toward(up1, np.full(up1.shape, np.inf)), z[:, qk], wq)) | \
           (dn_ok & _rounding_ok(_neighbour_toward(dn1, np.full(dn1.shape, -np.inf)), z[:, qk], wq))
    ratio = np.zeros((M, N))
    for m in range(M):
        cs_row = None if cos_sin is None else np.asarray(cos_sin)[int(positions[m])]
        for h in range(nq + nkv):
            cols = slice(h * HEAD_DIM, (h + 1) * HEAD_DIM)
            gh = y_gpu[m, cols]
            base = np.array(p[m, cols], copy=True)
            pv = bf16_to_float(base)
            r = 1.0 / np.sqrt(float(np.mean(pv * pv)) + eps)
            # the projection values each element may take, split into those
            # enumerated and those whose spread goes into the output windows
            soft = np.zeros(HEAD_DIM)
            hard = []
            for i in np.flatnonzero(multi[m, cols]):
                col = h * HEAD_DIM + int(i)
                if deep[m, col]:
                    cand = _candidates(int(p[m, col]), float(z[m, col]),
                                       float(_p_window(z[m, col], a[m, col])))
                else:
                    cand = [int(p[m, col])] + ([int(up1[m, col])] if up_ok[m, col] else []) + \
                           ([int(dn1[m, col])] if dn_ok[m, col] else [])
                if len(cand) == 1:
                    continue
                spread = max(abs(float(bf16_to_float(np.uint16(v))) - float(pv[i]))
                             for v in cand)
                hard.append((spread * r, int(i), cand))
            hard.sort(reverse=True)
            enum = [(i, cand) for eff, i, cand in hard if eff >= SMALL_EFFECT][:MAX_ENUM]
            enumerated = {i for i, _ in enum}
            for eff, i, cand in hard:
                if i not in enumerated:
                    soft[i] = eff / r
            ok, out, od, nalt = _head_matches(gh, base, cs_row, eps, soft)
            rescued = False
            if not ok:
                for choice in itertools.product(*[range(len(cand)) for _, cand in enum]):
                    if not any(choice):
                        continue
                    ph = base.copy()
                    for (i, cand), k in zip(enum, choice):
                        ph[i] = cand[k]
                    ok, out, od, nalt = _head_matches(gh, ph, cs_row, eps, soft)
                    if ok:
                        rescued = True
                        break
            if not ok:
                ok0 = _head_matches(gh, base, cs_row, eps, soft)
                bad = np.flatnonzero(gh != ok0[1])
                c = h * HEAD_DIM + int(bad[0]) if bad.size else h * HEAD_DIM
                raise ParityError(
                    f"q/k head mismatch at token {m} head {h} column {c}: gpu {yg[m, c]!r} "
                    f"oracle {yr[m, c]!r} ({len(bad)} of 64 values differ; {len(enum)} "
                    f"projection near-ties enumerated)")
            want = bf16_to_float(out)
            if not _within(yg[m, cols], want).all():
                raise ParityError(f"token {m} head {h}: matched rounding beyond the tolerance")
            ratio[m, cols] = np.abs(yg[m, cols] - want) / (RTOL * np.abs(want) + ATOL)
            if rescued:
                report["tie_rescued_heads"] += 1
            else:
                report["qk_output_tie_alternatives"] += nalt
    ratio[:, vg] = np.abs(yg[:, vg] - yr[:, vg]) / (RTOL * np.abs(yr[:, vg]) + ATOL)
    report["max_ratio"] = float(ratio.max())

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
