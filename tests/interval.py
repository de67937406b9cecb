"""Interval checks of GPU results against the oracle's fp64 values.

The fp32 bar says a GPU value v_gpu lies within delta = 1e-5 * T of the
oracle's v64 (T the sum of |block terms|).  Where the GPU then takes a
discrete decision on that value (an int8 code, an argmax), the decision it
took must be one that some value inside the interval [v64 - delta,
v64 + delta] leads to.  These helpers check exactly that, element by
element, so no differing code or winner passes on a fraction or a margin
read off the observed drift.

Q8A32 of a vector v times a norm weight gamma (OpenJet, "One GPU launch for
a speculative cycle": the producer requantises its output for the next
consumer): per block of 32, d = max|v gamma| / 127, code = round(v gamma / d)
clamped to +-127; code sums per 16; the block's sum of v^2 (before gamma)
feeds the next RMS factor.
"""

from __future__ import annotations

import numpy as np

U32 = 2.0 ** -23      # two fp32 roundings' worth of relative error


def check_requant(v64, delta, gamma, q_g, d_g, s16_g, ss_g, orc=None):
    """Asserts that the GPU's Q8A32 output (codes q_g [M,N], scales d_g
    [M,N/32], code sums s16_g [M,N/16], partials ss_g [M,N/32]) is what a
    fp32 vector within delta [M,N] of v64 quantises to.  Returns the number
    of codes that differ from the oracle's own rounding of fp32(v64) (each
    of them a half-way tie within the interval), when orc is given."""
    v64 = np.asarray(v64, np.float64)
    M, N = v64.shape
    nb = N // 32
    g = np.asarray(gamma, np.float32).astype(np.float64)
    delta = np.broadcast_to(np.asarray(delta, np.float64), v64.shape)
    t = v64 * g
    et = delta * np.abs(g) + U32 * (np.abs(t) + delta * np.abs(g))
    tb, eb = t.reshape(M, nb, 32), et.reshape(M, nb, 32)
    lo = np.maximum(np.abs(tb) - eb, 0.0).max(2)
    hi = (np.abs(tb) + eb).max(2)
    d = np.asarray(d_g, np.float64).reshape(M, nb)
    # scale: max |v gamma| / 127 of a vector inside the interval
    ok_d = (d >= lo / 127 * (1 - U32)) & (d <= hi / 127 * (1 + U32))
    assert ok_d.all(), f"{(~ok_d).sum()} block scales outside the interval"
    # codes: round(t / d) with the GPU's own d for some t in the interval
    q = np.asarray(q_g, np.int64).reshape(M, nb, 32)
    assert np.abs(q).max(initial=0) <= 127
    dd = d[..., None]
    err = np.abs(q * dd - tb) - ((0.5 + 1e-4) * dd + eb)
    bad = err > 0
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{bad.sum()} codes no value in the interval rounds to; first at {tuple(i)}: "
                             f"code {q[tuple(i)]}, t/d {tb[tuple(i)] / dd[tuple(i[:2])][0]:.6f}")
    # code sums: exact integers of the GPU's own codes
    s16 = np.asarray(s16_g, np.int64).reshape(M, N // 16)
    assert np.array_equal(s16, q.reshape(M, N // 16, 16).sum(2)), "code sums differ from the codes"
    # partials: sum of v^2 per block (before gamma)
    vb, db = v64.reshape(M, nb, 32), delta.reshape(M, nb, 32)
    ref = (vb * vb).sum(2)
    bound = (2 * np.abs(vb) * db + db * db).sum(2) + 32 * U32 * ((np.abs(vb) + db) ** 2).sum(2)
    ss = np.asarray(ss_g, np.float64).reshape(M, nb)
    ok_s = np.abs(ss - ref) <= bound
    assert ok_s.all(), f"{(~ok_s).sum()} RMS partials outside the interval"
    if orc is None:
        return None
    q_or = orc.quantize_act(v64.astype(np.float32), np.asarray(gamma, np.float32))[0]
    return int(np.count_nonzero(q_or.reshape(M, nb, 32) != q))


def pair_bound(g64, Tg, u64, Tu, tol):
    """Bound on |fp32(g_gpu) * fp32(u_gpu) - g64 * u64| when each factor is
    within tol * T of the oracle's value (the product rounded once)."""
    dg, du = tol * Tg, tol * Tu
    return np.abs(u64) * dg + np.abs(g64) * du + dg * du + U32 * (np.abs(g64) + dg) * (np.abs(u64) + du)


def check_winner(idx, y64, delta):
    """Each row's winner idx must be a row that can be the maximum for some
    values inside the intervals: y64[idx] + delta[idx] >= max(y64 - delta).
    Returns the number of rows whose winner is decided by the intervals
    alone (one row's lower bound above every other row's upper bound)."""
    y64 = np.atleast_2d(np.asarray(y64, np.float64))
    delta = np.broadcast_to(np.asarray(delta, np.float64), y64.shape)
    rows = np.arange(y64.shape[0])
    up = y64[rows, idx] + delta[rows, idx]
    floor = (y64 - delta).max(1)
    assert np.all(up >= floor), "a winner no value inside the intervals makes the maximum"
    top = y64.argmax(1)
    hi = y64 + delta
    hi[rows, top] = -np.inf
    decided = (y64[rows, top] - delta[rows, top]) > hi.max(1)
    assert np.array_equal(np.asarray(idx)[decided], top[decided])
    return int(decided.sum())
