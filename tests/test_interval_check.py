"""CPU pins of the interval checks the GPU tests rely on: the oracle's own
quantiser output passes them, and each plausible GPU mistake (a code off by
one away from a tie, a wrong block scale, code sums not of the codes, an
RMS partial of the wrong vector, a winner outside the intervals) fails."""

import numpy as np
import pytest

import interval
import synth


def _case(seed, M=3, N=256):
    v = synth.activations(M, N, seed, "v").astype(np.float64) * 3.0
    g = synth.rms_weight(N, seed, "g")
    return v, g


def _quant(orc, v, g):
    q, d, s16, _ = orc.quantize_act(v.astype(np.float32), g)
    ss = (v.astype(np.float32).astype(np.float64) ** 2).reshape(v.shape[0], -1, 32).sum(2)
    return q, d, s16, ss


def test_oracle_output_passes(orc):
    v, g = _case(1)
    q, d, s16, ss = _quant(orc, v, g)
    assert interval.check_requant(v, 0.0, g, q, d, s16, ss, orc) == 0


def test_value_inside_interval_passes_with_its_own_codes(orc):
    """Codes of a perturbed vector (within delta) pass against the exact one,
    and some of them differ from the exact vector's codes (ties moved)."""
    v, g = _case(2, M=8, N=2048)
    delta = 2e-3 * np.abs(v).max()
    rng = np.random.default_rng(0)
    w = v + rng.uniform(-1, 1, v.shape) * delta
    q, d, s16, _ = orc.quantize_act(w.astype(np.float32), g)
    ss = (w.astype(np.float32).astype(np.float64) ** 2).reshape(8, -1, 32).sum(2)
    n = interval.check_requant(v, delta, g, q, d, s16, ss, orc)
    assert n > 0


def test_code_off_by_one_fails(orc):
    v, g = _case(3)
    q, d, s16, ss = _quant(orc, v, g)
    # the element whose scaled value sits farthest from a half-way point
    t = (v.astype(np.float32) * g).astype(np.float64) / np.repeat(d.astype(np.float64), 32, 1)
    far = np.argmax(np.abs(np.abs(t - np.trunc(t)) - 0.5) * (np.abs(q) < 127))
    i, j = np.unravel_index(far, q.shape)
    bad = q.copy()
    bad[i, j] += 1
    s = s16.copy()
    s[i, j // 16] += 1
    with pytest.raises(AssertionError, match="codes"):
        interval.check_requant(v, 1e-6, g, bad, d, s, ss)


def test_wrong_scale_fails(orc):
    v, g = _case(4)
    q, d, s16, ss = _quant(orc, v, g)
    bad = d.copy()
    bad[1, 2] *= 1.001
    with pytest.raises(AssertionError, match="scales"):
        interval.check_requant(v, 1e-6, g, q, bad, s16, ss)


def test_code_sums_must_be_of_the_codes(orc):
    v, g = _case(5)
    q, d, s16, ss = _quant(orc, v, g)
    bad = s16.copy()
    bad[0, 3] += 1
    with pytest.raises(AssertionError, match="code sums"):
        interval.check_requant(v, 0.0, g, q, d, bad, ss)


def test_partials_of_scaled_vector_fail(orc):
    """Partials taken after the norm weight, not before it."""
    v, g = _case(6)
    q, d, s16, _ = _quant(orc, v, g)
    vg = (v.astype(np.float32) * g).astype(np.float64)
    ss = (vg ** 2).reshape(v.shape[0], -1, 32).sum(2)
    with pytest.raises(AssertionError, match="partials"):
        interval.check_requant(v, 1e-6, g, q, d, s16, ss)


def test_winner_rules():
    y = np.array([[1.0, 3.0, 2.9999, 0.0], [5.0, 1.0, 2.0, 4.0]])
    delta = np.full_like(y, 1e-3)
    # row 0: 1 and 2 overlap (either may win), row 1: 0 is decided
    assert interval.check_winner(np.array([2, 0]), y, delta) == 1
    assert interval.check_winner(np.array([1, 0]), y, delta) == 1
    with pytest.raises(AssertionError):
        interval.check_winner(np.array([0, 0]), y, delta)
    with pytest.raises(AssertionError):
        interval.check_winner(np.array([1, 3]), y, delta)


def test_pair_bound_covers_the_rounded_product():
    rng = np.random.default_rng(7)
    g, u = rng.standard_normal(1000), rng.standard_normal(1000)
    Tg, Tu = np.abs(g) * 10, np.abs(u) * 10
    tol = 1e-5
    gg = (g + rng.uniform(-1, 1, 1000) * tol * Tg).astype(np.float32)
    uu = (u + rng.uniform(-1, 1, 1000) * tol * Tu).astype(np.float32)
    p = (gg * uu).astype(np.float64)
    assert np.all(np.abs(p - g * u) <= interval.pair_bound(g, Tg, u, Tu, tol))
