"""Pins for the oracle's activation quantiser (Q8A32) and RMS factor.

Closed forms: a block whose largest magnitude is exactly 127 has d = 1, so
q = round(x) and half-way values expose the rounding mode; an all-zero block
gives d = 0, q = 0; a block with one nonzero value gives +-127 there.
Invariants on random data: |q| <= 127, |x - d q| <= d/2, the block maximum
maps to +-127, and the per-16 sums are the sums of the codes.
"""

import numpy as np
import pytest


def test_unit_scale_rounding_half_away(orc):
    x = np.zeros((1, 32), np.float32)
    x[0, 0] = 127.0
    vals = [2.5, -2.5, 0.5, -0.5, 1.5, -1.5, 3.49, -3.51, 126.5, -126.5]
    x[0, 1:1 + len(vals)] = vals
    q, d, s16, _ = orc.quantize_act(x)
    assert d[0, 0] == 1.0
    want = [127, 3, -3, 1, -1, 2, -2, 3, -4, 127, -127]
    assert list(q[0, :len(want)]) == want


def test_zero_block(orc):
    x = np.zeros((2, 64), np.float32)
    x[1, 40] = -0.25
    q, d, s16, ss = orc.quantize_act(x)
    assert d[0, 0] == 0 and d[0, 1] == 0 and not q[0].any()
    assert d[1, 0] == 0 and not q[1, :32].any()
    assert q[1, 40] == -127 and np.count_nonzero(q[1]) == 1
    assert d[1, 1] == np.float32(0.25) / np.float32(127.0)
    assert ss[1] == 0.0625


@pytest.mark.parametrize("seed", [0, 1])
def test_invariants_random(orc, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((5, 1024)).astype(np.float32) * np.float32(3.0)
    q, d, s16, ss = orc.quantize_act(x)
    xb = x.reshape(5, 32, 32).astype(np.float64)
    qb = q.reshape(5, 32, 32).astype(np.float64)
    assert np.abs(q).max() <= 127
    # reconstruction error at most half a step (plus fp32 rounding slack)
    err = np.abs(xb - d[:, :, None] * qb)
    assert np.all(err <= d[:, :, None] * (0.5 + 1e-5))
    # the largest magnitude in each block lands on +-127
    amax_idx = np.abs(xb).argmax(axis=2)
    assert np.all(np.abs(np.take_along_axis(qb, amax_idx[:, :, None], 2)) == 127)
    assert np.array_equal(s16, q.reshape(5, 64, 16).astype(np.int32).sum(axis=2))
    assert np.allclose(ss, (x.astype(np.float64) ** 2).sum(axis=1), rtol=1e-12)
    # d is the fp32 quotient amax / 127
    amax = np.abs(x.reshape(5, 32, 32)).max(axis=2)
    assert np.array_equal(d, amax / np.float32(127.0))


def test_gamma_is_one_fp32_product(orc):
    rng = np.random.default_rng(3)
    x = rng.standard_normal((3, 256)).astype(np.float32)
    g = (1 + 0.1 * rng.standard_normal(256)).astype(np.float32)
    a = orc.quantize_act(x, g)
    b = orc.quantize_act(x * g)
    for u, v in zip(a[:3], b[:3]):
        assert np.array_equal(u, v)
    # sumsq is taken before gamma
    assert np.allclose(a[3], (x.astype(np.float64) ** 2).sum(1), rtol=1e-12)


def test_scale_invariance_of_codes(orc):
    """Scaling a block by a power of two leaves the codes unchanged and
    scales d exactly (every fp32 step is exact under such a scaling)."""
    rng = np.random.default_rng(4)
    x = rng.standard_normal((2, 128)).astype(np.float32)
    q1, d1, _, _ = orc.quantize_act(x)
    q2, d2, _, _ = orc.quantize_act(x * np.float32(8.0))
    assert np.array_equal(q1, q2)
    assert np.array_equal(d2, d1 * np.float32(8.0))


def test_rms_factor_closed_form(orc):
    # constant vector c of length n: r = 1/sqrt(c^2 + eps)
    n, c, eps = 2560, 3.0, 1e-6
    r = orc.rms_factor(n * c * c, n, eps)[0]
    assert r == 1.0 / np.sqrt(c * c + eps)
