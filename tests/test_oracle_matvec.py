"""Pins for the oracle's projection (decode + exact integer block sums +
fp64 terms and row sum).

* Brute force: weights are built from chosen integer fields by the test-side
  encoders, so their exact fp64 values are known without any decoder; the
  activations' values are d_a * q_a.  numpy's fp64 matmul of the two is the
  reference, and the oracle must agree to ~1e-12 of T = sum |terms|.
* Unit scales: with every float scale 1.0 (Q4_K: sub-scale 1, min 0) and
  integer activations whose block maximum is 127 (so d_a = 1), the output and
  the integer block sums are an exact integer matrix product.
* The row split over threads does not change a single bit.
"""

import numpy as np
import pytest

import gguf_encode as ge

QT = [8, 12, 14]


def _acts(orc, rng, M, K, integer=False):
    if integer:
        x = rng.integers(-127, 128, (M, K)).astype(np.float32)
        x.reshape(M, K // 32, 32)[:, :, 0] = 127.0
    else:
        x = rng.standard_normal((M, K)).astype(np.float32)
    q, d, s16, _ = orc.quantize_act(x)
    return q, d


@pytest.mark.parametrize("qt", QT)
@pytest.mark.parametrize("M", [1, 3, 5])
def test_bruteforce_fp64(orc, qt, M):
    rng = np.random.default_rng(100 + qt + M)
    N, K = 7, 512
    Wb, Wf = ge.random_fields(qt, N, K, rng)
    q, d = _acts(orc, rng, M, K)
    A = (d.astype(np.float64).repeat(32, axis=1) * q.astype(np.float64))
    ref = A @ Wf.T
    y, T = orc.matvec(qt, Wb, K, q, d)
    assert np.all(np.abs(y - ref) <= 1e-12 * T + 1e-300)
    # T really is the sum of |block terms|: it bounds |y|
    assert np.all(np.abs(y) <= T * (1 + 1e-12))


@pytest.mark.parametrize("qt", QT)
def test_unit_scale_integer_gemm(orc, qt):
    rng = np.random.default_rng(7 + qt)
    N, K, M = 9, 512, 4
    Wb, Wf = ge.random_fields(qt, N, K, rng, unit=True)
    q, d = _acts(orc, rng, M, K, integer=True)
    assert np.all(d == 1.0)
    wi = np.rint(Wf).astype(np.int64)  # exact integers by construction
    y, T, bs = orc.matvec(qt, Wb, K, q, d, block_sums=True)
    ref = q.astype(np.int64) @ wi.T
    assert np.array_equal(y, ref.astype(np.float64))
    blocks = np.einsum("mbi,nbi->mnb", q.astype(np.int64).reshape(M, K // 32, 32),
                       wi.reshape(N, K // 32, 32))
    assert np.array_equal(bs, blocks)


def test_q4_k_min_term_only(orc):
    """All quants zero: each weight is -dmin*m_j, so y = -sum_j dmin m_j
    d_a sum(q_a over sub-block j)."""
    rng = np.random.default_rng(11)
    K, M = 512, 2
    ns = K // 256
    dm = ge.half_bits(np.full(ns, 0.5))
    m = rng.integers(0, 64, (ns, 8))
    row = ge.encode_q4_k(ge.half_bits(np.full(ns, 2.0)), dm, rng.integers(0, 64, (ns, 8)), m,
                         np.zeros((ns, 256), np.int64))
    q, d = _acts(orc, rng, M, K)
    y, _ = orc.matvec(12, row[None, :], K, q, d)
    sub = q.astype(np.int64).reshape(M, K // 32, 32).sum(2)
    ref = -(0.5 * m.reshape(-1)[None, :] * d.astype(np.float64) * sub).sum(1)
    assert np.allclose(y[:, 0], ref, rtol=1e-13, atol=0)


def test_q6_k_offset(orc):
    """All stored quants 32 give zero weights whatever the scales."""
    rng = np.random.default_rng(12)
    K = 512
    row = ge.encode_q6_k(ge.half_bits(np.full(2, 0.3)), rng.integers(-128, 128, (2, 16)),
                         np.full((2, 256), 32))
    q, d = _acts(orc, rng, 3, K)
    y, T = orc.matvec(14, row[None, :], K, q, d)
    assert not y.any() and not T.any()


@pytest.mark.parametrize("qt", QT)
def test_threads_and_row_ids(orc, qt):
    rng = np.random.default_rng(13)
    N, K, M = 33, 512, 5
    Wb, _ = ge.random_fields(qt, N, K, rng)
    q, d = _acts(orc, rng, M, K)
    y1, T1 = orc.matvec(qt, Wb, K, q, d, threads=1)
    y8, T8 = orc.matvec(qt, Wb, K, q, d, threads=8)
    assert np.array_equal(y1, y8) and np.array_equal(T1, T8)
    ids = np.array([32, 0, 5, 5, 17], np.int32)
    yr, _ = orc.matvec(qt, Wb, K, q, d, row_ids=ids)
    assert np.array_equal(yr, y1[:, ids])
    # per-position rows are independent: row m alone equals row m of the batch
    for m in range(M):
        ym, _ = orc.matvec(qt, Wb, K, q[m:m + 1], d[m:m + 1])
        assert np.array_equal(ym[0], y1[m])


def test_scale_vector(orc):
    rng = np.random.default_rng(14)
    Wb, _ = ge.random_fields(8, 4, 256, rng)
    q, d = _acts(orc, rng, 2, 256)
    y, T = orc.matvec(8, Wb, 256, q, d)
    ys, Ts = orc.matvec(8, Wb, 256, q, d, scale=[0.5, -2.0])
    assert np.array_equal(ys[0], y[0] * 0.5) and np.array_equal(ys[1], y[1] * -2.0)
    assert np.array_equal(Ts[1], T[1] * 2.0)
