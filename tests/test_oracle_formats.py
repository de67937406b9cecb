"""Pins for the oracle's GGUF block decoders.

What fixes the expected values:
  * fp16 conversion: numpy's IEEE half conversion, all 65536 bit patterns.
  * Block layouts: blocks are built from chosen integer fields by the
    test-side encoders (tests/gguf_encode.py, the inverse operation written
    from the public ggml layout) and by the hand-written golden blocks in
    tests/golden/; the decoder must return exactly those fields.
Format fidelity to real GGUF files stays unpinned here (no GGUF file or ggml
source is available to compare against).
"""

import json
import os

import numpy as np
import pytest

import gguf_encode as ge

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_half_all_patterns(orc):
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([orc.half(int(b)) for b in bits])
    finite = np.isfinite(ref)
    assert np.array_equal(got[finite], ref[finite])
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    assert np.array_equal(got[np.isinf(ref)], ref[np.isinf(ref)])


def test_half_subnormal_closed_form(orc):
    # smallest subnormal 2^-24, largest subnormal 1023 * 2^-24, smallest normal 2^-14
    assert orc.half(0x0001) == 2.0 ** -24
    assert orc.half(0x03FF) == 1023 * 2.0 ** -24
    assert orc.half(0x0400) == 2.0 ** -14
    assert orc.half(0x8400) == -(2.0 ** -14)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_q8_0_roundtrip(orc, seed):
    rng = np.random.default_rng(seed)
    nb = 8
    d = ge.half_bits(np.abs(rng.normal(0, 0.02, nb)))
    q = rng.integers(-128, 128, (nb, 32))
    row = ge.encode_q8_0(d, q)
    assert row.size == nb * 34
    gq, gd = orc.decode_q8_0(row, nb * 32)
    assert np.array_equal(gq, q.reshape(-1))
    assert np.array_equal(gd, ge.half_value(d))


@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_q4_k_roundtrip(orc, seed):
    rng = np.random.default_rng(seed)
    ns = 3
    d = ge.half_bits(np.abs(rng.normal(0, 0.02, ns)))
    dm = ge.half_bits(np.abs(rng.normal(0, 0.02, ns)))
    sc = rng.integers(0, 64, (ns, 8))
    m = rng.integers(0, 64, (ns, 8))
    q = rng.integers(0, 16, (ns, 256))
    row = ge.encode_q4_k(d, dm, sc, m, q)
    assert row.size == ns * 144
    gq, gd, gdm, gsc, gm = orc.decode_q4_k(row, ns * 256)
    assert np.array_equal(gq, q.reshape(-1))
    assert np.array_equal(gsc, sc.reshape(-1))
    assert np.array_equal(gm, m.reshape(-1))
    assert np.array_equal(gd, ge.half_value(d))
    assert np.array_equal(gdm, ge.half_value(dm))


def test_q4_k_positions_distinct(orc):
    """Every element position carries its own value: a transposed nibble or
    swapped sub-block would move a value and fail."""
    ns = 1
    q = (np.arange(256) * 7 + 3) % 16
    sc = np.arange(8) * 9 % 64
    m = (np.arange(8) * 5 + 60) % 64
    row = ge.encode_q4_k([0x3C00], [0x3800], sc, m, q)
    gq, _, _, gsc, gm = orc.decode_q4_k(row, 256)
    assert np.array_equal(gq, q)
    assert np.array_equal(gsc, sc)
    assert np.array_equal(gm, m)


@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_q6_k_roundtrip(orc, seed):
    rng = np.random.default_rng(seed)
    ns = 3
    d = ge.half_bits(np.abs(rng.normal(0, 0.02, ns)))
    sc = rng.integers(-128, 128, (ns, 16))
    q = rng.integers(0, 64, (ns, 256))
    row = ge.encode_q6_k(d, sc, q)
    assert row.size == ns * 210
    gq, gd, gsc = orc.decode_q6_k(row, ns * 256)
    assert np.array_equal(gq, q.reshape(-1))
    assert np.array_equal(gsc, sc.reshape(-1))
    assert np.array_equal(gd, ge.half_value(d))


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_golden_q4_k_block(orc):
    """Hand-written Q4_K block (tests/golden/q4_k_block.json): byte values
    and the sub-scales, mins and quants they stand for, worked out by hand
    from the ggml bit layout."""
    g = _golden("q4_k_block.json")
    row = np.array(g["bytes"], np.uint8)
    gq, gd, gdm, gsc, gm = orc.decode_q4_k(row, 256)
    assert list(gsc) == g["sc"]
    assert list(gm) == g["m"]
    assert gd[0] == g["d"] and gdm[0] == g["dmin"]
    for pos, val in g["q_at"].items():
        assert gq[int(pos)] == val


def test_golden_q6_k_block(orc):
    """Hand-written Q6_K block (tests/golden/q6_k_block.json)."""
    g = _golden("q6_k_block.json")
    row = np.array(g["bytes"], np.uint8)
    gq, gd, gsc = orc.decode_q6_k(row, 256)
    assert list(gsc) == g["sc"]
    assert gd[0] == g["d"]
    for pos, val in g["q_at"].items():
        assert gq[int(pos)] == val


def test_golden_q8_0_block(orc):
    g = _golden("q8_0_block.json")
    row = np.array(g["bytes"], np.uint8)
    gq, gd = orc.decode_q8_0(row, 32)
    assert gd[0] == g["d"]
    assert list(gq) == g["q"]
