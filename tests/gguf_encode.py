"""Test-side GGUF block encoders: integer fields -> canonical block bytes.

These build weights whose exact dequantised values are known by construction
(the fields themselves), so the oracle's decoders and projection can be
checked without going through any decoder.  They follow the public ggml
block layouts (the formats the Kinetic page's references attribute to ggml).
"""

from __future__ import annotations

import numpy as np


def half_bits(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float16).view(np.uint16)


def half_value(bits) -> np.ndarray:
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def encode_q8_0(d_bits, q) -> np.ndarray:
    """d_bits: [nb] uint16 fp16 scales; q: [nb, 32] int in [-128, 127]."""
    d_bits = np.asarray(d_bits, np.uint16).reshape(-1)
    q = np.asarray(q).reshape(d_bits.size, 32)
    out = np.zeros((d_bits.size, 34), np.uint8)
    out[:, 0] = d_bits & 0xFF
    out[:, 1] = d_bits >> 8
    out[:, 2:] = q.astype(np.int8).view(np.uint8)
    return out.reshape(-1)


def dequant_q8_0(d_bits, q) -> np.ndarray:
    return (half_value(d_bits)[:, None] * np.asarray(q, np.float64).reshape(-1, 32)).reshape(-1)


def encode_q4_k(d_bits, dmin_bits, sc, m, q) -> np.ndarray:
    """One row of super-blocks.  d_bits, dmin_bits: [ns]; sc, m: [ns, 8] in
    [0, 63]; q: [ns, 256] in [0, 15]."""
    d_bits = np.asarray(d_bits, np.uint16).reshape(-1)
    ns = d_bits.size
    dmin_bits = np.asarray(dmin_bits, np.uint16).reshape(ns)
    sc = np.asarray(sc, np.int64).reshape(ns, 8)
    m = np.asarray(m, np.int64).reshape(ns, 8)
    q = np.asarray(q, np.int64).reshape(ns, 256)
    out = np.zeros((ns, 144), np.uint8)
    for s in range(ns):
        b = out[s]
        b[0], b[1] = d_bits[s] & 0xFF, d_bits[s] >> 8
        b[2], b[3] = dmin_bits[s] & 0xFF, dmin_bits[s] >> 8
        packed = [0] * 12
        # Bytes 0-3: low 6 bits = scale j, top 2 bits = high bits of scale j+4.
        # Bytes 4-7: low 6 bits = min j,   top 2 bits = high bits of min j+4.
        # Bytes 8-11: low nibble = low 4 bits of scale j+4, high nibble = low
        # 4 bits of min j+4.
        for j in range(4):
            packed[j] = (sc[s, j] & 63) | ((sc[s, j + 4] >> 4) << 6)
            packed[j + 4] = (m[s, j] & 63) | ((m[s, j + 4] >> 4) << 6)
            packed[j + 8] = (sc[s, j + 4] & 15) | ((m[s, j + 4] & 15) << 4)
        b[4:16] = packed
        # Elements 64c .. 64c+31 are low nibbles of bytes 32c .. 32c+31,
        # elements 64c+32 .. 64c+63 the high nibbles of the same bytes.
        for c in range(4):
            lo = q[s, 64 * c: 64 * c + 32]
            hi = q[s, 64 * c + 32: 64 * c + 64]
            b[16 + 32 * c: 16 + 32 * c + 32] = (lo | (hi << 4)).astype(np.uint8)
    return out.reshape(-1)


def dequant_q4_k(d_bits, dmin_bits, sc, m, q) -> np.ndarray:
    d = half_value(d_bits).reshape(-1)
    dmin = half_value(dmin_bits).reshape(-1)
    ns = d.size
    sc = np.asarray(sc, np.float64).reshape(ns, 8)
    m = np.asarray(m, np.float64).reshape(ns, 8)
    q = np.asarray(q, np.float64).reshape(ns, 8, 32)
    w = d[:, None, None] * sc[:, :, None] * q - dmin[:, None, None] * m[:, :, None]
    return w.reshape(-1)


def encode_q6_k(d_bits, sc, q) -> np.ndarray:
    """One row of super-blocks.  d_bits: [ns]; sc: [ns, 16] int8; q: [ns, 256]
    in [0, 63] (the stored value; the weight is d*sc*(q-32))."""
    d_bits = np.asarray(d_bits, np.uint16).reshape(-1)
    ns = d_bits.size
    sc = np.asarray(sc, np.int64).reshape(ns, 16)
    q = np.asarray(q, np.int64).reshape(ns, 256)
    out = np.zeros((ns, 210), np.uint8)
    for s in range(ns):
        ql = np.zeros(128, np.int64)
        qh = np.zeros(64, np.int64)
        # Within each 128-element half h: element 32g + l (g = 0..3) keeps its
        # low 4 bits in ql[64h + l + 32*(g & 1)] (low nibble for g < 2, high
        # nibble for g >= 2) and its high 2 bits at bit 2g of qh[32h + l].
        for h in range(2):
            for g in range(4):
                for l in range(32):
                    v = q[s, 128 * h + 32 * g + l]
                    idx = 64 * h + l + 32 * (g & 1)
                    ql[idx] |= (v & 15) << (0 if g < 2 else 4)
                    qh[32 * h + l] |= ((v >> 4) & 3) << (2 * g)
        b = out[s]
        b[0:128] = ql.astype(np.uint8)
        b[128:192] = qh.astype(np.uint8)
        b[192:208] = sc[s].astype(np.int8).view(np.uint8)
        b[208], b[209] = d_bits[s] & 0xFF, d_bits[s] >> 8
    return out.reshape(-1)


def dequant_q6_k(d_bits, sc, q) -> np.ndarray:
    d = half_value(d_bits).reshape(-1)
    ns = d.size
    sc = np.asarray(sc, np.float64).reshape(ns, 16)
    q = np.asarray(q, np.float64).reshape(ns, 16, 16)
    return (d[:, None, None] * sc[:, :, None] * (q - 32.0)).reshape(-1)


def random_fields(qtype: int, rows: int, K: int, rng: np.random.Generator, unit: bool = False):
    """Random integer fields for a [rows, K] matrix, plus its bytes and its
    exact fp64 dequantisation.  unit=True sets every float scale to 1.0 and
    (Q4_K) every sub-scale to 1 and min to 0, so the projection reduces to
    an integer product."""
    one = int(half_bits(1.0))
    rows_b, rows_w = [], []
    for _ in range(rows):
        if qtype == 8:
            nb = K // 32
            d = np.full(nb, one, np.uint16) if unit else half_bits(np.abs(rng.normal(0, 0.02, nb)))
            q = rng.integers(-127, 128, (nb, 32))
            rows_b.append(encode_q8_0(d, q))
            rows_w.append(dequant_q8_0(d, q))
        elif qtype == 12:
            ns = K // 256
            d = np.full(ns, one, np.uint16) if unit else half_bits(np.abs(rng.normal(0, 0.02, ns)))
            dm = np.zeros(ns, np.uint16) if unit else half_bits(np.abs(rng.normal(0, 0.02, ns)))
            sc = np.ones((ns, 8), np.int64) if unit else rng.integers(0, 64, (ns, 8))
            m = np.zeros((ns, 8), np.int64) if unit else rng.integers(0, 64, (ns, 8))
            q = rng.integers(0, 16, (ns, 256))
            rows_b.append(encode_q4_k(d, dm, sc, m, q))
            rows_w.append(dequant_q4_k(d, dm, sc, m, q))
        else:
            ns = K // 256
            d = np.full(ns, one, np.uint16) if unit else half_bits(np.abs(rng.normal(0, 0.02, ns)))
            sc = np.ones((ns, 16), np.int64) if unit else rng.integers(-128, 128, (ns, 16))
            q = rng.integers(0, 64, (ns, 256))
            rows_b.append(encode_q6_k(d, sc, q))
            rows_w.append(dequant_q6_k(d, sc, q))
    return np.stack(rows_b), np.stack(rows_w)
