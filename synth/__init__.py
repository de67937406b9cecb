"""Seeded synthetic inputs for the verification pass.

This module is shared by the CPU oracle side (tests, bench baseline) and the
GPU side (tests, bench, smoke).  It holds no arithmetic of the method: it only
draws random numbers and places them where the input formats expect them.

* Weights are canonical GGUF block bytes (the formats ggml defines, named on
  the Kinetic page "How Kinetic is fast", section "References").  Quant fields
  are uniform random bytes; the fp16 block scales are |N(0, 0.02)| written as
  IEEE half at the field offsets of each block type.  Only field offsets are
  known here, never how a block decodes.
* Activations are N(0, 1) fp32 rows; RMSNorm weights are 1 + N(0, 0.1^2).
* Drafts are token ids; uniforms are k * 2^-53 with k a 53-bit integer, so they
  are exact doubles in [0, 1).

Every tensor is drawn from its own PCG64 stream, keyed by (seed, name), so a
tensor does not change when another one is added or resized.
"""

from __future__ import annotations

import hashlib

import numpy as np

# GGUF type ids and block geometry: (elements per block, bytes per block).
Q8_0, Q4_K, Q6_K = 8, 12, 14
BLOCK = {Q8_0: (32, 34), Q4_K: (256, 144), Q6_K: (256, 210)}
QTYPE_NAME = {Q8_0: "Q8_0", Q4_K: "Q4_K", Q6_K: "Q6_K"}

# Offsets of the fp16 scale fields inside one block.
_HALF_FIELDS = {Q8_0: (0,), Q4_K: (0, 2), Q6_K: (208,)}


def stream(seed: int, *key) -> np.random.Generator:
    """Independent PCG64 generator for (seed, key...)."""
    h = hashlib.sha256(repr((int(seed),) + tuple(key)).encode()).digest()
    words = [int.from_bytes(h[i:i + 4], "little") for i in range(0, 32, 4)]
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(words)))


def row_bytes(qtype: int, cols: int) -> int:
    blk, nb = BLOCK[qtype]
    if cols % blk:
        raise ValueError(f"{QTYPE_NAME[qtype]} needs cols % {blk} == 0, got {cols}")
    return cols // blk * nb


def gguf_weights(qtype: int, rows: int, cols: int, seed: int, *key,
                 scale_sigma: float = 0.02) -> np.ndarray:
    """Canonical GGUF bytes, shape [rows, row_bytes] uint8.

    Q8_0 quants are int8 uniform in [-127, 127]; K-quant fields are raw
    uniform bytes; every fp16 scale is |N(0, scale_sigma)|.
    """
    blk, nb = BLOCK[qtype]
    rb = row_bytes(qtype, cols)
    nblocks = rows * (cols // blk)
    g = stream(seed, "w", QTYPE_NAME[qtype], rows, cols, *key)
    raw = g.integers(0, 256, size=(nblocks, nb), dtype=np.uint8)
    if qtype == Q8_0:
        raw[:, 2:] = g.integers(-127, 128, size=(nblocks, 32), dtype=np.int8).view(np.uint8)
    for off in _HALF_FIELDS[qtype]:
        h = np.abs(g.standard_normal(nblocks) * scale_sigma).astype(np.float16)
        raw[:, off:off + 2] = h.view(np.uint8).reshape(nblocks, 2)
    return raw.reshape(rows, rb)


def activations(M: int, K: int, seed: int, *key, sigma: float = 1.0) -> np.ndarray:
    """fp32 [M, K] rows drawn from N(0, sigma^2)."""
    g = stream(seed, "x", M, K, *key)
    return (g.standard_normal((M, K)) * sigma).astype(np.float32)


def rms_weight(n: int, seed: int, *key) -> np.ndarray:
    """RMSNorm weight 1 + N(0, 0.1^2), fp32 [n]."""
    g = stream(seed, "gamma", n, *key)
    return (1.0 + 0.1 * g.standard_normal(n)).astype(np.float32)


def uniforms(shape, seed: int, *key) -> np.ndarray:
    """Exact doubles k * 2^-53 in [0, 1)."""
    g = stream(seed, "u", tuple(np.atleast_1d(shape)), *key)
    k = g.integers(0, 1 << 53, size=shape, dtype=np.int64)
    return k.astype(np.float64) * (2.0 ** -53)


def normals(shape, seed: int, *key, sigma: float = 1.0, dtype=np.float32) -> np.ndarray:
    g = stream(seed, "n", tuple(np.atleast_1d(shape)), *key)
    return (g.standard_normal(shape) * sigma).astype(dtype)


def drafts_from(target: np.ndarray, vocab: int, p_match: float, seed: int, *key) -> np.ndarray:
    """Draft ids equal to target[i] with probability p_match, else uniform
    over the vocabulary (which may coincide with the target by chance)."""
    target = np.asarray(target, dtype=np.int64)
    g = stream(seed, "drafts", target.shape, vocab, p_match, *key)
    keep = g.random(target.shape) < p_match
    other = g.integers(0, vocab, size=target.shape)
    return np.where(keep, target, other).astype(np.int32)


def token_ids(n: int, vocab: int, seed: int, *key, distinct: bool = False,
              exclude=None) -> np.ndarray:
    """n token ids in [0, vocab); sorted and distinct when asked."""
    g = stream(seed, "ids", n, vocab, distinct, *key)
    if not distinct:
        return g.integers(0, vocab, size=n).astype(np.int32)
    pool = np.arange(vocab, dtype=np.int64)
    if exclude is not None:
        pool = np.setdiff1d(pool, np.asarray(exclude, dtype=np.int64))
    pick = g.choice(pool.size, size=n, replace=False)
    return np.sort(pool[pick]).astype(np.int32)
