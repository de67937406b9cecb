"""Pins for the oracle's reading of the layer chain (oracle.chain_pass).

The probe makes every step exact and checkable by hand:
* every weight matrix is Q8_0 with one block scale D for all blocks and one
  nonzero integer code per row (a scaled partial permutation), built by the
  test-side encoder, so a projection moves each input entry to one output
  row, times its code and D;
* every activation vector holds at most one nonzero per 32-element block,
  so Q8A32 quantises it exactly (code +-127, scale |v| / 127) and the
  dequantised vector equals the vector to fp32 rounding.

The chain then reduces to a short recurrence (OpenJet, "One GPU launch for a
speculative cycle": each producer requantises the next input with the next
norm's weight folded in, the RMS factor of the normalised vector scaling the
consumer's output).  The closed form below is written from that recurrence,
not from the oracle's code: per layer

    r1 = rms_H(x);   v = r1 * Wv (g1 * x)
    r2 = rms_H(v);   o = r2 * Wo (g2 * v)
    r3 = rms_H(o);   g = r3 * Wg (g3 * o),  u = r3 * Wu (g3 * o),  p = g * u
    r4 = rms_F(p);   x = r4 * Wd (g4 * p)
    logits = rms_H(x) * Wh (gf * x)

with rms_n(v) = 1 / sqrt(sum(v^2) / n + eps) of the vector before its norm
weight.

Every stage after a norm is scale-invariant in that norm's input, except
through eps, so a wrong RMS factor in the middle of the chain would only show
at the end when eps is not negligible there.  D = 2^-14 keeps every stage's
mean square within a decade or two of eps, so each factor's eps share is a few
percent and a factor taken from the wrong vector moves the logits.  Mutated
oracles (norm weights swapped, RMS factor of the scaled vector or of the
previous vector, o reading k or q, eps dropped) must all miss the closed form.
"""

import numpy as np
import pytest

import gguf_encode as ge

H, F, V, EPS = 128, 256, 64, 1e-6
D = 2.0 ** -14
D_BITS = int(ge.half_bits(D))


def _perm_matrix(rows, cols, mapping):
    """Q8_0 GGUF bytes of a rows x cols matrix whose row i has code c at
    column j for every (j, i, c) in mapping, zeros elsewhere, every block
    scale D; also its dense fp64 value."""
    q = np.zeros((rows, cols), np.int64)
    for j, i, c in mapping:
        assert not q[i].any()
        q[i, j] = c
    nb = cols // 32
    out = [ge.encode_q8_0(np.full(nb, D_BITS, np.uint16), q[i].reshape(nb, 32)) for i in range(rows)]
    return np.stack(out), q.astype(np.float64) * D


def _build(seed):
    """Layers and head of the probe, the dense matrices the closed form uses,
    and M = 3 input positions of different magnitudes."""
    rng = np.random.default_rng(seed)
    pos_x = [32 * b + int(rng.integers(0, 32)) for b in range(H // 32)]

    def code():
        return int(rng.integers(16, 128)) * (1 if rng.random() < 0.5 else -1)

    def spread(src_pos, out_len):
        """Each source position to its own output block (so the output keeps
        one nonzero per block), at a random offset, with a random code."""
        blocks = rng.permutation(out_len // 32)[:len(src_pos)]
        assert len(blocks) == len(src_pos)
        return [(j, 32 * int(b) + int(rng.integers(0, 32)), code()) for j, b in zip(src_pos, blocks)]

    dense = {}
    layers = []
    pos = pos_x
    for li in range(2):
        mq, mk, mv = spread(pos, H), spread(pos, H), spread(pos, H)
        mo = spread([i for _, i, _ in mv], H)
        mg = spread([i for _, i, _ in mo], F)
        # up lands on the gate's rows (the product needs both), other codes
        mu = [(j, i, code()) for j, i, _ in mg]
        md = spread([i for _, i, _ in mg], H)
        pos = [i for _, i, _ in md]
        lw = {}
        for name, r, c, mp in (("q", H, H, mq), ("k", H, H, mk), ("v", H, H, mv), ("o", H, H, mo),
                               ("gate", F, H, mg), ("up", F, H, mu), ("down", H, F, md)):
            raw, Wd = _perm_matrix(r, c, mp)
            lw[name] = (8, raw)
            dense[(li, name)] = Wd
        # norm weights in disjoint ranges, so a swap changes every entry
        lw["g1"] = rng.uniform(0.5, 0.9, H).astype(np.float32)
        lw["g2"] = rng.uniform(1.1, 1.6, H).astype(np.float32)
        lw["g3"] = rng.uniform(1.7, 2.2, H).astype(np.float32)
        lw["g4"] = rng.uniform(0.2, 0.45, F).astype(np.float32)
        layers.append(lw)
    rows = rng.permutation(V)[:len(pos)]
    hraw, Wh = _perm_matrix(V, H, [(j, int(i), code()) for j, i in zip(pos, rows)])
    dense["head"] = Wh
    gf = rng.uniform(0.6, 1.4, H).astype(np.float32)
    # positions: eps-dominated, eps-comparable, eps-negligible at the input
    x = np.zeros((3, H), np.float32)
    for j in pos_x:
        for m, (lo, hi) in enumerate(((0.5e-3, 2e-3), (5e-3, 2e-2), (0.05, 0.2))):
            x[m, j] = rng.uniform(lo, hi) * (1 if rng.random() < 0.5 else -1)
    return layers, (8, hraw, gf), dense, x


def _closed_form(layers, head, dense, x, eps=EPS):
    """The recurrence above in fp64, with fp32 rounding where the chain
    stores a value (each quantiser's input and the gate/up product)."""
    f32 = lambda a: np.asarray(a, np.float64).astype(np.float32)

    def rms(v, n):
        v = f32(v).astype(np.float64)
        return 1.0 / np.sqrt((v * v).sum(1, keepdims=True) / n + eps)

    def proj(W, v, gamma):
        return (f32(v) * gamma).astype(np.float64) @ W.T

    cur = x.astype(np.float64)
    for li, lw in enumerate(layers):
        v = rms(cur, H) * proj(dense[(li, "v")], cur, lw["g1"])
        o = rms(v, H) * proj(dense[(li, "o")], v, lw["g2"])
        r3 = rms(o, H)
        g = r3 * proj(dense[(li, "gate")], o, lw["g3"])
        u = r3 * proj(dense[(li, "up")], o, lw["g3"])
        p = (f32(g) * f32(u)).astype(np.float64)
        cur = rms(p, F) * proj(dense[(li, "down")], p, lw["g4"])
    z = rms(cur, H) * proj(dense["head"], cur, head[2])
    return cur, z


def _close(a, b, rtol):
    scale = np.abs(b).max(axis=1, keepdims=True)
    return bool(np.all(np.abs(a - b) <= rtol * scale))


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_chain_pass_closed_form(orc, seed):
    layers, head, dense, x = _build(seed)
    xo, lo = orc.chain_pass(layers, x, H, F, head=head, eps=EPS)
    xc, lc = _closed_form(layers, head, dense, x)
    # a handful of fp32 roundings per stage: 2e-5 of the row's largest entry
    assert _close(xo, xc, 2e-5), np.abs(xo - xc).max()
    assert _close(lo, lc, 2e-5), np.abs(lo - lc).max()
    # the probe is not degenerate: every row carries four nonzero logits
    assert np.all((np.abs(lc) > 0).sum(1) == H // 32)


def test_eps_share_is_visible(orc):
    """The probe's premise: eps moves the logits by more than a percent, so
    a factor from the wrong vector is seen at the end of the chain."""
    layers, head, dense, x = _build(7)
    _, l1 = _closed_form(layers, head, dense, x, eps=EPS)
    _, l0 = _closed_form(layers, head, dense, x, eps=0.0)
    assert not _close(l0, l1, 1e-2)


def _missed(orc, probe, layers=None, head=None, eps=EPS):
    """True when the oracle, run on a mutated copy of the probe's layers or
    head (or with another eps), misses the true probe's closed form by more
    than 1e-3 of a row's largest logit, fifty times the parity bar."""
    L, hd, dense, x = probe
    _, lo = orc.chain_pass(layers or L, x, H, F, head=head or hd, eps=eps)
    _, lc = _closed_form(L, hd, dense, x)
    return not _close(lo, lc, 1e-3)


def test_mutation_swapped_norm_weights_is_caught(orc):
    probe = _build(3)
    layers, head = probe[0], probe[1]
    assert _missed(orc, probe, [dict(lw, g1=lw["g2"], g2=lw["g1"]) for lw in layers])
    assert _missed(orc, probe, [dict(lw, g2=lw["g3"], g3=lw["g2"]) for lw in layers])
    assert _missed(orc, probe, head=(head[0], head[1], layers[-1]["g1"]))


def test_mutation_qkv_mixup_is_caught(orc):
    probe = _build(4)
    layers = probe[0]
    assert _missed(orc, probe, [dict(lw, v=lw["k"]) for lw in layers])
    assert _missed(orc, probe, [dict(lw, v=lw["q"]) for lw in layers])
    assert _missed(orc, probe, [dict(lw, up=lw["gate"]) for lw in layers])


def test_mutation_rms_of_scaled_vector_is_caught(orc, monkeypatch):
    """An RMS factor taken from the vector after its norm weight."""
    probe = _build(5)
    real = orc.quantize_act

    def after_gamma(v, gamma=None):
        q, d, s16, ss = real(v, gamma)
        if gamma is not None:
            vg = np.atleast_2d(v).astype(np.float32) * np.asarray(gamma, np.float32)
            ss = (vg.astype(np.float64) ** 2).sum(1)
        return q, d, s16, ss

    monkeypatch.setattr(orc, "quantize_act", after_gamma)
    assert _missed(orc, probe)


def test_mutation_rms_of_previous_vector_is_caught(orc, monkeypatch):
    """Each consumer scaled by the RMS factor of the stage before its input
    (the factor one hand-off late)."""
    probe = _build(6)
    real = orc.quantize_act
    prev = {}

    def stale(v, gamma=None):
        q, d, s16, ss = real(v, gamma)
        n = np.atleast_2d(v).shape[1]
        out = prev.get("ss", ss) if prev.get("n") == n else ss
        prev.update(ss=ss, n=n)
        return q, d, s16, out

    monkeypatch.setattr(orc, "quantize_act", stale)
    assert _missed(orc, probe)


def test_mutation_eps_dropped_is_caught(orc):
    assert _missed(orc, _build(8), eps=0.0)
