"""Pins for the oracle's argmax and acceptance rules.

* Greedy: the worked example of the Kinetic page ("How Kinetic is fast",
  RAD-1: four drafts kept plus the model's own token = five tokens from one
  pass), the depth semantics of the dasLLAMA page ("What we tried": one draft
  means two positions, the round yields one token plus one more if the draft
  matched), and the invariant accepted length = number of leading drafts
  equal to the argmax.
* Rejection (micrologics page, "Mathematical Integrity"): on tiny
  vocabularies the emitted token follows p exactly (chi-square), the
  acceptance rate is sum_x min(p, q), and after a rejection the token follows
  norm(max(0, p - q)); q = p never rejects, disjoint supports always reject.
* Certain drafter (Kinetic page, "Why the output does not change"): the
  drafted tokens equal plain inverse-CDF sampling with the same uniforms,
  cycle by cycle.
"""

import json
import os

import numpy as np
import pytest
from scipy import stats

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _onehot_logits(top, V, hi=5.0):
    z = np.zeros((len(top), V), np.float32)
    z[np.arange(len(top)), top] = hi
    return z


def test_argmax_ties_lowest(orc):
    z = np.array([[1.0, 3.0, 3.0, 2.0], [0.0, 0.0, 0.0, 0.0], [-1.0, -2.0, -1.0, -0.5]])
    assert list(orc.argmax(z)) == [1, 0, 3]


def test_kinetic_worked_example(orc):
    """Tokens of the example mapped to ids (tests/golden/kinetic_rad1.json)."""
    with open(os.path.join(GOLDEN, "kinetic_rad1.json")) as f:
        g = json.load(f)
    vocab = {t: i for i, t in enumerate(g["vocab"])}
    ids = lambda ts: [vocab[t] for t in ts]
    # Reading 1: four drafts n + 1 ; verified in five rows; the fifth row's
    # own token closes the round.
    out = orc.accept_greedy(ids(g["model"]), ids(g["draft"][:4]))
    assert out[0] == 4 and list(out[1:6]) == ids(g["kept"])
    # Reading 2: all five drafts verified (six rows); the fifth draft
    # mismatches and is replaced by the model's token.  Same kept tokens.
    out = orc.accept_greedy(ids(g["model"]) + [0], ids(g["draft"]))
    assert out[0] == 4 and list(out[1:6]) == ids(g["kept"])
    assert out[0] + 1 == g["tokens_per_pass"]


def test_depth_one_semantics(orc):
    # one draft = two rows; a match yields two tokens, a mismatch one
    assert list(orc.accept_greedy([7, 9], [7])) == [1, 7, 9]
    out = orc.accept_greedy([7, 9], [8])
    assert out[0] == 0 and out[1] == 7


@pytest.mark.parametrize("seed", range(5))
def test_greedy_invariant(orc, seed):
    rng = np.random.default_rng(seed)
    for _ in range(200):
        K = int(rng.integers(0, 16))
        top = rng.integers(0, 4, K + 1)
        drafts = np.where(rng.random(K) < 0.7, top[:K], rng.integers(0, 4, K))
        out = orc.accept_greedy(top, drafts)
        n = 0
        while n < K and drafts[n] == top[n]:
            n += 1
        assert out[0] == n
        assert list(out[1:n + 1]) == list(drafts[:n]) and out[n + 1] == top[n]


def test_greedy_all_match(orc):
    top = np.arange(6)
    out = orc.accept_greedy(top, top[:5])
    assert out[0] == 5 and list(out[1:]) == list(range(6))


def test_temperature_must_be_positive(orc):
    with pytest.raises(ValueError):
        orc.accept_rejection(np.zeros((2, 4)), [0], np.zeros(4), temperature=0.0)


def _softmax64(z, T=1.0):
    z = np.asarray(z, np.float64) / T
    e = np.exp(z - z.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


def _draw(cdf_src, u):
    c = np.cumsum(cdf_src)
    return int(np.searchsorted(c, u * c[-1], side="right"))


@pytest.mark.parametrize("V,seed", [(4, 0), (8, 1), (16, 2)])
def test_rejection_distribution(orc, V, seed):
    """One-draft rounds: emitted first token ~ p, acceptance rate
    sum min(p, q), rejected-branch token ~ norm(max(0, p - q))."""
    rng = np.random.default_rng(seed)
    z = (rng.standard_normal((2, V)) * 1.5).astype(np.float32)
    qv = rng.dirichlet(np.ones(V)).astype(np.float32)
    p = _softmax64(z[0])
    trials = 60000
    u = rng.integers(0, 1 << 53, (trials, 2, 2)).astype(np.float64) * 2.0 ** -53
    ux = rng.random(trials)
    qc = qv.astype(np.float64)
    first = np.empty(trials, np.int64)
    acc = np.zeros(trials, bool)
    for t in range(trials):
        x = _draw(qc, ux[t])
        out = orc.accept_rejection(z, [x], u[t], 1.0, q=qv[None, :])
        first[t] = out[1]
        acc[t] = out[0] == 1
    counts = np.bincount(first, minlength=V)
    assert stats.chisquare(counts, p * trials).pvalue > 1e-4
    rate = np.minimum(p, qc).sum()
    assert abs(acc.mean() - rate) < 5 * np.sqrt(rate * (1 - rate) / trials)
    res = np.maximum(p - qc, 0.0)
    res /= res.sum()
    rc = np.bincount(first[~acc], minlength=V)
    keep = res > 0
    assert rc[~keep].sum() == 0
    assert stats.chisquare(rc[keep], res[keep] * rc.sum()).pvalue > 1e-4


def test_rejection_q_equals_p_never_rejects(orc):
    # q is p rounded to fp32; with p = 1/8, 1/8, 1/4, 1/2 the rounding is at
    # most one fp64 ulp, so only a uniform within ~1e-15 of 1 could reject.
    z = np.log(np.array([[1, 1, 2, 4], [1, 2, 4, 1]], np.float64)).astype(np.float32)
    p = _softmax64(z[0]).astype(np.float32)
    rng = np.random.default_rng(5)
    for _ in range(500):
        u = rng.random(4)
        x = int(rng.integers(0, 4))
        out = orc.accept_rejection(z, [x], u, 1.0, q=p[None, :])
        assert out[0] == 1


def test_rejection_disjoint_supports_always_reject(orc):
    V = 8
    z = np.full((2, V), -3e38, np.float32)
    z[:, :4] = 0.0
    qv = np.zeros(V, np.float32)
    qv[4:] = 0.25
    rng = np.random.default_rng(6)
    for _ in range(300):
        x = int(rng.integers(4, 8))
        out = orc.accept_rejection(z, [x], rng.random(4), 1.0, q=qv[None, :])
        assert out[0] == 0 and out[1] < 4


@pytest.mark.parametrize("seed", range(3))
def test_certain_drafter_equals_plain_sampling(orc, seed):
    rng = np.random.default_rng(seed)
    V, K = 12, 4
    for _ in range(400):
        z = (rng.standard_normal((K + 1, V)) * 2).astype(np.float32)
        u = rng.random((K + 1, 2))
        e = np.exp(z.astype(np.float64) - z.astype(np.float64).max(1, keepdims=True))
        plain = [_draw(e[i], u[i, 0]) for i in range(K + 1)]
        drafts = [plain[i] if rng.random() < 0.6 else int(rng.integers(0, V)) for i in range(K)]
        out = orc.accept_rejection(z, drafts, u, 1.0, q=None)
        n = out[0]
        k = 0
        while k < K and drafts[k] == plain[k]:
            k += 1
        assert n == k
        assert list(out[1:n + 2]) == plain[:n + 1]


def test_certain_drafter_acceptance_rate(orc):
    """The guess x survives with probability p(x)."""
    rng = np.random.default_rng(9)
    V = 6
    z = (rng.standard_normal((2, V))).astype(np.float32)
    p = _softmax64(z[0])
    x = 2
    trials = 40000
    u = rng.random((trials, 2, 2))
    acc = sum(orc.accept_rejection(z, [x], u[t], 1.0)[0] for t in range(trials)) / trials
    assert abs(acc - p[x]) < 5 * np.sqrt(p[x] * (1 - p[x]) / trials)


def test_bonus_from_last_row(orc):
    """All drafts accepted: one more token is sampled from row K."""
    V = 5
    z = np.full((3, V), -3e38, np.float32)
    z[0, 1] = z[1, 3] = 0.0   # rows 0, 1 certain of tokens 1 and 3
    z[2, 4] = 0.0             # row 2 certain of token 4
    out = orc.accept_rejection(z, [1, 3], np.full(6, 0.5), 1.0)
    assert list(out) == [2, 1, 3, 4]
    q = np.zeros((2, V), np.float32)
    q[0, 1] = q[1, 3] = 1.0
    out = orc.accept_rejection(z, [1, 3], np.full(6, 0.5), 1.0, q=q)
    assert list(out) == [2, 1, 3, 4]
