"""GPU parity of the verification pass against the CPU oracle, through the
C ABI.  Bars: bit-exact for bytes, codes, integer block sums, argmax and
accepted tokens; |y_gpu - y_oracle| <= 1e-5 * T for fp32 outputs, with T the
sum of |block terms| (the bound reordering error scales with); bit-identical
rows between an M-row call and the same row alone."""

import numpy as np
import pytest

import synth
import gguf_encode as ge
import interval

pytestmark = pytest.mark.gpu

QT = [8, 12, 14]
TOL = 1e-5


@pytest.fixture(scope="module")
def gu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gpu_util
    import speculative_decoding_verification_amd as sv
    sv.lib()
    return gpu_util


def _oracle_act(orc, x, gamma=None):
    q, d, s16, ss = orc.quantize_act(x, gamma)
    return q, d, s16


# ------------------------------------------------------------------ a1
@pytest.mark.parametrize("qt,N,K", [(8, 96, 1024), (12, 64, 2560), (14, 33, 5120), (14, 7, 256), (12, 3, 768)])
def test_repack_roundtrip(gu, qt, N, K):
    import speculative_decoding_verification_amd as sv
    import torch
    raw = synth.gguf_weights(qt, N, K, seed=11)
    W, buf = gu.upload_weight(qt, raw, K)
    back = torch.empty(raw.size, dtype=torch.uint8, device="cuda")
    sv.unpack_weights(qt, buf, back, N, K)
    assert np.array_equal(gu.host(back).reshape(N, -1), raw)


# ------------------------------------------------------------------ a2
@pytest.mark.parametrize("M,K", [(1, 32), (5, 1024), (16, 2560), (3, 17408)])
def test_quantize_bitexact(gu, orc, M, K):
    rng = np.random.default_rng(M * 1000 + K)
    x = synth.activations(M, K, 3, K)
    x[0, :32] = 0.0                                 # zero block
    if K >= 64:
        x[0, 32:64] = np.arange(32) - 15.5          # exact halves after scaling
        x[0, 63] = 127.0
    g = synth.rms_weight(K, seed=4)
    for gamma in (None, g):
        b = gu.quantize(x, gamma)
        q, d, s16, ss = orc.quantize_act(x, gamma)
        assert np.array_equal(gu.host(b.q), q)
        assert np.array_equal(gu.host(b.d), d)
        assert np.array_equal(gu.host(b.s16), s16)
        parts = gu.host(b.sumsq).astype(np.float64)
        ref = (x.astype(np.float64) ** 2).reshape(M, K // 32, 32).sum(2)
        assert np.allclose(parts, ref, rtol=1e-6, atol=0)


# ------------------------------------------------------------------ a3 exact integer probes
@pytest.mark.parametrize("qt", QT)
@pytest.mark.parametrize("M", [1, 5])
def test_unit_scale_integer_exact(gu, orc, qt, M):
    """Unit scales and integer activations with block maximum 127: every
    output is an exact integer; with one nonzero weight block per row the
    output is that row's int32 block sum."""
    import speculative_decoding_verification_amd as sv
    rng = np.random.default_rng(qt * 7 + M)
    N, K = 64, 1024
    Wb, Wf = ge.random_fields(qt, N, K, rng, unit=True)
    x = rng.integers(-127, 128, (M, K)).astype(np.float32)
    x.reshape(M, K // 32, 32)[:, :, 5] = 127.0
    b = gu.quantize(x)
    assert np.all(gu.host(b.d) == 1.0)
    W, wbuf = gu.upload_weight(qt, Wb, K)
    y = gu.empty((M, N), gu.torch().float32)
    sv.verify_matvec([W], b.act(), [y])
    ref = x.astype(np.int64) @ np.rint(Wf).astype(np.int64).T
    assert np.array_equal(gu.host(y), ref.astype(np.float32))
    # single nonzero block per row -> the row's exact int32 block sum
    q, d, s16 = _oracle_act(orc, x)
    _, _, bs = orc.matvec(qt, Wb, K, q, d, block_sums=True)
    nb = K // 32
    blk = rng.integers(0, nb, N)
    Wz = np.rint(Wf).astype(np.int64).reshape(N, nb, 32)
    keep = np.zeros_like(Wz)
    keep[np.arange(N), blk] = Wz[np.arange(N), blk]
    Wb2 = _encode_unit(qt, keep.reshape(N, K))
    W2, wbuf2 = gu.upload_weight(qt, Wb2, K)
    sv.verify_matvec([W2], b.act(), [y])
    got = gu.host(y)
    want = bs[:, np.arange(N), blk]
    if qt != 14:
        assert np.array_equal(got, want.astype(np.float32))
    else:  # Q6_K block sums fold the two int8 sub-scales (1 here)
        assert np.array_equal(got, want.astype(np.float32))


def _encode_unit(qt, w):
    """Encode an integer matrix whose values fit the format with unit
    scales (Q8_0: any int8; Q4_K: 0..15; Q6_K: -32..31)."""
    N, K = w.shape
    one = int(ge.half_bits(1.0))
    rows = []
    for r in range(N):
        if qt == 8:
            nb = K // 32
            rows.append(ge.encode_q8_0(np.full(nb, one, np.uint16), w[r].reshape(nb, 32)))
        elif qt == 12:
            ns = K // 256
            rows.append(ge.encode_q4_k(np.full(ns, one, np.uint16), np.zeros(ns, np.uint16),
                                       np.ones((ns, 8)), np.zeros((ns, 8)), w[r].reshape(ns, 256)))
        else:
            ns = K // 256
            rows.append(ge.encode_q6_k(np.full(ns, one, np.uint16), np.ones((ns, 16)), w[r].reshape(ns, 256) + 32))
    return np.stack(rows)


# ------------------------------------------------------------------ a3 tolerance parity
# K = 1056 and 5152 (Q8_0 only): K chunks whose scale and code-sum rows are
# not whole 16-byte pieces (33 and 81 sub-blocks), staged row by row
SHAPES = [(96, 1024), (64, 2560), (160, 5120), (32, 768), (64, 9728), (32, 17408), (64, 1056), (32, 5152)]


@pytest.mark.parametrize("qt", QT)
@pytest.mark.parametrize("N,K", SHAPES)
@pytest.mark.parametrize("M", [1, 2, 5, 8, 16])
def test_matvec_parity(gu, orc, qt, N, K, M):
    _check_matvec(gu, orc, qt, N, K, M)


@pytest.mark.parametrize("qt", QT)
@pytest.mark.parametrize("N,K", [(64, 9728), (32, 17408)])
@pytest.mark.parametrize("M", [7, 10, 12, 13])
def test_matvec_parity_split_combine(gu, orc, qt, N, K, M):
    """Tiles split over K (two and four chunks) where the tile's last unit
    reloads the partials in rounds of two position pairs (M = 7..12: at
    M = 10 the last round holds one pair, at M = 7 the last pair has one
    position past M, at M = 12 every round is full) or one pair at a time
    (M = 13)."""
    _check_matvec(gu, orc, qt, N, K, M)


def _check_matvec(gu, orc, qt, N, K, M):
    import speculative_decoding_verification_amd as sv
    if qt != 8 and K % 256:
        pytest.skip("K-quants need K % 256 == 0")
    raw = synth.gguf_weights(qt, N, K, 21, M)
    x = synth.activations(M, K, 22, N)
    b = gu.quantize(x)
    q, d, s16 = _oracle_act(orc, x)
    assert np.array_equal(gu.host(b.q), q)
    W, wbuf = gu.upload_weight(qt, raw, K)
    y = gu.empty((M, N), gu.torch().float32)
    sv.verify_matvec([W], b.act(), [y])
    y64, T = orc.matvec(qt, raw, K, q, d)
    err = np.abs(gu.host(y).astype(np.float64) - y64)
    assert np.all(err <= TOL * T + 1e-30), (err / np.maximum(T, 1e-30)).max()


@pytest.mark.parametrize("qt", QT)
def test_batch_invariance_and_determinism(gu, qt):
    import speculative_decoding_verification_amd as sv
    N, K = 192, 5120 if qt != 8 else 2048
    raw = synth.gguf_weights(qt, N, K, seed=31)
    W, wbuf = gu.upload_weight(qt, raw, K)
    x = synth.activations(16, K, seed=32)
    full = {}
    for M in (16, 8, 5, 2):
        b = gu.quantize(x[:M])
        y = gu.empty((M, N), gu.torch().float32)
        sv.verify_matvec([W], b.act(), [y])
        full[M] = gu.host(y)
    for m in range(16):
        b = gu.quantize(x[m:m + 1])
        y = gu.empty((1, N), gu.torch().float32)
        sv.verify_matvec([W], b.act(), [y])
        alone = gu.host(y)[0]
        for M, ys in full.items():
            if m < M:
                assert np.array_equal(ys[m].view(np.uint32), alone.view(np.uint32)), (M, m)
    b = gu.quantize(x[:5])
    y2 = gu.empty((5, N), gu.torch().float32)
    sv.verify_matvec([W], b.act(), [y2])
    assert np.array_equal(gu.host(y2).view(np.uint32), full[5].view(np.uint32))


def test_shared_input_three_matrices(gu, orc):
    import speculative_decoding_verification_amd as sv
    qt, N, K, M = 12, 128, 2560, 5
    raws = [synth.gguf_weights(qt, N, K, 41, i) for i in range(3)]
    ups = [gu.upload_weight(qt, r, K) for r in raws]
    x = synth.activations(M, K, seed=42)
    b = gu.quantize(x)
    q, d, _ = _oracle_act(orc, x)
    ys = [gu.empty((M, N), gu.torch().float32) for _ in range(3)]
    sv.verify_matvec([u[0] for u in ups], b.act(), ys)
    for r, y in zip(raws, ys):
        y64, T = orc.matvec(qt, r, K, q, d)
        assert np.all(np.abs(gu.host(y) - y64) <= TOL * T)
    # each matrix alone gives the same bits
    for i, u in enumerate(ups):
        y1 = gu.empty((M, N), gu.torch().float32)
        sv.verify_matvec([u[0]], b.act(), [y1])
        assert np.array_equal(gu.host(y1).view(np.uint32), gu.host(ys[i]).view(np.uint32))


# ------------------------------------------------------------------ a4 epilogue
@pytest.mark.parametrize("qt", [12, 14])
def test_epilogue_quant_and_rms_fold(gu, orc, qt):
    import speculative_decoding_verification_amd as sv
    import torch
    N, K, M = 256, 2560, 5
    raw = synth.gguf_weights(qt, N, K, seed=51)
    W, wbuf = gu.upload_weight(qt, raw, K)
    x = synth.activations(M, K, seed=52)
    g_in = synth.rms_weight(K, seed=53)
    b = gu.quantize(x, g_in)                  # int8 of x * gamma, partials of x^2
    parts = b.sumsq
    gamma = synth.rms_weight(N, seed=54)
    out = gu.ActBuf(M, N)
    y = gu.empty((M, N), torch.float32)
    ep = sv.epilogue(sv.SV_EP_QUANT, out.q, out.d, out.s16, out.sumsq, gamma=gu.dev(gamma), src=0)
    sv.verify_matvec([W], b.act(parts, K // 32, 1e-6), [y], ep)
    q, d, s16 = _oracle_act(orc, x, g_in)
    ss = gu.host(parts).astype(np.float64).sum(1)
    r = 1.0 / np.sqrt(ss / K + 1e-6)
    y64, T = orc.matvec(qt, raw, K, q, d, scale=r)
    yg = gu.host(y).astype(np.float64)
    assert np.all(np.abs(yg - y64) <= TOL * T)
    interval.check_requant(y64, TOL * T, gamma, gu.host(out.q), gu.host(out.d), gu.host(out.s16),
                           gu.host(out.sumsq))


@pytest.mark.parametrize("N,K,M", [(512, 2560, 5), (512, 2560, 9), (9728, 2560, 16), (2048, 6144, 9)])
def test_epilogue_pair(gu, orc, N, K, M):
    """Gate/up pair with the product's requantisation: fused units up to
    M = 8, two matrices joined through the K-split partials above (M = 9,
    16), a balanced decomposition at 9728 rows, two K chunks at K = 6144."""
    import speculative_decoding_verification_amd as sv
    import torch
    qt = 12
    rg = synth.gguf_weights(qt, N, K, 61, "g")
    ru = synth.gguf_weights(qt, N, K, 61, "u")
    Wg, bg = gu.upload_weight(qt, rg, K)
    Wu, bu = gu.upload_weight(qt, ru, K)
    x = synth.activations(M, K, seed=62)
    b = gu.quantize(x)
    gamma = synth.rms_weight(N, seed=63)
    out = gu.ActBuf(M, N)
    yg = gu.empty((M, N), torch.float32)
    yu = gu.empty((M, N), torch.float32)
    ep = sv.epilogue(sv.SV_EP_PAIR, out.q, out.d, out.s16, out.sumsq, gamma=gu.dev(gamma))
    sv.verify_matvec([Wg, Wu], b.act(), [yg, yu], ep)
    q, d, _ = _oracle_act(orc, x)
    g64, Tg = orc.matvec(qt, rg, K, q, d)
    u64, Tu = orc.matvec(qt, ru, K, q, d)
    hg, hu = gu.host(yg), gu.host(yu)
    assert np.all(np.abs(hg - g64) <= TOL * Tg) and np.all(np.abs(hu - u64) <= TOL * Tu)
    # the product the epilogue quantises is fp32(g) * fp32(u) of the outputs
    interval.check_requant(g64 * u64, interval.pair_bound(g64, Tg, u64, Tu, TOL), gamma, gu.host(out.q),
                           gu.host(out.d), gu.host(out.s16), gu.host(out.sumsq))
    # each row of an M-row call equals the same row alone
    if M > 1:
        b1 = gu.quantize(x[M - 1:M])
        out1 = gu.ActBuf(1, N)
        y1 = [gu.empty((1, N), torch.float32) for _ in range(2)]
        ep1 = sv.epilogue(sv.SV_EP_PAIR, out1.q, out1.d, out1.s16, out1.sumsq, gamma=gu.dev(gamma))
        sv.verify_matvec([Wg, Wu], b1.act(), y1, ep1)
        assert np.array_equal(gu.host(y1[0]).view(np.uint32), hg[M - 1:].view(np.uint32))
        assert np.array_equal(gu.host(out1.q), gu.host(out.q)[M - 1:])
        assert np.array_equal(gu.host(out1.d).view(np.uint32), gu.host(out.d)[M - 1:].view(np.uint32))


# ------------------------------------------------------------------ a6 / a9 head
@pytest.mark.parametrize("qt,V,K", [(8, 4096, 1024), (14, 3000, 5120), (14, 151936, 5120)])
def test_head_logits_argmax(gu, orc, qt, V, K):
    import speculative_decoding_verification_amd as sv
    import torch
    M = 5
    raw = synth.gguf_weights(qt, V, K, seed=71)
    H, hb = gu.upload_weight(qt, raw, K)
    x = synth.activations(M, K, seed=72)
    b = gu.quantize(x)
    logits = gu.empty((M, V), torch.float32)
    am = gu.zeros((M,), torch.int64)
    sv.head_logits(H, b.act(), logits, am)
    lg = gu.host(logits)
    packed = gu.host(am).view(np.uint64)
    idx = np.array([sv.argmax_index(int(p)) for p in packed])
    # argmax must be exactly the first maximum of the GPU's own logits
    assert np.array_equal(idx, lg.argmax(1))
    q, d, _ = _oracle_act(orc, x)
    if V <= 5000:
        y64, T = orc.matvec(qt, raw, K, q, d)
        assert np.all(np.abs(lg - y64) <= TOL * T)
        top = orc.argmax(y64)
        # decided rows: top-2 margin larger than twice the tolerance
        s = np.sort(y64, 1)
        margin = s[:, -1] - s[:, -2]
        tol = 2 * TOL * T.max(1)
        decided = margin > tol
        assert np.array_equal(idx[decided], top[decided])
    else:
        # full vocabulary: oracle on a seeded sample of rows plus the GPU's winners
        ids = np.unique(np.concatenate([synth.token_ids(512, V, seed=73), idx])).astype(np.int32)
        y64, T = orc.matvec(qt, raw, K, q, d, row_ids=ids)
        assert np.all(np.abs(lg[:, ids] - y64) <= TOL * T)


def test_restricted_head_rows_bitwise(gu, orc):
    """A restricted head (row gather) scores each row exactly as the full
    head does; the argmax returns the position inside the id list."""
    import speculative_decoding_verification_amd as sv
    import torch
    qt, V, K, M = 8, 4096, 1024, 3
    raw = synth.gguf_weights(qt, V, K, seed=81)
    H, hb = gu.upload_weight(qt, raw, K)
    x = synth.activations(M, K, seed=82)
    b = gu.quantize(x)
    full = gu.empty((M, V), torch.float32)
    sv.head_logits(H, b.act(), full, None)
    ids = synth.token_ids(700, V, seed=83, distinct=True)
    ids_d = gu.dev(ids)
    part = gu.empty((M, ids.size), torch.float32)
    am = gu.zeros((M,), torch.int64)
    sv.head_logits(H, b.act(), part, am, row_ids=ids_d)
    fl, pl = gu.host(full), gu.host(part)
    assert np.array_equal(pl.view(np.uint32), fl[:, ids].view(np.uint32))
    pos = np.array([sv.argmax_index(int(p)) for p in gu.host(am).view(np.uint64)])
    assert np.array_equal(pos, pl.argmax(1))


# ------------------------------------------------------------------ a7 / a8 acceptance
def _packed(logits_rows):
    """Host packing of the first maximum of each row (for greedy inputs)."""
    out = []
    for r in logits_rows:
        i = int(np.argmax(r))
        f = np.float32(r[i]) + np.float32(0.0)
        u = int(np.array([f], np.float32).view(np.uint32)[0])
        key = (~u & 0xFFFFFFFF) if (u & 0x80000000) else (u | 0x80000000)
        out.append((key << 32) | (0xFFFFFFFF - i))
    return np.array(out, np.uint64)


@pytest.mark.parametrize("seed", range(4))
def test_accept_greedy(gu, orc, seed):
    import speculative_decoding_verification_amd as sv
    import torch
    rng = np.random.default_rng(seed)
    for K in (0, 1, 4, 15):
        V = 50
        z = rng.standard_normal((K + 1, V)).astype(np.float32)
        top = z.argmax(1)
        drafts = synth.drafts_from(top[:K], V, 0.75, seed, K)
        out = gu.zeros((K + 2,), torch.int32)
        am = gu.dev(_packed(z).view(np.int64))
        dd = gu.dev(drafts) if K else None
        sv.accept_greedy(am, dd, out, V)
        assert np.array_equal(gu.host(out), orc.accept_greedy(top, drafts))
    # restricted head: argmax positions map through the id list
    ids = np.array([5, 9, 11, 40], np.int32)
    z = np.full((3, 4), -1.0, np.float32)
    z[0, 1] = z[1, 2] = z[2, 3] = 1.0
    out = gu.zeros((4,), torch.int32)
    sv.accept_greedy(gu.dev(_packed(z).view(np.int64)), gu.dev(np.array([9, 11], np.int32)), out, ids.size,
                     row_ids=gu.dev(ids))
    assert list(gu.host(out)) == [2, 9, 11, 40]


@pytest.mark.parametrize("V,T,mode,seed", [(997, 1.0, "general", 0), (997, 0.7, "certain", 1),
                                           (151936, 1.0, "general", 2), (151936, 1.0, "certain", 3),
                                           (4096, 1.3, "general", 4)])
def test_accept_rejection(gu, orc, V, T, mode, seed):
    import speculative_decoding_verification_amd as sv
    import torch
    K = 4
    ws = gu.empty((sv.accept_workspace_bytes(V, K),), torch.uint8)
    uncertified = 0
    cycles = 12 if V > 100000 else 40
    for c in range(cycles):
        z = synth.normals((K + 1, V), seed, c, sigma=2.0)
        qd = None
        if mode == "general":
            zq = z[:K].astype(np.float64) + synth.normals((K, V), seed, c, "q", sigma=0.5, dtype=np.float64)
            e = np.exp(zq - zq.max(1, keepdims=True))
            qd = (e / e.sum(1, keepdims=True)).astype(np.float32)
            drafts = np.array([int(np.searchsorted(np.cumsum(qd[i].astype(np.float64)),
                                                   synth.uniforms((), seed, c, i) * qd[i].sum(dtype=np.float64),
                                                   side="right")) for i in range(K)], np.int32)
            drafts = np.minimum(drafts, V - 1)
        else:
            drafts = synth.drafts_from(z[:K].argmax(1), V, 0.6, seed, c)
        u = synth.uniforms((K + 1, 2), seed, c, "acc")
        want, mg = orc.accept_rejection(z, drafts, u, T, q=qd, with_margin=True)
        out = gu.zeros((K + 2,), torch.int32)
        sv.accept_rejection(gu.dev(z), gu.dev(drafts), gu.dev(u), out, ws, temperature=T,
                            q=None if qd is None else gu.dev(qd))
        got = gu.host(out)
        n = want[0]
        if np.all(mg[:n + 1] > 1e-9):
            assert np.array_equal(got, want), (c, got, want)
        else:
            uncertified += 1
    assert uncertified <= 1


def _softmax64(z):
    e = np.exp(z.astype(np.float64) - z.astype(np.float64).max())
    return e / e.sum()


def _rejection_both(gu, orc, z, drafts, u, q, T=1.0):
    """GPU and oracle acceptance on the same inputs; returns (gpu, oracle,
    oracle margins).  For the general drafter at K = 0 the GPU gets a
    one-row q it never reads (a null q selects the certain drafter)."""
    import speculative_decoding_verification_amd as sv
    import torch
    K, V = len(drafts), z.shape[1]
    ws = gu.empty((sv.accept_workspace_bytes(V, K),), torch.uint8)
    out = gu.zeros((K + 2,), torch.int32)
    dd = np.asarray(drafts, np.int32)
    qg = None if q is None else gu.dev(q if K else np.zeros((1, V), np.float32))
    sv.accept_rejection(gu.dev(z), gu.dev(dd) if K else None, gu.dev(u), out, ws, temperature=T, q=qg)
    want, mg = orc.accept_rejection(z, dd, u, T, q=None if q is None else np.asarray(q, np.float32).reshape(K, V),
                                    with_margin=True)
    return gu.host(out), want, mg


def test_accept_rejection_edges(gu, orc):
    """Edge cases of the rejection rule (micrologics, "Mathematical Integrity:
    Rejection Sampling for LLMs"), GPU against oracle bit for bit."""
    rng = np.random.default_rng(17)
    V = 97
    # K = 0: one token from row 0; the certain drafter draws it with u[0][0],
    # the general one as the bonus with u[0][1]
    for t in range(40):
        z = (rng.standard_normal((1, V)) * 2).astype(np.float32)
        u = rng.random((1, 2))
        for q in (None, np.zeros((0, V), np.float32)):
            got, want, _ = _rejection_both(gu, orc, z, [], u, q)
            assert np.array_equal(got, want) and got[0] == 0
    # q = p (p exactly representable): every draft is kept
    z = np.tile(np.log(np.array([1, 1, 2, 4], np.float64)).astype(np.float32), (5, 1))
    p = _softmax64(z[0]).astype(np.float32)
    for t in range(100):
        drafts = rng.integers(0, 4, 4)
        got, want, _ = _rejection_both(gu, orc, z, drafts, rng.random((5, 2)), np.tile(p, (4, 1)))
        assert np.array_equal(got, want) and got[0] == 4
    # disjoint supports: p on 0..3, q on 4..7: the first draft is rejected
    # and the token comes from the residual, which is p
    z = np.full((3, 8), -3e38, np.float32)
    z[:, :4] = 0.0
    q = np.zeros((2, 8), np.float32)
    q[:, 4:] = 0.25
    for t in range(100):
        got, want, _ = _rejection_both(gu, orc, z, rng.integers(4, 8, 2), rng.random((3, 2)), q)
        assert np.array_equal(got, want) and got[0] == 0 and got[1] < 4
    # R = 0: q = 2p leaves no residual mass; a rejection (u0 q(x) >= p(x),
    # i.e. u0 >= 1/2) then draws from p itself with u[i][1]
    rejected = 0
    for t in range(200):
        z = (rng.standard_normal((3, 50)) * 1.5).astype(np.float32)
        q = np.stack([(2 * _softmax64(z[i])).astype(np.float32) for i in range(2)])
        drafts = rng.integers(0, 50, 2)
        u = rng.random((3, 2))
        u[:, 0] = np.where(np.abs(u[:, 0] - 0.5) < 1e-6, 0.25, u[:, 0])
        got, want, mg = _rejection_both(gu, orc, z, drafts, u, q)
        assert np.all(mg[:want[0] + 1] > 1e-9)
        assert np.array_equal(got, want)
        rejected += int(want[0] < 2)
    assert rejected > 50


def test_restricted_drafter_head_vs_oracle(gu, orc):
    """Q8_0 drafter head over 32768 seeded distinct tokens plus 256 appended
    tokens outside that set, in arbitrary order (OpenJet, "Cheap drafting,
    careful state management": a fixed bundle of frequent tokens with the
    sequence's own tokens added as they appear), read from a 151936-token
    Q8_0 head through row_ids.  Logits against the oracle's row_ids path
    within 1e-5 * T, bit-identical to the same rows of the full head, and
    the argmax position checked by interval on every row."""
    import speculative_decoding_verification_amd as sv
    import torch
    qt, V, K = 8, 151936, 5120
    raw = synth.gguf_weights(qt, V, K, seed=91)
    H, hb = gu.upload_weight(qt, raw, K)
    bundle = synth.token_ids(32768, V, seed=92, distinct=True)
    rest = np.setdiff1d(np.arange(V), bundle)
    tail = synth.stream(93, "tail").permutation(rest)[:256]
    ids = np.concatenate([bundle, tail]).astype(np.int32)
    ids_d = gu.dev(ids)
    for M in (5, 16):
        x = synth.activations(M, K, seed=94)
        b = gu.quantize(x)
        part = gu.empty((M, ids.size), torch.float32)
        am = gu.zeros((M,), torch.int64)
        sv.head_logits(H, b.act(), part, am, row_ids=ids_d)
        full = gu.empty((M, V), torch.float32)
        sv.head_logits(H, b.act(), full, None)
        pl, fl = gu.host(part), gu.host(full)
        assert np.array_equal(pl.view(np.uint32), fl[:, ids].view(np.uint32))
        q, d, _ = _oracle_act(orc, x)
        y64, T = orc.matvec(qt, raw, K, q, d, row_ids=ids)
        assert np.all(np.abs(pl - y64) <= TOL * T)
        pos = np.array([sv.argmax_index(int(p)) for p in gu.host(am).view(np.uint64)])
        assert np.array_equal(pos, pl.argmax(1))
        assert interval.check_winner(pos, y64, TOL * T) == M


def test_restricted_head_tie_rule(gu, orc):
    """Equal logits resolve to the lowest position in the id list, not the
    lowest token id: a bundle row beats an appended row it ties with, and of
    two tied appended rows the earlier one wins although its token id is the
    larger.  The tied rows are byte copies of one dominant row (scale 1, codes
    127 times the sign of the input's codes)."""
    import speculative_decoding_verification_amd as sv
    import torch
    qt, V, K = 8, 4096, 1024
    x = synth.activations(1, K, seed=95)
    xq = orc.quantize_act(x)[0][0]
    nb = K // 32
    dom = ge.encode_q8_0(np.full(nb, int(ge.half_bits(1.0)), np.uint16),
                         (np.where(xq >= 0, 127, -127)).reshape(nb, 32))
    bundle = synth.token_ids(3000, V, seed=96, distinct=True)
    rest = np.setdiff1d(np.arange(V), bundle)
    tail = synth.stream(97, "tail").permutation(rest)[:256]
    ids = np.concatenate([bundle, tail]).astype(np.int32)
    # tail positions a < b with ids[a] > ids[b]
    a = next(i for i in range(3000, ids.size - 1) if ids[i] > ids[i + 1])
    b = a + 1
    cases = [((10, a), 10), ((a, b), a)]
    b_act = gu.quantize(x)
    for (p0, p1), want in cases:
        raw = synth.gguf_weights(qt, V, K, seed=98)
        raw[ids[p0]] = dom
        raw[ids[p1]] = dom
        H, hb = gu.upload_weight(qt, raw, K)
        part = gu.empty((1, ids.size), torch.float32)
        am = gu.zeros((1,), torch.int64)
        sv.head_logits(H, b_act.act(), part, am, row_ids=gu.dev(ids))
        pl = gu.host(part)[0]
        assert pl[p0] == pl[p1] and pl[p0] == pl.max()
        assert sv.argmax_index(int(gu.host(am).view(np.uint64)[0])) == want
        # greedy acceptance maps the position to its token
        out = gu.zeros((2,), torch.int32)
        sv.accept_greedy(am, None, out, ids.size, row_ids=gu.dev(ids))
        assert list(gu.host(out)) == [0, int(ids[want])]
