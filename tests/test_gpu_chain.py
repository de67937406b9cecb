"""GPU tests of the whole verification pass over a projection stack.

* The persistent one-launch pass equals the eager phase-by-phase calls bit
  for bit (same units, same order of every fp32 operation).
* Graph replays of the pass, with eager work in between, repeat the same bits.
* Whole-stack batch invariance: the logits of row m of an M-row pass are
  bit-identical to a 1-row pass of that row alone.
* Against the oracle's plain reading of the chain (fp64 projections, fp32
  quantiser decisions), run free: every int8 code both sides quantise can
  differ only at half-way ties, so the final logits agree to a small fraction
  of their scale and the argmax agrees wherever the top-2 margin is clear.
"""

import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import speculative_decoding_verification_amd as sv
    sv.lib()
    return sv


def _weights_fn(seed, keep):
    def fn(layer, name, qtype, rows, cols):
        if name.startswith("gamma:"):
            return synth.rms_weight(rows, seed, layer, name)
        raw = synth.gguf_weights(qtype, rows, cols, seed, layer, name)
        keep[(layer, name)] = (qtype, raw)
        return raw
    return fn


def _stack(env, shape, seed, max_M=16):
    from speculative_decoding_verification_amd.chain import VerifyStack
    keep = {}
    st = VerifyStack(shape, _weights_fn(seed, keep), max_M=max_M)
    return st, keep


def _set_x(st, x):
    import torch
    st.x[:x.shape[0]].copy_(torch.from_numpy(x).cuda())


def _oracle_chain(orc, keep, shape, seed, x):
    H, F = shape.hidden, shape.ffn
    layers = []
    for li in range(shape.layers):
        lw = {n: keep[(li, n)] for n in ("q", "k", "v", "o", "gate", "up", "down")}
        for g, n in (("g1", H), ("g2", H), ("g3", H), ("g4", F)):
            lw[g] = synth.rms_weight(n, seed, li, "gamma:" + g)
        layers.append(lw)
    hq, hraw = keep[(-1, "head")]
    head = (hq, hraw, synth.rms_weight(H, seed, -1, "gamma:final"))
    return orc.chain_pass(layers, x, H, F, head=head)


SMALL = dict(hidden=512, ffn=1536, layers=3, vocab=4096)


def test_pass_equals_eager_and_graph_replays(env):
    import torch

    from speculative_decoding_verification_amd.chain import StackShape
    sv = env
    shape = StackShape(**SMALL)
    st, _ = _stack(env, shape, 101)
    M = 5
    x = synth.activations(M, shape.hidden, 101, "x")
    _set_x(st, x)
    st.run(M)
    torch.cuda.synchronize()
    eager = st.logits[:M].cpu().numpy().copy()
    eager_am = st.argmax[:M].cpu().numpy().copy()
    eager_q = st.a_final.q[:M].cpu().numpy().copy()
    p = st.make_pass(M)
    st.logits.zero_()
    st.run_pass(M, p)
    torch.cuda.synchronize()
    assert p.status() == 0
    assert np.array_equal(st.logits[:M].cpu().numpy().view(np.uint32), eager.view(np.uint32))
    assert np.array_equal(st.argmax[:M].cpu().numpy(), eager_am)
    assert np.array_equal(st.a_final.q[:M].cpu().numpy(), eager_q)
    g = st.capture(M)
    for _ in range(3):
        st.logits.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(st.logits[:M].cpu().numpy().view(np.uint32), eager.view(np.uint32))
        st.run(M)               # eager work between replays
        torch.cuda.synchronize()


@pytest.mark.parametrize("shape_kw", [SMALL, dict(hidden=1024, ffn=2048, layers=2, vocab=3000)])
def test_stack_batch_invariance(env, shape_kw):
    import torch

    from speculative_decoding_verification_amd.chain import StackShape
    shape = StackShape(**shape_kw)
    st, _ = _stack(env, shape, 102)
    x = synth.activations(8, shape.hidden, 102, "x")
    res = {}
    for M in (8, 5, 1):
        p = st.make_pass(M)
        _set_x(st, x[:M])
        st.run_pass(M, p)
        torch.cuda.synchronize()
        res[M] = st.logits[:M].cpu().numpy().copy()
    for m in range(8):
        p = st.make_pass(1)
        _set_x(st, x[m:m + 1])
        st.run_pass(1, p)
        torch.cuda.synchronize()
        alone = st.logits[0].cpu().numpy()
        for M, lg in res.items():
            if m < M:
                assert np.array_equal(lg[m].view(np.uint32), alone.view(np.uint32)), (M, m)


C2 = dict(hidden=2560, ffn=9728, layers=36, vocab=151936)


@pytest.mark.parametrize("shape_kw,M,bound", [(SMALL, 5, 1e-3), (C2, 5, None)])
def test_chain_against_oracle(env, orc, shape_kw, M, bound):
    """Free-running pass vs the oracle's chain.  Wherever a value to be
    requantised lies within rounding of a half-way point, the int8 code the
    GPU takes (fp32 arithmetic in its own fixed order) and the oracle's
    (fp32 rounding of fp64 values) can differ by one, and the difference
    propagates down the chain; per-phase parity on identical inputs is
    pinned by test_chain_oracle_forced_phases.  Here the drift is reported,
    its mean over all logits is bounded on the short chain, and the argmax
    must agree wherever the top-2 gap exceeds twice the largest drift."""
    import torch

    from speculative_decoding_verification_amd.chain import StackShape
    shape = StackShape(**shape_kw)
    seed = 103
    st, keep = _stack(env, shape, seed)
    x = synth.activations(M, shape.hidden, seed, "x")
    _set_x(st, x)
    p = st.make_pass(M)
    st.run_pass(M, p)
    torch.cuda.synchronize()
    lg = st.logits[:M].cpu().numpy().astype(np.float64)
    am = np.array([env.argmax_index(int(v)) for v in st.argmax[:M].cpu().numpy().view(np.uint64)])
    xo, lo = _oracle_chain(orc, keep, shape, seed, x)
    scale = np.abs(lo).max(axis=1, keepdims=True)
    rel = np.abs(lg - lo) / scale
    print(f"free-running logit drift: max {rel.max():.3e}, mean {rel.mean():.3e} (relative to max |logit|)")
    if bound is not None:
        assert rel.mean() < bound
    top = lo.argmax(1)
    s = np.sort(lo, 1)
    clear = (s[:, -1] - s[:, -2]) > 2 * rel.max() * scale[:, 0]
    assert np.array_equal(am[clear], top[clear])
    assert np.array_equal(am, lg.argmax(1))


def test_chain_oracle_forced_phases(env, orc):
    """Each phase of the 4B-class layer (real shapes, first two layers) run
    through the C ABI on the oracle's own quantised input: outputs within
    1e-5 of T, the requantised codes equal to the oracle's except at
    half-way ties."""
    import torch
    sv = env
    H, F, M, seed = 2560, 9728, 5, 104
    eps = 1e-6
    x = synth.activations(M, H, seed, "x").astype(np.float64)

    def gpu_phase(qt, raws, q, d, s16, ss, K, gamma, mode):
        A = [torch.from_numpy(np.ascontiguousarray(a)).cuda() for a in (q, d, s16)]
        parts = torch.from_numpy(np.asarray(ss, np.float32).reshape(M, 1)).cuda()
        ups = []
        for raw in raws:
            n = sv.repacked_bytes(qt, raw.shape[0], K)
            src = torch.from_numpy(raw.reshape(-1)).cuda()
            dst = torch.empty(n, dtype=torch.uint8, device="cuda")
            sv.repack_weights(qt, src, dst, raw.shape[0], K)
            ups.append((sv.weight(qt, raw.shape[0], K, dst), dst))
        N = raws[0].shape[0]
        ys = [torch.empty((M, N), dtype=torch.float32, device="cuda") for _ in raws]
        oq = torch.empty((M, N), dtype=torch.int8, device="cuda")
        od = torch.empty((M, N // 32), dtype=torch.float32, device="cuda")
        o16 = torch.empty((M, N // 16), dtype=torch.int32, device="cuda")
        oss = torch.empty((M, N // 32), dtype=torch.float32, device="cuda")
        ep = sv.epilogue(mode, oq, od, o16, oss, gamma=torch.from_numpy(gamma).cuda(), src=len(raws) - 1)
        sv.verify_matvec([u[0] for u in ups], sv.act(M, K, A[0], A[1], A[2], parts, 1, eps), ys, ep)
        torch.cuda.synchronize()
        return [y.cpu().numpy() for y in ys], oq.cpu().numpy()

    def check(y_gpu, y64, T):
        assert np.all(np.abs(y_gpu.astype(np.float64) - y64) <= 1e-5 * T)

    def codes_close(q_gpu, v64, gamma):
        q_or, _, _, _ = orc.quantize_act(v64.astype(np.float32), gamma)
        diff = q_gpu.astype(np.int32) - q_or.astype(np.int32)
        assert np.abs(diff).max(initial=0) <= 1 and np.count_nonzero(diff) <= 4e-3 * diff.size

    for layer in range(2):
        g = {k: synth.rms_weight(n, seed, layer, k) for k, n in (("g1", H), ("g2", H), ("g3", H), ("g4", F))}
        W = {n: synth.gguf_weights(qt, r, c, seed, layer, n) for n, qt, r, c in
             [("q", 12, H, H), ("k", 12, H, H), ("v", 12, H, H), ("o", 12, H, H), ("gate", 12, F, H),
              ("up", 12, F, H), ("down", 14, H, F)]}
        q, d, s16, ss = orc.quantize_act(x.astype(np.float32), g["g1"])
        r = orc.rms_factor(ss, H, eps)
        (yq, yk, yv), qv = gpu_phase(12, [W["q"], W["k"], W["v"]], q, d, s16, ss, H, g["g2"], sv.SV_EP_QUANT)
        for name, yg in (("q", yq), ("k", yk), ("v", yv)):
            y64, T = orc.matvec(12, W[name], H, q, d, scale=r)
            check(yg, y64, T)
        v64, _ = orc.matvec(12, W["v"], H, q, d, scale=r)
        codes_close(qv, v64, g["g2"])
        q, d, s16, ss = orc.quantize_act(v64.astype(np.float32), g["g2"])
        r = orc.rms_factor(ss, H, eps)
        (yo,), qo = gpu_phase(12, [W["o"]], q, d, s16, ss, H, g["g3"], sv.SV_EP_QUANT)
        o64, T = orc.matvec(12, W["o"], H, q, d, scale=r)
        check(yo, o64, T)
        codes_close(qo, o64, g["g3"])
        q, d, s16, ss = orc.quantize_act(o64.astype(np.float32), g["g3"])
        r = orc.rms_factor(ss, H, eps)
        (yg_, yu_), qh = gpu_phase(12, [W["gate"], W["up"]], q, d, s16, ss, H, g["g4"], sv.SV_EP_PAIR)
        gg, Tg = orc.matvec(12, W["gate"], H, q, d, scale=r)
        uu, Tu = orc.matvec(12, W["up"], H, q, d, scale=r)
        check(yg_, gg, Tg)
        check(yu_, uu, Tu)
        p64 = (gg.astype(np.float32) * uu.astype(np.float32)).astype(np.float64)
        codes_close(qh, p64, g["g4"])
        q, d, s16, ss = orc.quantize_act(p64.astype(np.float32), g["g4"])
        r = orc.rms_factor(ss, F, eps)
        nxt = synth.rms_weight(H, seed, layer + 1, "g1")
        (yd,), _ = gpu_phase(14, [W["down"]], q, d, s16, ss, F, nxt, sv.SV_EP_QUANT)
        x, T = orc.matvec(14, W["down"], F, q, d, scale=r)
        check(yd, x, T)
