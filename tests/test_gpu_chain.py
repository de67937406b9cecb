"""GPU tests of the whole verification pass over a projection stack.

* The persistent one-launch pass equals the eager phase-by-phase calls bit
  for bit (same units, same order of every fp32 operation).
* Graph replays of the pass, with eager work in between, repeat the same bits.
* Whole-stack batch invariance: the logits of row m of an M-row pass are
  bit-identical to a 1-row pass of that row alone.
(The pass against the oracle, phase by phase at the real layer shapes, is
in test_gpu_pass_shapes.py.)
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
