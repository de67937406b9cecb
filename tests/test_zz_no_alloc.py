"""The allocation-free rejection round (sv_accept_rejection_noalloc, static
scratch) against sv_accept_rejection with a workspace, through the C ABI:
the same outputs bit for bit, on consecutive calls, the second one smaller
(fewer tokens and drafts) so that it runs on the scratch the first one
left behind."""

import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gpu_util
    import speculative_decoding_verification_amd as sv
    sv.lib()
    return gpu_util


def _round(gu, V, K, T, general, seed):
    z = synth.normals((K + 1, V), seed, "z", sigma=2.0)
    drafts = synth.token_ids(K, V, seed, "d")
    u = synth.uniforms((K + 1, 2), seed, "u")
    q = None
    if general:
        zq = z[:K].astype(np.float64) + synth.normals((K, V), seed, "q", sigma=0.5, dtype=np.float64)
        e = np.exp(zq - zq.max(1, keepdims=True))
        q = (e / e.sum(1, keepdims=True)).astype(np.float32)
    return z, drafts, u, q


@pytest.mark.parametrize("general", [True, False])
def test_noalloc_matches_workspace_call(gu, general):
    import speculative_decoding_verification_amd as sv
    import torch
    for i, (V, K, T) in enumerate([(151936, 15, 1.0), (151936, 4, 0.8), (50000, 2, 1.3), (997, 0, 1.0)]):
        z, drafts, u, q = _round(gu, V, K, T, general, 40 + i)
        zd, ud = gu.dev(z), gu.dev(u)
        dd = gu.dev(drafts) if K else None
        qd = gu.dev(q if K else np.zeros((1, V), np.float32)) if general else None
        ws = gu.empty((sv.accept_workspace_bytes(V, K),), torch.uint8)
        ref = gu.zeros((K + 2,), torch.int32)
        sv.accept_rejection(zd, dd, ud, ref, ws, temperature=T, q=qd)
        got = gu.zeros((K + 2,), torch.int32)
        sv.accept_rejection_noalloc(zd, dd, ud, got, temperature=T, q=qd)
        r, g = gu.host(ref), gu.host(got)
        assert np.array_equal(r, g), (V, K, r, g)
        assert 0 <= r[0] <= K
