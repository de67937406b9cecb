"""Helpers for the GPU tests: device buffers and uploads (torch is only the
memory provider; every computation goes through the C ABI)."""

from __future__ import annotations

import numpy as np

import speculative_decoding_verification_amd as sv


def torch():
    import torch as _t
    return _t


def dev(a, dtype=None):
    t = torch()
    x = t.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        x = x.to(dtype)
    return x.cuda()


def host(t):
    torch().cuda.synchronize()
    return t.detach().cpu().numpy()


def empty(shape, dtype):
    t = torch()
    return t.empty(shape, dtype=dtype, device="cuda")


def zeros(shape, dtype):
    t = torch()
    return t.zeros(shape, dtype=dtype, device="cuda")


class ActBuf:
    """Device buffers of one int8 activation [M][K]."""

    def __init__(self, M, K):
        t = torch()
        self.M, self.K = M, K
        self.q = empty((M, K), t.int8)
        self.d = empty((M, K // 32), t.float32)
        self.s16 = empty((M, K // 16), t.int32)
        self.sumsq = empty((M, K // 32), t.float32)

    def act(self, parts=None, n_parts=0, eps=1e-6):
        return sv.act(self.M, self.K, self.q, self.d, self.s16, parts, n_parts, eps)

    @classmethod
    def from_host(cls, q, d, s16):
        M, K = q.shape
        b = cls(M, K)
        t = torch()
        b.q.copy_(t.from_numpy(np.ascontiguousarray(q)))
        b.d.copy_(t.from_numpy(np.ascontiguousarray(d)))
        b.s16.copy_(t.from_numpy(np.ascontiguousarray(s16)))
        return b


def quantize(x, gamma=None):
    """GPU quantiser on host fp32 x; returns an ActBuf."""
    t = torch()
    M, K = x.shape
    b = ActBuf(M, K)
    xd = dev(x.astype(np.float32))
    g = None if gamma is None else dev(gamma.astype(np.float32))
    sv.quantize_act_q8(xd, b.q, b.d, b.s16, gamma=g, sumsq=b.sumsq)
    return b


def upload_weight(qtype, gguf_rows: np.ndarray, K: int):
    """Copy GGUF bytes [N, row_bytes] to the GPU and repack; returns
    (sv.Weight, device buffer keeping it alive)."""
    t = torch()
    N = gguf_rows.shape[0]
    src = dev(gguf_rows.reshape(-1))
    nbytes = sv.repacked_bytes(qtype, N, K)
    assert gguf_rows.size == sv.gguf_bytes(qtype, N, K)
    dst = t.empty(nbytes + 256, dtype=t.uint8, device="cuda")
    off = (-dst.data_ptr()) % 256
    dst = dst[off:off + nbytes]
    sv.repack_weights(qtype, src, dst, N, K)
    t.cuda.synchronize()
    del src
    return sv.weight(qtype, N, K, dst), dst
