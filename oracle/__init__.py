"""CPU oracle for the verification pass: Python face of ``oracle.c``.

TEST INFRASTRUCTURE ONLY: tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py may import this package; the product path
(``speculative_decoding_verification_amd``) never does, and the two share no
code.  See the header of oracle.c for what each function computes and which
page passage it follows; ``chain_pass`` documents the reading of the layer
chain.
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

Q8_0, Q4_K, Q6_K = 8, 12, 14
BLOCK = {Q8_0: (32, 34), Q4_K: (256, 144), Q6_K: (256, 210)}


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc (plain -O2, no FMA contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + f".tmp{os.getpid()}"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
                               "-fPIC", "-shared", "-pthread", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i32, i64, f64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_double
        L.or_half.restype = f64
        L.or_half.argtypes = [ctypes.c_uint16]
        L.or_decode_q8_0.argtypes = [P, i64, P, P]
        L.or_decode_q4_k.argtypes = [P, i64, P, P, P, P, P]
        L.or_decode_q6_k.argtypes = [P, i64, P, P, P]
        L.or_quantize_act.argtypes = [P, P, i32, i64, P, P, P, P]
        L.or_matvec.restype = ctypes.c_int
        L.or_matvec.argtypes = [ctypes.c_int, P, i64, i64, P, P, P, i32, P, P, P, P, i32]
        L.or_rms_factor.restype = f64
        L.or_rms_factor.argtypes = [f64, i64, f64]
        L.or_argmax.argtypes = [P, i32, i64, P]
        L.or_accept_greedy.argtypes = [P, P, i32, P]
        L.or_accept_rejection.restype = ctypes.c_int
        L.or_accept_rejection.argtypes = [P, i64, P, P, i32, P, f64, P, P]
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def default_threads() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


# ---------------------------------------------------------------- decode
def half(bits: int) -> float:
    return lib().or_half(int(bits) & 0xFFFF)


def decode_q8_0(row: np.ndarray, K: int):
    row = _c(row, np.uint8)
    q = np.empty(K, np.int32)
    d = np.empty(K // 32, np.float64)
    lib().or_decode_q8_0(_p(row), K, _p(q), _p(d))
    return q, d


def decode_q4_k(row: np.ndarray, K: int):
    row = _c(row, np.uint8)
    q = np.empty(K, np.int32)
    d = np.empty(K // 256, np.float64)
    dmin = np.empty(K // 256, np.float64)
    sc = np.empty(K // 32, np.int32)
    m = np.empty(K // 32, np.int32)
    lib().or_decode_q4_k(_p(row), K, _p(q), _p(d), _p(dmin), _p(sc), _p(m))
    return q, d, dmin, sc, m


def decode_q6_k(row: np.ndarray, K: int):
    row = _c(row, np.uint8)
    q = np.empty(K, np.int32)
    d = np.empty(K // 256, np.float64)
    sc = np.empty(K // 16, np.int32)
    lib().or_decode_q6_k(_p(row), K, _p(q), _p(d), _p(sc))
    return q, d, sc


# ---------------------------------------------------------------- quantiser
def quantize_act(x: np.ndarray, gamma: np.ndarray | None = None):
    """Q8A32 of x (times gamma).  Returns q int8 [M,K], d fp32 [M,K/32],
    s16 int32 [M,K/16], sumsq fp64 [M] (sum of x^2 before gamma)."""
    x = _c(np.atleast_2d(x), np.float32)
    M, K = x.shape
    if K % 32:
        raise ValueError("K must be a multiple of 32")
    g = None if gamma is None else _c(gamma, np.float32)
    q = np.empty((M, K), np.int8)
    d = np.empty((M, K // 32), np.float32)
    s16 = np.empty((M, K // 16), np.int32)
    ss = np.empty(M, np.float64)
    lib().or_quantize_act(_p(x), _p(g), M, K, _p(q), _p(d), _p(s16), _p(ss))
    return q, d, s16, ss


def rms_factor(sumsq, n: int, eps: float = 1e-6):
    return np.array([lib().or_rms_factor(float(s), n, eps) for s in np.atleast_1d(sumsq)])


# ---------------------------------------------------------------- projection
def matvec(qtype: int, W: np.ndarray, K: int, q: np.ndarray, d: np.ndarray,
           scale=None, row_ids=None, block_sums: bool = False, threads: int | None = None):
    """fp64 Y[M, N] = scale[m] * W_deq . A_deq for GGUF rows W[N, row_bytes].

    Returns (y, T) or (y, T, bsum) with T = scale * sum|block term| and bsum
    the exact integer block sums [M, N, K/32]."""
    W = _c(W, np.uint8)
    q = _c(np.atleast_2d(q), np.int8)
    d = _c(np.atleast_2d(d), np.float32)
    M = q.shape[0]
    ids = None if row_ids is None else _c(row_ids, np.int32)
    N = W.shape[0] if ids is None else ids.size
    sc = None if scale is None else _c(np.broadcast_to(np.asarray(scale, np.float64), (M,)), np.float64)
    y = np.empty((M, N), np.float64)
    T = np.empty((M, N), np.float64)
    bs = np.empty((M, N, K // 32), np.int64) if block_sums else None
    rc = lib().or_matvec(qtype, _p(W), N, K, _p(ids), _p(q), _p(d), M, _p(sc), _p(y), _p(T),
                         _p(bs), threads or default_threads())
    if rc:
        raise ValueError(f"or_matvec failed ({rc})")
    return (y, T, bs) if block_sums else (y, T)


# ---------------------------------------------------------------- acceptance
def argmax(logits: np.ndarray) -> np.ndarray:
    z = _c(np.atleast_2d(logits), np.float64)
    out = np.empty(z.shape[0], np.int64)
    lib().or_argmax(_p(z), z.shape[0], z.shape[1], _p(out))
    return out


def accept_greedy(top, drafts) -> np.ndarray:
    top = _c(top, np.int64)
    drafts = _c(drafts, np.int32)
    K = drafts.size
    if top.size != K + 1:
        raise ValueError("need K+1 top tokens")
    out = np.zeros(K + 2, np.int32)
    lib().or_accept_greedy(_p(top), _p(drafts), K, _p(out))
    return out


def accept_rejection(logits, drafts, u, temperature: float = 1.0, q=None, with_margin=False):
    """Rejection acceptance; q=None selects the certain-drafter rule."""
    z = _c(np.atleast_2d(logits), np.float32)
    drafts = _c(drafts, np.int32)
    K = drafts.size
    V = z.shape[1]
    if z.shape[0] != K + 1:
        raise ValueError("need K+1 logit rows")
    uu = _c(u, np.float64).reshape(K + 1, 2)
    qq = None if q is None else _c(q, np.float32).reshape(K, V)
    out = np.zeros(K + 2, np.int32)
    mg = np.full(K + 1, np.inf)
    rc = lib().or_accept_rejection(_p(z), V, _p(qq), _p(drafts), K, _p(uu), float(temperature),
                                   _p(out), _p(mg))
    if rc:
        raise ValueError("temperature must be > 0")
    return (out, mg) if with_margin else out


# ---------------------------------------------------------------- layer chain
def chain_pass(layers, x0, hidden: int, ffn: int, head=None, eps: float = 1e-6, threads=None):
    """Plain reading of the verification pass over a projection stack.

    layers: list of dicts with 'q','k','v','o','gate','up','down' ->
    (qtype, GGUF bytes) and 'g1'..'g4' -> fp32 norm weights; head: None or
    (qtype, GGUF bytes, gamma_final).  Per layer (the producer requantises
    the next input including the next norm's weight; the RMS factor r of the
    normalised vector multiplies the consumer's output):
        a = Q8A32(x*g1);  q,k,v = r(x) W a;  b = Q8A32(v*g2);  o = r(v) Wo b;
        c = Q8A32(o*g3);  g,u = r(o) W c;    h = Q8A32((g*u)*g4);
        x = r(g*u) Wd h
    Projections are fp64; every quantiser input is the fp32 rounding of the
    fp64 value (the codes are fp32 decisions).  Returns (x_last fp64 [M,H],
    logits fp64 [M,V] or None)."""
    H, F = hidden, ffn

    def fold(v64, gamma, n):
        v32 = np.asarray(v64, np.float64).astype(np.float32)
        q, d, _, ss = quantize_act(v32, gamma)
        return q, d, rms_factor(ss, n, eps)

    x = np.asarray(x0, np.float64)
    for lw in layers:
        q, d, r = fold(x, lw["g1"], H)
        mv = lambda name, q=q, d=d, r=r, K=H: matvec(lw[name][0], lw[name][1], K, q, d, scale=r,
                                                     threads=threads)[0]
        mv("q")
        mv("k")
        v = mv("v")
        q, d, r = fold(v, lw["g2"], H)
        o = matvec(lw["o"][0], lw["o"][1], H, q, d, scale=r, threads=threads)[0]
        q, d, r = fold(o, lw["g3"], H)
        g = matvec(lw["gate"][0], lw["gate"][1], H, q, d, scale=r, threads=threads)[0]
        u = matvec(lw["up"][0], lw["up"][1], H, q, d, scale=r, threads=threads)[0]
        p = (g.astype(np.float32) * u.astype(np.float32)).astype(np.float64)
        q, d, r = fold(p, lw["g4"], F)
        x = matvec(lw["down"][0], lw["down"][1], F, q, d, scale=r, threads=threads)[0]
    logits = None
    if head is not None:
        hq, hraw, gf = head
        q, d, r = fold(x, gf, H)
        logits = matvec(hq, hraw, H, q, d, scale=r, threads=threads)[0]
    return x, logits
