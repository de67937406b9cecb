"""Python binding of libspecverify (the C ABI in include/specverify.h).

Argument marshalling only: every step of the verification pass runs in the
HIP kernels of the shared library.  Tensors are torch tensors on the GPU
(torch provides device memory and streams); each function passes their
data pointers and the current HIP stream to the C call of the same name and
raises SpecVerifyError on a non-zero status.  If the shared library is not
built, importing the functions fails loudly; nothing falls back to the CPU.
"""

from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libspecverify.so")

SV_OK, SV_ERR_ARG, SV_ERR_SHAPE, SV_ERR_ALIGN, SV_ERR_QTYPE, SV_ERR_WORKSPACE, SV_ERR_HIP = 0, -1, -2, -3, -4, -5, -6
SV_Q8_0, SV_Q4_K, SV_Q6_K = 8, 12, 14
SV_EP_NONE, SV_EP_QUANT, SV_EP_PAIR = 0, 1, 2
MAX_M = 16

EXPORTS = [
    "sv_last_error", "sv_version", "sv_repacked_bytes", "sv_repack_weights", "sv_unpack_weights",
    "sv_quantize_act_q8", "sv_verify_matvec", "sv_head_logits", "sv_argmax_index",
    "sv_accept_greedy", "sv_accept_workspace_bytes", "sv_accept_rejection",
]


class SpecVerifyError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"specverify error {code}: {msg}")
        self.code = code


class Weight(ctypes.Structure):
    _fields_ = [("qtype", ctypes.c_int32), ("rows", ctypes.c_int64), ("cols", ctypes.c_int64),
                ("data", ctypes.c_void_p)]


class Act(ctypes.Structure):
    _fields_ = [("M", ctypes.c_int32), ("K", ctypes.c_int64), ("q", ctypes.c_void_p), ("d", ctypes.c_void_p),
                ("s16", ctypes.c_void_p), ("sumsq_parts", ctypes.c_void_p), ("n_parts", ctypes.c_int32),
                ("eps", ctypes.c_float)]


class Epilogue(ctypes.Structure):
    _fields_ = [("mode", ctypes.c_int32), ("src", ctypes.c_int32), ("gamma", ctypes.c_void_p),
                ("q", ctypes.c_void_p), ("d", ctypes.c_void_p), ("s16", ctypes.c_void_p),
                ("sumsq", ctypes.c_void_p)]


_lib = None


def lib():
    """The loaded shared library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                              "(the verification pass has no CPU fallback)")
        L = ctypes.CDLL(LIB_PATH)
        P, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
        L.sv_last_error.restype = ctypes.c_char_p
        L.sv_version.restype = ctypes.c_char_p
        L.sv_repacked_bytes.restype = ctypes.c_size_t
        L.sv_repacked_bytes.argtypes = [i32, i64, i64]
        L.sv_repack_weights.argtypes = [i32, P, P, i64, i64, P]
        L.sv_unpack_weights.argtypes = [i32, P, P, i64, i64, P]
        L.sv_quantize_act_q8.argtypes = [P, i32, i64, P, P, P, P, P, P]
        L.sv_verify_matvec.argtypes = [ctypes.POINTER(Weight), i32, ctypes.POINTER(Act),
                                       ctypes.POINTER(ctypes.c_void_p), ctypes.POINTER(Epilogue), P]
        L.sv_head_logits.argtypes = [ctypes.POINTER(Weight), ctypes.POINTER(Act), P, i64, P, P, P]
        L.sv_argmax_index.restype = i64
        L.sv_argmax_index.argtypes = [ctypes.c_uint64]
        L.sv_accept_greedy.argtypes = [P, P, P, i32, P, P]
        L.sv_accept_workspace_bytes.restype = ctypes.c_size_t
        L.sv_accept_workspace_bytes.argtypes = [i64, i32]
        L.sv_accept_rejection.argtypes = [P, i64, P, P, i32, P, ctypes.c_float, P, ctypes.c_size_t, P, P]
        for f in ("sv_repack_weights", "sv_unpack_weights", "sv_quantize_act_q8", "sv_verify_matvec",
                  "sv_head_logits", "sv_accept_greedy", "sv_accept_rejection"):
            getattr(L, f).restype = ctypes.c_int
        _lib = L
    return _lib


def _check(rc):
    if rc != SV_OK:
        raise SpecVerifyError(rc, lib().sv_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    if stream is not None:
        return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def version() -> str:
    return lib().sv_version().decode()


def repacked_bytes(qtype: int, rows: int, cols: int) -> int:
    return int(lib().sv_repacked_bytes(qtype, rows, cols))


def repack_weights(qtype, gguf, dst, rows, cols, stream=None):
    _check(lib().sv_repack_weights(qtype, _ptr(gguf), _ptr(dst), rows, cols, _stream(stream)))


def unpack_weights(qtype, repacked, dst, rows, cols, stream=None):
    _check(lib().sv_unpack_weights(qtype, _ptr(repacked), _ptr(dst), rows, cols, _stream(stream)))


def quantize_act_q8(x, q, d, s16, gamma=None, sumsq=None, stream=None):
    M, K = x.shape
    _check(lib().sv_quantize_act_q8(_ptr(x), M, K, _ptr(gamma), _ptr(q), _ptr(d), _ptr(s16), _ptr(sumsq),
                                    _stream(stream)))


def weight(qtype, rows, cols, data) -> Weight:
    return Weight(qtype, rows, cols, data.data_ptr())


def act(M, K, q, d, s16, sumsq_parts=None, n_parts=0, eps=1e-6) -> Act:
    return Act(M, K, q.data_ptr(), d.data_ptr(), s16.data_ptr(),
               None if sumsq_parts is None else sumsq_parts.data_ptr(), int(n_parts), float(eps))


def epilogue(mode, q, d, s16, sumsq, gamma=None, src=0) -> Epilogue:
    return Epilogue(mode, src, None if gamma is None else gamma.data_ptr(), q.data_ptr(), d.data_ptr(),
                    s16.data_ptr(), sumsq.data_ptr())


def verify_matvec(weights, A: Act, ys, ep: Epilogue | None = None, stream=None):
    n = len(weights)
    W = (Weight * n)(*weights)
    Y = (ctypes.c_void_p * n)(*[None if y is None else y.data_ptr() for y in ys])
    _check(lib().sv_verify_matvec(W, n, ctypes.byref(A), Y, None if ep is None else ctypes.byref(ep),
                                  _stream(stream)))


def head_logits(H: Weight, A: Act, logits=None, argmax=None, row_ids=None, n_rows=None, stream=None):
    n = H.rows if row_ids is None else (n_rows if n_rows is not None else row_ids.numel())
    _check(lib().sv_head_logits(ctypes.byref(H), ctypes.byref(A), _ptr(row_ids), n, _ptr(logits), _ptr(argmax),
                                _stream(stream)))


def argmax_index(packed: int) -> int:
    return int(lib().sv_argmax_index(ctypes.c_uint64(int(packed) & 0xFFFFFFFFFFFFFFFF)))


def accept_greedy(argmax, drafts, out, row_ids=None, stream=None):
    K = 0 if drafts is None else drafts.numel()
    _check(lib().sv_accept_greedy(_ptr(argmax), _ptr(row_ids), _ptr(drafts), K, _ptr(out), _stream(stream)))


def accept_workspace_bytes(V: int, K: int) -> int:
    return int(lib().sv_accept_workspace_bytes(V, K))


def accept_rejection(logits, drafts, u, out, workspace, temperature=1.0, q=None, stream=None):
    V = logits.shape[-1]
    K = 0 if drafts is None else drafts.numel()
    _check(lib().sv_accept_rejection(_ptr(logits), V, _ptr(q), _ptr(drafts), K, _ptr(u), float(temperature),
                                     _ptr(workspace), workspace.numel() * workspace.element_size(), _ptr(out),
                                     _stream(stream)))
