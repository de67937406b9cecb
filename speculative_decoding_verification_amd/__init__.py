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
    "sv_quantize_act_q8", "sv_matvec_workspace_bytes", "sv_verify_matvec", "sv_head_workspace_bytes",
    "sv_head_logits", "sv_argmax_index", "sv_pass_workspace_bytes", "sv_pass_schedule", "sv_pass_create",
    "sv_pass_run", "sv_pass_status", "sv_pass_trace", "sv_pass_destroy", "sv_accept_greedy",
    "sv_accept_workspace_bytes", "sv_accept_rejection", "sv_accept_noalloc_max_bytes",
    "sv_accept_rejection_noalloc", "sv_read_bandwidth",
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


class Phase(ctypes.Structure):
    _fields_ = [("W", ctypes.POINTER(Weight)), ("n_w", ctypes.c_int32), ("A", Act),
                ("y", ctypes.c_void_p * 3), ("ep", Epilogue), ("row_ids", ctypes.c_void_p),
                ("n_rows", ctypes.c_int64), ("argmax", ctypes.c_void_p)]


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
        L.sv_matvec_workspace_bytes.restype = ctypes.c_size_t
        L.sv_matvec_workspace_bytes.argtypes = [ctypes.POINTER(Weight), i32, ctypes.POINTER(Act)]
        L.sv_verify_matvec.argtypes = [ctypes.POINTER(Weight), i32, ctypes.POINTER(Act),
                                       ctypes.POINTER(ctypes.c_void_p), ctypes.POINTER(Epilogue), P,
                                       ctypes.c_size_t, P]
        L.sv_head_workspace_bytes.restype = ctypes.c_size_t
        L.sv_head_workspace_bytes.argtypes = [ctypes.POINTER(Weight), ctypes.POINTER(Act), i64]
        L.sv_head_logits.argtypes = [ctypes.POINTER(Weight), ctypes.POINTER(Act), P, i64, P, P, P,
                                     ctypes.c_size_t, P]
        L.sv_pass_workspace_bytes.restype = ctypes.c_size_t
        L.sv_pass_workspace_bytes.argtypes = [ctypes.POINTER(Phase), i32]
        L.sv_pass_schedule.restype = ctypes.c_size_t
        L.sv_pass_schedule.argtypes = [ctypes.POINTER(Phase), i32, i32, ctypes.c_void_p, ctypes.c_size_t]
        L.sv_pass_create.argtypes = [ctypes.POINTER(Phase), i32, P, ctypes.c_size_t, ctypes.POINTER(P)]
        L.sv_pass_run.argtypes = [P, P]
        L.sv_pass_status.argtypes = [P, ctypes.POINTER(ctypes.c_uint32)]
        L.sv_pass_trace.restype = ctypes.c_int
        L.sv_pass_trace.argtypes = [P, ctypes.c_int, P, ctypes.c_size_t, ctypes.POINTER(ctypes.c_int32)]
        L.sv_pass_destroy.restype = None
        L.sv_pass_destroy.argtypes = [P]
        L.sv_argmax_index.restype = i64
        L.sv_argmax_index.argtypes = [ctypes.c_uint64]
        L.sv_accept_greedy.argtypes = [P, P, i64, P, i32, P, P]
        L.sv_accept_workspace_bytes.restype = ctypes.c_size_t
        L.sv_accept_workspace_bytes.argtypes = [i64, i32]
        L.sv_accept_rejection.argtypes = [P, i64, P, P, i32, P, ctypes.c_float, P, ctypes.c_size_t, P, P]
        L.sv_accept_noalloc_max_bytes.restype = ctypes.c_size_t
        L.sv_accept_noalloc_max_bytes.argtypes = []
        L.sv_accept_rejection_noalloc.argtypes = [P, i64, P, P, i32, P, ctypes.c_float, P, P]
        L.sv_read_bandwidth.argtypes = [P, ctypes.c_size_t, P, i32, P]
        for f in ("sv_repack_weights", "sv_unpack_weights", "sv_quantize_act_q8", "sv_verify_matvec",
                  "sv_head_logits", "sv_accept_greedy", "sv_accept_rejection", "sv_accept_rejection_noalloc",
                  "sv_pass_create",
                  "sv_pass_run", "sv_pass_status", "sv_read_bandwidth"):
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


_GGUF_BLOCK = {8: (32, 34), 12: (256, 144), 14: (256, 210)}   # elements, bytes per GGUF block


def gguf_bytes(qtype: int, rows: int, cols: int) -> int:
    """Bytes of a rows x cols matrix in its canonical GGUF blocks (the
    weight bytes a projection has to read)."""
    n, b = _GGUF_BLOCK[qtype]
    return rows * (cols // n) * b


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


_ws = {}


def workspace(nbytes: int):
    """A zero-filled, 256-byte aligned device scratch buffer of at least
    nbytes, shared by the single-phase calls of this process (the library
    leaves it zero-filled after every call)."""
    import torch
    dev = torch.cuda.current_device()
    buf = _ws.get(dev)
    if nbytes == 0:
        return None
    if buf is None or buf.numel() < nbytes + 256:
        buf = torch.zeros(max(nbytes, 1 << 20) + 256, dtype=torch.uint8, device="cuda")
        _ws[dev] = buf
    off = (-buf.data_ptr()) % 256
    return buf[off:off + nbytes]


def _ws_args(nbytes, ws):
    if nbytes == 0:
        return None, 0
    if ws is None:
        ws = workspace(nbytes)
    return ctypes.c_void_p(ws.data_ptr()), ws.numel() * ws.element_size()


def verify_matvec(weights, A: Act, ys, ep: Epilogue | None = None, workspace_buf=None, stream=None):
    n = len(weights)
    W = (Weight * n)(*weights)
    Y = (ctypes.c_void_p * n)(*[None if y is None else y.data_ptr() for y in ys])
    need = lib().sv_matvec_workspace_bytes(W, n, ctypes.byref(A))
    wp, wn = _ws_args(need, workspace_buf)
    _check(lib().sv_verify_matvec(W, n, ctypes.byref(A), Y, None if ep is None else ctypes.byref(ep), wp, wn,
                                  _stream(stream)))


def head_logits(H: Weight, A: Act, logits=None, argmax=None, row_ids=None, n_rows=None, workspace_buf=None,
                stream=None):
    n = H.rows if row_ids is None else (n_rows if n_rows is not None else row_ids.numel())
    need = lib().sv_head_workspace_bytes(ctypes.byref(H), ctypes.byref(A), 0 if row_ids is None else n)
    wp, wn = _ws_args(need, workspace_buf)
    _check(lib().sv_head_logits(ctypes.byref(H), ctypes.byref(A), _ptr(row_ids), n, _ptr(logits), _ptr(argmax),
                                wp, wn, _stream(stream)))


def phase(weights, A: Act, ys=(), ep: Epilogue | None = None, row_ids=None, n_rows=0, argmax=None) -> Phase:
    """Descriptor of one phase of a whole-pass launch (see Pass)."""
    n = len(weights)
    ph = Phase()
    arr = (Weight * n)(*weights)
    ph._keep = arr
    ph.W = ctypes.cast(arr, ctypes.POINTER(Weight))
    ph.n_w = n
    ph.A = A
    for i, y in enumerate(list(ys)[:3]):
        ph.y[i] = None if y is None else y.data_ptr()
    if ep is not None:
        ph.ep = ep
    ph.row_ids = None if row_ids is None else row_ids.data_ptr()
    ph.n_rows = int(n_rows if row_ids is not None else 0)
    ph.argmax = None if argmax is None else argmax.data_ptr()
    return ph


def pass_schedule(phases, grid: int):
    """The unit lists a pass over `phases` runs with `grid` workgroups (host
    only): (offsets [grid + 1], entries) as uint32 arrays, each entry
    (phase << 20) | unit."""
    import numpy as np
    n = len(phases)
    arr = (Phase * n)(*phases)
    need = lib().sv_pass_schedule(arr, n, int(grid), None, 0)
    if need == 0:
        raise SpecVerifyError(SV_ERR_ARG, lib().sv_last_error().decode())
    out = np.zeros(need, np.uint32)
    got = lib().sv_pass_schedule(arr, n, int(grid), out.ctypes.data_as(ctypes.c_void_p), need)
    if got != need:
        raise SpecVerifyError(SV_ERR_ARG, lib().sv_last_error().decode())
    return out[:grid + 1].copy(), out[grid + 1:].copy()


class Pass:
    """A chain of phases run as one persistent launch (sv_pass_*)."""

    def __init__(self, phases):
        import torch
        n = len(phases)
        arr = (Phase * n)(*phases)
        self._phases = (arr, phases)
        need = lib().sv_pass_workspace_bytes(arr, n)
        if need == 0:
            raise SpecVerifyError(SV_ERR_ARG, lib().sv_last_error().decode())
        buf = torch.zeros(need + 256, dtype=torch.uint8, device="cuda")
        off = (-buf.data_ptr()) % 256
        self._ws = buf[off:off + need]
        h = ctypes.c_void_p()
        _check(lib().sv_pass_create(arr, n, ctypes.c_void_p(self._ws.data_ptr()), need, ctypes.byref(h)))
        self._h = h

    def run(self, stream=None):
        _check(lib().sv_pass_run(self._h, _stream(stream)))

    def status(self) -> int:
        v = ctypes.c_uint32()
        _check(lib().sv_pass_status(self._h, ctypes.byref(v)))
        return v.value

    def trace(self, enable=True):
        """Enable per-phase timestamps for later runs; returns the grid size."""
        g = ctypes.c_int32()
        _check(lib().sv_pass_trace(self._h, int(enable), None, 0, ctypes.byref(g)))
        return g.value

    def read_trace(self, n_phases):
        """[grid, n_phases, 16] uint64 record of the last traced run."""
        import numpy as np
        g = ctypes.c_int32()
        _check(lib().sv_pass_trace(self._h, 1, None, 0, ctypes.byref(g)))
        buf = np.zeros((g.value, n_phases, 16), np.uint64)
        _check(lib().sv_pass_trace(self._h, 1, buf.ctypes.data_as(ctypes.c_void_p), buf.nbytes, None))
        return buf

    def __del__(self):
        if getattr(self, "_h", None) and _lib is not None:
            _lib.sv_pass_destroy(self._h)
            self._h = None


def argmax_index(packed: int) -> int:
    return int(lib().sv_argmax_index(ctypes.c_uint64(int(packed) & 0xFFFFFFFFFFFFFFFF)))


def accept_greedy(argmax, drafts, out, n_rows, row_ids=None, stream=None):
    """n_rows: rows of the head the argmax words index (the vocabulary, or
    the number of row_ids of a restricted head)."""
    K = 0 if drafts is None else drafts.numel()
    _check(lib().sv_accept_greedy(_ptr(argmax), _ptr(row_ids), int(n_rows), _ptr(drafts), K, _ptr(out),
                                  _stream(stream)))


def accept_workspace_bytes(V: int, K: int) -> int:
    return int(lib().sv_accept_workspace_bytes(V, K))


def accept_rejection(logits, drafts, u, out, workspace, temperature=1.0, q=None, stream=None):
    V = logits.shape[-1]
    K = 0 if drafts is None else drafts.numel()
    _check(lib().sv_accept_rejection(_ptr(logits), V, _ptr(q), _ptr(drafts), K, _ptr(u), float(temperature),
                                     _ptr(workspace), workspace.numel() * workspace.element_size(), _ptr(out),
                                     _stream(stream)))


def accept_noalloc_max_bytes() -> int:
    return int(lib().sv_accept_noalloc_max_bytes())


def accept_rejection_noalloc(logits, drafts, u, out, temperature=1.0, q=None, stream=None):
    """accept_rejection on the library's static scratch (no workspace, no
    allocation); calls that overlap on one GPU must not be made."""
    V = logits.shape[-1]
    K = 0 if drafts is None else drafts.numel()
    _check(lib().sv_accept_rejection_noalloc(_ptr(logits), V, _ptr(q), _ptr(drafts), K, _ptr(u),
                                             float(temperature), _ptr(out), _stream(stream)))


def read_bandwidth(src, sink, stream=None):
    """Pure-read measurement kernel over the bytes of `src` (see
    sv_read_bandwidth); one workgroup per element of `sink` (uint32/int32)."""
    _check(lib().sv_read_bandwidth(_ptr(src), src.numel() * src.element_size(), _ptr(sink), sink.numel(),
                                   _stream(stream)))
