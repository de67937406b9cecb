"""Host-side tests of the C ABI (no GPU needed): the library loads, exports
every function include/specverify.h declares, sizes are right, and invalid
arguments are rejected with the documented status before any launch."""

import ctypes
import os
import re
import subprocess

import pytest

import speculative_decoding_verification_amd as sv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "specverify.h")

pytestmark = pytest.mark.skipif(not os.path.exists(sv.LIB_PATH), reason="libspecverify.so not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sv_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert len(names) >= 12
    out = subprocess.run(["nm", "-D", "--defined-only", sv.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (sv_\w+)", out))
    assert set(names) <= exported, set(names) - exported
    L = sv.lib()
    for n in names:
        assert hasattr(L, n)
    assert set(sv.EXPORTS) == set(names)


def test_version():
    assert "gfx950" in sv.version()


def _blocked(qt, rows, cols):
    """Tile-blocked size: rows rounded up to 16, cols to 256, one block of
    16 rows x 256 columns each (the GGUF bytes of those elements), and 64
    zero bytes after the last block."""
    per_256 = {8: 8 * 34, 12: 144, 14: 210}[qt]
    return -(-rows // 16) * 16 * -(-cols // 256) * per_256 + 64


@pytest.mark.parametrize("qt,rows,cols,expect", [
    (8, 1024, 1024, _blocked(8, 1024, 1024)),
    (12, 2560, 2560, _blocked(12, 2560, 2560)),
    (14, 151936, 5120, _blocked(14, 151936, 5120)),
    (14, 5120, 17408, _blocked(14, 5120, 17408)),
    (8, 100, 96, _blocked(8, 100, 96)),      # ragged rows and a partial step
    (8, 3, 48, 0),      # cols not a multiple of 32
    (12, 4, 128, 0),    # cols not a multiple of 256
    (3, 4, 256, 0),     # unsupported type
    (8, 0, 32, 0),
])
def test_repacked_bytes(qt, rows, cols, expect):
    assert sv.repacked_bytes(qt, rows, cols) == expect
    if expect:
        # the blocks hold exactly the GGUF bytes of the padded matrix
        per_256 = {8: 8 * 34, 12: 144, 14: 210}[qt]
        assert expect - 64 == -(-rows // 16) * 16 * -(-cols // 256) * per_256


FAKE = ctypes.c_void_p(1 << 20)        # never dereferenced: validation fails first
FAKE_ODD = ctypes.c_void_p((1 << 20) + 4)


def _err(rc, code):
    assert rc == code, (rc, sv.lib().sv_last_error())
    assert sv.lib().sv_last_error()


def test_quantize_rejects():
    L = sv.lib()
    _err(L.sv_quantize_act_q8(FAKE, 0, 64, None, FAKE, FAKE, FAKE, None, None), sv.SV_ERR_ARG)
    _err(L.sv_quantize_act_q8(FAKE, 17, 64, None, FAKE, FAKE, FAKE, None, None), sv.SV_ERR_ARG)
    _err(L.sv_quantize_act_q8(FAKE, 2, 48, None, FAKE, FAKE, FAKE, None, None), sv.SV_ERR_SHAPE)
    _err(L.sv_quantize_act_q8(None, 2, 64, None, FAKE, FAKE, FAKE, None, None), sv.SV_ERR_ARG)
    _err(L.sv_quantize_act_q8(ctypes.c_void_p((1 << 20) + 2), 2, 64, None, FAKE, FAKE, FAKE, None, None),
         sv.SV_ERR_ALIGN)


def test_repack_rejects():
    L = sv.lib()
    _err(L.sv_repack_weights(5, FAKE, FAKE, 4, 256, None), sv.SV_ERR_QTYPE)
    _err(L.sv_repack_weights(12, FAKE, FAKE, 4, 128, None), sv.SV_ERR_SHAPE)
    _err(L.sv_repack_weights(12, FAKE, FAKE_ODD, 4, 256, None), sv.SV_ERR_ALIGN)
    _err(L.sv_repack_weights(12, None, FAKE, 4, 256, None), sv.SV_ERR_ARG)
    # overlapping source and destination
    _err(L.sv_repack_weights(8, ctypes.c_void_p((1 << 20) + 256), FAKE, 4, 256, None), sv.SV_ERR_ARG)


def _act(M=5, K=256, q=FAKE):
    return sv.Act(M, K, q.value, FAKE.value, FAKE.value, None, 0, 1e-6)


def _w(qt=12, rows=64, cols=256, data=FAKE):
    return sv.Weight(qt, rows, cols, data.value)


def _mv(ws, A, ep=None):
    n = len(ws)
    W = (sv.Weight * n)(*ws)
    Y = (ctypes.c_void_p * n)(*([FAKE.value] * n))
    return sv.lib().sv_verify_matvec(W, n, ctypes.byref(A), Y, None if ep is None else ctypes.byref(ep), None, 0,
                                     None)


def test_matvec_rejects():
    _err(_mv([_w()], _act(M=0)), sv.SV_ERR_ARG)
    _err(_mv([_w()], _act(M=17)), sv.SV_ERR_ARG)
    _err(_mv([_w(qt=2)], _act()), sv.SV_ERR_QTYPE)
    _err(_mv([_w(cols=512)], _act()), sv.SV_ERR_SHAPE)          # cols != K
    _err(_mv([_w(cols=32)], _act(K=32)), sv.SV_ERR_SHAPE)       # Q4_K needs 256
    _err(_mv([_w(data=FAKE_ODD)], _act()), sv.SV_ERR_ALIGN)
    _err(_mv([_w()], _act(q=FAKE_ODD)), sv.SV_ERR_ALIGN)
    _err(_mv([_w(), _w(rows=32)], _act()), sv.SV_ERR_SHAPE)     # rows differ
    _err(_mv([_w(), _w(qt=14)], _act()), sv.SV_ERR_SHAPE)       # qtypes differ
    W = (sv.Weight * 4)(*([_w()] * 4))
    rc = sv.lib().sv_verify_matvec(W, 4, ctypes.byref(_act()), None, None, None, 0, None)
    _err(rc, sv.SV_ERR_ARG)
    ep = sv.Epilogue(7, 0, None, FAKE.value, FAKE.value, FAKE.value, FAKE.value)
    _err(_mv([_w()], _act(), ep), sv.SV_ERR_ARG)
    ep = sv.Epilogue(sv.SV_EP_PAIR, 0, None, FAKE.value, FAKE.value, FAKE.value, FAKE.value)
    _err(_mv([_w()], _act(), ep), sv.SV_ERR_ARG)                 # pair needs two
    ep = sv.Epilogue(sv.SV_EP_QUANT, 0, None, FAKE.value, FAKE.value, FAKE.value, FAKE.value)
    _err(_mv([_w(rows=48)], _act(), ep), sv.SV_ERR_SHAPE)       # rows % 32
    ep = sv.Epilogue(sv.SV_EP_QUANT, 3, None, FAKE.value, FAKE.value, FAKE.value, FAKE.value)
    _err(_mv([_w()], _act(), ep), sv.SV_ERR_ARG)                 # src out of range


def test_head_and_accept_rejects():
    L = sv.lib()
    H = _w(qt=14)
    _err(L.sv_head_logits(ctypes.byref(H), ctypes.byref(_act()), None, 0, None, None, None, 0, None),
         sv.SV_ERR_ARG)
    _err(L.sv_head_logits(ctypes.byref(H), ctypes.byref(_act()), FAKE, 0, FAKE, None, None, 0, None),
         sv.SV_ERR_SHAPE)
    # a head whose K is split over units (K > 5120) needs a workspace
    H2 = _w(qt=14, rows=4096, cols=10240)
    A2 = _act(K=10240)
    need = L.sv_head_workspace_bytes(ctypes.byref(H2), ctypes.byref(A2), 0)
    assert need > 0
    _err(L.sv_head_logits(ctypes.byref(H2), ctypes.byref(A2), None, 0, FAKE, None, None, 0, None),
         sv.SV_ERR_WORKSPACE)
    _err(L.sv_accept_greedy(FAKE, None, 4096, FAKE, 16, FAKE, None), sv.SV_ERR_ARG)
    _err(L.sv_accept_greedy(FAKE, None, 0, FAKE, 4, FAKE, None), sv.SV_ERR_ARG)      # no rows
    _err(L.sv_accept_greedy(FAKE_ODD, None, 4096, FAKE, 4, FAKE, None), sv.SV_ERR_ALIGN)
    ws = sv.accept_workspace_bytes(151936, 4)
    assert ws > 0 and ws % 256 == 0
    assert sv.accept_workspace_bytes(10, 16) == 0
    _err(L.sv_accept_rejection(FAKE, 151936, None, FAKE, 4, FAKE, ctypes.c_float(0.0), FAKE, ws, FAKE, None),
         sv.SV_ERR_ARG)
    _err(L.sv_accept_rejection(FAKE, 151936, None, FAKE, 4, FAKE, ctypes.c_float(1.0), FAKE, ws - 8, FAKE, None),
         sv.SV_ERR_WORKSPACE)
    _err(L.sv_accept_rejection(FAKE, 0, None, FAKE, 4, FAKE, ctypes.c_float(1.0), FAKE, ws, FAKE, None),
         sv.SV_ERR_SHAPE)
    # the allocation-free variant refuses a round larger than its static
    # scratch before any runtime call
    cap = sv.accept_noalloc_max_bytes()
    assert cap == 256 * 1024 and sv.accept_workspace_bytes(860160, 15) <= cap
    assert sv.accept_workspace_bytes(860161, 15) > cap
    _err(L.sv_accept_rejection_noalloc(FAKE, 860161, None, FAKE, 15, FAKE, ctypes.c_float(1.0), FAKE, None),
         sv.SV_ERR_WORKSPACE)
    _err(L.sv_accept_rejection_noalloc(FAKE, 151936, None, FAKE, 16, FAKE, ctypes.c_float(1.0), FAKE, None),
         sv.SV_ERR_ARG)
    _err(L.sv_accept_rejection_noalloc(FAKE, 0, None, FAKE, 4, FAKE, ctypes.c_float(1.0), FAKE, None),
         sv.SV_ERR_SHAPE)


def _chunking(rows, cols, balance=True, grid=256, max_s=8):
    """K chunks of a phase: S = ceil(steps / 20) for every tile; a balanced
    phase (not a head) with at least one round of `grid` tile-chunks and a
    partial last round cuts the last ceil(R / S) tiles (R = the remainder of
    tile-chunks over whole rounds) into S1 = f S chunks, f = the largest
    factor that keeps those tiles within one round, chunks of at least one
    step and at most 8 chunks.  Returns (S, S1, tiles cut into S)."""
    steps = -(-cols // 256)
    S = -(-steps // 20)
    T = -(-rows // 32)
    if balance and T * S >= grid and (T * S) % grid:
        tr = -(-((T * S) % grid) // S)
        f = min(grid // (tr * S), max_s // S, steps // S)
        if f >= 2:
            return S, S * f, T - tr
    return S, S, T


def test_workspace_sizes():
    """Partial sums (after a fixed 256 KiB counter region, [n_w][S1][M][rows]
    fp32) are needed when some tile's K is split over units, or when two
    matrices may be paired at M > 8 (then each matrix of a pair is a unit of
    its own and the tile's last unit forms the product; at M <= 8 a unit
    covers both), and nothing otherwise.  A head keeps one chunking for all
    tiles."""
    L = sv.lib()
    cases = [(2560, 2560, 12, 3, 5, (1, 1)), (2560, 9728, 14, 1, 5, (2, 2)), (9728, 2560, 12, 2, 16, (1, 5)),
             (5120, 17408, 14, 1, 5, (4, 8)), (17408, 5120, 12, 1, 8, (1, 8)), (2560, 2560, 14, 2, 5, (1, 1)),
             (17408, 5120, 12, 2, 5, (1, 8)), (4096, 10240, 14, 1, 3, (2, 2)), (8192, 5120, 12, 1, 5, (1, 1)),
             (8192 + 32, 2048, 8, 1, 2, (1, 8)), (2048, 1024, 8, 1, 1, (1, 1))]
    for rows, cols, qt, n_w, M, (S, S1) in cases:
        assert _chunking(rows, cols)[:2] == (S, S1), (rows, cols)
        W = (sv.Weight * n_w)(*([_w(qt=qt, rows=rows, cols=cols)] * n_w))
        need = L.sv_matvec_workspace_bytes(W, n_w, ctypes.byref(_act(M=M, K=cols)))
        if S1 == 1 and (n_w != 2 or M <= 8):
            assert need == 0, (rows, cols)
        else:
            assert need == 256 * 1024 + n_w * S1 * M * rows * 4, (rows, cols)
    # a head is never rebalanced: 17408 rows of K = 5120 stay in one chunk
    H = _w(qt=12, rows=17408, cols=5120)
    assert L.sv_head_workspace_bytes(ctypes.byref(H), ctypes.byref(_act(M=5, K=5120)), 0) == 0


def _phase(W, A, ep=None, argmax=None):
    ph = sv.Phase()
    ph.W, ph.n_w, ph.A = ctypes.cast(W, ctypes.POINTER(sv.Weight)), len(W), A
    if ep is not None:
        ph.ep = ep
    ph.argmax = argmax
    return ph


def test_pass_rejects():
    L = sv.lib()
    W1 = (sv.Weight * 1)(_w(qt=12, rows=64, cols=256))
    W2 = (sv.Weight * 1)(_w(qt=12, rows=64, cols=512))
    a1, a2 = _act(K=256), _act(M=3, K=512)
    ph = (sv.Phase * 2)(_phase(W1, a1), _phase(W2, a2))
    assert L.sv_pass_workspace_bytes(ph, 2) == 0          # M differs
    h = ctypes.c_void_p()
    _err(L.sv_pass_create(ph, 2, FAKE, 1 << 30, ctypes.byref(h)), sv.SV_ERR_SHAPE)
    ok = (sv.Phase * 1)(_phase(W1, a1))
    need = L.sv_pass_workspace_bytes(ok, 1)
    assert need > 0
    _err(L.sv_pass_create(ok, 1, FAKE, need - 1, ctypes.byref(h)), sv.SV_ERR_WORKSPACE)
    _err(L.sv_pass_create(ok, 1, FAKE_ODD, need, ctypes.byref(h)), sv.SV_ERR_ALIGN)
    _err(L.sv_pass_create(ph, 0, FAKE, 1 << 30, ctypes.byref(h)), sv.SV_ERR_ARG)


def _buf(i):
    """A fake, 256-byte aligned device address well apart from the others."""
    return (1 << 32) + i * (1 << 24)


def _ep(i, mode=sv.SV_EP_QUANT):
    return sv.Epilogue(mode, 0, None, _buf(i), _buf(i) + (1 << 20), _buf(i) + (2 << 20), _buf(i) + (3 << 20))


def _act_at(i, M=5, K=64, parts=False):
    return sv.Act(M, K, _buf(i), _buf(i) + (1 << 20), _buf(i) + (2 << 20),
                  _buf(i) + (3 << 20) if parts else None, K // 32 if parts else 0, 1e-6)


def test_pass_dependency_rules():
    """Rules sv_pass_create checks on the host before touching the device:
    a consumer reads exactly its producer's outputs; inputs written by no
    earlier phase share no 256-byte block with anything the pass writes;
    requantised outputs never share blocks; at most four argmax phases."""
    L = sv.lib()
    W = (sv.Weight * 1)(_w(qt=8, rows=64, cols=64))
    h = ctypes.c_void_p()

    def create(phs):
        arr = (sv.Phase * len(phs))(*phs)
        return L.sv_pass_create(arr, len(phs), FAKE, 1 << 30, ctypes.byref(h))

    # consumer takes the producer's codes but other scales
    bad = _act_at(1, K=64, parts=True)
    bad.d = _buf(7)
    _err(create([_phase(W, _act_at(0), _ep(1)), _phase(W, bad, _ep(2))]), sv.SV_ERR_ARG)
    # a phase's input is a later phase's output (written during the launch)
    _err(create([_phase(W, _act_at(0), _ep(1)), _phase(W, _act_at(1), _ep(0))]), sv.SV_ERR_ARG)
    # two phases requantise into the same buffers
    _err(create([_phase(W, _act_at(0), _ep(1)), _phase(W, _act_at(1), _ep(1))]), sv.SV_ERR_ARG)
    # a phase input that shares a block with an argmax the pass writes
    _err(create([_phase(W, _act_at(0), _ep(1), argmax=_buf(0) + 128)]), sv.SV_ERR_ARG)
    # five phases with an argmax
    heads = [_phase(W, _act_at(0), argmax=_buf(10 + i)) for i in range(5)]
    _err(create(heads), sv.SV_ERR_ARG)


def test_argmax_index_decode():
    for idx in (0, 1, 151935, (1 << 31) - 1):
        packed = (0xC0000000 << 32) | (0xFFFFFFFF - idx)
        assert sv.argmax_index(packed) == idx


def test_missing_library_fails_loudly(tmp_path, monkeypatch):
    import importlib
    mod = importlib.import_module("speculative_decoding_verification_amd")
    monkeypatch.setattr(mod, "LIB_PATH", str(tmp_path / "absent.so"))
    monkeypatch.setattr(mod, "_lib", None)
    with pytest.raises(ImportError):
        mod.lib()
