"""Host tests of the unit lists a pass runs (sv_pass_schedule, no device).

The phases are wired as the verification stacks wire them (the 27B-class
stack: v, q/k, o, gate/up, down per layer, then the head; the 4B-class chain:
one q/k/v phase with v's epilogue), but every buffer is a synthetic address:
the schedule only compares addresses.  Checked: every (phase, unit) exactly
once, every list in phase order, the same lists on every call, and where the
units of the narrow phases go (v and o on different workgroups as far as
their sizes allow, q/k spread over the workgroups the two leave idle).
"""

import ctypes

import numpy as np
import pytest

import speculative_decoding_verification_amd as sv

Q4K, Q6K = sv.SV_Q4_K, sv.SV_Q6_K
MAX_M = 16


class _Space:
    """Bump allocator of 256-byte aligned synthetic addresses with a gap
    between buffers (nothing is ever read at them)."""

    def __init__(self):
        self.next = 0x7F0000000000

    def take(self, nbytes):
        a = self.next
        self.next += (nbytes + 255) // 256 * 256 + 4096
        return a


def _act_bufs(sp, K):
    return dict(q=sp.take(MAX_M * K), d=sp.take(MAX_M * K // 8), s16=sp.take(MAX_M * K // 4),
                sumsq=sp.take(MAX_M * K // 8), K=K)


def _act(b, M):
    return sv.Act(M, b["K"], b["q"], b["d"], b["s16"], b["sumsq"], b["K"] // 32, 1e-6)


def _ep(b, mode, gamma, src=0):
    return sv.Epilogue(mode, src, gamma, b["q"], b["d"], b["s16"], b["sumsq"])


def _phase(keep, weights, A, ys=(), ep=None, argmax=None):
    arr = (sv.Weight * len(weights))(*weights)
    keep.append(arr)
    ph = sv.Phase()
    ph.W = ctypes.cast(arr, ctypes.POINTER(sv.Weight))
    ph.n_w = len(weights)
    ph.A = A
    for i, y in enumerate(ys):
        ph.y[i] = y
    if ep is not None:
        ph.ep = ep
    ph.argmax = argmax
    return ph


def _weight(sp, qt, rows, cols):
    return sv.Weight(qt, rows, cols, sp.take(sv.repacked_bytes(qt, rows, cols)))


def _stack(M, H, F, L, vocab, v_q, sp=None):
    """(phases, labels, keep-alive list) of a stack pass at M positions."""
    sp = sp or _Space()
    keep, phases, labels = [], [], []
    a_in = _act_bufs(sp, H)
    for li in range(L):
        g = {k: sp.take(4 * n) for k, n in (("g2", H), ("g3", H), ("g4", F), ("g1", H))}
        wq, wk, wv, wo = (_weight(sp, Q4K if n != "v" else v_q, H, H) for n in "qkvo")
        wg, wu, wd = _weight(sp, Q4K, F, H), _weight(sp, Q4K, F, H), _weight(sp, Q6K, H, F)
        ys = {n: sp.take(4 * MAX_M * H) for n in "qkv"}
        b_v, b_o, b_h = _act_bufs(sp, H), _act_bufs(sp, H), _act_bufs(sp, F)
        nxt = _act_bufs(sp, H)
        if v_q == Q4K:
            phases.append(_phase(keep, [wq, wk, wv], _act(a_in, M), [ys["q"], ys["k"], ys["v"]],
                                 _ep(b_v, sv.SV_EP_QUANT, g["g2"], src=2)))
            labels.append("qkv")
        else:
            phases.append(_phase(keep, [wv], _act(a_in, M), [ys["v"]], _ep(b_v, sv.SV_EP_QUANT, g["g2"])))
            labels.append("v")
            phases.append(_phase(keep, [wq, wk], _act(a_in, M), [ys["q"], ys["k"]]))
            labels.append("qk")
        phases.append(_phase(keep, [wo], _act(b_v, M), [0], _ep(b_o, sv.SV_EP_QUANT, g["g3"])))
        labels.append("o")
        phases.append(_phase(keep, [wg, wu], _act(b_o, M), [0, 0], _ep(b_h, sv.SV_EP_PAIR, g["g4"])))
        labels.append("gate_up")
        phases.append(_phase(keep, [wd], _act(b_h, M), [0], _ep(nxt, sv.SV_EP_QUANT, g["g1"])))
        labels.append("down")
        a_in = nxt
    head = _weight(sp, Q6K, vocab, H)
    phases.append(_phase(keep, [head], _act(a_in, M), [sp.take(4 * MAX_M * vocab)], argmax=sp.take(8 * MAX_M)))
    labels.append("head")
    return phases, labels, keep


def _lists(offsets, entries):
    return [entries[offsets[w]:offsets[w + 1]] for w in range(len(offsets) - 1)]


@pytest.fixture(scope="module")
def lib():
    return sv.lib()


def _check_lists(offsets, entries, n_phases):
    assert offsets[0] == 0 and np.all(np.diff(offsets.astype(np.int64)) >= 0)
    assert offsets[-1] == len(entries)
    for lst in _lists(offsets, entries):
        ph = lst >> 20
        assert np.all(np.diff(ph.astype(np.int64)) >= 0), "a list is not in phase order"
    pairs = entries.astype(np.uint64)
    assert len(np.unique(pairs)) == len(pairs), "a unit is listed twice"
    assert np.all((entries >> 20) < n_phases)


@pytest.mark.parametrize("M", [1, 5, 16])
def test_stack27b_lists(lib, M):
    phases, labels, keep = _stack(M, 5120, 17408, 4, 151936, Q6K)
    G = 256
    off, ent = sv.pass_schedule(phases, G)
    _check_lists(off, ent, len(phases))
    # (every unit exactly once is also checked inside the call, which fails
    # otherwise); every phase has units, and a second call gives the same lists
    counts = np.bincount(ent >> 20, minlength=len(phases))
    assert np.all(counts > 0)
    off2, ent2 = sv.pass_schedule(phases, G)
    assert np.array_equal(off, off2) and np.array_equal(ent, ent2)
    lists = _lists(off, ent)
    wgs = {p: {w for w, lst in enumerate(lists) if np.any((lst >> 20) == p)} for p in range(len(phases))}
    for p, lab in enumerate(labels):
        if lab != "v":
            continue
        v, qk, o = wgs[p], wgs[p + 1], wgs[p + 2]
        assert labels[p + 1] == "qk" and labels[p + 2] == "o"
        # 160 units each: at most 160 + 160 - 256 = 64 workgroups run both
        assert len(v & o) <= 64, (M, p, len(v & o))
        # q/k goes to workgroups around v and o, over most of the grid
        assert len(qk) >= 150, (M, p, len(qk))
        # on a workgroup that runs o, its q/k units come before its o units
        for w in qk & o:
            ph = lists[w] >> 20
            assert np.max(np.nonzero(ph == p + 1)[0]) < np.min(np.nonzero(ph == p + 2)[0])


def test_chain4b_lists(lib):
    phases, labels, keep = _stack(5, 2560, 9728, 3, 151936, Q4K)
    assert "qk" not in labels
    off, ent = sv.pass_schedule(phases, 256)
    _check_lists(off, ent, len(phases))


def test_grid_sizes(lib):
    phases, labels, keep = _stack(5, 5120, 17408, 1, 4096, Q6K)
    for G in (1, 7, 256, 1024):
        off, ent = sv.pass_schedule(phases, G)
        assert len(off) == G + 1
        _check_lists(off, ent, len(phases))
        if G == 1:
            # one workgroup runs every unit, phase by phase
            assert np.array_equal(np.sort(ent >> 20), ent >> 20)


def test_schedule_errors(lib):
    phases, labels, keep = _stack(5, 5120, 17408, 1, 4096, Q6K)
    arr = (sv.Phase * len(phases))(*phases)
    n = len(phases)
    for G in (0, 1025, -1):
        assert lib.sv_pass_schedule(arr, n, G, None, 0) == 0
        assert b"grid" in lib.sv_last_error()
    need = lib.sv_pass_schedule(arr, n, 256, None, 0)
    assert need > 257
    buf = np.zeros(need, np.uint32)
    assert lib.sv_pass_schedule(arr, n, 256, buf.ctypes.data_as(ctypes.c_void_p), need - 1) == 0
    assert b"holds" in lib.sv_last_error()
    assert lib.sv_pass_schedule(arr, n, 256, buf.ctypes.data_as(ctypes.c_void_p), need) == need
    # an input that is not exactly an earlier phase's output but overlaps one
    bad = list(phases)
    A = bad[2].A    # o reads v's output: shift its scales by one block
    A.d = A.d + 256
    bad[2].A = A
    arr = (sv.Phase * n)(*bad)
    assert lib.sv_pass_schedule(arr, n, 256, None, 0) == 0
    assert b"shares 256-byte blocks" in lib.sv_last_error() or b"exactly" in lib.sv_last_error()
