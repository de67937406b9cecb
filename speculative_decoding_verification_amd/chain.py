"""A verification pass over a stack of quantised projection layers.

Host-side sequencing of C-ABI calls only (no arithmetic here): per layer
four phases, each one launch of sv_verify_matvec whose fused epilogue
requantises the next phase's input ("Inside OpenJet Engine: making
speculative decoding pay", section "One GPU launch for a speculative cycle":
the producing phase requantises activations for the next consumer,
including the next RMS normalisation's weight):

    x  -> a   = Q8A32(x * g1)                 (RMS factor of x folded below)
    a  -> q, k, v = r(x) W{q,k,v} a           epilogue: b = Q8A32(v * g2)
          (when v's format differs from q and k's: one phase for v with
          the epilogue, then one for q and k, both on a; o waits for v only)
    b  -> o   = r(v) Wo b                     epilogue: c = Q8A32(o * g3)
    c  -> g, u = r(o) W{g,u} c                epilogue: h = Q8A32((g*u) * g4)
    h  -> x'  = r(g*u) Wd h                   epilogue: Q8A32(x' * next norm)

then the head (logits + fused argmax) and acceptance.  With no attention
history the single-key attention of each position returns its own v, so o
reads v; q and k are computed and written but have no consumer.  There are
no residual adds.  The whole pass can be captured once in a HIP graph (the
calls are stream-ordered and allocate nothing) and replayed per cycle.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from . import (SV_EP_PAIR, SV_EP_QUANT, SV_Q4_K, SV_Q6_K, SV_Q8_0, Pass, accept_greedy, act, epilogue,
               gguf_bytes, head_logits, phase, quantize_act_q8, repack_weights, repacked_bytes, verify_matvec, weight)


@dataclass
class StackShape:
    hidden: int
    ffn: int
    layers: int
    vocab: int
    attn_q: int = SV_Q4_K      # q, k, o
    v_q: int = SV_Q4_K
    gate_up_q: int = SV_Q4_K
    down_q: int = SV_Q6_K
    head_q: int = SV_Q6_K

    def layer_mats(self):
        H, F = self.hidden, self.ffn
        return [("q", self.attn_q, H, H), ("k", self.attn_q, H, H), ("v", self.v_q, H, H),
                ("o", self.attn_q, H, H), ("gate", self.gate_up_q, F, H), ("up", self.gate_up_q, F, H),
                ("down", self.down_q, H, F)]

    def layer_bytes(self) -> int:
        return sum(gguf_bytes(qt, r, c) for _, qt, r, c in self.layer_mats())

    def head_bytes(self) -> int:
        return gguf_bytes(self.head_q, self.vocab, self.hidden) if self.vocab else 0

    def pass_bytes(self) -> int:
        return self.layers * self.layer_bytes() + self.head_bytes()


# The 4B-class chain (hidden 2560, FFN 9728, 36 layers, Q4_K attention and
# gate/up, Q6_K down) with a Q6_K head over a 151936-token vocabulary.
CHAIN_4B = StackShape(hidden=2560, ffn=9728, layers=36, vocab=151936)
# The 27B-class stack: Q4_K q, k, o, gate, up; Q6_K v and down.
STACK_27B = StackShape(hidden=5120, ffn=17408, layers=64, vocab=151936, v_q=SV_Q6_K)


def _torch():
    import torch
    return torch


class _Act:
    def __init__(self, M, K):
        t = _torch()
        self.M, self.K = M, K
        self.q = t.empty((M, K), dtype=t.int8, device="cuda")
        self.d = t.empty((M, K // 32), dtype=t.float32, device="cuda")
        self.s16 = t.empty((M, K // 16), dtype=t.int32, device="cuda")
        self.sumsq = t.empty((M, K // 32), dtype=t.float32, device="cuda")

    def desc(self, M, eps):
        return act(M, self.K, self.q, self.d, self.s16, self.sumsq, self.K // 32, eps)

    def ep(self, mode, gamma, src=0):
        return epilogue(mode, self.q, self.d, self.s16, self.sumsq, gamma=gamma, src=src)


@dataclass
class LayerWeights:
    mats: dict = field(default_factory=dict)    # name -> (sv.Weight, buffer)
    gammas: dict = field(default_factory=dict)  # g1..g4 -> device fp32


def upload_gguf(qtype: int, raw: np.ndarray, rows: int, cols: int, staging=None):
    """Copy canonical GGUF bytes to the GPU and repack them (load time)."""
    t = _torch()
    g = gguf_bytes(qtype, rows, cols)
    assert g == raw.size, (g, raw.size)
    src = t.from_numpy(raw.reshape(-1)).cuda() if staging is None else staging[:g].copy_(
        t.from_numpy(raw.reshape(-1)), non_blocking=False)
    dst = t.empty(repacked_bytes(qtype, rows, cols), dtype=t.uint8, device="cuda")
    assert dst.data_ptr() % 256 == 0
    repack_weights(qtype, src, dst, rows, cols)
    return weight(qtype, rows, cols, dst), dst


class VerifyStack:
    """Device weights and buffers of one stack plus the pass itself."""

    def __init__(self, shape: StackShape, weights_fn, max_M: int = 16, eps: float = 1e-6, workers: int = 0):
        """weights_fn(layer, name, qtype, rows, cols) -> GGUF bytes;
        weights_fn(-1, 'gamma:<name>', ...) -> fp32 norm weights.  It is
        called from `workers` threads (0: one per core, at most 16), the
        next layer's matrices being drawn while this layer's upload."""
        t = _torch()
        self.shape, self.eps, self.max_M = shape, eps, max_M
        H, F = shape.hidden, shape.ffn
        staging = t.empty(max(gguf_bytes(qt, r, c) for _, qt, r, c in shape.layer_mats()) + 256,
                          dtype=t.uint8, device="cuda")
        self.layers = []
        n_workers = workers or max(1, min(16, os.cpu_count() or 1))
        with ThreadPoolExecutor(n_workers) as ex:
            def submit(layer):
                return [(name, qt, r, c, ex.submit(weights_fn, layer, name, qt, r, c))
                        for name, qt, r, c in shape.layer_mats()]
            pending = submit(0) if shape.layers else []
            for layer in range(shape.layers):
                nxt = submit(layer + 1) if layer + 1 < shape.layers else []
                lw = LayerWeights()
                for name, qt, r, c, fut in pending:
                    raw = fut.result()
                    lw.mats[name] = upload_gguf(qt, raw, r, c, staging)
                    del raw
                for g, n in (("g1", H), ("g2", H), ("g3", H), ("g4", F)):
                    lw.gammas[g] = t.from_numpy(weights_fn(layer, "gamma:" + g, None, n, 0)).cuda()
                self.layers.append(lw)
                pending = nxt
        self.gamma_f = t.from_numpy(weights_fn(-1, "gamma:final", None, H, 0)).cuda()
        self.head = None
        if shape.vocab:
            raw = weights_fn(-1, "head", shape.head_q, shape.vocab, H)
            self.head = upload_gguf(shape.head_q, raw, shape.vocab, H)
            del raw
        del staging
        M = max_M
        self.x = t.empty((M, H), dtype=t.float32, device="cuda")
        # Every phase writes its requantised output to buffers of its own:
        # within one persistent launch an address is written once, so no
        # reader's cache can hold a stale copy of it.
        self.acts = []
        for _ in range(shape.layers):
            self.acts.append({"in": _Act(M, H), "v": _Act(M, H), "o": _Act(M, H), "h": _Act(M, F)})
        self.a_final = _Act(M, H)
        self.a_in = self.acts[0]["in"]
        # Each layer writes its q, k and v outputs to buffers of its own: a
        # pass does not order two phases' writes to one y buffer, and a
        # layer's q/k units fill idle workgroups wherever the schedule finds
        # them, so a buffer shared by the layers could end with an earlier
        # layer's rows.  yq, yk and yv are the last layer's.
        self.ys = [{n: t.empty((M, H), dtype=t.float32, device="cuda") for n in "qkv"}
                   for _ in range(max(shape.layers, 1))]
        self.yq, self.yk, self.yv = self.ys[-1]["q"], self.ys[-1]["k"], self.ys[-1]["v"]
        self.logits = t.empty((M, shape.vocab or 1), dtype=t.float32, device="cuda")
        self.argmax = t.zeros((M,), dtype=t.int64, device="cuda")
        self.drafts = t.zeros((max(M - 1, 1),), dtype=t.int32, device="cuda")
        self.out = t.zeros((M + 1,), dtype=t.int32, device="cuda")

    # ----------------------------------------------------------- phases
    def _specs(self, M: int):
        """(label, weights, act, ys, epilogue, head?) of every projection
        phase of one pass at M positions, in order."""
        eps = self.eps
        L = self.layers
        specs = []
        for li, lw in enumerate(L):
            m = lw.mats
            a = self.acts[li]
            y = self.ys[li]
            last = li + 1 == len(L)
            nxt = self.gamma_f if last else L[li + 1].gammas["g1"]
            out = self.a_final if last else self.acts[li + 1]["in"]
            if self.shape.attn_q == self.shape.v_q:
                specs.append(("qkv", [m["q"][0], m["k"][0], m["v"][0]], a["in"].desc(M, eps),
                              [y["q"], y["k"], y["v"]], a["v"].ep(SV_EP_QUANT, lw.gammas["g2"], src=2)))
            else:
                # v (its own format) first: o waits for it alone; q and k
                # read the same input and have no reader
                specs.append(("v", [m["v"][0]], a["in"].desc(M, eps), [y["v"]],
                              a["v"].ep(SV_EP_QUANT, lw.gammas["g2"], src=0)))
                specs.append(("qk", [m["q"][0], m["k"][0]], a["in"].desc(M, eps), [y["q"], y["k"]], None))
            specs.append(("o", [m["o"][0]], a["v"].desc(M, eps), [None],
                          a["o"].ep(SV_EP_QUANT, lw.gammas["g3"])))
            specs.append(("gate_up", [m["gate"][0], m["up"][0]], a["o"].desc(M, eps), [None, None],
                          a["h"].ep(SV_EP_PAIR, lw.gammas["g4"])))
            specs.append(("down", [m["down"][0]], a["h"].desc(M, eps), [None], out.ep(SV_EP_QUANT, nxt)))
        return specs

    def _quant_in(self, M):
        quantize_act_q8(self.x[:M], self.a_in.q[:M], self.a_in.d[:M], self.a_in.s16[:M],
                        gamma=self.layers[0].gammas["g1"], sumsq=self.a_in.sumsq[:M])

    def _accept(self, M):
        accept_greedy(self.argmax[:M], self.drafts[:M - 1] if M > 1 else None, self.out[:M + 1], self.shape.vocab)

    def phases(self, M: int):
        """(label, callable) of every launch of one eager pass at M positions
        (one sv_verify_matvec / sv_head_logits call per phase)."""
        ph = [("quant_in", lambda: self._quant_in(M))]
        for label, ws, a, ys, ep in self._specs(M):
            ph.append((label, lambda ws=ws, a=a, ys=ys, ep=ep: verify_matvec(ws, a, ys, ep)))
        if self.head is not None:
            ph.append(("head", lambda: head_logits(self.head[0], self.a_final.desc(M, self.eps), self.logits[:M],
                                                   self.argmax[:M])))
            ph.append(("accept", lambda: self._accept(M)))
        return ph

    def run(self, M: int):
        for _, f in self.phases(M):
            f()

    def make_pass(self, M: int) -> Pass:
        """The projection phases and the head as one persistent launch."""
        phs = [phase(ws, a, ys, ep) for _, ws, a, ys, ep in self._specs(M)]
        if self.head is not None:
            phs.append(phase([self.head[0]], self.a_final.desc(M, self.eps), [self.logits[:M]],
                             argmax=self.argmax[:M]))
        return Pass(phs)

    def run_pass(self, M: int, p: Pass):
        self._quant_in(M)
        p.run()
        if self.head is not None:
            self._accept(M)

    def capture(self, M: int, persistent: bool = True):
        """Capture one pass at M positions in a HIP graph (torch.cuda.CUDAGraph)."""
        t = _torch()
        p = self.make_pass(M) if persistent else None
        fn = (lambda: self.run_pass(M, p)) if persistent else (lambda: self.run(M))
        s = t.cuda.Stream()
        s.wait_stream(t.cuda.current_stream())
        with t.cuda.stream(s):
            fn()          # warm-up on the side stream (sizes the shared workspace)
        t.cuda.current_stream().wait_stream(s)
        t.cuda.synchronize()
        g = t.cuda.CUDAGraph()
        with t.cuda.graph(g):
            fn()
        t.cuda.synchronize()
        g._keep_pass = p
        return g

    def phase_bytes(self, label: str) -> int:
        sh = self.shape
        H, F = sh.hidden, sh.ffn
        if label == "qkv":
            return 2 * gguf_bytes(sh.attn_q, H, H) + gguf_bytes(sh.v_q, H, H)
        if label == "v":
            return gguf_bytes(sh.v_q, H, H)
        if label == "qk":
            return 2 * gguf_bytes(sh.attn_q, H, H)
        if label == "o":
            return gguf_bytes(sh.attn_q, H, H)
        if label == "gate_up":
            return 2 * gguf_bytes(sh.gate_up_q, F, H)
        if label == "down":
            return gguf_bytes(sh.down_q, H, F)
        if label == "head":
            return sh.head_bytes()
        return 0
