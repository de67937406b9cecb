#!/usr/bin/env python3
"""Benchmark of the verification pass on one MI355X.

A step is one verification pass at M positions (current token + M-1
drafts) over a quantised projection stack, the requantising epilogue
between every pair of projections, a Q6_K output head over 151936 tokens
with fused argmax, and greedy acceptance.  The default workload is the
27B-class stack: hidden 5120, FFN 17408, 64 layers, Q4_K q/k/o/gate/up and
Q6_K v/down, plus the Q6_K head (15,942,097,920 weight bytes per pass); the
4B-class chain (hidden 2560, FFN 9728, 36 layers) is --config chain4b.
Weights and inputs are seeded synthetic data resident in HBM before timing
starts.  Each pass is one persistent launch, captured once in a HIP graph
(with the input quantiser and the acceptance) and replayed.

Output: one JSON line.  `value` is the weight-stream rate in GB/s (the
repacked weight bytes one pass reads / time per pass) at the headline M; the
M sweep reports time per pass (median, p10, p90 over single replays), GB/s,
% of the 8 TB/s HBM peak and of the pure-read rate measured in the same
run, verified positions/s, t(M)/t(1), and the implied tokens/s
E(M, a) / t(M) with E(M, a) = (1 - a^M) / (1 - a) expected tokens per
cycle at per-draft acceptance a.  `roofline` gives the pass kernel's rate
from live per-launch HIP-event timing; `cpu_baseline` times the CPU oracle
on the same pass on the host cores; `manifest` records the GPU, software,
clocks and power before and after.
"""

from __future__ import annotations

import argparse
import json
import os
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
METRIC = "weight-stream GB/s (% HBM peak) and verified positions/s at M=1..5"
SEED_BASE = 0x5EED0000
ACCEPT_RATES = (0.6, 0.75, 0.9)
CONFIGS = {"chain4b": 1, "stack27b": 3}   # index of the workload in the configuration list


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def make_weights_fn(seed, keep=None):
    import synth

    def fn(layer, name, qtype, rows, cols):
        if name.startswith("gamma:"):
            return synth.rms_weight(rows, seed, layer, name)
        raw = synth.gguf_weights(qtype, rows, cols, seed, layer, name)
        if keep is not None:
            keep[(layer, name)] = (qtype, raw)
        return raw
    return fn


def expected_tokens(M, a):
    """Tokens per cycle when each of the M-1 drafts is accepted with
    probability a independently until the first rejection, plus the bonus
    or correction token: 1 + a + ... + a^(M-1)."""
    return sum(a ** k for k in range(M))


def time_replays(g, steps, warmup):
    """Warm up, then time exactly `steps` replays between two synchronised
    events, with an event pair around every replay for the spread."""
    import numpy as np
    import torch
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    t0 = time.perf_counter()
    ev[0].record()
    for i in range(steps):
        g.replay()
        ev[i + 1].record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps * 1e3
    per = np.array([ev[i].elapsed_time(ev[i + 1]) for i in range(steps)])
    total = ev[0].elapsed_time(ev[-1])
    return {"ms_per_pass": total / steps, "ms_median": float(np.median(per)),
            "ms_p10": float(np.percentile(per, 10)), "ms_p90": float(np.percentile(per, 90)),
            "wall_ms_per_pass": wall}


def time_sweep(stack, Ms, steps, warmup):
    rows = []
    for M in Ms:
        g = stack.capture(M)
        p = g._keep_pass
        p.status()                       # clears what capture's warm-up run left
        grid = p.trace(False)
        r = time_replays(g, steps, warmup)
        r["grid"] = grid
        st = p.status()
        if st != 0:
            raise RuntimeError(f"pass at M={M} reported status {st} during the timed replays")
        r["M"] = M
        rows.append(r)
        log(f"M={M}: {r['ms_per_pass']:.4f} ms/pass (median {r['ms_median']:.4f}, p10 {r['ms_p10']:.4f}, "
            f"p90 {r['ms_p90']:.4f}; grid {grid}; status ok)")
        del g
    return rows


def calibrate_sleep():
    import torch
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(1000)
    e0.record()
    torch.cuda._sleep(2_000_000)
    e1.record()
    torch.cuda.synchronize()
    return 2_000_000 / max(e0.elapsed_time(e1), 1e-3)   # cycles per ms


def pass_launch_timing(stack, M, launches, cycles_per_ms):
    """Duration of individual launches of the one-launch pass kernel, each
    bracketed by its own HIP events on the launching stream and preceded by
    ~60 us of queued GPU work, so host enqueue time never falls inside a
    measured interval."""
    import torch
    p = stack.make_pass(M)
    stack.run_pass(M, p)            # warm
    torch.cuda.synchronize()
    p.status()
    sleep = int(cycles_per_ms * 0.06)
    recs = []
    for _ in range(launches):
        stack._quant_in(M)
        torch.cuda._sleep(sleep)
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        p.run()
        b.record()
        recs.append((a, b))
    torch.cuda.synchronize()
    st = p.status()
    if st != 0:
        raise RuntimeError(f"pass reported status {st} in the roofline launches")
    return [a.elapsed_time(b) * 1e3 for a, b in recs]   # us


def per_phase_timing(stack, M, passes, cycles_per_ms):
    """Per-phase launches (one sv_verify_matvec call per phase), each timed
    alone as above: the phase breakdown of the same pass."""
    import torch
    sleep = int(cycles_per_ms * 0.06)
    recs = []
    for _ in range(passes):
        for label, f in stack.phases(M):
            torch.cuda._sleep(sleep)
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            f()
            b.record()
            recs.append((label, a, b))
    torch.cuda.synchronize()
    out = {}
    for label, a, b in recs:
        out.setdefault(label, []).append(a.elapsed_time(b) * 1e3)
    return out


def read_roofline(nbytes=1 << 30, reps=10):
    """Plain read rate of the device: the pure-read kernel over 1 GiB,
    median of `reps` timed launches."""
    import numpy as np
    import torch

    import speculative_decoding_verification_amd as sv
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    src.fill_(3)
    props = torch.cuda.get_device_properties(0)
    sink = torch.empty(props.multi_processor_count * 8, dtype=torch.int32, device="cuda")
    for _ in range(2):
        sv.read_bandwidth(src, sink)
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        sv.read_bandwidth(src, sink)
        b.record()
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b))
    del src, sink
    ms = float(np.median(ts))
    return {"bytes": nbytes, "ms_median": round(ms, 4), "gbps": round(nbytes / (ms * 1e-3) / 1e9, 1),
            "kernel": "sv::read_kernel (sv_read_bandwidth), 16-byte streaming loads"}


def copy_calibration(nbytes=1 << 30, reps=3):
    """A plain device-to-device copy of a known size, so that a profiler
    run over this script records FETCH_SIZE / WRITE_SIZE of a kernel whose
    traffic is known exactly (the scale factor for the pass's counters)."""
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    return nbytes


# the pass kernel and what decides its work: the decomposition and the
# schedule of units (matvec.hip) set which units run where and how often an
# input is staged, so they change a launch's traffic as much as its code does
KERNEL_SOURCES = [os.path.join(ROOT, "speculative_decoding_verification_amd", "csrc", f)
                  for f in ("matvec_dev.h", "matvec_launch.h", "matvec_inst.hip", "sv_internal.h", "matvec.hip")]


def traffic_file(config, M):
    return os.path.join(ROOT, "profiles", f"pass_kernel_{config}_m{M}_traffic.md")


def kernel_source_hash():
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def recorded_traffic(config, M):
    """HBM bytes per pass launch from the committed FETCH_SIZE/WRITE_SIZE
    summary, if it was taken on the kernel sources as they are now (else
    None)."""
    try:
        text = open(traffic_file(config, M)).read()
    except OSError:
        return None
    fields = {}
    for line in text.splitlines():
        if line.startswith("- ") and ":" in line:
            k, v = line[2:].split(":", 1)
            fields[k.strip()] = v.strip().strip("`")
    if fields.get("kernel_source_sha256") != kernel_source_hash():
        return None
    if fields.get("config") != config or fields.get("M") != str(M):
        return None
    try:
        return int(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def _under_profiler():
    return any(k.startswith(("ROCPROF", "ROCPROFILER")) for k in os.environ)


def _smi():
    # rocm-smi is a launcher that replaces itself with python; under
    # rocprofv3 every child process has the GPU initialised by the
    # profiler's library first, so no smi reading is taken there
    if _under_profiler():
        return {"skipped": "under rocprofv3"}
    try:
        r = subprocess.run(["rocm-smi", "--showclocks", "--showpower", "--showtemp", "--json"],
                           capture_output=True, text=True, timeout=30)
        data = json.loads(r.stdout) if r.returncode == 0 else {}
    except (OSError, subprocess.SubprocessError, ValueError):
        return None
    card = next(iter(data.values()), {}) if isinstance(data, dict) and data else {}
    keep = {}
    for k, v in card.items():
        kl = k.lower()
        if any(s in kl for s in ("sclk", "mclk", "fclk", "power", "temperature")):
            keep[k] = v
    return keep


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def manifest_base():
    import torch
    rocm = None
    try:
        rocm = open("/opt/rocm/.info/version").read().strip()
    except OSError:
        pass
    props = torch.cuda.get_device_properties(0)
    return {"gpu": torch.cuda.get_device_name(0), "gcn_arch": getattr(props, "gcnArchName", None),
            "compute_units": props.multi_processor_count, "hbm_bytes": props.total_memory,
            "rocm": rocm, "torch": torch.__version__, "hip": torch.version.hip,
            "cpu": cpu_model(), "host_cores": len(os.sched_getaffinity(0)),
            "kernel_source_sha256": kernel_source_hash()}


def cpu_baseline(keep, shape, seed, Ms, budget_s):
    """The oracle's plain reading of the same pass (C, fp64 projections) on
    the host cores, full passes of the same weights at each M in Ms, within
    about budget_s seconds per M (at least one pass)."""
    import numpy as np

    import oracle
    import synth
    H, F = shape.hidden, shape.ffn
    layers = []
    for li in range(shape.layers):
        lw = {n: keep[(li, n)] for n in ("q", "k", "v", "o", "gate", "up", "down")}
        for g, n in (("g1", H), ("g2", H), ("g3", H), ("g4", F)):
            lw[g] = synth.rms_weight(n, seed, li, "gamma:" + g)
        layers.append(lw)
    head = None
    if shape.vocab:
        hq, hraw = keep[(-1, "head")]
        head = (hq, hraw, synth.rms_weight(H, seed, -1, "gamma:final"))
    threads = oracle.default_threads()
    out = {}
    for M in Ms:
        x = synth.activations(max(Ms), H, seed, "x0")[:M]
        times = []
        t_start = time.perf_counter()
        while True:
            t0 = time.perf_counter()
            oracle.chain_pass(layers, x, H, F, head=head, threads=threads)
            times.append(time.perf_counter() - t0)
            if time.perf_counter() - t_start >= budget_s or len(times) >= 20:
                break
        out[M] = (float(np.median(times)), len(times))
        log(f"oracle M={M}: {out[M][0]:.2f} s per pass ({len(times)} passes, {threads} threads)")
    return out, threads


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="stack27b", choices=sorted(CONFIGS))
    ap.add_argument("--m", default="1,2,3,4,5", help="M sweep (positions per pass)")
    ap.add_argument("--headline-m", type=int, default=5)
    ap.add_argument("--roofline-launches", type=int, default=10)
    ap.add_argument("--phase-breakdown", action="store_true", help="also time every phase as its own launch")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="oracle time budget per M")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-read-roofline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a 1 GiB device copy (the known-size kernel for counter scaling)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU; --gpus {args.gpus} is not supported "
              "(the verification pass of one sequence is not sharded)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import speculative_decoding_verification_amd as sv
    from speculative_decoding_verification_amd.chain import CHAIN_4B, STACK_27B, VerifyStack

    shape = CHAIN_4B if args.config == "chain4b" else STACK_27B
    seed = SEED_BASE + CONFIGS[args.config]
    Ms = [int(m) for m in args.m.split(",")]
    hm = args.headline_m if args.headline_m in Ms else Ms[-1]
    torch.cuda.set_device(0)
    sv.lib()
    manifest = manifest_base()
    manifest["smi_before"] = _smi()
    keep = {} if not args.no_cpu_baseline else None
    t0 = time.perf_counter()
    stack = VerifyStack(shape, make_weights_fn(seed, keep), max_M=max(Ms))
    torch.cuda.synchronize()
    log(f"loaded {args.config}: {shape.pass_bytes() / 1e9:.3f} GB in {time.perf_counter() - t0:.1f} s")
    import synth
    stack.x.copy_(torch.from_numpy(synth.activations(max(Ms), shape.hidden, seed, "x0")).cuda())
    drafts = synth.token_ids(max(Ms) - 1 or 1, shape.vocab, seed, "drafts")
    stack.drafts.copy_(torch.from_numpy(drafts).cuda())

    read = None if args.no_read_roofline else read_roofline()
    if read:
        log(f"pure-read kernel: {read['gbps']} GB/s")

    pass_bytes = shape.pass_bytes()
    sweep = time_sweep(stack, Ms, args.steps, args.warmup)
    t1 = next((r["ms_per_pass"] for r in sweep if r["M"] == 1), None)
    for r in sweep:
        r["gbps"] = pass_bytes / (r["ms_per_pass"] * 1e-3) / 1e9
        r["pct_hbm_peak"] = 100.0 * r["gbps"] / HBM_PEAK_GBPS
        r["pct_read_roofline"] = 100.0 * r["gbps"] / read["gbps"] if read else None
        r["positions_per_s"] = r["M"] / (r["ms_per_pass"] * 1e-3)
        r["t_over_t1"] = (r["ms_per_pass"] / t1) if t1 else None
        r["implied_tok_s"] = {str(a): expected_tokens(r["M"], a) / (r["ms_per_pass"] * 1e-3) for a in ACCEPT_RATES}
    head_row = next(r for r in sweep if r["M"] == hm)

    # dominant kernel: the one-launch pass kernel, timed live per launch
    cpm = calibrate_sleep()
    us = pass_launch_timing(stack, hm, args.roofline_launches, cpm)
    avg_us = float(np.mean(us))
    achieved = pass_bytes / (avg_us * 1e-6) / 1e9
    roofline = {
        "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
        "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": recorded_traffic(args.config, hm),
        "kernel": f"sv::pass_kernel<{hm}> (all projection phases and the head in one launch)",
        "avg_launch_us": round(avg_us, 2), "p10_us": round(float(np.percentile(us, 10)), 2),
        "p90_us": round(float(np.percentile(us, 90)), 2), "launches": len(us),
        "alg_bytes_per_launch": pass_bytes, "kernel_source_sha256": kernel_source_hash(),
    }
    log(f"roofline: pass_kernel<{hm}> {avg_us:.1f} us per launch, {achieved:.1f} GB/s")
    if args.phase_breakdown:
        per = per_phase_timing(stack, hm, 1, cpm)
        roofline["eager_phases"] = {
            k: {"avg_us": round(float(np.mean(v)), 2), "launches_per_pass": len(v),
                "gbps": round(stack.phase_bytes(k) / (np.mean(v) * 1e-6) / 1e9, 1) if stack.phase_bytes(k) else None}
            for k, v in per.items()}

    if args.copy_calibration:
        copy_calibration()
    manifest["smi_after"] = _smi()

    cpu = None
    if not args.no_cpu_baseline:
        cms = [hm] + ([1] if hm != 1 else [])
        res, threads = cpu_baseline(keep, shape, seed, cms, args.cpu_seconds)
        t_cpu, n_cpu = res[hm]
        cpu = {"value": round(pass_bytes / t_cpu / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
               "sample": f"{n_cpu} full {args.config} pass(es) at M={hm} ({shape.layers} layers + head), median "
                         f"{t_cpu:.2f} s per pass, C oracle with {threads} threads on {manifest['cpu']}",
               "positions_per_s": round(hm / t_cpu, 4),
               "per_M": {str(M): {"s_per_pass": round(t, 3), "passes": n, "gbps": round(pass_bytes / t / 1e9, 4),
                                  "positions_per_s": round(M / t, 4)} for M, (t, n) in res.items()}}
        del keep

    def rnd(v):
        if isinstance(v, float):
            return round(v, 4)
        if isinstance(v, dict):
            return {k: rnd(x) for k, x in v.items()}
        return v

    res = {
        "metric": METRIC,
        "value": round(head_row["gbps"], 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head_row["ms_per_pass"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": f"{args.config}: hidden {shape.hidden}, ffn {shape.ffn}, {shape.layers} layers "
                               f"(Q4_K q/k/o/gate/up, {'Q6_K' if shape.v_q == 14 else 'Q4_K'} v, Q6_K down), "
                               f"Q6_K head {shape.vocab}x{shape.hidden}, greedy acceptance",
                   "M": hm, "drafts": hm - 1, "bytes_per_pass": pass_bytes},
        "pct_hbm_peak": round(head_row["pct_hbm_peak"], 2),
        "pct_read_roofline": round(head_row["pct_read_roofline"], 2) if read else None,
        "read_roofline": read,
        "growth_t5_over_t1": next((round(r["t_over_t1"], 4) for r in sweep if r["M"] == 5 and r["t_over_t1"]), None),
        "positions_per_s": round(head_row["positions_per_s"], 1),
        "sweep": [rnd(r) for r in sweep],
        "roofline": roofline,
        "cpu_baseline": cpu,
        "manifest": manifest,
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
