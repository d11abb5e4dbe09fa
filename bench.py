#!/usr/bin/env python3
"""Benchmark of the diagonal-precision scan forward on one MI355X.

Default workload: B=2, H=16, T=16384, d_k=d_v=128, bf16 inputs, fp32 state
and output: the largest single-GPU diagonal configuration, a long sequence
that the plan cuts into segments (segment composites + ordered carry + the
main pass).  A step is one kdn_diag_scan_fwd call over that batch, inputs
already resident in HBM.  Prints one JSON line with tokens/s (tokens = B*T
positions, all heads) from the wall clock, the roofline of the dominant
kernel (the main pass, timed live by HIP events that the library records
around that launch on the launch stream), the whole call's event times, the
fp64 CPU oracle timed on a bounded sample of the same workload, and the
error of the GPU output on that sample against the oracle.

Other workloads (--workload) print the same fields for the short-sequence
batch (B=8, H=16, T=2048), Palimpsa-M gating, the packed variable-length
batch (also a skewed one whose long sequence runs in segments) and its gradient, the backward
pass, the process-noise variant, the decode step and the
isotropic scan; they are not the headline line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, GB/s
# MI355X fp32 vector peak: 256 CU x 128 FMA lanes/clk x 2 flop x 2.4 GHz.  Plain (non-packed)
# v_fmac_f32 measured on the device sustains ~86 lane-instr/clk/CU (106 TFLOP/s), above a
# one-wave64-op-per-4-clocks model (78.6), so the published figure is the ceiling used.
# MI355X lists the same 157.3 TFLOP/s for dense fp32 MFMA.
PEAK_FP32_VALU_TFLOPS = 157.3
DIAG_FLOPS_PER_ENTRY_STEP = 11   # I update 4, eta update 3, reciprocal+multiply 2, read-out 2
ISO_FLOPS_PER_ENTRY_STEP = 5     # mean update 3, read-out 2
# gradient: state recurrences 4, mu = eta / I 2, adjoint updates 4 (g = q dout, g / I, g mu / I),
# dq 2, dk 4, dbeta / dv row sums 4, dalpha 4
BWD_FLOPS_PER_ENTRY_STEP = 24
# Diagonal KDN (residual write): predict 3 (a^2 sig + p, a mu), the two sums over j 4,
# mean write 3 (sp gain, fma), projected variance 5 (beta k^2, fma, reciprocal, multiply),
# read-out 2
NOISE_FLOPS_PER_ENTRY_STEP = 17


def _args():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # about 0.6 s of timed and warm-up work on the default workload: enough for
    # the clocks to settle, far inside a minute
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default="diag_b2h16t16384d128_bf16")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target CPU time of the oracle sample")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle leg")
    ap.add_argument("--segments", type=int, default=0,
                    help="packed batches: 0 splits sequences longer than a fair share, 1 never")
    return ap.parse_args()


def _traffic(kernel_file: str, profile_json: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, or None if the
    kernel source changed since they were taken."""
    path = os.path.join(ROOT, "profiles", profile_json)
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    src = open(os.path.join(ROOT, "bayesian_memory_scan_amd", "csrc", kernel_file), "rb").read()
    if rec.get("source_sha256") != hashlib.sha256(src).hexdigest():
        return None
    return rec.get("traffic_bytes_per_launch")


def _up(x, torch, dev):
    import numpy as np
    x = np.ascontiguousarray(x)
    return torch.from_numpy(x.view(np.int16) if x.dtype == np.uint16 else x).to(dev)


def _stats(ms):
    v = sorted(ms)
    n = len(v)
    med = v[n // 2] if n % 2 else 0.5 * (v[n // 2 - 1] + v[n // 2])
    return {"avg": sum(v) / n, "median": med, "min": v[0], "max": v[-1]}


class Timing:
    """Wall clock of the timed steps, per-step HIP events around the whole
    call, and (for calls that take them) per-step events that the library
    records right before and after its main pass, all on the current stream
    (the stream every launch goes to)."""

    def __init__(self, wall, call, main):
        self.wall, self.call, self.main = wall, call, main

    def kernel(self):
        """Event statistics of the dominant kernel: the main pass where the
        call records it, else the whole call."""
        return self.main or self.call

    def fields(self):
        k = self.kernel()
        out = {"launch_ms_avg": k["avg"], "launch_ms_median": k["median"], "launch_ms_min": k["min"],
               "call_ms_avg": self.call["avg"], "call_ms_median": self.call["median"],
               "call_ms_min": self.call["min"],
               "timed_kernel": "main pass" if self.main else "whole call"}
        return out


def _time_steps(torch, step, steps, warmup, main_events=False):
    """Warmup, then `steps` timed steps.  step(timing) runs one call; with
    main_events it passes the call a pair of events to record around its main
    pass, else None."""
    for _ in range(warmup):
        step(None)
    torch.cuda.synchronize()
    mk = lambda: torch.cuda.Event(enable_timing=True)
    ev = [(mk(), mk()) for _ in range(steps)]
    mev = [(mk(), mk()) for _ in range(steps)] if main_events else [None] * steps
    if main_events:   # create the library's events before the clock starts
        for a, b in mev:
            a.record()
            b.record()
        torch.cuda.synchronize()
    t0 = time.perf_counter()
    for (e0, e1), m in zip(ev, mev):
        e0.record()
        step(m)
        e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    call = _stats([e0.elapsed_time(e1) for e0, e1 in ev])
    main = _stats([a.elapsed_time(b) for a, b in mev]) if main_events else None
    return Timing(wall, call, main)


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _cpu_threads():
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


def cpu_baseline_diag(inp, spec, target_s):
    """fp64 oracle on whole heads of the same workload; tokens/s scaled to all H heads."""
    import oracle
    threads = _cpu_threads()
    heads_all = [(b, h) for b in range(spec.B) for h in range(spec.H)]
    # calibrate on one head, then size the sample to about target_s of wall time
    with oracle.Timer() as t1:
        oracle.diag_scan(inp, heads=heads_all[:1], threads=1)
    n = max(1, min(len(heads_all), int(target_s / max(t1.seconds, 1e-3) * threads)))
    heads = heads_all[:n]
    with oracle.Timer() as t:
        ref = oracle.diag_scan(inp, heads=heads, threads=threads)
    T = spec.prefix + spec.T
    tokens = n * T / spec.H
    return {"value": tokens / t.seconds, "unit": "tokens/s", "cores": min(threads, n),
            "kind": "oracle", "cpu_model": _cpu_model(),
            "sample": f"{n} of {len(heads_all)} heads x {T} tokens, fp64 sequential oracle, "
                      f"{t.seconds:.1f} s wall, heads in parallel on {min(threads, n)} threads"}, ref


def parity_report(o_gpu, ref, what="o"):
    """The GPU output of the sampled heads against the oracle's: the acceptance
    measure max |o - o_ref| / s_ref (s_ref = sum_j |q_j mu_ref[j,i]|, which
    bounds |o_ref|), and the plain relative error over the elements with
    |o_ref| >= 1e-2 rms(o_ref), where it is well posed."""
    import numpy as np
    worst_s, worst_rel, n_large, n_all, rels = 0.0, 0.0, 0, 0, []
    for (b, h), r in ref.items():
        og = o_gpu[b, h].astype(np.float64)
        oref = np.asarray(r["o"], dtype=np.float64)
        err = np.abs(og - oref)
        worst_s = max(worst_s, float(np.max(err / (np.asarray(r["s"]) + 1e-30))))
        rms = float(np.sqrt(np.mean(oref * oref)))
        big = np.abs(oref) >= 1e-2 * rms
        if big.any():
            rel = err[big] / np.abs(oref[big])
            worst_rel = max(worst_rel, float(np.max(rel)))
            rels.append(rel)
        n_large += int(big.sum())
        n_all += oref.size
    allrel = np.concatenate(rels) if rels else np.zeros(1)
    return {"of": what, "heads": len(ref), "max_err_over_s_ref": worst_s,
            "acceptance": "max_err_over_s_ref <= 1e-4",
            "max_rel_err_large": worst_rel, "median_rel_err_large": float(np.median(allrel)),
            "p999_rel_err_large": float(np.quantile(allrel, 0.999)),
            "large_elements": n_large, "elements": n_all}


def cpu_baseline_bwd(inp, grads, spec, target_s):
    """fp64 oracle gradient on whole heads of the same workload; tokens/s scaled to all heads."""
    import oracle
    threads = _cpu_threads()
    heads_all = [(b, h) for b in range(spec.B) for h in range(spec.H)]
    with oracle.Timer() as t1:
        oracle.diag_scan_bwd(inp, grads["d_o"], heads=heads_all[:1], threads=1)
    # whole rounds of `threads` heads, each round taking about t1
    rounds = max(1, int(target_s / max(t1.seconds, 1e-3)))
    n = max(1, min(len(heads_all), rounds * threads))
    with oracle.Timer() as t:
        oracle.diag_scan_bwd(inp, grads["d_o"], heads=heads_all[:n], threads=threads)
    return {"value": n * spec.T / spec.H / t.seconds, "unit": "tokens/s",
            "cores": min(threads, n), "kind": "oracle", "cpu_model": _cpu_model(),
            "sample": f"{n} of {len(heads_all)} heads x {spec.T} tokens, fp64 sequential oracle "
                      f"gradient, {t.seconds:.1f} s wall, heads in parallel on {min(threads, n)} threads"}


def _varlen_seq(inp, cu, s):
    """Sequence s of a packed batch as a one-row batch (the oracle's input form)."""
    import numpy as np
    sub = dict(inp)
    for n in ("q", "k", "v", "beta", "d"):
        if inp.get(n) is not None:
            sub[n] = np.ascontiguousarray(inp[n][:, :, cu[s]:cu[s + 1]])
    return sub


def cpu_baseline_varlen_bwd(inp, d_o, spec, target_s):
    """fp64 oracle gradient of the packed batch, sequence by sequence (every
    head of a sequence in parallel), over a prefix of the sequences sized to
    about target_s; tokens/s over the prefix's packed tokens."""
    import oracle
    threads = _cpu_threads()
    cu = [int(x) for x in inp["cu_seqlens"]]
    heads = [(0, h) for h in range(spec.H)]

    def run(n):
        for s in range(n):
            oracle.diag_scan_bwd(_varlen_seq(inp, cu, s), d_o[:, :, cu[s]:cu[s + 1]], heads=heads,
                                 threads=threads)

    with oracle.Timer() as t1:
        run(1)
    per_token = t1.seconds / max(1, cu[1])
    n = 1
    while n < spec.N and cu[n + 1] * per_token < target_s:
        n += 1
    with oracle.Timer() as t:
        run(n)
    return {"value": cu[n] / t.seconds, "unit": "tokens/s", "cores": min(threads, spec.H),
            "kind": "oracle", "cpu_model": _cpu_model(),
            "sample": f"first {n} of {spec.N} sequences ({cu[n]} of {spec.total_T} packed tokens) x "
                      f"{spec.H} heads, fp64 sequential oracle gradient, {t.seconds:.1f} s wall, "
                      f"heads of a sequence in parallel"}


def cpu_baseline_varlen(inp, spec, target_s):
    """fp64 oracle over the packed batch's (sequence, head) runs; a prefix of
    the sequences sized to about target_s, scaled by its share of tokens."""
    import oracle
    threads = _cpu_threads()
    cu = [int(x) for x in inp["cu_seqlens"]]
    with oracle.Timer() as t1:
        oracle.diag_scan_varlen(inp, cu[:2], threads=1)
    per_token = t1.seconds / max(1, cu[1]) / spec.H * 1.0
    n = 1
    while n < spec.N and (cu[n + 1] * spec.H * per_token) / threads < target_s:
        n += 1
    with oracle.Timer() as t:
        oracle.diag_scan_varlen(inp, cu[:n + 1], threads=threads)
    return {"value": cu[n] / t.seconds, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "cpu_model": _cpu_model(),
            "sample": f"first {n} of {spec.N} sequences ({cu[n]} of {spec.total_T} packed tokens) x "
                      f"{spec.H} heads, fp64 sequential oracle, {t.seconds:.1f} s wall"}


def cpu_baseline_noise(inp, spec, target_s):
    import oracle
    threads = _cpu_threads()
    heads_all = [(b, h) for b in range(spec.B) for h in range(spec.H)]
    with oracle.Timer() as t1:
        oracle.diag_noise_scan(inp, heads=heads_all[:1], threads=1)
    n = max(1, min(len(heads_all), int(target_s / max(t1.seconds, 1e-3) * threads)))
    with oracle.Timer() as t:
        oracle.diag_noise_scan(inp, heads=heads_all[:n], threads=threads)
    return {"value": n * spec.T / spec.H / t.seconds, "unit": "tokens/s",
            "cores": min(threads, n), "kind": "oracle", "cpu_model": _cpu_model(),
            "sample": f"{n} of {len(heads_all)} heads x {spec.T} tokens, fp64 sequential oracle, "
                      f"{t.seconds:.1f} s wall, heads in parallel on {min(threads, n)} threads"}


def cpu_baseline_iso(inp, spec, target_s):
    import oracle
    threads = _cpu_threads()
    heads_all = [(b, h) for b in range(spec.B) for h in range(spec.H)]
    with oracle.Timer() as t1:
        oracle.iso_scan(inp, heads=heads_all[:1], threads=1)
    n = max(1, min(len(heads_all), int(target_s / max(t1.seconds, 1e-3) * threads)))
    with oracle.Timer() as t:
        oracle.iso_scan(inp, heads=heads_all[:n], threads=threads)
    return {"value": n * spec.T / spec.H / t.seconds, "unit": "tokens/s",
            "cores": min(threads, n), "kind": "oracle", "cpu_model": _cpu_model(),
            "sample": f"{n} of {len(heads_all)} heads x {spec.T} tokens, fp64 sequential oracle, "
                      f"{t.seconds:.1f} s wall"}


def main():
    a = _args()
    if a.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {a.gpus}); the scans shard over "
              "(batch, head) with no communication, so there is no multi-GPU step to time.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from bayesian_memory_scan_amd import kdnscan as kdn
    from bayesian_memory_scan_amd import synth

    dev = torch.device("cuda:0")
    spec = synth.workload(a.workload) if a.workload in synth.WORKLOADS else None
    out = {"metric": "tokens/s per MI355X, diag-precision scan fwd; % of HBM/FP32 roofline",
           "n_gpus": 1, "steps": a.steps, "warmup": a.warmup, "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic"}

    if a.workload.startswith("diag_"):
        inp = synth.diag_inputs(spec)
        x = {n: _up(inp[n], torch, dev) for n in ("q", "k", "v", "beta", "d", "A")}
        o = torch.empty((spec.B, spec.H, spec.T, spec.d_v), dtype=torch.float32, device=dev)
        st = torch.empty((2, spec.B, spec.H, spec.d_k, spec.d_v), dtype=torch.float32, device=dev)
        _, S, _, _ = kdn.kdn_diag_plan(spec.B, spec.H, spec.T, spec.d_k, spec.d_v)

        def step(m):
            kdn.kdn_diag_scan_fwd(x["q"], x["k"], x["v"], x["beta"], x["d"], x["A"],
                                  spec.I_prior, o=o, I_T=st[0], mu_T=st[1], timing=m)

        tm = _time_steps(torch, step, a.steps, a.warmup, main_events=True)
        wall, ev_ms = tm.wall, tm.kernel()["avg"]
        tokens = spec.B * spec.T
        flops = DIAG_FLOPS_PER_ENTRY_STEP * spec.B * spec.H * spec.T * spec.d_k * spec.d_v
        achieved = flops / (ev_ms * 1e-3) / 1e12
        out.update({
            "value": tokens / (wall / a.steps), "unit": "tokens/s",
            "ms_per_step": wall / a.steps * 1e3,
            "config": {"workload": spec.name, "B": spec.B, "H": spec.H, "T": spec.T,
                       "d_k": spec.d_k, "d_v": spec.d_v, "inputs": spec.dtype, "state": "fp32",
                       "segments": S, "parallelism": "single GPU"},
            "roofline": {"bound": "alu", "achieved": achieved, "peak": PEAK_FP32_VALU_TFLOPS,
                         "unit": "TFLOP/s", "frac": achieved / PEAK_FP32_VALU_TFLOPS,
                         "traffic": _traffic("diag_scan.hip", f"traffic_{spec.name}.json"),
                         **tm.fields(),
                         "kernels_per_step": 2 if S == 1 else 4,
                         "note": "achieved: algorithmic flops of every entry-step over the main "
                                 "pass's own event time; call_ms_*: the whole call (frame "
                                 "scalars + main pass, + composite and carry passes when "
                                 "segments > 1)"},
        })
        if not a.no_cpu:
            out["cpu_baseline"], ref = cpu_baseline_diag(inp, spec, a.cpu_seconds)
            out["parity"] = parity_report(o.cpu().numpy(), ref)
    elif a.workload.startswith("diagm_"):
        # Palimpsa-M gating: the step gate d_t is also the input gate (no beta input)
        inp = synth.diag_inputs(spec)
        inp["beta"] = None
        x = {n: _up(inp[n], torch, dev) for n in ("q", "k", "v", "d", "A")}
        o = torch.empty((spec.B, spec.H, spec.T, spec.d_v), dtype=torch.float32, device=dev)
        st = torch.empty((2, spec.B, spec.H, spec.d_k, spec.d_v), dtype=torch.float32, device=dev)

        def step(m):
            kdn.kdn_diag_scan_fwd(x["q"], x["k"], x["v"], None, x["d"], x["A"], spec.I_prior,
                                  o=o, I_T=st[0], mu_T=st[1], timing=m)

        tm = _time_steps(torch, step, a.steps, a.warmup, main_events=True)
        wall, ev_ms = tm.wall, tm.kernel()["avg"]
        flops = DIAG_FLOPS_PER_ENTRY_STEP * spec.B * spec.H * spec.T * spec.d_k * spec.d_v
        achieved = flops / (ev_ms * 1e-3) / 1e12
        out.update({
            "metric": "tokens/s per MI355X, diag-precision scan fwd under Palimpsa-M gating",
            "value": spec.B * spec.T / (wall / a.steps), "unit": "tokens/s",
            "ms_per_step": wall / a.steps * 1e3,
            "config": {"workload": spec.name, "B": spec.B, "H": spec.H, "T": spec.T,
                       "d_k": spec.d_k, "d_v": spec.d_v, "inputs": spec.dtype,
                       "gating": "beta_t = d_t", "parallelism": "single GPU"},
            "roofline": {"bound": "alu", "achieved": achieved, "peak": PEAK_FP32_VALU_TFLOPS,
                         "unit": "TFLOP/s", "frac": achieved / PEAK_FP32_VALU_TFLOPS,
                         "traffic": _traffic("diag_scan.hip", f"traffic_{spec.name}.json"),
                         **tm.fields()},
        })
        if not a.no_cpu:
            out["cpu_baseline"], ref = cpu_baseline_diag(inp, spec, a.cpu_seconds)
            out["parity"] = parity_report(o.cpu().numpy(), ref)
    elif a.workload.startswith(("varlen_", "varlenskew_")):
        inp = synth.varlen_inputs(spec)
        x = {n: _up(inp[n][0], torch, dev) for n in ("q", "k", "v", "beta", "d")}
        A = _up(inp["A"], torch, dev)
        cu = torch.from_numpy(inp["cu_seqlens"]).to(dev)
        seg_tokens = kdn.kdn_diag_varlen_plan(spec.N, spec.H, spec.total_T, spec.d_k, spec.d_v,
                                              a.segments)[0]

        def step(m):
            kdn.kdn_diag_scan_varlen_fwd(x["q"], x["k"], x["v"], x["beta"], x["d"], A,
                                         spec.I_prior, cu, segments=a.segments, timing=m)

        tm = _time_steps(torch, step, a.steps, a.warmup, main_events=True)
        wall, ev_ms = tm.wall, tm.kernel()["avg"]
        flops = DIAG_FLOPS_PER_ENTRY_STEP * spec.H * spec.total_T * spec.d_k * spec.d_v
        achieved = flops / (ev_ms * 1e-3) / 1e12
        lens = [int(b - a_) for a_, b in zip(inp["cu_seqlens"][:-1], inp["cu_seqlens"][1:])]
        out.update({
            "metric": "tokens/s per MI355X, diag-precision scan fwd over a packed variable-length batch",
            "value": spec.total_T / (wall / a.steps), "unit": "tokens/s",
            "ms_per_step": wall / a.steps * 1e3,
            "config": {"workload": spec.name, "sequences": spec.N, "H": spec.H,
                       "packed_T": spec.total_T, "d_k": spec.d_k, "d_v": spec.d_v,
                       "inputs": spec.dtype, "length_min": min(lens), "length_max": max(lens),
                       "segment_tokens": seg_tokens, "parallelism": "single GPU"},
            "roofline": {"bound": "alu", "achieved": achieved, "peak": PEAK_FP32_VALU_TFLOPS,
                         "unit": "TFLOP/s", "frac": achieved / PEAK_FP32_VALU_TFLOPS,
                         "traffic": _traffic("diag_scan.hip", f"traffic_{spec.name}.json"),
                         **tm.fields()},
        })
        if not a.no_cpu:
            out["cpu_baseline"] = cpu_baseline_varlen(inp, spec, a.cpu_seconds)
    elif a.workload.startswith("noise_"):
        inp = synth.noise_inputs(spec)
        x = {n: _up(inp[n], torch, dev) for n in ("q", "k", "v", "beta", "a", "p")}

        def step(_m):
            kdn.kdn_diag_noise_scan_fwd(x["q"], x["k"], x["v"], x["beta"], x["a"], x["p"])

        tm = _time_steps(torch, step, a.steps, a.warmup)
        wall, ev_ms = tm.wall, tm.kernel()["avg"]
        flops = NOISE_FLOPS_PER_ENTRY_STEP * spec.B * spec.H * spec.T * spec.d_k * spec.d_v
        achieved = flops / (ev_ms * 1e-3) / 1e12
        out.update({
            "metric": "tokens/s per MI355X, diagonal KDN with process noise, forward",
            "value": spec.B * spec.T / (wall / a.steps), "unit": "tokens/s",
            "ms_per_step": wall / a.steps * 1e3,
            "config": {"workload": spec.name, "B": spec.B, "H": spec.H, "T": spec.T,
                       "d_k": spec.d_k, "d_v": spec.d_v, "inputs": spec.dtype, "state": "fp32",
                       "parallelism": "single GPU"},
            "roofline": {"bound": "alu", "achieved": achieved, "peak": PEAK_FP32_VALU_TFLOPS,
                         "unit": "TFLOP/s", "frac": achieved / PEAK_FP32_VALU_TFLOPS,
                         "traffic": _traffic("diag_noise.hip", f"traffic_{spec.name}.json"),
                         **tm.fields()},
        })
        if not a.no_cpu:
            out["cpu_baseline"] = cpu_baseline_noise(inp, spec, a.cpu_seconds)
    elif a.workload.startswith("bwd_"):
        inp = synth.diag_inputs(spec)
        grads = synth.grad_inputs(spec, final_state=False)
        x = {n: _up(inp[n], torch, dev) for n in ("q", "k", "v", "beta", "d", "A")}
        d_o = _up(grads["d_o"], torch, dev)

        def step(_m):
            kdn.kdn_diag_scan_bwd(x["q"], x["k"], x["v"], x["beta"], x["d"], x["A"],
                                  spec.I_prior, d_o)

        tm = _time_steps(torch, step, a.steps, a.warmup)
        wall, ev_ms = tm.wall, tm.kernel()["avg"]
        flops = BWD_FLOPS_PER_ENTRY_STEP * spec.B * spec.H * spec.T * spec.d_k * spec.d_v
        achieved = flops / (ev_ms * 1e-3) / 1e12
        out.update({
            "metric": "tokens/s per MI355X, diag-precision scan backward (gradient of all inputs)",
            "value": spec.B * spec.T / (wall / a.steps), "unit": "tokens/s",
            "ms_per_step": wall / a.steps * 1e3,
            "config": {"workload": spec.name, "B": spec.B, "H": spec.H, "T": spec.T,
                       "d_k": spec.d_k, "d_v": spec.d_v, "inputs": spec.dtype,
                       "gradients": "fp32, loss on o only",
                       "segments": kdn.kdn_diag_plan(spec.B, spec.H, spec.T, spec.d_k, spec.d_v)[1],
                       "parallelism": "single GPU"},
            "roofline": {"bound": "alu", "achieved": achieved, "peak": PEAK_FP32_VALU_TFLOPS,
                         "unit": "TFLOP/s", "frac": achieved / PEAK_FP32_VALU_TFLOPS,
                         "traffic": _traffic("diag_bwd_kernels.h", f"traffic_{spec.name}.json"),
                         **tm.fields(),
                         "note": "events bracket the whole call: frame scalars, checkpoints, "
                                 "reverse pass and finishing sums; traffic is the reverse pass"},
        })
        if not a.no_cpu:
            out["cpu_baseline"] = cpu_baseline_bwd(inp, grads, spec, a.cpu_seconds)
    elif a.workload.startswith(("varlenbwd_", "varlenskewbwd_")):
        inp = synth.varlen_inputs(spec)
        d_o_h = synth.varlen_grad_inputs(spec)["d_o"]
        x = {n: _up(inp[n][0], torch, dev) for n in ("q", "k", "v", "beta", "d")}
        A = _up(inp["A"], torch, dev)
        cu = torch.from_numpy(inp["cu_seqlens"]).to(dev)
        d_o = _up(d_o_h[0], torch, dev)

        def step(_m):
            kdn.kdn_diag_scan_varlen_bwd(x["q"], x["k"], x["v"], x["beta"], x["d"], A,
                                         spec.I_prior, cu, d_o)

        tm = _time_steps(torch, step, a.steps, a.warmup)
        wall, ev_ms = tm.wall, tm.kernel()["avg"]
        flops = BWD_FLOPS_PER_ENTRY_STEP * spec.H * spec.total_T * spec.d_k * spec.d_v
        achieved = flops / (ev_ms * 1e-3) / 1e12
        lens = [int(b - a_) for a_, b in zip(inp["cu_seqlens"][:-1], inp["cu_seqlens"][1:])]
        out.update({
            "metric": "tokens/s per MI355X, diag-precision scan backward over a packed "
                      "variable-length batch",
            "value": spec.total_T / (wall / a.steps), "unit": "tokens/s",
            "ms_per_step": wall / a.steps * 1e3,
            "config": {"workload": spec.name, "sequences": spec.N, "H": spec.H,
                       "packed_T": spec.total_T, "d_k": spec.d_k, "d_v": spec.d_v,
                       "inputs": spec.dtype, "length_min": min(lens), "length_max": max(lens),
                       "gradients": "fp32, loss on o only", "parallelism": "single GPU"},
            "roofline": {"bound": "alu", "achieved": achieved, "peak": PEAK_FP32_VALU_TFLOPS,
                         "unit": "TFLOP/s", "frac": achieved / PEAK_FP32_VALU_TFLOPS,
                         "traffic": _traffic("diag_bwd_kernels.h", f"traffic_{spec.name}.json"),
                         **tm.fields(),
                         "note": "events bracket the whole call: sequence plan, frame scalars, "
                                 "checkpoints, reverse pass and finishing sums"},
        })
        if not a.no_cpu:
            out["cpu_baseline"] = cpu_baseline_varlen_bwd(inp, d_o_h, spec, a.cpu_seconds)
    elif a.workload.startswith("decode_"):
        inp = synth.diag_inputs(spec)
        P = spec.prefix
        x = {n: _up(inp[n][:, :, :P], torch, dev) for n in ("q", "k", "v", "beta", "d")}
        A = _up(inp["A"], torch, dev)
        _, I, mu = kdn.kdn_diag_scan_fwd(x["q"], x["k"], x["v"], x["beta"], x["d"], A,
                                         spec.I_prior)
        del x
        y = {n: _up(inp[n][:, :, P], torch, dev) for n in ("q", "k", "v", "beta", "d")}
        o = torch.empty((spec.B, spec.H, spec.d_v), dtype=torch.float32, device=dev)

        def step(_m):
            kdn.kdn_decode_step(y["q"], y["k"], y["v"], y["beta"], y["d"], A, spec.I_prior,
                                I, mu, o=o)

        tm = _time_steps(torch, step, a.steps, a.warmup)
        wall, ev_ms = tm.wall, tm.kernel()["avg"]
        BH = spec.B * spec.H
        nbytes = BH * (4 * 4 * spec.d_k * spec.d_v + 2 * (2 * spec.d_k + 2 * spec.d_v + 1)
                       + 4 * spec.d_v)
        achieved = nbytes / (ev_ms * 1e-3) / 1e9
        out.update({
            "metric": "tokens/s per MI355X, diag-precision decode step; % of HBM roofline",
            "value": spec.B / (wall / a.steps), "unit": "tokens/s",
            "ms_per_step": wall / a.steps * 1e3,
            "config": {"workload": spec.name, "B": spec.B, "H": spec.H, "d_k": spec.d_k,
                       "d_v": spec.d_v, "state": "fp32, in place", "prefix": P},
            "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": achieved / PEAK_HBM_GBS,
                         "traffic": _traffic("decode.hip", f"traffic_{spec.name}.json"),
                         **tm.fields()},
        })
        if not a.no_cpu:
            out["cpu_baseline"], _ = cpu_baseline_diag(inp, spec.with_(B=8), a.cpu_seconds)
    elif a.workload.startswith("iso_"):
        inp = synth.iso_inputs(spec)
        x = {n: _up(inp[n], torch, dev) for n in ("a", "p", "Lambda", "q", "k", "v", "lambda0")}

        def step(m):
            kdn.kdn_mobius_precision_scan(x["a"], x["p"], x["Lambda"], x["lambda0"], x["q"],
                                          x["k"], x["v"], timing=m)

        tm = _time_steps(torch, step, a.steps, a.warmup, main_events=True)
        wall, ev_ms = tm.wall, tm.kernel()["avg"]
        flops = ISO_FLOPS_PER_ENTRY_STEP * spec.B * spec.H * spec.T * spec.d_k * spec.d_v
        achieved = flops / (ev_ms * 1e-3) / 1e12
        out.update({
            "metric": "tokens/s per MI355X, isotropic Mobius scan + gated mean scan",
            "value": spec.B * spec.T / (wall / a.steps), "unit": "tokens/s",
            "ms_per_step": wall / a.steps * 1e3,
            "config": {"workload": spec.name, "B": spec.B, "H": spec.H, "T": spec.T,
                       "d_k": spec.d_k, "d_v": spec.d_v, "inputs": "fp32"},
            # the dominant kernel (the chunked mean scan) runs on fp32 MFMA, whose
            # MI355X peak equals the fp32 vector peak
            "roofline": {"bound": "mfma", "achieved": achieved, "peak": PEAK_FP32_VALU_TFLOPS,
                         "unit": "TFLOP/s", "frac": achieved / PEAK_FP32_VALU_TFLOPS,
                         "traffic": _traffic("iso_scan.hip", f"traffic_{spec.name}.json"),
                         **tm.fields(),
                         "note": "achieved: algorithmic flops over the main mean-scan pass's "
                                 "own event time; call_ms_*: the whole call (Mobius scan, "
                                 "segment composites, carry and main pass)"},
        })
        if not a.no_cpu:
            out["cpu_baseline"] = cpu_baseline_iso(inp, spec, a.cpu_seconds)
    elif a.workload == "copy_1gib":
        # plain device-to-device copy of 1 GiB: the reference for HBM counters
        # (read 1 GiB + write 1 GiB per step) and for attainable copy bandwidth
        n = 1 << 28
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)

        def step(_m):
            dst.copy_(src)

        tm = _time_steps(torch, step, a.steps, a.warmup)
        wall, ev_ms = tm.wall, tm.kernel()["avg"]
        gbs = 2 * 4 * n / (ev_ms * 1e-3) / 1e9
        out.update({"metric": "copy GB/s (read + write)", "value": gbs, "unit": "GB/s",
                    "ms_per_step": wall / a.steps * 1e3,
                    "config": {"workload": "copy_1gib", "bytes_read": 4 * n, "bytes_written": 4 * n},
                    "roofline": {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                 "frac": gbs / PEAK_HBM_GBS, "traffic": None,
                                 **tm.fields()}})
    else:
        raise SystemExit(f"unknown workload {a.workload}")

    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
