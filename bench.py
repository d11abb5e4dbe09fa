#!/usr/bin/env python3
"""Benchmark of the diagonal-precision scan forward on one MI355X.

Default workload: B=8, H=16, T=2048, d_k=d_v=128, bf16 inputs, fp32 state
and output (a 760M-class layer shape).  A step is one kdn_diag_scan_fwd call
over that batch, inputs already resident in HBM.  Prints one JSON line with
tokens/s (tokens = B*T positions, all heads), the roofline of the dominant
kernel (timed live with HIP events on the launch stream) and the fp64 CPU
oracle timed on a bounded sample of the same workload.

Other workloads (--workload) print the same fields for the decode step and
the isotropic scan; they are not the headline line.
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
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="diag_b8h16t2048d128_bf16")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target CPU time of the oracle sample")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle leg")
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


def _time_steps(torch, step, steps, warmup):
    """Warmup, then `steps` timed steps; wall clock plus per-step HIP events on
    the current stream (the stream every launch goes to)."""
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    t0 = time.perf_counter()
    for e0, e1 in ev:
        e0.record()
        step()
        e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = [e0.elapsed_time(e1) for e0, e1 in ev]
    return wall, sum(per) / len(per), min(per)


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
        oracle.diag_scan(inp, heads=heads, threads=threads)
    T = spec.prefix + spec.T
    tokens = n * T / spec.H
    return {"value": tokens / t.seconds, "unit": "tokens/s", "cores": min(threads, n),
            "kind": "oracle",
            "sample": f"{n} of {len(heads_all)} heads x {T} tokens, fp64 sequential oracle, "
                      f"{t.seconds:.1f} s wall, heads in parallel on {min(threads, n)} threads"}


def cpu_baseline_bwd(inp, grads, spec, target_s):
    """fp64 oracle gradient on whole heads of the same workload; tokens/s scaled to all heads."""
    import oracle
    threads = _cpu_threads()
    heads_all = [(b, h) for b in range(spec.B) for h in range(spec.H)]
    with oracle.Timer() as t1:
        oracle.diag_scan_bwd(inp, grads["d_o"], heads=heads_all[:1], threads=1)
    n = max(1, min(len(heads_all), int(target_s / max(t1.seconds, 1e-3) * threads)))
    with oracle.Timer() as t:
        oracle.diag_scan_bwd(inp, grads["d_o"], heads=heads_all[:n], threads=threads)
    return {"value": n * spec.T / spec.H / t.seconds, "unit": "tokens/s",
            "cores": min(threads, n), "kind": "oracle",
            "sample": f"{n} of {len(heads_all)} heads x {spec.T} tokens, fp64 sequential oracle "
                      f"gradient, {t.seconds:.1f} s wall, heads in parallel on {min(threads, n)} threads"}


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
            "cores": min(threads, n), "kind": "oracle",
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
            "cores": min(threads, n), "kind": "oracle",
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

        def step():
            kdn.kdn_diag_scan_fwd(x["q"], x["k"], x["v"], x["beta"], x["d"], x["A"],
                                  spec.I_prior, o=o, I_T=st[0], mu_T=st[1])

        wall, ev_ms, ev_min = _time_steps(torch, step, a.steps, a.warmup)
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
                         "launch_ms_avg": ev_ms, "launch_ms_min": ev_min,
                         "kernels_per_step": 2 if S == 1 else 4,
                         "note": "events bracket the whole call: prep (<1 %) + main pass "
                                 "(+ composite and carry passes when segments > 1)"},
        })
        if not a.no_cpu:
            out["cpu_baseline"] = cpu_baseline_diag(inp, spec, a.cpu_seconds)
    elif a.workload.startswith("diagm_"):
        # Palimpsa-M gating: the step gate d_t is also the input gate (no beta input)
        inp = synth.diag_inputs(spec)
        inp["beta"] = None
        x = {n: _up(inp[n], torch, dev) for n in ("q", "k", "v", "d", "A")}
        o = torch.empty((spec.B, spec.H, spec.T, spec.d_v), dtype=torch.float32, device=dev)
        st = torch.empty((2, spec.B, spec.H, spec.d_k, spec.d_v), dtype=torch.float32, device=dev)

        def step():
            kdn.kdn_diag_scan_fwd(x["q"], x["k"], x["v"], None, x["d"], x["A"], spec.I_prior,
                                  o=o, I_T=st[0], mu_T=st[1])

        wall, ev_ms, ev_min = _time_steps(torch, step, a.steps, a.warmup)
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
                         "launch_ms_avg": ev_ms, "launch_ms_min": ev_min},
        })
        if not a.no_cpu:
            out["cpu_baseline"] = cpu_baseline_diag(inp, spec, a.cpu_seconds)
    elif a.workload.startswith("varlen_"):
        inp = synth.varlen_inputs(spec)
        x = {n: _up(inp[n][0], torch, dev) for n in ("q", "k", "v", "beta", "d")}
        A = _up(inp["A"], torch, dev)
        cu = torch.from_numpy(inp["cu_seqlens"]).to(dev)

        def step():
            kdn.kdn_diag_scan_varlen_fwd(x["q"], x["k"], x["v"], x["beta"], x["d"], A,
                                         spec.I_prior, cu)

        wall, ev_ms, ev_min = _time_steps(torch, step, a.steps, a.warmup)
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
                       "parallelism": "single GPU"},
            "roofline": {"bound": "alu", "achieved": achieved, "peak": PEAK_FP32_VALU_TFLOPS,
                         "unit": "TFLOP/s", "frac": achieved / PEAK_FP32_VALU_TFLOPS,
                         "traffic": _traffic("diag_scan.hip", f"traffic_{spec.name}.json"),
                         "launch_ms_avg": ev_ms, "launch_ms_min": ev_min},
        })
        if not a.no_cpu:
            out["cpu_baseline"] = cpu_baseline_varlen(inp, spec, a.cpu_seconds)
    elif a.workload.startswith("noise_"):
        inp = synth.noise_inputs(spec)
        x = {n: _up(inp[n], torch, dev) for n in ("q", "k", "v", "beta", "a", "p")}

        def step():
            kdn.kdn_diag_noise_scan_fwd(x["q"], x["k"], x["v"], x["beta"], x["a"], x["p"])

        wall, ev_ms, ev_min = _time_steps(torch, step, a.steps, a.warmup)
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
                         "launch_ms_avg": ev_ms, "launch_ms_min": ev_min},
        })
        if not a.no_cpu:
            out["cpu_baseline"] = cpu_baseline_noise(inp, spec, a.cpu_seconds)
    elif a.workload.startswith("bwd_"):
        inp = synth.diag_inputs(spec)
        grads = synth.grad_inputs(spec, final_state=False)
        x = {n: _up(inp[n], torch, dev) for n in ("q", "k", "v", "beta", "d", "A")}
        d_o = _up(grads["d_o"], torch, dev)

        def step():
            kdn.kdn_diag_scan_bwd(x["q"], x["k"], x["v"], x["beta"], x["d"], x["A"],
                                  spec.I_prior, d_o)

        wall, ev_ms, ev_min = _time_steps(torch, step, a.steps, a.warmup)
        flops = BWD_FLOPS_PER_ENTRY_STEP * spec.B * spec.H * spec.T * spec.d_k * spec.d_v
        achieved = flops / (ev_ms * 1e-3) / 1e12
        out.update({
            "metric": "tokens/s per MI355X, diag-precision scan backward (gradient of all inputs)",
            "value": spec.B * spec.T / (wall / a.steps), "unit": "tokens/s",
            "ms_per_step": wall / a.steps * 1e3,
            "config": {"workload": spec.name, "B": spec.B, "H": spec.H, "T": spec.T,
                       "d_k": spec.d_k, "d_v": spec.d_v, "inputs": spec.dtype,
                       "gradients": "fp32, loss on o only", "parallelism": "single GPU"},
            "roofline": {"bound": "alu", "achieved": achieved, "peak": PEAK_FP32_VALU_TFLOPS,
                         "unit": "TFLOP/s", "frac": achieved / PEAK_FP32_VALU_TFLOPS,
                         "traffic": _traffic("diag_bwd.hip", f"traffic_{spec.name}.json"),
                         "launch_ms_avg": ev_ms, "launch_ms_min": ev_min,
                         "note": "events bracket the whole call: frame scalars, checkpoints, "
                                 "reverse pass and finishing sums; traffic is the reverse pass"},
        })
        if not a.no_cpu:
            out["cpu_baseline"] = cpu_baseline_bwd(inp, grads, spec, a.cpu_seconds)
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

        def step():
            kdn.kdn_decode_step(y["q"], y["k"], y["v"], y["beta"], y["d"], A, spec.I_prior,
                                I, mu, o=o)

        wall, ev_ms, ev_min = _time_steps(torch, step, a.steps, a.warmup)
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
                         "launch_ms_avg": ev_ms, "launch_ms_min": ev_min},
        })
        if not a.no_cpu:
            out["cpu_baseline"] = cpu_baseline_diag(inp, spec.with_(B=8), a.cpu_seconds)
    elif a.workload.startswith("iso_"):
        inp = synth.iso_inputs(spec)
        x = {n: _up(inp[n], torch, dev) for n in ("a", "p", "Lambda", "q", "k", "v", "lambda0")}

        def step():
            kdn.kdn_mobius_precision_scan(x["a"], x["p"], x["Lambda"], x["lambda0"], x["q"],
                                          x["k"], x["v"])

        wall, ev_ms, ev_min = _time_steps(torch, step, a.steps, a.warmup)
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
                         "launch_ms_avg": ev_ms, "launch_ms_min": ev_min,
                         "note": "whole step (all kernels) timed by events; traffic is the "
                                 "main mean-scan pass"},
        })
        if not a.no_cpu:
            out["cpu_baseline"] = cpu_baseline_iso(inp, spec, a.cpu_seconds)
    elif a.workload == "copy_1gib":
        # plain device-to-device copy of 1 GiB: the reference for HBM counters
        # (read 1 GiB + write 1 GiB per step) and for attainable copy bandwidth
        n = 1 << 28
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)

        def step():
            dst.copy_(src)

        wall, ev_ms, ev_min = _time_steps(torch, step, a.steps, a.warmup)
        gbs = 2 * 4 * n / (ev_ms * 1e-3) / 1e9
        out.update({"metric": "copy GB/s (read + write)", "value": gbs, "unit": "GB/s",
                    "ms_per_step": wall / a.steps * 1e3,
                    "config": {"workload": "copy_1gib", "bytes_read": 4 * n, "bytes_written": 4 * n},
                    "roofline": {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                 "frac": gbs / PEAK_HBM_GBS, "traffic": None,
                                 "launch_ms_avg": ev_ms, "launch_ms_min": ev_min}})
    else:
        raise SystemExit(f"unknown workload {a.workload}")

    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
