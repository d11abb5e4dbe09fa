"""Print the gfx950 VALU issue-rate table measured by libkdnprobe.so.

    python -m bayesian_memory_scan_amd.issue_rates [--iters N] [--wps 2,4,8]

Measurement only (csrc/issue_rates.hip describes the kernels).  For each
probe and occupancy it prints, as a markdown table: the VGPRs the kernel
uses, the timed launch's milliseconds, the shader clock workgroup 0 ran at
(its s_memtime ticks over its s_memrealtime ticks at 100 MHz), and the rate
per clock per CU, both at the nominal 2.4 GHz and at that measured clock:
lane-instructions for the single-instruction chains, entry-steps (one key row
x value column x token of the scan) for the scan mixes, whose fp32 work is
also shown as TFLOP/s at 11 flop per entry-step.
"""
from __future__ import annotations

import argparse
import ctypes
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libkdnprobe.so")
NOMINAL_HZ = 2.4e9
CUS = 256
THREADS = 256
FLOP_PER_ENTRY_STEP = 11


def load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: run bayesian_memory_scan_amd._build first")
    try:  # bind to the HIP runtime torch ships, as libkdnscan does
        import torch  # noqa: F401
    except ImportError:  # pragma: no cover
        pass
    lib = ctypes.CDLL(LIB_PATH)
    lib.kdn_probe_count.restype = ctypes.c_int
    lib.kdn_probe_name.argtypes = [ctypes.c_int]
    lib.kdn_probe_name.restype = ctypes.c_char_p
    lib.kdn_probe_per_iter.argtypes = [ctypes.c_int]
    lib.kdn_probe_per_iter.restype = ctypes.c_int
    lib.kdn_probe_run.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                  ctypes.POINTER(ctypes.c_float), ctypes.POINTER(ctypes.c_uint64),
                                  ctypes.POINTER(ctypes.c_uint64), ctypes.POINTER(ctypes.c_int)]
    lib.kdn_probe_run.restype = ctypes.c_int
    return lib


def run(lib, i: int, wps: int, iters: int) -> dict:
    ms, clk, tick, vg = ctypes.c_float(), ctypes.c_uint64(), ctypes.c_uint64(), ctypes.c_int()
    rc = lib.kdn_probe_run(i, wps, iters, ctypes.byref(ms), ctypes.byref(clk), ctypes.byref(tick),
                           ctypes.byref(vg))
    if rc != 0:
        raise RuntimeError(f"probe {i} at {wps} waves/SIMD failed: {rc}")
    name = lib.kdn_probe_name(i).decode()
    per_iter = lib.kdn_probe_per_iter(i)
    work = per_iter * iters * 256 * wps * THREADS
    per_s_cu = work / (ms.value * 1e-3) / CUS
    mhz = clk.value / (tick.value / 100.0) if tick.value else float("nan")
    r = {"name": name, "wps": wps, "vgprs": vg.value, "ms": ms.value, "mhz": mhz,
         "rate_nominal": per_s_cu / NOMINAL_HZ, "rate_clock": per_s_cu / (mhz * 1e6),
         "mix": " " in name}
    if r["mix"]:
        r["tflops"] = work * FLOP_PER_ENTRY_STEP / (ms.value * 1e-3) / 1e12
    return r


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--iters", type=int, default=2048)
    ap.add_argument("--wps", default="2,4,8")
    ap.add_argument("--only", default=None, help="run only the probes whose name contains this")
    a = ap.parse_args(argv)
    lib = load()
    print("| probe | waves/SIMD | VGPRs | ms | clock MHz | per clk per CU @2.4 GHz | "
          "per clk per CU @clock | TFLOP/s (11 flop/entry-step) |")
    print("|---|---|---|---|---|---|---|---|")
    for i in range(lib.kdn_probe_count()):
        if a.only and a.only not in lib.kdn_probe_name(i).decode():
            continue
        for wps in (int(x) for x in a.wps.split(",")):
            r = run(lib, i, wps, a.iters)
            tf = f"{r['tflops']:.1f}" if r["mix"] else ""
            print(f"| {r['name']} | {wps} | {r['vgprs']} | {r['ms']:.3f} | {r['mhz']:.0f} | "
                  f"{r['rate_nominal']:.1f} | {r['rate_clock']:.1f} | {tf} |", flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
