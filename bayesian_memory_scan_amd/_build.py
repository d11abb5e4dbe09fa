"""Build libkdnscan.so (gfx950 only) in-tree with hipcc, and next to it the
measurement-only issue-rate probe libkdnprobe.so.

Every translation unit is compiled for gfx950 with packed fp32 math disabled
(``-Xclang -target-feature -Xclang -packed-fp32-ops``), then linked into one
shared library next to this file.
"""
from __future__ import annotations

import os
import re
import subprocess
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libkdnscan.so")
# measurement-only library (issue-rate probe); not linked into libkdnscan
PROBE_LIB = os.path.join(HERE, "libkdnprobe.so")
PROBE_SOURCES = ["issue_rates.hip"]
BUILD = os.path.join(HERE, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["kdnscan_api.hip", "diag_scan.hip", "decode.hip", "mobius_scan.hip", "iso_scan.hip", "diag_comp.hip",
           "diag_bwd.hip", "diag_bwd_seg.hip", "diag_noise.hip"]

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17",
    # code object v5: loadable by the HIP runtime torch ships as well as the system one
    "-mcode-object-version=5",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
]


def dpp_hazards(asm: str) -> list[str]:
    """VALU writes of a VGPR read by a following DPP instruction (as its
    permuted source) with fewer than two wait states between them.

    The compiler pads hazards of the DPP instructions it emits itself but
    cannot see inside inline assembly, so the build checks the generated
    gfx950 code of this library (our own output) and refuses it on a hit.
    """
    found = []
    func, prev = "", []
    for raw in asm.splitlines():
        m = re.match(r"^(_Z\w+):", raw)
        if m:
            func, prev = m.group(1), []
            continue
        line = raw.split(";")[0].strip()
        if not line or line.startswith(".") or line.endswith(":"):
            continue
        d = re.match(r"v_\w+_dpp\s+v\d+,\s*(v\d+)", line)
        if d:
            waits = 0
            for p in reversed(prev[-2:]):
                if p.startswith("s_nop"):
                    parts = p.split()
                    waits += (int(parts[1], 0) if len(parts) > 1 else 0) + 1
                else:
                    w = re.match(r"(v_\w+)\s+(v\d+)\b", p)
                    if w and w.group(2) == d.group(1) and not w.group(1).startswith(("v_readfirstlane", "v_cmp")):
                        found.append(f"{func}: '{p}' then '{line}'")
                        break
                    waits += 1
                if waits >= 2:
                    break
        prev.append(line)
    return found


def build(verbose: bool = False) -> str:
    """Compile every source and link libkdnscan.so; returns the library path."""
    os.makedirs(BUILD, exist_ok=True)

    def compile_one(src: str) -> str:
        obj = os.path.join(BUILD, src.replace(".hip", ".o"))
        cmd = [HIPCC, *FLAGS, "-save-temps=obj", "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True, cwd=BUILD)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
        asm = os.path.join(BUILD, src.replace(".hip", "-hip-amdgcn-amd-amdhsa-gfx950.s"))
        hz = dpp_hazards(open(asm).read())
        if hz:
            raise RuntimeError(f"DPP read-after-write hazard in {src}:\n" + "\n".join(hz[:10]))
        return obj

    with ThreadPoolExecutor(len(SOURCES) + len(PROBE_SOURCES)) as ex:
        objs = list(ex.map(compile_one, SOURCES + PROBE_SOURCES))
    for out, group in ((LIB, objs[:len(SOURCES)]), (PROBE_LIB, objs[len(SOURCES):])):
        tmp = out + ".tmp"
        cmd = [HIPCC, "--offload-arch=gfx950", "-mcode-object-version=5", "-shared", "-fPIC", "-o", tmp,
               *group]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        os.replace(tmp, out)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
