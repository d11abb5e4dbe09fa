"""AddressSanitizer / UndefinedBehaviorSanitizer runs on the CPU.

Two executables are built in a temporary folder and run:
  * the fp64 oracle (oracle/kdn_oracle.c) with tests/sanitize/oracle_driver.c,
    every oracle function on small seeded inputs in exactly sized heap
    blocks, optional arguments given and NULL, T = 0 and degenerate heads;
  * the host code of the C ABI (kdnscan_api.hip, host side instrumented, the
    device code and the kernel objects of the library as built) with
    tests/sanitize/abi_driver.cpp, which walks the argument checks, the plan,
    the workspace and echo-size queries and the status strings: calls that
    all return before any HIP call, so no GPU is needed.
Any out-of-bounds access, leak or undefined operation aborts the executable
with a sanitizer report; the test fails on a non-zero exit.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# host-side instrumentation only; the device code is built as usual
HOST_SANITIZE = ["-Xarch_host", "-fsanitize=address",
                 "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=all",
                 "-Xarch_host", "-fno-omit-frame-pointer"]
GCC_SANITIZE = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def _run(cmd, cwd, env=None):
    r = subprocess.run(cmd, cwd=cwd, capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0, f"{' '.join(cmd[:3])} ... failed ({r.returncode}):\n{r.stdout[-3000:]}\n{r.stderr[-6000:]}"
    return r


def test_oracle_under_asan_ubsan(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    exe = str(tmp_path / "oracle_driver")
    _run(["gcc", "-std=c99", "-g", "-O1", "-ffp-contract=off", *GCC_SANITIZE, "-o", exe,
          os.path.join(ROOT, "oracle", "kdn_oracle.c"), os.path.join(HERE, "oracle_driver.c"), "-lm"],
         cwd=tmp_path)
    r = _run([exe], cwd=tmp_path)
    assert "ok" in r.stdout


def test_host_validation_under_asan_ubsan(tmp_path):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    from bayesian_memory_scan_amd import _build
    others = [s for s in _build.SOURCES if s != "kdnscan_api.hip"]
    objs = [os.path.join(_build.BUILD, s.replace(".hip", ".o")) for s in others]
    if not all(os.path.exists(o) for o in objs):
        _build.build()
    flags = ["--offload-arch=gfx950", "-mcode-object-version=5", "-std=c++17", "-g", "-O1", "-fPIC",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wno-unused-command-line-argument"]
    api = str(tmp_path / "api_san.o")
    _run([HIPCC, *flags, *HOST_SANITIZE, "-c", os.path.join(_build.CSRC, "kdnscan_api.hip"), "-o", api],
         cwd=tmp_path)
    drv = str(tmp_path / "abi_driver.o")
    _run([HIPCC, "-std=c++17", "-g", "-O1", *HOST_SANITIZE, "-x", "c++", "-c",
          os.path.join(HERE, "abi_driver.cpp"), "-o", drv], cwd=tmp_path)
    exe = str(tmp_path / "abi_driver")
    _run([HIPCC, "--offload-arch=gfx950", "-mcode-object-version=5", *HOST_SANITIZE, "-o", exe, drv, api,
          *objs], cwd=tmp_path)
    r = _run([exe], cwd=tmp_path, env={**os.environ, "ASAN_OPTIONS": "detect_leaks=1"})
    assert "ok" in r.stdout
