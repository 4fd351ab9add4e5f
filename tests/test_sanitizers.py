"""AddressSanitizer and UndefinedBehaviorSanitizer builds of the CPU-side code, driven on the CPU.

- The oracle (oracle/moe_oracle.c, gcc) under tests/sanitize/oracle_driver.c: every entry point
  on small layers in every weight format and both activation modes, plus rejected arguments.
- libmoe's host code (every csrc/*.hip, sanitizers on the host side only) under
  tests/sanitize/abi_driver.cpp: the argument validation of every entry point; no call
  reaches a launch, so no GPU is used.
Any sanitizer report makes the driver exit non-zero.
"""
import concurrent.futures
import glob
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OUT = os.path.join(ROOT, "_build", "sanitize")
CSRC = os.path.join(ROOT, "routed_expert_grouped_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANG = "/opt/rocm/lib/llvm/bin/clang++"
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout[-3000:]}\n{r.stderr[-3000:]}"
    return r


def test_oracle_under_sanitizers():
    os.makedirs(OUT, exist_ok=True)
    exe = os.path.join(OUT, "oracle_driver")
    _run(["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-ffp-contract=off",
          "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-o", exe,
          os.path.join(ROOT, "tests", "sanitize", "oracle_driver.c"),
          os.path.join(ROOT, "oracle", "moe_oracle.c"), "-lm"])
    r = _run([exe], env=ENV)
    assert "0 failures" in r.stdout


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="no ROCm clang")
def test_host_validation_under_sanitizers():
    os.makedirs(OUT, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(OUT, os.path.basename(src) + ".o")
        _run([HIPCC, "--offload-arch=gfx950", "-std=c++17", "-Xarch_device", "-O1", "-g0",
              "-Xarch_host", "-O1", "-fPIC",
              "-Xarch_host", "-fsanitize=address",
              "-Xarch_host", "-fsanitize=undefined",
              "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
              "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-c", src, "-o", obj])
        return obj

    with concurrent.futures.ThreadPoolExecutor(max_workers=8) as ex:
        objs = list(ex.map(compile_one, sorted(glob.glob(os.path.join(CSRC, "*.hip")))))
    drv = os.path.join(OUT, "abi_driver.o")
    _run([CLANG, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
          "-I", os.path.join(ROOT, "include"), "-c",
          os.path.join(ROOT, "tests", "sanitize", "abi_driver.cpp"), "-o", drv])
    exe = os.path.join(OUT, "abi_driver")
    _run([CLANG, "-fsanitize=address,undefined", drv, *objs, "-L/opt/rocm/lib", "-lamdhip64",
          "-Wl,-rpath,/opt/rocm/lib", "-o", exe])
    r = _run([exe], env=dict(ENV, ASAN_OPTIONS="detect_leaks=0"))
    assert "0 failures" in r.stdout
