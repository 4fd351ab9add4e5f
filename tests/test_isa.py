"""Invariants of the compiled prefill GEMMs (bf16 and FP8 activations) that their hand-counted
load waits rely on (CPU only: hipcc cross-compiles gfx950 device code without a GPU).

The direct-to-LDS loads are issued from inline assembly, so the compiler neither knows that
they write M0 nor counts them when it inserts its own load waits; the kernel waits for them
explicitly with s_waitcnt vmcnt(n), n = loads issued after the ones it needs.  That is correct
only if
  * no compiler-generated instruction reads or writes M0 (the asm clobbers it), and
  * no other vector-memory instruction is issued while those loads are in flight (it would
    shift the counts).
"""
import os
import re
import subprocess

import pytest

from routed_expert_grouped_amd import build

SRCS = [os.path.join(build.CSRC, f) for f in ("moe_gemm.hip", "moe_gemm_a8.hip")]
KERNELS = ("gemm_fp8_q256_kernel", "gemm_a8_kernel")  # the kernels with direct-to-LDS loads

pytestmark = pytest.mark.skipif(not os.path.exists(build.HIPCC), reason="hipcc not available")

_VMEM = re.compile(r"^\s*(global_|buffer_|scratch_|flat_)\w*")


@pytest.fixture(scope="module")
def isa(tmp_path_factory):
    funcs = {}
    for src in SRCS:
        out = tmp_path_factory.mktemp("isa") / (os.path.basename(src) + ".s")
        subprocess.run([build.HIPCC, *build.FLAGS, "-S", "--cuda-device-only", "-o", str(out),
                        src], check=True, capture_output=True)
        text = out.read_text()
        for m in re.finditer(r"^(_Z\w+):[^\n]*\n(.*?)^\.Lfunc_end", text, re.S | re.M):
            funcs[m.group(1)] = m.group(2).splitlines()
    assert any("gemm" in n for n in funcs), "no kernels found in the assembly"
    return funcs


def _code(lines):
    """(instruction, inside inline asm) pairs, comments and directives dropped."""
    inasm = False
    for line in lines:
        if "ASMSTART" in line:
            inasm = True
            continue
        if "ASMEND" in line:
            inasm = False
            continue
        t = line.split(";")[0].strip()
        if t and not t.startswith(".") and not t.endswith(":"):
            yield t, inasm


def test_kernels_present(isa):
    for kernel in KERNELS:
        names = [n for n in isa if kernel in n]
        assert len(names) == 4, names  # 2 phases x (grouped, identity)


def test_m0_only_in_inline_asm(isa):
    checked = 0
    for name, lines in isa.items():
        if "gemm" not in name:
            continue
        checked += 1
        bad = [t for t, inasm in _code(lines) if not inasm and re.search(r"\bm0\b", t)]
        assert not bad, (name, bad[:5])
    assert checked >= 12


def test_no_other_vector_memory_between_direct_loads(isa):
    checked = 0
    for name, lines in isa.items():
        if not any(k in name for k in KERNELS):
            continue
        checked += 1
        code = list(_code(lines))
        dma = [i for i, (t, _) in enumerate(code) if t.startswith("global_load_lds")]
        assert dma, name
        inside = [t for t, _ in code[dma[0]:dma[-1] + 1]
                  if _VMEM.match(t) and not t.startswith("global_load_lds")]
        assert not inside, (name, inside[:5])
    assert checked == 8
