"""Invariants of the compiled kernels with direct-to-LDS loads (the prefill GEMMs with bf16 and FP8
activations, and the MXFP4 decode kernel's scale staging) that their hand-counted load waits rely
on (CPU only: hipcc cross-compiles gfx950 device code without a GPU).

The direct-to-LDS loads are issued from inline assembly, so the compiler neither knows that
they write M0 nor counts them when it inserts its own load waits; the kernel waits for them
explicitly with s_waitcnt vmcnt(n), n = loads issued after the ones it needs.  That is correct
only if
  * no compiler-generated instruction reads or writes M0 (the asm clobbers it), and
  * no other vector-memory load is issued while those loads are in flight (it would shift the
    counts); the only stores are the epilogue's, after the last wait.
"""
import os
import re
import subprocess

import pytest

from routed_expert_grouped_amd import build

SRCS = [os.path.join(build.CSRC, f)
        for f in ("moe_gemm.hip", "moe_gemm_wide.hip", "moe_gemm_a8.hip", "moe_gemm_a8_wide.hip",
                  "moe_gemm_w4.hip", "moe_gemm_w4a8.hip", "moe_ffn.hip")]
# the GEMMs with direct-to-LDS loads (and their instantiation counts: 2 phases x (grouped,
# identity); the FP8-activation 160 x 512 kernel is a down projection only)
KERNELS = {"gemm_fp8_q256_kernel": 4, "gemm_fp8_wide_kernel": 4, "gemm_a8_kernel": 4,
           "gemm_a8_wide_kernel": 2, "gemm_w4_kernel": 4, "gemm_w4a8_kernel": 4}

pytestmark = pytest.mark.skipif(not os.path.exists(build.HIPCC), reason="hipcc not available")

_VMEM = re.compile(r"^\s*(global_|buffer_|scratch_|flat_)\w*")


@pytest.fixture(scope="module")
def isa(tmp_path_factory):
    funcs = {}
    for src in SRCS:
        out = tmp_path_factory.mktemp("isa") / (os.path.basename(src) + ".s")
        subprocess.run([build.HIPCC, *build.flags_for(src), "-S", "--cuda-device-only", "-o",
                        str(out), src], check=True, capture_output=True)
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
    for kernel, count in KERNELS.items():
        names = [n for n in isa if kernel in n]
        assert len(names) == count, names


def test_m0_only_in_inline_asm(isa):
    checked = 0
    for name, lines in isa.items():
        if "gemm" not in name and "gemv" not in name:
            continue
        checked += 1
        bad = [t for t, inasm in _code(lines) if not inasm and re.search(r"\bm0\b", t)]
        assert not bad, (name, bad[:5])
    assert checked >= 32


def test_no_other_vector_memory_between_direct_loads(isa):
    checked = 0
    for name, lines in isa.items():
        if not any(k in name for k in KERNELS):
            continue
        checked += 1
        code = list(_code(lines))
        dma = [i for i, (t, _) in enumerate(code) if t.startswith("global_load_lds")]
        assert dma, name
        # the kernels store only in their epilogue, after the K loop's last vmcnt(0) wait; the
        # compiler may lay that code out between the loop's variants, so stores are allowed
        inside = [t for t, _ in code[dma[0]:dma[-1] + 1]
                  if _VMEM.match(t) and not t.startswith("global_load_lds")
                  and not re.match(r"(global|buffer|flat)_store", t)]
        assert not inside, (name, inside[:5])
    assert checked == sum(KERNELS.values())


def _vmcnt(t):
    m = re.match(r"s_waitcnt\b.*\bvmcnt\((\d+)\)", t)
    return int(m.group(1)) if m else None


def test_mxfp4_scale_loads_waited_for_before_their_lds_reads(isa):
    """The MXFP4 decode kernel copies its scales to LDS with direct loads and reads them back with
    8-byte LDS reads (the only ds_read_b64 in the kernel).  Between a direct load and the next
    such read there must be an s_waitcnt vmcnt(n) with at least n ordinary loads issued after the
    direct load (completion is in issue order, so only those n can still be outstanding)."""
    checked = 0
    for name, lines in isa.items():
        if "gemv_kernelILi2E" not in name:
            continue
        checked += 1
        pending, younger, reads = False, 0, 0
        for t, _ in _code(lines):
            n = _vmcnt(t)
            if t.startswith("global_load_lds"):
                pending, younger = True, 0
            elif _VMEM.match(t):
                younger += 1
            elif n is not None and pending and younger >= n:
                pending = False
            elif t.startswith("ds_read_b64"):
                assert not pending, (name, t)
                reads += 1
        assert reads >= 2, name
    assert checked == 10  # two or four weight groups a wave (four: K split in two in phase 1)


def _issue_model(K, sps, per_slot, per_stage, load_a):
    """Loads of a two-ring direct-to-LDS GEMM in issue order, and each stage's wait, as its
    source states them: weight slots of sps 64-K stages (per_slot loads a wave), activation stages
    of 64 K (per_stage loads); prologue weight slots 0, 1 then activation stages 0, 1; at stage q:
    wait, then weight slot q / sps + 2 (first stage of a slot), activation stage q + 2.  Yields
    (loads issued so far, the stage's wait, the loads it needs)."""
    nq, nslots = K // 64, -(-K // (64 * sps))
    seq = [("B", 0)] * per_slot
    if nslots > 1:
        seq += [("B", 1)] * per_slot
    if load_a:
        seq += [("A", 0)] * per_stage + [("A", 1)] * per_stage
    for q in range(nq):
        hs, sl = q % sps, q // sps
        b1, b2, a1 = sl + 1 < nslots, sl + 2 < nslots, q + 1 < nq
        if load_a:  # the kernels' wait immediates
            if hs == 1:
                n = (per_slot + per_stage if b2 and a1 else per_slot if b2
                     else per_stage if a1 else 0)
            else:
                n = per_stage if a1 else 0
        else:
            n = 2 * per_slot if hs >= 1 and b1 and b2 else per_slot if b1 else 0
        yield list(seq), n, {("B", sl)} | ({("A", q)} if load_a else set())
        if hs == 0 and b2:
            seq += [("B", sl + 2)] * per_slot
        if load_a and q + 2 < nq:
            seq += [("A", q + 2)] * per_stage


@pytest.mark.parametrize("kernel,sps,per_slot,per_stage", [
    ("FP8-activation GEMM, FP8 weights", 2, 4, 2),
    ("4-bit GEMM, bf16 activations", 2, 3, 4),
])
@pytest.mark.parametrize("load_a", [False, True])
def test_gemm_waits_cover_exactly_the_needed_loads(kernel, sps, per_slot, per_stage, load_a):
    """Loads land in issue order, so vmcnt(n) leaves exactly the last n issued in flight: each
    stage's n must leave none of the loads it reads, and (for speed) no more than needed, at
    every K the kernel takes."""
    for K in range(128, 8192 + 1, 128):
        for seq, n, need in _issue_model(K, sps, per_slot, per_stage, load_a):
            newest = max(i for i, x in enumerate(seq) if x in need)
            assert n == len(seq) - 1 - newest, (K, n, len(seq) - 1 - newest)


def _issue_model_w4a8(K, na):
    """The one-wave-per-SIMD W4A8 GEMM's loads in issue order, as its source states them, and each
    stage's wait: prologue exponent parts 0, 1 (those that exist), weight slot 0 (10 loads) and
    part 0 of weight slot 1 (5), activation slots 0, 1 (128 K, 2 na loads each); at stage q, after
    the wait: exponent part q / 32 + 2 when q % 32 == 31 (if it exists), part 0 of weight slot
    q / 4 + 2 when q % 4 == 3, part 1 of weight slot q / 4 + 1 when q % 4 == 0, activation slot
    (q + 3) / 2 when q is odd (weight and activation loads are issued past the end of K too: they
    reload into free slots).  Yields (loads issued so far, the wait before reading stage s's
    fragments, the loads stage s reads), s = 0 (the prologue's wait) and s = q + 1."""
    nq, nparts = K // 64, -(-(K // 128) // 16)
    seq = [("E", 0)] + ([("E", 1)] if nparts > 1 else [])
    seq += [("B", 0)] * 10 + [("B", 1)] * 5 + [("A", 0)] * (2 * na) + [("A", 1)] * (2 * na)
    yield list(seq), 2 * na, {("A", 0), ("B", 0), ("E", 0)}
    for q in range(nq):
        if q + 1 < nq:  # the kernel's wait immediate
            if q % 2:
                n = 5 if q % 4 == 1 else 0
            else:
                n = 2 * na if q == 0 else (2 * na + 5 + (1 if q % 32 == 0 and q // 32 + 1 < nparts
                                                          else 0))
            yield list(seq), n, {("A", (q + 1) // 2), ("B", (q + 1) // 4), ("E", (q + 1) // 32)}
        if q % 32 == 31 and q // 32 + 2 < nparts:
            seq += [("E", q // 32 + 2)]
        if q % 4 == 3:
            seq += [("B", q // 4 + 2)] * 5
        if q % 4 == 0:
            seq += [("B", q // 4 + 1)] * 5
        if q % 2:
            seq += [("A", (q + 3) // 2)] * (2 * na)


@pytest.mark.parametrize("na", [1, 2, 3, 4])
def test_w4a8_waits_cover_exactly_the_needed_loads(na):
    """As above for the W4A8 GEMM, whose waves all issue 2 na loads per activation slot (na = the
    64-row blocks holding tile rows) and whose waits come before reading the next stage's
    fragments: every wait leaves exactly the loads issued after the newest one it needs."""
    for K in range(128, 8192 + 1, 128):
        for seq, n, need in _issue_model_w4a8(K, na):
            newest = max(i for i, x in enumerate(seq) if x in need)
            assert n == len(seq) - 1 - newest, (K, n, len(seq) - 1 - newest)
