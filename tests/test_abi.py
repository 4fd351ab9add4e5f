"""The C-ABI library loads, exports every declared entry point, and rejects bad arguments on the
host before anything is enqueued (no GPU needed: no call here reaches a kernel launch).

The validation tests pass a fake device address that no call may dereference.  They run only
where no GPU is visible: there a validation bug cannot turn into a device fault, and the same
bug fails the test instead (the pointer is never mapped)."""
import ctypes
import os
import re

import pytest
import torch

import routed_expert_grouped_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "libmoe.h")

pytestmark = pytest.mark.skipif(not os.path.exists(moe.LIB_PATH), reason="libmoe.so not built")

# counting devices does not initialise the runtime
cpu_only = pytest.mark.skipif(torch.cuda.device_count() > 0,
                              reason="fake device pointers: run only where no GPU is visible")

# A non-null, 16-byte aligned address that is never dereferenced by the calls below: each of
# them fails validation (or has T == 0) before any device work is enqueued.
FAKE = ctypes.c_void_p(0x1000)


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^(?:moe_status|const char\*)\s+(moe_\w+)\(", text, re.M)))


def test_header_declares_the_boundary():
    assert declared_functions() == sorted(moe.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(moe.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings():
    assert moe.moe_status_string(moe.MOE_OK) == "MOE_OK"
    assert moe.moe_status_string(moe.MOE_ERR_WORKSPACE) == "MOE_ERR_WORKSPACE"
    assert moe.moe_status_string(99) == "MOE_ERR_UNKNOWN"


def _w(dtype=0, n=4, H=256, I=128, ptr=FAKE, scales=True):
    s = ptr if scales else None
    return moe.MoeExpertWeights(dtype, n, H, I, ptr.value, ptr.value, ptr.value,
                                s.value if s else None, s.value if s else None,
                                s.value if s else None)


@cpu_only
def test_route_validation():
    L = moe.lib()
    st = None
    assert L.moe_route(None, 4, 8, 2, 0, 1, FAKE, FAKE, st) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_route(FAKE, 4, 8, 9, 0, 1, FAKE, FAKE, st) == moe.MOE_ERR_INVALID_ARG  # k > E
    assert L.moe_route(FAKE, 4, 8, 0, 0, 1, FAKE, FAKE, st) == moe.MOE_ERR_INVALID_ARG  # k < 1
    assert L.moe_route(FAKE, -1, 8, 2, 0, 1, FAKE, FAKE, st) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_route(FAKE, 4, 8, 2, 7, 1, FAKE, FAKE, st) == moe.MOE_ERR_INVALID_ARG  # score_fn
    assert L.moe_route(FAKE, 4, 2048, 2, 0, 1, FAKE, FAKE, st) == moe.MOE_ERR_UNSUPPORTED  # E
    assert L.moe_route(FAKE, 4, 64, 33, 0, 1, FAKE, FAKE, st) == moe.MOE_ERR_UNSUPPORTED  # k
    assert L.moe_route(FAKE, 0, 8, 2, 0, 1, FAKE, FAKE, st) == moe.MOE_OK  # T == 0: no-op


@cpu_only
def test_permute_validation():
    L = moe.lib()
    P = L.moe_permute
    assert P(None, 4, 2, 8, FAKE, FAKE, FAKE, FAKE, None, 0, None) == moe.MOE_ERR_INVALID_ARG
    assert P(FAKE, 4, 0, 8, FAKE, FAKE, FAKE, FAKE, None, 0, None) == moe.MOE_ERR_INVALID_ARG
    assert P(FAKE, 4, 2, 0, FAKE, FAKE, FAKE, FAKE, None, 0, None) == moe.MOE_ERR_INVALID_ARG
    assert P(FAKE, 4, 2, 8, FAKE, FAKE, None, FAKE, None, 0, None) == moe.MOE_ERR_INVALID_ARG
    assert P(FAKE, 4, 2, 1025, FAKE, FAKE, FAKE, FAKE, None, 0, None) == moe.MOE_ERR_UNSUPPORTED
    assert P(FAKE, 1 << 28, 16, 8, FAKE, FAKE, FAKE, FAKE, None, 0, None) == moe.MOE_ERR_UNSUPPORTED
    assert P(FAKE, 0, 2, 8, FAKE, FAKE, FAKE, FAKE, None, 0, None) == moe.MOE_OK


def _permute_ws(T, k, E):
    n = ctypes.c_size_t(12345)
    st = moe.lib().moe_permute_workspace_size(T, k, E, ctypes.byref(n))
    return st, n.value


def test_permute_workspace_size():
    """No workspace up to 2048 assignments; above, one int32 count per (block of 2048, expert)."""
    assert _permute_ws(16, 8, 256) == (moe.MOE_OK, 0)
    assert _permute_ws(256, 8, 256) == (moe.MOE_OK, 0)        # 2048 assignments
    assert _permute_ws(2049, 1, 256) == (moe.MOE_OK, 2 * 256 * 4)
    assert _permute_ws(4096, 8, 256) == (moe.MOE_OK, 16 * 256 * 4)
    assert _permute_ws(32768, 8, 256) == (moe.MOE_OK, 128 * 256 * 4)
    assert _permute_ws(8192, 8, 384) == (moe.MOE_OK, 32 * 384 * 4)
    assert _permute_ws(0, 8, 256) == (moe.MOE_OK, 0)
    assert _permute_ws(-1, 8, 256)[0] == moe.MOE_ERR_INVALID_ARG
    assert _permute_ws(4, 0, 256)[0] == moe.MOE_ERR_INVALID_ARG
    assert _permute_ws(4, 2, 0)[0] == moe.MOE_ERR_INVALID_ARG
    assert _permute_ws(4, 2, 1025)[0] == moe.MOE_ERR_UNSUPPORTED
    assert _permute_ws(1 << 28, 16, 8)[0] == moe.MOE_ERR_UNSUPPORTED
    assert moe.lib().moe_permute_workspace_size(4, 2, 8, None) == moe.MOE_ERR_INVALID_ARG


@cpu_only
def test_permute_workspace_errors():
    """Above 2048 assignments a missing or short workspace is MOE_ERR_WORKSPACE and an unaligned
    one INVALID_ARG, before anything is enqueued; up to 2048 none is needed."""
    P = moe.lib().moe_permute
    _, need = _permute_ws(4096, 8, 256)
    assert P(FAKE, 4096, 8, 256, FAKE, FAKE, FAKE, FAKE, None, 0, None) == moe.MOE_ERR_WORKSPACE
    assert P(FAKE, 4096, 8, 256, FAKE, FAKE, FAKE, FAKE, None, need, None) == moe.MOE_ERR_WORKSPACE
    assert P(FAKE, 4096, 8, 256, FAKE, FAKE, FAKE, FAKE, FAKE, need - 1,
             None) == moe.MOE_ERR_WORKSPACE
    assert P(FAKE, 4096, 8, 256, FAKE, FAKE, FAKE, FAKE, ctypes.c_void_p(0x1004), need,
             None) == moe.MOE_ERR_INVALID_ARG


@cpu_only
def test_expert_validation():
    L = moe.lib()
    gu, dn = L.moe_expert_gate_up, L.moe_expert_down
    ok = _w()
    assert gu(FAKE, 4, 2, FAKE, FAKE, ctypes.byref(ok), None, None) == moe.MOE_ERR_INVALID_ARG
    assert gu(FAKE, 4, 2, FAKE, FAKE, None, FAKE, None) == moe.MOE_ERR_INVALID_ARG
    assert gu(FAKE, 4, 2, FAKE, None, ctypes.byref(ok), FAKE, None) == moe.MOE_ERR_INVALID_ARG
    # identity grouping needs k == 1 and one group
    assert gu(FAKE, 4, 2, None, None, ctypes.byref(ok), FAKE, None) == moe.MOE_ERR_INVALID_ARG
    assert gu(FAKE, 4, 1, None, None, ctypes.byref(ok), FAKE, None) == moe.MOE_ERR_INVALID_ARG
    bad_dtype = _w(dtype=5)
    assert gu(FAKE, 4, 2, FAKE, FAKE, ctypes.byref(bad_dtype), FAKE, None) == moe.MOE_ERR_INVALID_ARG
    no_scales = _w(scales=False)
    assert gu(FAKE, 4, 2, FAKE, FAKE, ctypes.byref(no_scales), FAKE, None) == moe.MOE_ERR_INVALID_ARG
    fp4_no_scales = _w(dtype=2, scales=False)
    assert gu(FAKE, 4, 2, FAKE, FAKE, ctypes.byref(fp4_no_scales), FAKE, None) == moe.MOE_ERR_INVALID_ARG
    fp4 = _w(dtype=2)
    assert gu(FAKE, 0, 2, FAKE, FAKE, ctypes.byref(fp4), FAKE, None) == moe.MOE_OK
    bad_dtype3 = _w(dtype=3)
    assert gu(FAKE, 4, 2, FAKE, FAKE, ctypes.byref(bad_dtype3), FAKE, None) == moe.MOE_ERR_INVALID_ARG
    bf16_no_scales = _w(dtype=1, scales=False)
    assert gu(FAKE, 0, 2, FAKE, FAKE, ctypes.byref(bf16_no_scales), FAKE, None) == moe.MOE_OK
    odd = _w(H=200)
    assert gu(FAKE, 4, 2, FAKE, FAKE, ctypes.byref(odd), FAKE, None) == moe.MOE_ERR_UNSUPPORTED
    huge = _w(H=16384 + 128)
    assert gu(FAKE, 4, 2, FAKE, FAKE, ctypes.byref(huge), FAKE, None) == moe.MOE_ERR_UNSUPPORTED
    many = _w(n=2000)
    assert gu(FAKE, 4, 2, FAKE, FAKE, ctypes.byref(many), FAKE, None) == moe.MOE_ERR_UNSUPPORTED
    unaligned = _w(ptr=ctypes.c_void_p(0x1004))
    assert gu(FAKE, 4, 2, FAKE, FAKE, ctypes.byref(unaligned), FAKE, None) == moe.MOE_ERR_INVALID_ARG
    assert gu(FAKE, 0, 2, FAKE, FAKE, ctypes.byref(ok), FAKE, None) == moe.MOE_OK
    assert dn(FAKE, 4, 0, FAKE, ctypes.byref(ok), FAKE, None) == moe.MOE_ERR_INVALID_ARG
    assert dn(None, 4, 2, FAKE, ctypes.byref(ok), FAKE, None) == moe.MOE_ERR_INVALID_ARG
    assert dn(FAKE, 0, 2, FAKE, ctypes.byref(ok), FAKE, None) == moe.MOE_OK


@cpu_only
def test_shared_expert_calls_validation():
    """moe_expert_gate_up_shared / moe_expert_down_shared: the shared expert must be one expert
    of the routed experts' dtype and shape; perm and offsets are required."""
    L = moe.lib()
    gu, dn = L.moe_expert_gate_up_shared, L.moe_expert_down_shared
    w, ws = _w(), _w(n=1)
    assert gu(FAKE, 4, 2, FAKE, FAKE, ctypes.byref(w), None, FAKE, None) == moe.MOE_ERR_INVALID_ARG
    two = _w(n=2)
    assert gu(FAKE, 4, 2, FAKE, FAKE, ctypes.byref(w), ctypes.byref(two), FAKE, None) == moe.MOE_ERR_INVALID_ARG
    other_dtype = _w(dtype=1, n=1)
    assert gu(FAKE, 4, 2, FAKE, FAKE, ctypes.byref(w), ctypes.byref(other_dtype), FAKE,
              None) == moe.MOE_ERR_INVALID_ARG
    other_h = _w(n=1, H=384)
    assert gu(FAKE, 4, 2, FAKE, FAKE, ctypes.byref(w), ctypes.byref(other_h), FAKE,
              None) == moe.MOE_ERR_INVALID_ARG
    assert gu(FAKE, 4, 2, None, FAKE, ctypes.byref(w), ctypes.byref(ws), FAKE, None) == moe.MOE_ERR_INVALID_ARG
    assert gu(FAKE, 4, 2, FAKE, None, ctypes.byref(w), ctypes.byref(ws), FAKE, None) == moe.MOE_ERR_INVALID_ARG
    assert gu(FAKE, 4, 2, FAKE, FAKE, ctypes.byref(w), ctypes.byref(ws), None, None) == moe.MOE_ERR_INVALID_ARG
    assert gu(FAKE, 0, 2, FAKE, FAKE, ctypes.byref(w), ctypes.byref(ws), FAKE, None) == moe.MOE_OK
    assert dn(FAKE, 4, 2, None, ctypes.byref(w), ctypes.byref(ws), FAKE, None) == moe.MOE_ERR_INVALID_ARG
    assert dn(FAKE, 4, 2, FAKE, ctypes.byref(w), ctypes.byref(two), FAKE, None) == moe.MOE_ERR_INVALID_ARG
    assert dn(FAKE, 4, 0, FAKE, ctypes.byref(w), ctypes.byref(ws), FAKE, None) == moe.MOE_ERR_INVALID_ARG
    assert dn(FAKE, 0, 2, FAKE, ctypes.byref(w), ctypes.byref(ws), FAKE, None) == moe.MOE_OK


@cpu_only
def test_ffn_workspace():
    L = moe.lib()
    w = _w()
    n = ctypes.c_size_t()
    assert L.moe_expert_ffn_workspace_size(16, 2, ctypes.byref(w), ctypes.byref(n)) == moe.MOE_OK
    assert n.value == 16 * 2 * 128 * 2
    assert L.moe_expert_ffn_workspace_size(16, 2, None, ctypes.byref(n)) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_expert_ffn(FAKE, 16, 2, FAKE, FAKE, ctypes.byref(w), FAKE, FAKE, n.value - 1,
                            None) == moe.MOE_ERR_WORKSPACE
    assert L.moe_expert_ffn(FAKE, 16, 2, FAKE, FAKE, ctypes.byref(w), FAKE, None, n.value,
                            None) == moe.MOE_ERR_WORKSPACE
    assert L.moe_expert_ffn(FAKE, 0, 2, FAKE, FAKE, ctypes.byref(w), FAKE, None, 0, None) == moe.MOE_OK


@cpu_only
def test_quantize_act_validation():
    q = moe.lib().moe_quantize_act
    assert q(None, 4, 256, FAKE, FAKE, 2, None) == moe.MOE_ERR_INVALID_ARG
    assert q(FAKE, 4, 256, None, FAKE, 2, None) == moe.MOE_ERR_INVALID_ARG
    assert q(FAKE, 4, 256, FAKE, None, 2, None) == moe.MOE_ERR_INVALID_ARG
    assert q(ctypes.c_void_p(0x1002), 4, 256, FAKE, FAKE, 2, None) == moe.MOE_ERR_INVALID_ARG
    assert q(FAKE, -1, 256, FAKE, FAKE, 2, None) == moe.MOE_ERR_INVALID_ARG
    assert q(FAKE, 4, 0, FAKE, FAKE, 2, None) == moe.MOE_ERR_INVALID_ARG
    assert q(FAKE, 4, 256, FAKE, FAKE, 1, None) == moe.MOE_ERR_INVALID_ARG  # pitch < K/128
    assert q(FAKE, 4, 200, FAKE, FAKE, 2, None) == moe.MOE_ERR_UNSUPPORTED
    assert q(FAKE, 1 << 30, 1024, FAKE, FAKE, 8, None) == moe.MOE_ERR_UNSUPPORTED
    assert q(None, 0, 256, None, None, 2, None) == moe.MOE_OK
    assert moe.exp_pitch(7168) == 64 and moe.exp_pitch(2048) == 16 and moe.exp_pitch(640) == 16


@cpu_only
def test_route_permute_validation():
    L = moe.lib()
    f = L.moe_route_permute
    args = lambda T, E, k, fn=1, c=FAKE: (FAKE, T, E, k, fn, 1, FAKE, FAKE, c, FAKE, FAKE, FAKE, None)
    assert f(*args(16, 256, 0)) == moe.MOE_ERR_INVALID_ARG           # k < 1
    assert f(*args(16, 8, 9)) == moe.MOE_ERR_INVALID_ARG             # k > E
    assert f(*args(16, 256, 8, fn=7)) == moe.MOE_ERR_INVALID_ARG     # unknown score function
    assert f(*args(16, 256, 8, c=None)) == moe.MOE_ERR_INVALID_ARG   # null grouping output
    assert f(*args(257, 256, 8)) == moe.MOE_ERR_UNSUPPORTED          # T*k > 2048
    assert f(*args(16, 2048, 8)) == moe.MOE_ERR_UNSUPPORTED          # E > MOE_MAX_EXPERTS
    assert f(None, 0, 256, 8, 1, 1, None, None, None, None, None, None, None) == moe.MOE_OK


@cpu_only
def test_combine_partial_validation():
    L = moe.lib()
    f = L.moe_combine_partial
    assert f(FAKE, FAKE, FAKE, FAKE, 4, 2, None, 16, 2, 256, FAKE, None) == moe.MOE_ERR_INVALID_ARG  # e_begin > e_end
    assert f(FAKE, FAKE, None, FAKE, 0, 8, None, 16, 2, 256, FAKE, None) == moe.MOE_ERR_INVALID_ARG  # null ids
    assert f(FAKE, FAKE, FAKE, FAKE, 0, 8, None, 16, 0, 256, FAKE, None) == moe.MOE_ERR_INVALID_ARG
    assert f(FAKE, FAKE, FAKE, FAKE, 0, 8, None, 16, 2, 250, FAKE, None) == moe.MOE_ERR_UNSUPPORTED
    assert f(None, None, None, None, 0, 8, None, 0, 2, 256, None, None) == moe.MOE_OK


@cpu_only
def test_a8_phase_validation():
    L = moe.lib()
    gu, dn = L.moe_expert_gate_up_a8, L.moe_expert_down_a8
    w = _w(n=4, H=256, I=384)
    big = (1024, 2)  # T*k = 2048 > 32 * 4 rows: the FP8-code GEMM applies
    assert gu(FAKE, FAKE, 16, *big, FAKE, FAKE, ctypes.byref(w), None, None) == moe.MOE_ERR_INVALID_ARG
    assert gu(None, FAKE, 16, *big, FAKE, FAKE, ctypes.byref(w), FAKE, None) == moe.MOE_ERR_INVALID_ARG
    assert gu(FAKE, FAKE, 1, *big, FAKE, FAKE, ctypes.byref(w), FAKE, None) == moe.MOE_ERR_INVALID_ARG
    assert gu(FAKE, FAKE, 24, *big, FAKE, FAKE, ctypes.byref(w), FAKE, None) == moe.MOE_ERR_UNSUPPORTED
    assert gu(FAKE, FAKE, 80, *big, FAKE, FAKE, ctypes.byref(w), FAKE, None) == moe.MOE_ERR_UNSUPPORTED
    assert gu(FAKE, FAKE, 16, 16, 2, FAKE, FAKE, ctypes.byref(w), FAKE, None) == moe.MOE_ERR_UNSUPPORTED
    bf16 = _w(dtype=1, scales=False)
    assert gu(FAKE, FAKE, 16, *big, FAKE, FAKE, ctypes.byref(bf16), FAKE, None) == moe.MOE_ERR_UNSUPPORTED
    # MXFP4 weights pass the format check (W4A8) and reach the later argument checks
    fp4 = _w(n=4, H=256, I=384, dtype=2)
    assert gu(FAKE, FAKE, 1, *big, FAKE, FAKE, ctypes.byref(fp4), FAKE, None) == moe.MOE_ERR_INVALID_ARG
    assert gu(FAKE, FAKE, 1, *big, FAKE, FAKE, ctypes.byref(bf16), FAKE, None) == moe.MOE_ERR_UNSUPPORTED
    wide = _w(n=4, H=8192 + 128, I=384)
    assert gu(FAKE, FAKE, 80, *big, FAKE, FAKE, ctypes.byref(wide), FAKE, None) == moe.MOE_ERR_UNSUPPORTED
    assert gu(None, None, 0, 0, 2, None, None, None, None, None) == moe.MOE_OK
    odd_h = _w(n=4, H=384, I=256)  # phase 2 needs H a multiple of 256
    assert dn(FAKE, FAKE, 16, *big, FAKE, ctypes.byref(odd_h), FAKE, None) == moe.MOE_ERR_UNSUPPORTED
    assert dn(FAKE, FAKE, 16, *big, FAKE, ctypes.byref(w), None, None) == moe.MOE_ERR_INVALID_ARG
    assert dn(FAKE, FAKE, 16, 1024, 0, FAKE, ctypes.byref(w), FAKE, None) == moe.MOE_ERR_INVALID_ARG
    assert dn(None, None, 0, 0, 2, None, None, None, None) == moe.MOE_OK


@cpu_only
def test_ffn_a8_validation():
    L = moe.lib()
    w = _w(H=256, I=384)
    n = ctypes.c_size_t()
    # many rows per expert (FP8-code GEMMs): h, then codes and E8M0 exponent rows (16-byte
    # pitch) of x and of h, each part 256-byte aligned
    big = ctypes.c_size_t()
    assert L.moe_expert_ffn_a8_workspace_size(1024, 2, ctypes.byref(w), ctypes.byref(big)) == moe.MOE_OK
    assert big.value == 2048 * 384 * 2 + 1024 * 256 + 1024 * 16 + 2048 * 384 + 2048 * 16
    # few rows per expert: h, then x and h dequantised to bf16
    assert L.moe_expert_ffn_a8_workspace_size(16, 2, ctypes.byref(w), ctypes.byref(n)) == moe.MOE_OK
    assert n.value == 32 * 384 * 2 + 16 * 256 * 2 + 32 * 384 * 2
    f = L.moe_expert_ffn_a8
    assert f(FAKE, 16, 2, FAKE, FAKE, ctypes.byref(w), FAKE, FAKE, n.value - 1,
             None) == moe.MOE_ERR_WORKSPACE
    assert f(FAKE, 16, 2, FAKE, FAKE, ctypes.byref(w), FAKE, None, n.value,
             None) == moe.MOE_ERR_WORKSPACE
    assert f(FAKE, 16, 2, FAKE, FAKE, ctypes.byref(w), None, FAKE, n.value,
             None) == moe.MOE_ERR_INVALID_ARG
    assert f(FAKE, 16, 2, FAKE, FAKE, ctypes.byref(w), FAKE, ctypes.c_void_p(0x1008), n.value,
             None) == moe.MOE_ERR_INVALID_ARG
    assert f(FAKE, 16, 2, None, FAKE, ctypes.byref(w), FAKE, FAKE, n.value,
             None) == moe.MOE_ERR_INVALID_ARG
    bf16 = _w(dtype=1, scales=False)
    assert f(FAKE, 16, 2, FAKE, FAKE, ctypes.byref(bf16), FAKE, FAKE, 1 << 30,
             None) == moe.MOE_ERR_UNSUPPORTED
    fp4 = _w(H=256, I=384, dtype=2)  # accepted: reaches the workspace check
    assert L.moe_expert_ffn_a8_workspace_size(16, 2, ctypes.byref(fp4), ctypes.byref(n)) == moe.MOE_OK
    assert f(FAKE, 16, 2, FAKE, FAKE, ctypes.byref(fp4), FAKE, FAKE, n.value - 1,
             None) == moe.MOE_ERR_WORKSPACE
    assert f(FAKE, 16, 0, FAKE, FAKE, ctypes.byref(w), FAKE, FAKE, n.value,
             None) == moe.MOE_ERR_INVALID_ARG
    assert f(None, 0, 2, None, None, None, None, None, 0, None) == moe.MOE_OK


@cpu_only
def test_combine_validation():
    L = moe.lib()
    c = L.moe_combine
    assert c(None, FAKE, FAKE, None, 4, 2, 64, FAKE, None) == moe.MOE_ERR_INVALID_ARG
    assert c(FAKE, FAKE, FAKE, None, 4, 0, 64, FAKE, None) == moe.MOE_ERR_INVALID_ARG
    assert c(FAKE, FAKE, FAKE, None, 4, 2, 60, FAKE, None) == moe.MOE_ERR_UNSUPPORTED
    assert c(FAKE, FAKE, FAKE, ctypes.c_void_p(0x1008), 4, 2, 64, FAKE, None) == moe.MOE_ERR_INVALID_ARG
    assert c(FAKE, FAKE, FAKE, None, 0, 2, 64, FAKE, None) == moe.MOE_OK


def test_binding_raises_on_error_status():
    with pytest.raises(moe.MoeError) as ei:
        moe._check("moe_route", moe.MOE_ERR_UNSUPPORTED)
    assert ei.value.status == moe.MOE_ERR_UNSUPPORTED and "MOE_ERR_UNSUPPORTED" in str(ei.value)
