"""ctypes binding of the plain C oracle (moe_oracle.c).

TEST INFRASTRUCTURE ONLY: only the tests, the smoke check and bench.py's cpu_baseline leg may
import this package.  The HIP library never does, and this package never imports it.

Every function takes host numpy arrays (or CPU torch tensors) and returns numpy arrays.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_DIR = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_DIR, "moe_oracle.c")
_LIB = os.path.join(_DIR, "_build", "libmoe_oracle.so")
_lib = None

SCORE_FN = {"softmax": 0, "sigmoid": 1}


def build(force: bool = False) -> str:
    """Compile moe_oracle.c with gcc (IEEE double arithmetic: no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        os.makedirs(os.path.dirname(_LIB), exist_ok=True)
        tmp = _LIB + f".tmp{os.getpid()}"
        subprocess.check_call(["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math",
                               "-fopenmp", "-shared", "-fPIC", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


class _Weights(ctypes.Structure):
    _fields_ = [("wdtype", ctypes.c_int32), ("n", ctypes.c_int32), ("H", ctypes.c_int32),
                ("I", ctypes.c_int32), ("gate", ctypes.c_void_p), ("up", ctypes.c_void_p),
                ("down", ctypes.c_void_p), ("s_gate", ctypes.c_void_p), ("s_up", ctypes.c_void_p),
                ("s_down", ctypes.c_void_p)]


def lib():
    global _lib
    if _lib is None:
        L = ctypes.CDLL(build())
        P = ctypes.c_void_p
        i32 = ctypes.c_int
        L.oracle_fp8_e4m3fn_to_double.restype = ctypes.c_double
        L.oracle_fp8_e4m3fn_to_double.argtypes = [ctypes.c_uint8]
        L.oracle_fp4_e2m1_to_double.restype = ctypes.c_double
        L.oracle_fp4_e2m1_to_double.argtypes = [ctypes.c_uint8]
        L.oracle_e8m0_to_double.restype = ctypes.c_double
        L.oracle_e8m0_to_double.argtypes = [ctypes.c_uint8]
        L.oracle_bf16_to_double.restype = ctypes.c_double
        L.oracle_bf16_to_double.argtypes = [ctypes.c_uint16]
        L.oracle_double_to_bf16.restype = ctypes.c_uint16
        L.oracle_double_to_bf16.argtypes = [ctypes.c_double]
        L.oracle_route.restype = i32
        L.oracle_route.argtypes = [P, i32, i32, i32, i32, i32, P, P]
        L.oracle_permute.restype = i32
        L.oracle_permute.argtypes = [P, i32, i32, i32, P, P, P, P]
        L.oracle_moe_layer.restype = i32
        L.oracle_moe_layer.argtypes = [P, P, i32, i32, i32, i32, i32, i32, i32,
                                       ctypes.POINTER(_Weights), P, ctypes.POINTER(_Weights),
                                       P, i32, P, P, P, P, P, P, i32, i32, P, i32, i32]
        L.oracle_float_to_e4m3fn.restype = ctypes.c_uint8
        L.oracle_float_to_e4m3fn.argtypes = [ctypes.c_float]
        L.oracle_act_scale_exp.restype = i32
        L.oracle_act_scale_exp.argtypes = [ctypes.c_double]
        L.oracle_quantize_rows.restype = None
        L.oracle_quantize_rows.argtypes = [P, i32, i32, P, P]
        L.oracle_expert_gate_up.restype = i32
        L.oracle_expert_gate_up.argtypes = [P, i32, i32, P, P, ctypes.POINTER(_Weights), P, i32]
        L.oracle_expert_down.restype = i32
        L.oracle_expert_down.argtypes = [P, i32, P, ctypes.POINTER(_Weights), P, i32]
        L.oracle_max_threads.restype = i32
        L.oracle_max_threads.argtypes = [i32]
        L.oracle_dequantize.restype = i32
        L.oracle_dequantize.argtypes = [ctypes.POINTER(_Weights), i32, i32, P, i32]
        L.oracle_silu_mul_bf16.restype = None
        L.oracle_silu_mul_bf16.argtypes = [P, P, ctypes.c_long, P]
        L.oracle_double_to_bf16_array.restype = None
        L.oracle_double_to_bf16_array.argtypes = [P, ctypes.c_long, P]
        L.oracle_quantize_dequantize.restype = None
        L.oracle_quantize_dequantize.argtypes = [P, ctypes.c_long, i32]
        _lib = L
    return _lib


def _np(a, dtype):
    """Contiguous host numpy view/copy of a numpy array or torch tensor with the given dtype."""
    if hasattr(a, "detach"):
        a = a.detach().cpu()
        import torch  # local: only needed for tensors
        tmap = {np.uint16: torch.int16, np.uint8: torch.uint8, np.float32: torch.float32,
                np.int32: torch.int32, np.float64: torch.float64}
        a = a.contiguous().view(tmap[dtype]).numpy()
    a = np.ascontiguousarray(a)
    return a.view(dtype) if a.dtype.itemsize == np.dtype(dtype).itemsize else a.astype(dtype)


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p) if a is not None else None


# ------------------------------------------------------------------ number formats

def fp8_e4m3fn_to_double(code: int) -> float:
    return lib().oracle_fp8_e4m3fn_to_double(int(code))


def bf16_to_double(bits: int) -> float:
    return lib().oracle_bf16_to_double(int(bits))


def double_to_bf16(v: float) -> int:
    return int(lib().oracle_double_to_bf16(float(v)))


# ------------------------------------------------------------------ steps

def route(scores, k: int, score_fn: str, renorm: int = 1):
    s = _np(scores, np.float32)
    T, E = s.shape
    ids = np.zeros((T, k), np.int32)
    w = np.zeros((T, k), np.float32)
    if lib().oracle_route(_ptr(s), T, E, k, SCORE_FN[score_fn], int(renorm), _ptr(ids), _ptr(w)):
        raise ValueError("oracle_route: invalid arguments")
    return ids, w


def permute(ids, E: int):
    a = _np(ids, np.int32)
    T, k = a.shape
    counts = np.zeros(E, np.int32)
    offsets = np.zeros(E + 1, np.int32)
    perm = np.zeros(T * k, np.int32)
    inv = np.zeros(T * k, np.int32)
    if lib().oracle_permute(_ptr(a), T, k, E, _ptr(counts), _ptr(offsets), _ptr(perm), _ptr(inv)):
        raise ValueError("oracle_permute: expert id out of range")
    return counts, offsets, perm, inv


WDTYPE = {"fp8": 0, "bf16": 1, "mxfp4": 2}


def _weights(ew, keep):
    """ctypes struct for a synth.ExpertWeights-like object (host copies kept alive in `keep`)."""
    wd = WDTYPE[ew.wdtype]
    mt = np.uint16 if wd == 1 else np.uint8
    mats = [_np(ew.gate, mt), _np(ew.up, mt), _np(ew.down, mt)]
    st = {0: np.float32, 2: np.uint8}.get(wd)
    scales = [None] * 3 if st is None else [_np(ew.s_gate, st), _np(ew.s_up, st), _np(ew.s_down, st)]
    keep.extend(mats + scales)
    n, I, H = mats[0].shape
    if wd == 2:  # two codes a byte along the input dimension
        H *= 2
    return _Weights(wd, n, H, I, *[_ptr(m) for m in mats], *[_ptr(s) for s in scales])


def fp4_e2m1_to_double(code: int) -> float:
    return lib().oracle_fp4_e2m1_to_double(code)


def e8m0_to_double(s: int) -> float:
    return lib().oracle_e8m0_to_double(s)


def float_to_e4m3fn(v: float) -> int:
    return lib().oracle_float_to_e4m3fn(float(v))


def act_scale_exp(amax: float) -> int:
    return lib().oracle_act_scale_exp(float(amax))


def quantize_rows(x, K: int):
    """bf16 bits [rows][K] -> (E4M3FN codes uint8 [rows][K], scale exponents int8 [rows][K/128])."""
    x = _np(x, np.uint16).reshape(-1, K)
    codes = np.zeros(x.shape, np.uint8)
    exps = np.zeros((x.shape[0], K // 128), np.int8)
    lib().oracle_quantize_rows(_ptr(x), x.shape[0], K, _ptr(codes), _ptr(exps))
    return codes, exps


def moe_layer(layer, rows=None, routed=None, expert_slot=None, with_shared=True, want_h=False,
              want_y=False, n_threads: int = 0, act_fp8: bool = False, expert_range=None):
    """Oracle of the whole layer for token rows `rows` (default: all).

    `layer` is a synth.Layer (its tensors may live on any device; they are copied to host).
    `routed` overrides layer.experts with a subset of experts (e.g. the ones the sampled rows
    select, copied from the device), in which case `expert_slot` maps expert id -> slot.
    Returns a dict with ids, w, out (bf16 bits, uint16) and optionally h and, with a shared
    expert, hS (its h) (uint16), y, S (float64).
    act_fp8: quantise the activations x and h to E4M3FN in 1x128 blocks first (the FP8 MFMA
    mode's arithmetic); h is reported before its quantisation.
    expert_range=(e_begin, e_end): evaluate and sum only those routed experts (one rank's local
    partial reduction under expert parallelism); the others' h and y are zeros.
    """
    keep = []
    scores = _np(layer.scores, np.float32)
    x = _np(layer.x, np.uint16)
    T, E, H, I, k = layer.T, layer.E, layer.H, layer.I, layer.k
    rw = _weights(routed if routed is not None else layer.experts, keep)
    sw = _weights(layer.shared, keep) if with_shared else None
    slot = None if expert_slot is None else _np(expert_slot, np.int32)
    r = None if rows is None else _np(np.asarray(rows), np.int32)
    n = T if r is None else len(r)
    res = dict(ids=np.zeros((n, k), np.int32), w=np.zeros((n, k), np.float32),
               out=np.zeros((n, H), np.uint16))
    if want_h:
        res["h"] = np.zeros((n, k, I), np.uint16)
        if sw is not None:
            res["hS"] = np.zeros((n, I), np.uint16)
    if want_y:
        res["y"] = np.zeros((n, k, H), np.float64)
        res["S"] = np.zeros((n, H), np.float64)
    rc = lib().oracle_moe_layer(
        _ptr(scores), _ptr(x), T, H, I, E, k, SCORE_FN[layer.score_fn], int(layer.renorm),
        ctypes.byref(rw), _ptr(slot), ctypes.byref(sw) if sw is not None else None,
        _ptr(r), n, _ptr(res["ids"]), _ptr(res["w"]), _ptr(res["out"]), _ptr(res.get("h")),
        _ptr(res.get("y")), _ptr(res.get("S")), int(n_threads), int(bool(act_fp8)),
        _ptr(res.get("hS")), *((0, E) if expert_range is None else map(int, expert_range)))
    if rc:
        raise ValueError("oracle_moe_layer: invalid arguments (row, k or expert slot)")
    return res


def expert_gate_up(x, token, slot, experts, n_threads: int = 0):
    """Phase 1 alone: h[p] = bf16(SiLU(Wg x_t) * (Wu x_t)) of expert slot[p] (a slot of
    `experts`, a synth.ExpertWeights) on token t = token[p] of x (bf16 bits [T][H]).  Returns
    bf16 bits [n, I]."""
    keep = []
    xb = _np(x, np.uint16)
    tok, sl = _np(np.asarray(token), np.int32), _np(np.asarray(slot), np.int32)
    W = _weights(experts, keep)
    h = np.zeros((len(tok), W.I), np.uint16)
    rc = lib().oracle_expert_gate_up(_ptr(xb), xb.shape[0], len(tok), _ptr(tok), _ptr(sl),
                                     ctypes.byref(W), _ptr(h), int(n_threads))
    if rc:
        raise ValueError("oracle_expert_gate_up: token or slot out of range")
    return h


def expert_down(h, slot, experts, n_threads: int = 0):
    """Phase 2 alone: y[p] = Wd h[p] (double) of expert slot[p] for bf16 rows h (bits [n][I])."""
    keep = []
    hb = _np(h, np.uint16)
    sl = _np(np.asarray(slot), np.int32)
    W = _weights(experts, keep)
    y = np.zeros((len(sl), W.H), np.float64)
    rc = lib().oracle_expert_down(_ptr(hb), len(sl), _ptr(sl), ctypes.byref(W), _ptr(y),
                                  int(n_threads))
    if rc:
        raise ValueError("oracle_expert_down: slot out of range")
    return y


def max_threads(n_threads: int = 0) -> int:
    return lib().oracle_max_threads(int(n_threads))


def bf16_bits_to_float(a) -> np.ndarray:
    """uint16 bf16 bit patterns -> float64 (host numpy)."""
    a = _np(a, np.uint16)
    return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


# ------------------------------------------------------------------ batched form


def dequantize(ew, which: int, n_threads: int = 0) -> np.ndarray:
    """Matrix `which` (0 gate [I, H], 1 up [I, H], 2 down [H, I]) of the single expert in `ew`
    (an ExpertWeights-like object holding one expert), dequantised exactly into float64."""
    keep = []
    W = _weights(ew, keep)
    if W.n != 1:
        raise ValueError("dequantize takes one expert")
    rows, cols = (W.H, W.I) if which == 2 else (W.I, W.H)
    out = np.empty((rows, cols), np.float64)
    if lib().oracle_dequantize(ctypes.byref(W), 0, int(which), _ptr(out), int(n_threads)):
        raise ValueError("oracle_dequantize: invalid arguments")
    return out


def silu_mul_bf16(g, u) -> np.ndarray:
    """bf16 bits of SiLU(g) * u element-wise (g, u float64 arrays of one shape)."""
    g = np.ascontiguousarray(g, np.float64)
    u = np.ascontiguousarray(u, np.float64)
    h = np.empty(g.shape, np.uint16)
    lib().oracle_silu_mul_bf16(_ptr(g), _ptr(u), g.size, _ptr(h))
    return h


def double_to_bf16_array(v) -> np.ndarray:
    v = np.ascontiguousarray(v, np.float64)
    out = np.empty(v.shape, np.uint16)
    lib().oracle_double_to_bf16_array(_ptr(v), v.size, _ptr(out))
    return out


def quantize_dequantize(v) -> np.ndarray:
    """The FP8 activation mode's 1x128 quantisation of rows of values (float64 [rows, K], each
    exact in fp32), returned dequantised (a new array)."""
    v = np.array(v, np.float64, copy=True, order="C")
    lib().oracle_quantize_dequantize(_ptr(v), v.shape[0], v.shape[1])
    return v


def _expert_on_rows(ew, X, act_fp8, n_threads):
    """One expert on activation rows X (float64 [n, H], already quantised in the FP8 mode):
    returns (h bf16 bits [n, I], y float64 [n, H]).  g = X Wg^T, u = X Wu^T and y = h Wd^T are
    float64 matrix products (the library's summation order instead of the plain loop's); the
    activation, its bf16 rounding and the FP8 mode's quantisation of h are the oracle's own."""
    Wg = dequantize(ew, 0, n_threads)
    G = X @ Wg.T
    del Wg
    Wu = dequantize(ew, 1, n_threads)
    U = X @ Wu.T
    del Wu
    hb = silu_mul_bf16(G, U)
    del G, U
    Hd = bf16_bits_to_float(hb)
    if act_fp8:
        Hd = quantize_dequantize(Hd)
    Wd = dequantize(ew, 2, n_threads)
    Y = Hd @ Wd.T
    return hb, Y


def moe_layer_batched(layer, rows=None, with_shared=True, want_h=False, want_y=False,
                      n_threads: int = 0, act_fp8: bool = False, expert_range=None):
    """The layer of moe_layer() for token rows `rows`, evaluated expert by expert: every expert
    that the rows select runs once over all of its (token, slot) assignments, found by scanning
    the rows' ids (no grouping is taken from anywhere), with its weights dequantised once and
    float64 matrix products for the sums.  Same definition, same roundings (h to bf16, out to
    bf16 from S + sum_j w_j y_j accumulated in double in that order) and same return dict as
    moe_layer(); only the order of the float64 sums inside the products differs.  This makes
    full-size layers cheap enough to check on every row."""
    T, E, H, I, k = layer.T, layer.E, layer.H, layer.I, layer.k
    r = np.arange(T, dtype=np.int64) if rows is None else np.asarray(rows, np.int64)
    n = len(r)
    scores = _np(layer.scores, np.float32)[r]
    ids, w = route(scores, k, layer.score_fn, layer.renorm)
    xb = _np(layer.x, np.uint16)[r]
    X = bf16_bits_to_float(xb)
    if act_fp8:
        X = quantize_dequantize(X)
    e0, e1 = (0, E) if expert_range is None else map(int, expert_range)
    y = np.zeros((n, k, H), np.float64)
    h = np.zeros((n, k, I), np.uint16) if want_h else None
    for e in np.unique(ids):
        if not e0 <= e < e1:
            continue
        ti, tj = np.nonzero(ids == e)  # the assignments (row, slot) that select expert e
        hb, Y = _expert_on_rows(layer.experts.select([int(e)]), X[ti], act_fp8, n_threads)
        y[ti, tj] = Y
        if want_h:
            h[ti, tj] = hb
    S = np.zeros((n, H), np.float64)
    hS = None
    if with_shared:
        hS, S = _expert_on_rows(layer.shared.select([0]), X, act_fp8, n_threads)
    acc = S.copy()
    wd = w.astype(np.float64)
    for j in range(k):
        local = (ids[:, j] >= e0) & (ids[:, j] < e1)
        acc += np.where(local, wd[:, j], 0.0)[:, None] * y[:, j]
    res = dict(ids=ids, w=w, out=double_to_bf16_array(acc))
    if want_h:
        res["h"] = h
        if with_shared:
            res["hS"] = hS
    if want_y:
        res["y"] = y
        res["S"] = S
    return res


def expert_gate_up_batched(x, token, slot, experts, n_threads: int = 0):
    """expert_gate_up() evaluated slot by slot (each slot's rows together, float64 library
    products); same definition and rounding."""
    xb = _np(x, np.uint16)
    tok, sl = np.asarray(token, np.int64), np.asarray(slot, np.int64)
    h = np.zeros((len(tok), experts.gate.shape[1]), np.uint16)
    for e in np.unique(sl):
        p = np.nonzero(sl == e)[0]
        one = experts.select([int(e)])
        X = bf16_bits_to_float(xb[tok[p]])
        G = X @ dequantize(one, 0, n_threads).T
        U = X @ dequantize(one, 1, n_threads).T
        h[p] = silu_mul_bf16(G, U)
    return h


def expert_down_batched(h, slot, experts, n_threads: int = 0):
    """expert_down() evaluated slot by slot; same definition (y = Wd h in float64)."""
    hb = _np(h, np.uint16)
    sl = np.asarray(slot, np.int64)
    H = experts.down.shape[1]
    y = np.zeros((len(sl), H), np.float64)
    for e in np.unique(sl):
        p = np.nonzero(sl == e)[0]
        y[p] = bf16_bits_to_float(hb[p]) @ dequantize(experts.select([int(e)]), 2, n_threads).T
    return y
