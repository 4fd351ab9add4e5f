"""Python binding of libmoe (include/libmoe.h): argument marshalling only.

Every function has the name of the C entry point it calls.  Tensors are torch tensors on the
GPU; calls enqueue on torch's current stream (or `stream=`) and do not synchronise.  Every step
of the MoE layer runs in libmoe's HIP kernels; this module only passes pointers and sizes.  A
missing libmoe.so is an error (build it with `python -m routed_expert_grouped_amd.build`).
"""
from __future__ import annotations

import ctypes
import os
import types

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_DEVICE = range(5)
MOE_SCORE_SOFTMAX, MOE_SCORE_SIGMOID = 0, 1
MOE_W_FP8_E4M3_B128, MOE_W_BF16, MOE_W_MXFP4_G32 = 0, 1, 2
SCORE_FN = {"softmax": MOE_SCORE_SOFTMAX, "sigmoid": MOE_SCORE_SIGMOID}

EXPORTS = ("moe_route", "moe_permute_workspace_size", "moe_permute", "moe_expert_gate_up", "moe_expert_down",
           "moe_expert_gate_up_shared", "moe_expert_down_shared",
           "moe_expert_ffn_workspace_size", "moe_expert_ffn", "moe_combine", "moe_quantize_act",
           "moe_expert_gate_up_a8", "moe_expert_down_a8", "moe_expert_ffn_a8_workspace_size",
           "moe_expert_ffn_a8", "moe_combine_partial", "moe_route_permute",
           "moe_permute_noalloc", "moe_status_string")


class MoeError(RuntimeError):
    def __init__(self, call: str, status: int):
        self.status = status
        super().__init__(f"{call} failed: {moe_status_string(status)} ({status})")


class MoeExpertWeights(ctypes.Structure):
    """ctypes mirror of moe_expert_weights."""
    _fields_ = [("dtype", ctypes.c_int32), ("n_groups", ctypes.c_int32), ("H", ctypes.c_int32),
                ("I", ctypes.c_int32), ("w_gate", ctypes.c_void_p), ("w_up", ctypes.c_void_p),
                ("w_down", ctypes.c_void_p), ("s_gate", ctypes.c_void_p), ("s_up", ctypes.c_void_p),
                ("s_down", ctypes.c_void_p)]


_lib = None


def lib():
    """The loaded libmoe.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libmoe.so not found at {LIB_PATH}; build it with "
                               "`python -m routed_expert_grouped_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P, i32, st = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int
        W = ctypes.POINTER(MoeExpertWeights)
        L.moe_route.argtypes = [P, i32, i32, i32, i32, i32, P, P, P]
        L.moe_permute_workspace_size.argtypes = [i32, i32, i32, ctypes.POINTER(ctypes.c_size_t)]
        L.moe_permute.argtypes = [P, i32, i32, i32, P, P, P, P, P, ctypes.c_size_t, P]
        L.moe_permute_noalloc.argtypes = [P, i32, i32, i32, P, P, P, P, P]
        L.moe_route_permute.argtypes = [P, i32, i32, i32, i32, i32, P, P, P, P, P, P, P]
        L.moe_expert_gate_up.argtypes = [P, i32, i32, P, P, W, P, P]
        L.moe_expert_down.argtypes = [P, i32, i32, P, W, P, P]
        L.moe_expert_gate_up_shared.argtypes = [P, i32, i32, P, P, W, W, P, P]
        L.moe_expert_down_shared.argtypes = [P, i32, i32, P, W, W, P, P]
        L.moe_expert_ffn_workspace_size.argtypes = [i32, i32, W, ctypes.POINTER(ctypes.c_size_t)]
        L.moe_expert_ffn.argtypes = [P, i32, i32, P, P, W, P, P, ctypes.c_size_t, P]
        L.moe_combine.argtypes = [P, P, P, P, i32, i32, i32, P, P]
        L.moe_combine_partial.argtypes = [P, P, P, P, i32, i32, P, i32, i32, i32, P, P]
        L.moe_quantize_act.argtypes = [P, i32, i32, P, P, i32, P]
        L.moe_expert_gate_up_a8.argtypes = [P, P, i32, i32, i32, P, P, W, P, P]
        L.moe_expert_down_a8.argtypes = [P, P, i32, i32, i32, P, W, P, P]
        L.moe_expert_ffn_a8_workspace_size.argtypes = [i32, i32, W,
                                                       ctypes.POINTER(ctypes.c_size_t)]
        L.moe_expert_ffn_a8.argtypes = [P, i32, i32, P, P, W, P, P, ctypes.c_size_t, P]
        for name in EXPORTS[:-1]:
            getattr(L, name).restype = st
        L.moe_status_string.argtypes = [st]
        L.moe_status_string.restype = ctypes.c_char_p
        _lib = L
    return _lib


def _p(t):
    """Device pointer of a tensor (None -> NULL)."""
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _s(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check(call, status):
    if status != MOE_OK:
        raise MoeError(call, status)


def moe_status_string(status: int) -> str:
    return lib().moe_status_string(int(status)).decode()


WDTYPE = {"fp8": MOE_W_FP8_E4M3_B128, "bf16": MOE_W_BF16, "mxfp4": MOE_W_MXFP4_G32}


def expert_weights(ew) -> MoeExpertWeights:
    """moe_expert_weights for an object with .wdtype ("fp8", "bf16" or "mxfp4"), .gate/.up/.down
    and .s_gate/.s_up/.s_down device tensors (the arrays must outlive the calls that use it)."""
    n, I, H = ew.gate.shape
    if ew.wdtype == "mxfp4":
        H *= 2  # two codes a byte along the input dimension
    scaled = ew.wdtype != "bf16"
    return MoeExpertWeights(WDTYPE[ew.wdtype], n, H, I,
                            ew.gate.data_ptr(), ew.up.data_ptr(), ew.down.data_ptr(),
                            ew.s_gate.data_ptr() if scaled else None,
                            ew.s_up.data_ptr() if scaled else None,
                            ew.s_down.data_ptr() if scaled else None)


def expert_slice(ew, e_begin: int, e_end: int):
    """Experts e_begin .. e_end - 1 of an object accepted by expert_weights(), as views of the
    same arrays (no copy): the weights one rank holds under expert parallelism."""
    return types.SimpleNamespace(
        wdtype=ew.wdtype, gate=ew.gate[e_begin:e_end], up=ew.up[e_begin:e_end],
        down=ew.down[e_begin:e_end],
        **{n: (None if getattr(ew, n) is None else getattr(ew, n)[e_begin:e_end])
           for n in ("s_gate", "s_up", "s_down")})


def moe_route(scores, k: int, score_fn="sigmoid", renorm: int = 1, topk_ids=None, topk_w=None,
              stream=None):
    T, E = scores.shape
    if topk_ids is None:
        topk_ids = torch.empty((T, k), dtype=torch.int32, device=scores.device)
    if topk_w is None:
        topk_w = torch.empty((T, k), dtype=torch.float32, device=scores.device)
    fn = SCORE_FN[score_fn] if isinstance(score_fn, str) else int(score_fn)
    _check("moe_route", lib().moe_route(_p(scores), T, E, k, fn, int(renorm), _p(topk_ids),
                                        _p(topk_w), _s(stream)))
    return topk_ids, topk_w


FUSED_ROUTE_PERMUTE_MAX = 2048  # assignments up to which moe_route_permute runs


def moe_route_permute(scores, k: int, score_fn="sigmoid", renorm: int = 1, topk_ids=None,
                      topk_w=None, counts=None, offsets=None, perm=None, inv=None, stream=None):
    """moe_route + moe_permute in one launch (T*k <= 2048); returns ids, w, counts, offsets,
    perm, inv."""
    T, E = scores.shape
    dev, i32 = scores.device, torch.int32
    topk_ids = torch.empty((T, k), dtype=i32, device=dev) if topk_ids is None else topk_ids
    topk_w = torch.empty((T, k), dtype=torch.float32, device=dev) if topk_w is None else topk_w
    counts = torch.empty(E, dtype=i32, device=dev) if counts is None else counts
    offsets = torch.empty(E + 1, dtype=i32, device=dev) if offsets is None else offsets
    perm = torch.empty(max(1, T * k), dtype=i32, device=dev) if perm is None else perm
    inv = torch.empty(max(1, T * k), dtype=i32, device=dev) if inv is None else inv
    fn = SCORE_FN[score_fn] if isinstance(score_fn, str) else int(score_fn)
    _check("moe_route_permute",
           lib().moe_route_permute(_p(scores), T, E, k, fn, int(renorm), _p(topk_ids), _p(topk_w),
                                   _p(counts), _p(offsets), _p(perm), _p(inv), _s(stream)))
    return topk_ids, topk_w, counts, offsets, perm, inv


def moe_permute_workspace_size(T: int, k: int, E: int) -> int:
    n = ctypes.c_size_t(0)
    _check("moe_permute_workspace_size",
           lib().moe_permute_workspace_size(T, k, E, ctypes.byref(n)))
    return n.value


def moe_permute(topk_ids, E: int, counts=None, offsets=None, perm=None, inv=None, ws=None,
                stream=None):
    """Returns counts, offsets, perm, inv.  `ws` (uint8 device tensor) is the call's workspace;
    None allocates one of moe_permute_workspace_size bytes (the caller must keep a passed one
    untouched until the stream has run the call)."""
    T, k = topk_ids.shape
    dev = topk_ids.device
    counts = torch.empty(E, dtype=torch.int32, device=dev) if counts is None else counts
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev) if offsets is None else offsets
    perm = torch.empty(T * k, dtype=torch.int32, device=dev) if perm is None else perm
    inv = torch.empty(T * k, dtype=torch.int32, device=dev) if inv is None else inv
    if ws is None:
        need = moe_permute_workspace_size(T, k, E)
        ws = torch.empty(need, dtype=torch.uint8, device=dev) if need else None
    _check("moe_permute", lib().moe_permute(_p(topk_ids), T, k, E, _p(counts), _p(offsets),
                                            _p(perm), _p(inv), _p(ws),
                                            0 if ws is None else ws.numel(), _s(stream)))
    return counts, offsets, perm, inv


PERMUTE_NOALLOC_MAX_BYTES = 1 << 20  # MOE_PERMUTE_NOALLOC_MAX_BYTES


def moe_permute_noalloc(topk_ids, E: int, counts, offsets, perm, inv, stream=None):
    """moe_permute with the library's static count table instead of a workspace (the caller
    passes every output buffer; nothing is allocated here or in the call)."""
    T, k = topk_ids.shape
    _check("moe_permute_noalloc",
           lib().moe_permute_noalloc(_p(topk_ids), T, k, E, _p(counts), _p(offsets), _p(perm),
                                     _p(inv), _s(stream)))
    return counts, offsets, perm, inv


def moe_expert_gate_up(x, k: int, perm, offsets, w: MoeExpertWeights, h=None, stream=None):
    T = x.shape[0]
    if h is None:
        h = torch.empty((T * k, w.I), dtype=torch.int16, device=x.device)
    _check("moe_expert_gate_up", lib().moe_expert_gate_up(
        _p(x), T, k, _p(perm), _p(offsets), ctypes.byref(w), _p(h), _s(stream)))
    return h


def moe_expert_down(h, T: int, k: int, offsets, w: MoeExpertWeights, y=None, stream=None):
    if y is None:
        y = torch.empty((T * k, w.H), dtype=torch.int16, device=h.device)
    _check("moe_expert_down", lib().moe_expert_down(
        _p(h), T, k, _p(offsets), ctypes.byref(w), _p(y), _s(stream)))
    return y


def moe_expert_gate_up_shared(x, k: int, perm, offsets, w: MoeExpertWeights, ws: MoeExpertWeights,
                              h=None, stream=None):
    """Routed gate/up over the T*k grouped rows and the shared expert's over T more rows (h has
    T*k + T rows; row T*k + t is token t's shared-expert h)."""
    T = x.shape[0]
    if h is None:
        h = torch.empty((T * k + T, w.I), dtype=torch.int16, device=x.device)
    _check("moe_expert_gate_up_shared", lib().moe_expert_gate_up_shared(
        _p(x), T, k, _p(perm), _p(offsets), ctypes.byref(w), ctypes.byref(ws), _p(h), _s(stream)))
    return h


def moe_expert_down_shared(h, T: int, k: int, offsets, w: MoeExpertWeights, ws: MoeExpertWeights,
                           y=None, stream=None):
    """Down projection of moe_expert_gate_up_shared's h: y has T*k + T rows, the shared expert's
    output from row T*k on."""
    if y is None:
        y = torch.empty((T * k + T, w.H), dtype=torch.int16, device=h.device)
    _check("moe_expert_down_shared", lib().moe_expert_down_shared(
        _p(h), T, k, _p(offsets), ctypes.byref(w), ctypes.byref(ws), _p(y), _s(stream)))
    return y


def moe_expert_ffn_workspace_size(T: int, k: int, w: MoeExpertWeights) -> int:
    n = ctypes.c_size_t(0)
    _check("moe_expert_ffn_workspace_size",
           lib().moe_expert_ffn_workspace_size(T, k, ctypes.byref(w), ctypes.byref(n)))
    return n.value


def moe_expert_ffn(x, k: int, perm, offsets, w: MoeExpertWeights, y=None, ws=None, stream=None):
    T = x.shape[0]
    if y is None:
        y = torch.empty((T * k, w.H), dtype=torch.int16, device=x.device)
    if ws is None:
        ws = torch.empty(max(1, moe_expert_ffn_workspace_size(T, k, w)), dtype=torch.uint8,
                         device=x.device)
    _check("moe_expert_ffn", lib().moe_expert_ffn(
        _p(x), T, k, _p(perm), _p(offsets), ctypes.byref(w), _p(y), _p(ws), ws.numel(),
        _s(stream)))
    return y, ws


def moe_combine(y, inv, topk_w, shared_y, T: int, k: int, H: int, out=None, stream=None):
    if out is None:
        out = torch.empty((T, H), dtype=torch.int16, device=y.device)
    _check("moe_combine", lib().moe_combine(_p(y), _p(inv), _p(topk_w), _p(shared_y), T, k, H,
                                            _p(out), _s(stream)))
    return out


def moe_combine_partial(y, inv, topk_ids, topk_w, e_begin: int, e_end: int, shared_y, T: int,
                        k: int, H: int, out=None, stream=None):
    if out is None:
        out = torch.empty((T, H), dtype=torch.int16, device=y.device)
    _check("moe_combine_partial",
           lib().moe_combine_partial(_p(y), _p(inv), _p(topk_ids), _p(topk_w), int(e_begin),
                                     int(e_end), _p(shared_y), T, k, H, _p(out), _s(stream)))
    return out


def exp_pitch(K: int) -> int:
    """Exponent row pitch that the FP8-activation phase calls take: K/128 rounded up to 16."""
    return (K // 128 + 15) // 16 * 16


def moe_quantize_act(x, codes=None, exps=None, pitch=None, stream=None):
    """FP8 activation quantisation of bf16 bits x [rows, K]: (codes uint8 [rows, K], exps int8
    [rows, pitch]; the exponents of row r are exps[r, :K/128])."""
    rows, K = x.shape
    pitch = exp_pitch(K) if pitch is None else pitch
    if codes is None:
        codes = torch.empty((rows, K), dtype=torch.uint8, device=x.device)
    if exps is None:
        exps = torch.empty((rows, max(1, pitch)), dtype=torch.int8, device=x.device)
    _check("moe_quantize_act", lib().moe_quantize_act(_p(x), rows, K, _p(codes), _p(exps), pitch,
                                                      _s(stream)))
    return codes, exps


def moe_expert_gate_up_a8(codes, exps, k: int, perm, offsets, w: MoeExpertWeights, h=None,
                          stream=None):
    T = codes.shape[0]
    if h is None:
        h = torch.empty((T * k, w.I), dtype=torch.int16, device=codes.device)
    _check("moe_expert_gate_up_a8", lib().moe_expert_gate_up_a8(
        _p(codes), _p(exps), exps.shape[1], T, k, _p(perm), _p(offsets), ctypes.byref(w), _p(h),
        _s(stream)))
    return h


def moe_expert_down_a8(codes, exps, T: int, k: int, offsets, w: MoeExpertWeights, y=None,
                       stream=None):
    if y is None:
        y = torch.empty((T * k, w.H), dtype=torch.int16, device=codes.device)
    _check("moe_expert_down_a8", lib().moe_expert_down_a8(
        _p(codes), _p(exps), exps.shape[1], T, k, _p(offsets), ctypes.byref(w), _p(y),
        _s(stream)))
    return y


def moe_expert_ffn_a8_workspace_size(T: int, k: int, w: MoeExpertWeights) -> int:
    n = ctypes.c_size_t(0)
    _check("moe_expert_ffn_a8_workspace_size",
           lib().moe_expert_ffn_a8_workspace_size(T, k, ctypes.byref(w), ctypes.byref(n)))
    return n.value


def moe_expert_ffn_a8(x, k: int, perm, offsets, w: MoeExpertWeights, y=None, ws=None,
                      stream=None):
    T = x.shape[0]
    if y is None:
        y = torch.empty((T * k, w.H), dtype=torch.int16, device=x.device)
    if ws is None:
        ws = torch.empty(max(1, moe_expert_ffn_a8_workspace_size(T, k, w)), dtype=torch.uint8,
                         device=x.device)
    _check("moe_expert_ffn_a8", lib().moe_expert_ffn_a8(
        _p(x), T, k, _p(perm), _p(offsets), ctypes.byref(w), _p(y), _p(ws), ws.numel(),
        _s(stream)))
    return y, ws


def _permute_ws(T, k, E, device):
    """moe_permute's workspace for T tokens (a 16-byte stand-in when none is needed)."""
    return torch.empty(max(16, moe_permute_workspace_size(T, k, E)), dtype=torch.uint8,
                       device=device)


class MoeLayer:
    """Buffers and the call sequence of one MoE layer forward: route -> permute (one launch,
    moe_route_permute, for T*k <= 2048) -> routed gate/up -> routed down -> combine on the
    caller's stream.  The shared expert (which only needs x) runs inside the routed launches at
    decode sizes (fuse_shared, below), and otherwise on a second stream that runs alongside the
    routed experts and joins before combine.

    `experts` and `shared` are objects accepted by expert_weights(); `x` is bf16 bits [T, H]
    (torch.int16) and `scores` fp32 [T, E], all on the GPU.

    fuse_shared: at decode sizes (T*k <= 32*E, bf16 activations) the shared expert can run inside
    the routed launches as an extra group (moe_expert_gate_up_shared / moe_expert_down_shared):
    one grid per phase, no second stream, no cross-stream waits; the extra group's tiles take the
    first workgroups, spread over the XCDs.  "auto" does so wherever it applies: the tiny layer
    0.035 against 0.092 ms a step, the DeepSeek-V3 decode layer 0.638 against 0.648 ms (FP8
    weights) and 0.363 against 0.372 ms (MXFP4) with the side stream.  True / False force it.
    `h`, `y`, `sh_h` and `sh_y` are then views of the shared buffers.

    overlap_shared=False runs the shared expert on the caller's stream after the routed experts
    instead of on the side stream (measured equal or slower at every layer size: the side stream
    fills CUs left idle by the routing kernels and by the routed GEMMs' last tiles).

    act="fp8" selects the FP8 activation mode (moe_expert_ffn_a8) for the routed and the shared
    experts; `h` then views the routed h inside the workspace, before its quantisation.

    capture(scores, x) records the forward into a HIP graph and replay() reruns it.
    """

    def __init__(self, T, H, I, E, k, experts, shared, score_fn="sigmoid", renorm=1, device="cuda",
                 overlap_shared=True, act="bf16", fuse_shared="auto"):
        if act not in ("bf16", "fp8"):
            raise ValueError(f"act must be 'bf16' or 'fp8', not {act!r}")
        self.T, self.H, self.I, self.E, self.k = T, H, I, E, k
        self.act = act
        self.score_fn, self.renorm = score_fn, renorm
        self.w = expert_weights(experts)
        self.ws_ = expert_weights(shared) if shared is not None else None
        self._keep = (experts, shared)
        d, i32 = device, torch.int32
        self.topk_ids = torch.empty((T, k), dtype=i32, device=d)
        self.topk_w = torch.empty((T, k), dtype=torch.float32, device=d)
        self.counts = torch.empty(E, dtype=i32, device=d)
        self.offsets = torch.empty(E + 1, dtype=i32, device=d)
        self.perm = torch.empty(max(1, T * k), dtype=i32, device=d)
        self.inv = torch.empty(max(1, T * k), dtype=i32, device=d)
        self.perm_ws = _permute_ws(T, k, E, d)
        if act == "fp8":
            self.ws = torch.empty(max(1, moe_expert_ffn_a8_workspace_size(T, k, self.w)),
                                  dtype=torch.uint8, device=d)
            # h (before its quantisation) opens the workspace
            self.h = self.ws[:max(1, T * k) * I * 2].view(torch.int16).view(-1, I)
            self.sh_ws = self.sh_h = None
            if shared is not None:
                self.sh_ws = torch.empty(max(1, moe_expert_ffn_a8_workspace_size(T, 1, self.ws_)),
                                         dtype=torch.uint8, device=d)
                self.sh_h = self.sh_ws[:max(1, T) * I * 2].view(torch.int16).view(-1, I)
        # the shared expert as an extra group of the routed decode launches
        if fuse_shared == "auto":
            fuse_shared = True
        self.fused = (bool(fuse_shared) and act == "bf16" and shared is not None and T > 0
                      and T * k <= 32 * E and self.ws_.dtype == self.w.dtype
                      and self.ws_.H == self.w.H and self.ws_.I == self.w.I)
        if self.fused:
            self.h_all = torch.empty((T * k + T, I), dtype=torch.int16, device=d)
            self.y_all = torch.empty((T * k + T, H), dtype=torch.int16, device=d)
            self.h, self.sh_h = self.h_all[:T * k], self.h_all[T * k:]
            self.y, self.sh_y = self.y_all[:T * k], self.y_all[T * k:]
        else:
            if act != "fp8":
                self.h = torch.empty((max(1, T * k), I), dtype=torch.int16, device=d)
                self.sh_h = torch.empty((max(1, T), I), dtype=torch.int16, device=d)
            self.y = torch.empty((max(1, T * k), H), dtype=torch.int16, device=d)
            self.sh_y = torch.empty((max(1, T), H), dtype=torch.int16, device=d)
        self.out = torch.empty((max(1, T), H), dtype=torch.int16, device=d)
        self.side = (torch.cuda.Stream(device=d)
                     if (overlap_shared and shared is not None and not self.fused) else None)

    def capture(self, scores, x):
        """Record one forward on the tensors `scores` and `x` into a HIP graph; replay() reruns it
        on whatever they hold then.  None of the layer's calls allocates or clears memory, so the
        whole sequence (both streams) can be captured."""
        warm = torch.cuda.Stream()
        warm.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(warm):
            self.forward(scores, x)
        torch.cuda.current_stream().wait_stream(warm)
        torch.cuda.synchronize()
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            self.forward(scores, x)
        return self.graph

    def replay(self):
        """Enqueue the captured forward on torch's current stream; returns `out`."""
        self.graph.replay()
        return self.out

    def _route_permute(self, scores, stream):
        """Routing and grouping; one launch for decode-sized batches."""
        k = self.k
        if self.T * k <= FUSED_ROUTE_PERMUTE_MAX:
            moe_route_permute(scores, k, self.score_fn, self.renorm, self.topk_ids, self.topk_w,
                              self.counts, self.offsets, self.perm, self.inv, stream)
        else:
            moe_route(scores, k, self.score_fn, self.renorm, self.topk_ids, self.topk_w, stream)
            moe_permute(self.topk_ids, self.E, self.counts, self.offsets, self.perm, self.inv,
                        self.perm_ws, stream)

    def _shared(self, x, st):
        if self.act == "fp8":
            moe_expert_ffn_a8(x, 1, None, None, self.ws_, self.sh_y, self.sh_ws, st)
        else:
            moe_expert_gate_up(x, 1, None, None, self.ws_, self.sh_h, st)
            moe_expert_down(self.sh_h, self.T, 1, None, self.ws_, self.sh_y, st)

    def forward(self, scores, x, stream=None, gate_up_events=None):
        """Enqueue the layer; returns `out` (bf16 bits [T, H]).  gate_up_events=(start, stop)
        records torch events around the routed gate/up kernel (for timing; bf16 mode only)."""
        T, k = self.T, self.k
        main = torch.cuda.current_stream() if stream is None else stream
        shared_y = None
        if self.ws_ is not None and self.side is not None:
            # shared expert on the side stream, ordered after everything already on `main`
            self.side.wait_stream(main)
            self._shared(x, self.side)
            shared_y = self.sh_y
        self._route_permute(scores, stream)
        if self.fused:
            if gate_up_events is not None:  # (here the routed and the shared gate/up)
                gate_up_events[0].record(stream)
            moe_expert_gate_up_shared(x, k, self.perm, self.offsets, self.w, self.ws_, self.h_all,
                                      stream)
            if gate_up_events is not None:
                gate_up_events[1].record(stream)
            moe_expert_down_shared(self.h_all, T, k, self.offsets, self.w, self.ws_, self.y_all,
                                   stream)
            moe_combine(self.y, self.inv, self.topk_w, self.sh_y, T, k, self.H, self.out, stream)
            return self.out
        if self.act == "fp8":
            moe_expert_ffn_a8(x, k, self.perm, self.offsets, self.w, self.y, self.ws, stream)
        else:
            if gate_up_events is not None:
                gate_up_events[0].record(stream)
            moe_expert_gate_up(x, k, self.perm, self.offsets, self.w, self.h, stream)
            if gate_up_events is not None:
                gate_up_events[1].record(stream)
            moe_expert_down(self.h, T, k, self.offsets, self.w, self.y, stream)
        if self.ws_ is not None and self.side is None:
            self._shared(x, stream)
            shared_y = self.sh_y
        elif self.side is not None:
            main.wait_stream(self.side)
        moe_combine(self.y, self.inv, self.topk_w, shared_y, T, k, self.H, self.out, stream)
        return self.out


class MoeRankShare:
    """One rank's share of the layer under expert parallelism over G ranks, as in the SmallEP
    scheme of the OSDI'26 hybrid-inference article (SmallEP section): after the tokens are
    all-gathered, every rank routes and groups all T tokens (redundantly), runs its local routed
    experts [e_begin, e_end) on the assignments that select them, and reduces their weighted
    outputs to a partial [T, H] (moe_combine_partial); the partials are then exchanged and
    summed.  The shared expert runs on the rank's own token rows [t_begin, t_end).

    `experts` holds all E experts' weights (only the local slice is ever read: expert_slice);
    forward() returns (partial [T, H], shared output [t_end - t_begin, H]), bf16 bits.  The
    collectives are not part of this single-GPU build.
    """

    def __init__(self, T, H, I, E, k, experts, shared, e_begin, e_end, t_begin, t_end,
                 score_fn="sigmoid", renorm=1, device="cuda"):
        if not (0 <= e_begin <= e_end <= E and 0 <= t_begin <= t_end <= T):
            raise ValueError("expert or token range out of bounds")
        self.T, self.H, self.I, self.E, self.k = T, H, I, E, k
        self.e0, self.e1, self.t0, self.t1 = e_begin, e_end, t_begin, t_end
        self.score_fn, self.renorm = score_fn, renorm
        local = expert_slice(experts, e_begin, e_end)
        self.w = expert_weights(local) if e_end > e_begin else None
        self.ws_ = expert_weights(shared) if shared is not None else None
        self._keep = (experts, shared, local)
        d, i32 = device, torch.int32
        self.topk_ids = torch.empty((T, k), dtype=i32, device=d)
        self.topk_w = torch.empty((T, k), dtype=torch.float32, device=d)
        self.counts = torch.empty(E, dtype=i32, device=d)
        self.offsets = torch.empty(E + 1, dtype=i32, device=d)
        self.perm = torch.empty(max(1, T * k), dtype=i32, device=d)
        self.inv = torch.empty(max(1, T * k), dtype=i32, device=d)
        self.perm_ws = _permute_ws(T, k, E, d)
        self.h = torch.empty((max(1, T * k), I), dtype=torch.int16, device=d)
        self.y = torch.empty((max(1, T * k), H), dtype=torch.int16, device=d)
        self.out = torch.empty((max(1, T), H), dtype=torch.int16, device=d)
        nt = max(1, t_end - t_begin)
        self.sh_h = torch.empty((nt, I), dtype=torch.int16, device=d)
        self.sh_y = torch.empty((nt, H), dtype=torch.int16, device=d)

    def forward(self, scores, x, stream=None, gate_up_events=None):
        T, k = self.T, self.k
        if T * k <= FUSED_ROUTE_PERMUTE_MAX:
            moe_route_permute(scores, k, self.score_fn, self.renorm, self.topk_ids, self.topk_w,
                              self.counts, self.offsets, self.perm, self.inv, stream)
        else:
            moe_route(scores, k, self.score_fn, self.renorm, self.topk_ids, self.topk_w, stream)
            moe_permute(self.topk_ids, self.E, self.counts, self.offsets, self.perm, self.inv,
                        self.perm_ws, stream)
        if self.w is not None:
            offs = self.offsets[self.e0:]  # the local experts' slice of the grouping
            if gate_up_events is not None:
                gate_up_events[0].record(stream)
            moe_expert_gate_up(x, k, self.perm, offs, self.w, self.h, stream)
            if gate_up_events is not None:
                gate_up_events[1].record(stream)
            moe_expert_down(self.h, T, k, offs, self.w, self.y, stream)
        moe_combine_partial(self.y, self.inv, self.topk_ids, self.topk_w, self.e0, self.e1, None,
                            T, k, self.H, self.out, stream)
        if self.ws_ is not None and self.t1 > self.t0:
            xs = x[self.t0:self.t1]
            moe_expert_gate_up(xs, 1, None, None, self.ws_, self.sh_h, stream)
            moe_expert_down(self.sh_h, self.t1 - self.t0, 1, None, self.ws_, self.sh_y, stream)
        return self.out, self.sh_y
