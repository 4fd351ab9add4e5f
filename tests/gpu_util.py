"""Helpers of the GPU tests: run the libmoe path on a synth.Layer and compare with the oracle."""
from __future__ import annotations

import numpy as np
import torch

import oracle
import routed_expert_grouped_amd as moe
import synth

ROW_TOL = 1e-2  # per-row relative L2 bound on float outputs (h, y, shared, out)
W_TOL = 1e-6  # absolute bound on the routing weights
# FP8 activation mode.  h is quantised to E4M3FN before the down projection, and h is itself a
# rounded result: the GPU's (fp32 sums) and the oracle's (double) may differ by a bf16 ulp, and
# where such an h value sits on an E4M3 rounding midpoint (or a block's largest magnitude on a
# scale boundary) the two sides quantise it one step apart -- both correctly for their own h.
# y is linear in the dequantised h, so the exact effect of those steps is added to the oracle's
# y (and through it to S and out) before the usual per-row bound is applied; see a8_correction.
DEV = "cuda"

_layers = {}


def layer_for(cfg, seed=0, **over):
    """Layers are cached per session (the large ones share their weights across configs)."""
    key = (cfg if isinstance(cfg, str) else tuple(sorted(cfg.items())), seed, tuple(sorted(over.items())))
    if key not in _layers:
        c = synth.CONFIGS[cfg] if isinstance(cfg, str) else cfg
        big = c["H"] * c["I"] * c["E"] > 1 << 26
        if big:
            _layers[key] = synth.make_layer(cfg, seed=seed, device=DEV, **over)
        else:  # small layers are drawn on the host, then copied
            _layers[key] = synth.make_layer(cfg, seed=seed, **over).to(DEV)
    return _layers[key]


def mid(**over):
    c = dict(T=200, H=512, I=384, E=24, k=4, score_fn="sigmoid", scores="uniform", wdtype="fp8")
    c.update(over)
    return c


GUARD = 4096  # bytes of sentinel before and after every output buffer of run_gpu
SENTINEL = 0xA5


def _guarded(L, name):
    """Replace tensor attribute `name` of L by a view of the same shape inside a buffer with
    GUARD sentinel bytes on both sides; returns the buffer."""
    t = getattr(L, name)
    nbytes = t.numel() * t.element_size()
    buf = torch.full((nbytes + 2 * GUARD,), SENTINEL, dtype=torch.uint8, device=t.device)
    setattr(L, name, buf[GUARD:GUARD + nbytes].view(t.dtype).view(t.shape))
    return buf


def _guard_layer(L):
    """Guard every buffer the layer's calls write (and re-derive the views into them)."""
    T, k, I = L.T, L.k, L.I
    names = ["out", "topk_ids", "topk_w", "counts", "offsets", "perm", "inv", "perm_ws"]
    if L.fused:
        names += ["h_all", "y_all"]
    elif L.act == "fp8":
        names += ["ws", "y"] + (["sh_ws", "sh_y"] if L.sh_ws is not None else [])
    else:
        names += ["h", "y", "sh_h", "sh_y"]
    bufs = {n: _guarded(L, n) for n in names}
    if L.fused:
        L.h, L.sh_h = L.h_all[:T * k], L.h_all[T * k:]
        L.y, L.sh_y = L.y_all[:T * k], L.y_all[T * k:]
    elif L.act == "fp8":
        L.h = L.ws[:max(1, T * k) * I * 2].view(torch.int16).view(-1, I)
        if L.sh_ws is not None:
            L.sh_h = L.sh_ws[:max(1, T) * I * 2].view(torch.int16).view(-1, I)
    return bufs


def _check_guards(bufs):
    for name, buf in bufs.items():
        for side, part in (("before", buf[:GUARD]), ("after", buf[-GUARD:])):
            bad = int((part != SENTINEL).sum())
            assert bad == 0, f"{bad} guard bytes {side} {name} were overwritten"


def run_gpu(layer, stream=None, act="bf16"):
    """Run the full layer through the C ABI; return host copies of every intermediate.  Every
    buffer the calls write sits between sentinel bytes, which must be untouched afterwards."""
    L = moe.MoeLayer(layer.T, layer.H, layer.I, layer.E, layer.k, layer.experts, layer.shared,
                     layer.score_fn, layer.renorm, act=act)
    bufs = _guard_layer(L)
    L.forward(layer.scores, layer.x, stream)
    torch.cuda.synchronize()
    _check_guards(bufs)
    T, k = layer.T, layer.k
    c = lambda t: t.detach().cpu().numpy()
    return dict(ids=c(L.topk_ids), w=c(L.topk_w), counts=c(L.counts), offsets=c(L.offsets),
                perm=c(L.perm[:T * k]), inv=c(L.inv[:T * k]),
                h=c(L.h[:T * k]).view(np.uint16), y=c(L.y[:T * k]).view(np.uint16),
                hS=c(L.sh_h[:T]).view(np.uint16), S=c(L.sh_y[:T]).view(np.uint16),
                out=c(L.out[:T]).view(np.uint16))


def block_exponents(h_bits, K):
    """Scale exponent of every 128-block of bf16 rows (bits [n, K]): the smallest e with
    max|v| <= 448 * 2^e, clamped to [-127, 127], 0 for an all-zero block; and the largest
    magnitude's bit pattern."""
    h = np.asarray(h_bits, np.uint16).reshape(-1, K // 128, 128)
    amax_bits = (h & 0x7FFF).max(-1)
    m, E = np.frexp(oracle.bf16_bits_to_float(amax_bits))  # exact: amax = m 2^E, m in [0.5, 1)
    e = np.where(m <= 0.875, E - 9, E - 8)
    e = np.where(amax_bits == 0, 0, np.clip(e, -127, 127))
    return e, amax_bits.astype(np.int64)


def quantise_dequantise(h_bits, K):
    """bf16 rows (bits [n, K]) through the FP8 mode's quantiser and back, in float64: exponents
    from block_exponents, codes from torch's E4M3FN cast (round to nearest even) of v * 2^-e in
    float32."""
    e, _ = block_exponents(h_bits, K)
    v = oracle.bf16_bits_to_float(h_bits).reshape(-1, K // 128, 128)
    s = np.exp2(-e.astype(np.float64))[..., None]
    q = torch.from_numpy((v * s).astype(np.float32)).to(torch.float8_e4m3fn).to(torch.float64)
    return (q.numpy() / s).reshape(-1, K)


_FP4 = None
_E8M0 = None


def down_columns(ew, e, cols):
    """Columns `cols` of expert e's down matrix [H][I], dequantised (FP8 code x block scale, or
    MXFP4 code x E8M0 group scale)."""
    idx = torch.as_tensor(cols, dtype=torch.long, device=ew.down.device)
    if ew.wdtype == "mxfp4":
        global _FP4, _E8M0
        if _FP4 is None:
            _FP4 = np.array([oracle.fp4_e2m1_to_double(c) for c in range(16)])
            _E8M0 = np.array([oracle.e8m0_to_double(v) for v in range(256)])
        b = ew.down[e].index_select(1, idx // 2).cpu().numpy()  # [H, n] bytes
        codes = (b >> (4 * (np.asarray(cols) % 2))) & 15
        s = ew.s_down[e].index_select(1, idx // 32).cpu().numpy()  # [H, n] E8M0
        return _FP4[codes] * _E8M0[s]
    q = ew.down[e].index_select(1, idx).cpu().view(torch.float8_e4m3fn).to(torch.float64).numpy()
    sc = ew.s_down[e].index_select(1, idx // 128).cpu().to(torch.float64).numpy()  # [H/128, n]
    return q * np.repeat(sc, 128, axis=0)


def a8_correction(ew, experts, h_gpu, h_ref, K):
    """[n, H] change of y = Wd h between the GPU's h and the oracle's h after each is quantised:
    Wd_e (deq(h_gpu) - deq(h_ref)), over the (few) positions where the two differ."""
    d = quantise_dequantise(h_gpu, K) - quantise_dequantise(h_ref, K)
    out = np.zeros((d.shape[0], ew.down.shape[1]))
    for p in np.nonzero(np.any(d != 0, axis=1))[0]:
        cols = np.nonzero(d[p])[0]
        out[p] = down_columns(ew, int(experts[p]), cols) @ d[p, cols]
    return out


A8_MAX_DIFF_FRACTION = 5e-3  # of h positions whose quantised value differs between the sides


def _ordered(bits):
    """bf16 bit patterns -> integers ordered like the values (adjacent values differ by 1)."""
    b = np.asarray(bits, np.int64)
    return np.where(b & 0x8000, -(b & 0x7FFF), b & 0x7FFF)


def _e4m3_spacing(v):
    """Spacing of the E4M3FN grid at magnitudes v (float64, in units of the block scale):
    2^(E-3) in the binade [2^E, 2^(E+1)), and 2^-9 below 2^-6 (the subnormals)."""
    v = np.asarray(v, np.float64)
    E = np.floor(np.log2(np.maximum(v, 2.0 ** -6)))
    return np.exp2(E - 3)


def check_a8_quantisation_steps(h_gpu, h_ref, K):
    """Bounds on where and how far the two sides' quantised h may differ (the mechanism of the
    layer comparison's correction).  Rounding to a grid is monotone, so two values a and b
    round at most |a - b| plus one grid step apart, the step taken at the larger magnitude and on
    the coarser of the two sides' grids (block exponents).  Asserted: every block whose exponent
    differs has largest magnitudes at most one bf16 ulp apart; at every position,
    |deq(h_gpu) - deq(h_ref)| <= |h_gpu - h_ref| + that step; and at most A8_MAX_DIFF_FRACTION
    of the positions differ.  Returns (differing fraction, per-row budget: the norm over the
    differing positions of |h_gpu - h_ref| + step, relative to the row's norm)."""
    hg = np.asarray(h_gpu, np.uint16).reshape(-1, K)
    hr = np.asarray(h_ref, np.uint16).reshape(-1, K)
    eg, ag = block_exponents(hg, K)
    er, ar = block_exponents(hr, K)
    flip = eg != er  # [n, K/128]
    assert np.all(np.abs(_ordered(ag[flip]) - _ordered(ar[flip])) <= 1), \
        "a block exponent differs with block maxima more than one bf16 ulp apart"
    qg, qr = quantise_dequantise(hg, K), quantise_dequantise(hr, K)
    d = qg != qr
    fg, fr = oracle.bf16_bits_to_float(hg), oracle.bf16_bits_to_float(hr)
    emax = np.repeat(np.maximum(eg, er), 128, axis=1)[d].astype(np.float64)
    scale = np.exp2(emax)
    step = _e4m3_spacing(np.maximum(np.abs(fg[d]), np.abs(fr[d])) / scale) * scale
    dh = np.abs(fg[d] - fr[d])
    worst = np.abs(qg[d] - qr[d]) - (dh + step)
    assert np.all(worst <= 1e-12 * step), \
        f"quantised h differs by more than its h difference plus one E4M3 step ({worst.max():.3g})"
    frac = float(d.mean())
    assert frac <= A8_MAX_DIFF_FRACTION, f"{frac:.2e} of the quantised h positions differ"
    budget = np.zeros(hg.shape)
    budget[d] = dh + step
    part = np.linalg.norm(budget, axis=1) / np.maximum(np.linalg.norm(fg, axis=1), 1e-30)
    return frac, part


def rel_l2_rows(got, ref):
    got = np.asarray(got, np.float64).reshape(-1, np.shape(got)[-1])
    ref = np.asarray(ref, np.float64).reshape(-1, np.shape(ref)[-1])
    num = np.linalg.norm(got - ref, axis=1)
    den = np.maximum(np.linalg.norm(ref, axis=1), 1e-30)
    return num / den


def assert_rows_close(name, got, ref, tol=ROW_TOL):
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    r = rel_l2_rows(got, ref)
    worst = int(np.argmax(r))
    assert r.max() <= tol, f"{name}: row {worst} relative L2 {r.max():.3e} > {tol}"
    return float(r.max())


def compare_with_oracle(layer, g, rows=None, routed=None, expert_slot=None, n_threads=0,
                        act_fp8=False, batched=False):
    """Check GPU results `g` against the oracle on token rows `rows` (default all).  batched:
    use the oracle's expert-by-expert form (full-size layers); else the per-token form."""
    if batched:
        ref = oracle.moe_layer_batched(layer, rows=rows, want_h=True, want_y=True,
                                       n_threads=n_threads, act_fp8=act_fp8)
    else:
        ref = oracle.moe_layer(layer, rows=rows, routed=routed, expert_slot=expert_slot,
                               want_h=True, want_y=True, n_threads=n_threads, act_fp8=act_fp8)
    T, k = layer.T, layer.k
    r = np.arange(T) if rows is None else np.asarray(rows)
    # routing: ids bit-exact, weights within W_TOL
    np.testing.assert_array_equal(g["ids"][r], ref["ids"])
    assert np.max(np.abs(g["w"][r].astype(np.float64) - ref["w"])) <= W_TOL
    # grouping: bit-exact (the oracle's permutation is computed from the GPU ids, which were
    # just shown identical to the oracle's on the checked rows)
    if rows is None:
        counts, offsets, perm, inv = oracle.permute(ref["ids"], layer.E)
        np.testing.assert_array_equal(g["counts"], counts)
        np.testing.assert_array_equal(g["offsets"], offsets)
        np.testing.assert_array_equal(g["perm"], perm)
        np.testing.assert_array_equal(g["inv"], inv)
    pos = g["inv"].reshape(T, k)[r]  # grouped row of (t, j)
    f = oracle.bf16_bits_to_float
    errs = {"rows": len(r)}
    errs["h"] = assert_rows_close("h", f(g["h"][pos.ravel()]), f(ref["h"]).reshape(-1, layer.I))
    errs["hS"] = assert_rows_close("shared h", f(g["hS"][r]), f(ref["hS"]))
    y_got, y_ref = f(g["y"][pos.ravel()]), ref["y"].reshape(-1, layer.H)
    S_got, S_ref = f(g["S"][r]), ref["S"]
    out_got, out_ref = f(g["out"][r]), f(ref["out"])
    if not act_fp8:
        errs["y"] = assert_rows_close("y", y_got, y_ref)
        errs["S"] = assert_rows_close("shared", S_got, S_ref)
        errs["out"] = assert_rows_close("out", out_got, out_ref)
        return errs
    # The two sides' h may quantise one step apart where they differ by a bf16 ulp: bound
    # where and how far, then add the exact effect of those steps to the oracle's y, S and out
    # (see a8_correction) before the usual per-row bound.
    h_g, h_r = g["h"][pos.ravel()], ref["h"].reshape(-1, layer.I)
    frac, part = check_a8_quantisation_steps(h_g, h_r, layer.I)
    fracS, partS = check_a8_quantisation_steps(g["hS"][r], ref["hS"], layer.I)
    jr = g["ids"][r].reshape(-1)  # expert of each checked (t, j)
    slots = jr if expert_slot is None else np.asarray(expert_slot)[jr]
    ew = routed if routed is not None else layer.experts
    dy = a8_correction(ew, slots, h_g, h_r, layer.I)
    dS = a8_correction(layer.shared, np.zeros(len(r), np.int64), g["hS"][r], ref["hS"], layer.I)
    w = ref["w"].astype(np.float64)
    dout = dS + np.einsum("tj,tjh->th", w, dy.reshape(len(r), k, -1))
    errs["y"] = assert_rows_close("y", y_got, y_ref + dy)
    errs["S"] = assert_rows_close("shared", S_got, S_ref + dS)
    errs["out"] = assert_rows_close("out", out_got, out_ref + dout)
    # Without the correction: the dequantised h of a row moves by at most its budget (the h
    # difference plus one E4M3 step at each differing position), so y moves by about that much
    # relative to the row (a factor 2 covers the spread of the random weights' column norms).
    # Rows must stay within the bar plus that.
    bound_y = ROW_TOL + 2 * part
    raw_y = rel_l2_rows(y_got, y_ref)
    assert np.all(raw_y <= bound_y), f"uncorrected y row {int(np.argmax(raw_y - bound_y))}"
    raw_S = rel_l2_rows(S_got, S_ref)
    assert np.all(raw_S <= ROW_TOL + 2 * partS), "uncorrected shared output"
    errs["corrected_rows"] = float(np.mean(np.any(dy != 0, axis=1)))
    errs["quantised_h_diff_fraction"] = max(frac, fracS)
    errs["uncorrected_y_max"] = float(raw_y.max())
    errs["uncorrected_out_max"] = float(rel_l2_rows(out_got, out_ref).max())
    return errs


def touched_experts(layer, g, rows):
    return sorted(set(g["ids"][np.asarray(rows)].ravel().tolist()))


def compare_sampled(layer, g, rows, n_threads=0, act_fp8=False):
    """Oracle on a few token rows of a large layer: only the experts they select are copied."""
    used = touched_experts(layer, g, rows)
    slot = np.full(layer.E, -1, np.int32)
    slot[used] = np.arange(len(used), dtype=np.int32)
    return compare_with_oracle(layer, g, rows=rows, routed=layer.experts.select(used),
                               expert_slot=slot, n_threads=n_threads, act_fp8=act_fp8)


# Heights of the kernels' m-tiles, by regime: few rows per expert (T*k <= 32*E) run the decode
# kernel's 16-row m-tiles (two of them per 32 rows); many rows run the prefill GEMMs, whose
# m-tiles are 128, 160 or 256 rows made of 32-row MFMA subtiles.
TILE_ROWS_FEW = (16, 32)
TILE_ROWS_MANY = (32, 128, 160, 256)


def stratified_tokens(layer, g, min_tokens=512, seed=0):
    """Tokens whose assignments cover, for every expert with rows, the first and last grouped
    row of the expert and of every m-tile (and 32-row subtile) of every tile height the layer's
    kernels use (TILE_ROWS_FEW or TILE_ROWS_MANY), topped up with seeded random tokens to at
    least min_tokens.  Through the rows they own, these tokens reach every (expert, m-tile) of
    every tiling, on both sides of each tile boundary."""
    offsets, perm, k = g["offsets"], g["perm"], layer.k
    heights = TILE_ROWS_FEW if layer.T * k <= 32 * layer.E else TILE_ROWS_MANY
    pos = []
    for e in range(layer.E):
        o, n = int(offsets[e]), int(offsets[e + 1] - offsets[e])
        if n == 0:
            continue
        pos += [o, o + n - 1]
        for bm in heights:
            m = np.arange(bm, n, bm)
            pos += list(o + m - 1) + list(o + m)
    tokens = set((perm[np.asarray(pos, np.int64)] // k).tolist())
    rng = np.random.default_rng(seed)
    for t in rng.permutation(layer.T):
        if len(tokens) >= min_tokens:
            break
        tokens.add(int(t))
    return sorted(tokens)
