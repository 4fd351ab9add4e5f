"""Helpers of the GPU tests: run the libmoe path on a synth.Layer and compare with the oracle."""
from __future__ import annotations

import numpy as np
import torch

import oracle
import routed_expert_grouped_amd as moe
import synth

ROW_TOL = 1e-2  # per-row relative L2 bound on float outputs (h, y, shared, out)
W_TOL = 1e-6  # absolute bound on the routing weights
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


def run_gpu(layer, stream=None, act="bf16"):
    """Run the full layer through the C ABI; return host copies of every intermediate."""
    L = moe.MoeLayer(layer.T, layer.H, layer.I, layer.E, layer.k, layer.experts, layer.shared,
                     layer.score_fn, layer.renorm, act=act)
    L.forward(layer.scores, layer.x, stream)
    torch.cuda.synchronize()
    T, k = layer.T, layer.k
    c = lambda t: t.detach().cpu().numpy()
    return dict(ids=c(L.topk_ids), w=c(L.topk_w), counts=c(L.counts), offsets=c(L.offsets),
                perm=c(L.perm[:T * k]), inv=c(L.inv[:T * k]),
                h=c(L.h[:T * k]).view(np.uint16), y=c(L.y[:T * k]).view(np.uint16),
                S=c(L.sh_y[:T]).view(np.uint16), out=c(L.out[:T]).view(np.uint16))


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
                        act_fp8=False):
    """Check GPU results `g` against the oracle on token rows `rows` (default all)."""
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
    errs = {}
    errs["h"] = assert_rows_close("h", f(g["h"][pos.ravel()]), f(ref["h"]).reshape(-1, layer.I))
    errs["y"] = assert_rows_close("y", f(g["y"][pos.ravel()]), ref["y"].reshape(-1, layer.H))
    errs["S"] = assert_rows_close("shared", f(g["S"][r]), ref["S"])
    errs["out"] = assert_rows_close("out", f(g["out"][r]), f(ref["out"]))
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
