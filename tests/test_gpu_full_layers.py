"""Full-size parity of the three large layers in every weight and activation mode.

DeepSeek-V3 prefill (T = 4096, 256 experts) is checked on every token row; Kimi-K2 (T = 8192,
384 experts) and the long Zipf-routed layer (T = 32768, 19 experts touched, the hottest with
32768 assignments) on a stratified token set (gpu_util.stratified_tokens): for every expert
with rows, the tokens that own the first and last grouped row of the expert and of every
m-tile and 32-row MFMA subtile of every tile height the prefill GEMMs use (32, 128, 160, 256
rows), topped up with seeded random tokens to at least 512.  Every (expert, m-tile) of every
tiling is thereby reached on both sides of each tile boundary, across all of its column tiles
(whole rows are compared).

Whole-layer routing (ids bit-exact, weights within 1e-6) and grouping (counts, offsets, perm,
inv bit-exact) are checked on every token in every case.  The float bars are the layer's:
h, y, the shared expert's h and output, and the layer output within 1e-2 relative L2 per row,
against the oracle's expert-by-expert form (oracle.moe_layer_batched, the same definition as
the per-token form with float64 library matrix products).  Grouped rows follow the
KTransformers article (2.2): the tokens that select one expert form one GEMM.
"""
import os

import numpy as np
import pytest

import oracle
from gpu_util import compare_with_oracle, layer_for, run_gpu, stratified_tokens

pytestmark = pytest.mark.gpu

MODES = [("fp8", "bf16"), ("fp8", "fp8"), ("mxfp4", "bf16"), ("mxfp4", "fp8")]
SEED = int(os.environ.get("MOE_FULL_SEED", "0"))  # the layers' seed (0; seed 1 passed as well)


@pytest.mark.parametrize("wdtype,act", MODES, ids=[f"{w}-{a}" for w, a in MODES])
@pytest.mark.parametrize("cfg", ["dsv3_prefill", "kimi_k2", "dsv3_long_zipf"])
def test_full_size_layer(cfg, wdtype, act):
    layer = (layer_for(cfg, seed=SEED) if wdtype == "fp8"
             else layer_for(cfg, seed=SEED, wdtype=wdtype))
    print(f"\n[{cfg} {wdtype} weights, {act} activations] GPU layer", flush=True)
    g = run_gpu(layer, act=act)
    rid, rw = oracle.route(layer.scores.cpu().numpy(), layer.k, layer.score_fn, layer.renorm)
    np.testing.assert_array_equal(g["ids"], rid)
    assert np.max(np.abs(g["w"].astype(np.float64) - rw)) <= 1e-6
    counts, offsets, perm, inv = oracle.permute(rid, layer.E)
    for key, ref in (("counts", counts), ("offsets", offsets), ("perm", perm), ("inv", inv)):
        np.testing.assert_array_equal(g[key], ref)
    rows = None if cfg == "dsv3_prefill" else stratified_tokens(layer, g)
    n = layer.T if rows is None else len(rows)
    print(f"  oracle on {n} token rows", flush=True)
    errs = compare_with_oracle(layer, g, rows=rows, act_fp8=act == "fp8", batched=True)
    print("  " + ", ".join(f"{k} {v:.3g}" for k, v in errs.items()), flush=True)
    assert rows is None or len(rows) >= 512
