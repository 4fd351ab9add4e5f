"""GPU parity of one rank's share of the layer under expert parallelism, as in the SmallEP scheme
of the OSDI'26 hybrid-inference article (SmallEP section): route and permute of all T tokens, the
routed experts of the rank's range on the assignments that select them, the local weighted
partial reduction (moe_combine_partial), and the shared expert on the rank's own token rows.
Bars as for the layer: ids bit-exact, partial and shared outputs within 1e-2 relative L2 per row
(tokens with no local expert: exactly zero)."""
import numpy as np
import pytest
import torch

import oracle
import routed_expert_grouped_amd as moe
from gpu_util import assert_rows_close, layer_for, mid

pytestmark = pytest.mark.gpu

f = oracle.bf16_bits_to_float


def _ranges(layer, G, r):
    E, T = layer.E, layer.T
    return r * E // G, (r + 1) * E // G, r * T // G, (r + 1) * T // G


def _run(layer, G, r):
    e0, e1, t0, t1 = _ranges(layer, G, r)
    R = moe.MoeRankShare(layer.T, layer.H, layer.I, layer.E, layer.k, layer.experts, layer.shared,
                         e0, e1, t0, t1, layer.score_fn, layer.renorm)
    part, sh = R.forward(layer.scores, layer.x)
    torch.cuda.synchronize()
    return (R.topk_ids.cpu().numpy(), part.cpu().numpy().view(np.uint16),
            sh[:t1 - t0].cpu().numpy().view(np.uint16))


@pytest.mark.parametrize("cfg,G", [
    ("tiny", 4),                                  # bf16 weights
    (mid(), 4),                                   # decode kernel, ragged expert ranges
    (mid(T=300, E=8, k=2), 8),                    # one expert per rank, GEMM shapes
    (mid(T=200, E=24, k=4, wdtype="mxfp4"), 3),   # 4-bit weights
])
def test_rank_partials_and_their_sum(cfg, G):
    layer = layer_for(cfg, seed=1)
    total = np.zeros((layer.T, layer.H))
    for r in range(G):
        e0, e1, t0, t1 = _ranges(layer, G, r)
        ids, part, sh = _run(layer, G, r)
        ref = oracle.moe_layer(layer, with_shared=False, expert_range=(e0, e1))
        np.testing.assert_array_equal(ids, ref["ids"])
        assert_rows_close("partial", f(part), f(ref["out"]))
        local = ((ref["ids"] >= e0) & (ref["ids"] < e1)).any(axis=1)
        assert not part[~local].any()
        refS = oracle.moe_layer(layer, rows=list(range(t0, t1)), want_y=True)["S"]
        assert_rows_close("shared", f(sh), refS)
        total += f(part)
        total[t0:t1] += f(sh)
    # every rank's partial plus its shared rows: the whole layer
    assert_rows_close("sum of the shares", total, f(oracle.moe_layer(layer)["out"]))


@pytest.mark.parametrize("cfg", ["dsv3_decode", "dsv3_prefill"])
def test_rank_share_at_full_size(cfg):
    """Rank 0 of 8 (32 of the 256 experts) at the DeepSeek-V3 shapes, every token (the oracle's
    expert-by-expert form at prefill; the local experts' weights are read in place)."""
    layer = layer_for(cfg)
    e0, e1, _, _ = _ranges(layer, 8, 0)
    ids, part, _ = _run(layer, 8, 0)
    ref = oracle.moe_layer_batched(layer, with_shared=False, expert_range=(e0, e1))
    np.testing.assert_array_equal(ids, ref["ids"])
    assert_rows_close("partial", f(part), f(ref["out"]))
    local = ((ids >= e0) & (ids < e1)).any(axis=1)
    assert not part[~local].any()


@pytest.mark.parametrize("cfg,G", [("dsv3_decode", 8), (mid(T=24, E=16, k=4), 4),
                                   (mid(T=37, E=64, k=8, wdtype="mxfp4"), 8)])
def test_shared_expert_calls_on_an_expert_slice(cfg, G):
    """moe_expert_gate_up_shared / moe_expert_down_shared on one rank's slice of the grouping
    (offsets + e0, weights of experts e0..e1-1): the shared expert's rows come after every
    grouped row (row T*k + t is token t) whichever slice is passed, and equal the separate
    identity-grouped calls bit for bit; the slice's routed rows equal the separate routed calls
    on the same slice."""
    layer = layer_for(cfg, seed=1)
    T, k = layer.T, layer.k
    ids, _ = moe.moe_route(layer.scores, k, layer.score_fn, layer.renorm)
    _, offsets, perm, _ = moe.moe_permute(ids, layer.E)
    ws = moe.expert_weights(layer.shared)
    h_s = moe.moe_expert_gate_up(layer.x, 1, None, None, ws)
    y_s = moe.moe_expert_down(h_s, T, 1, None, ws)
    for r in range(G):
        e0, e1, _, _ = _ranges(layer, G, r)
        if e1 == e0:
            continue
        local = moe.expert_slice(layer.experts, e0, e1)
        w = moe.expert_weights(local)
        offs = offsets[e0:]
        h_all = torch.zeros((T * k + T, layer.I), dtype=torch.int16, device="cuda")
        y_all = torch.zeros((T * k + T, layer.H), dtype=torch.int16, device="cuda")
        moe.moe_expert_gate_up_shared(layer.x, k, perm, offs, w, ws, h_all)
        moe.moe_expert_down_shared(h_all, T, k, offs, w, ws, y_all)
        h_r = torch.zeros((T * k, layer.I), dtype=torch.int16, device="cuda")
        y_r = torch.zeros((T * k, layer.H), dtype=torch.int16, device="cuda")
        moe.moe_expert_gate_up(layer.x, k, perm, offs, w, h_r)
        moe.moe_expert_down(h_r, T, k, offs, w, y_r)
        torch.cuda.synchronize()
        assert torch.equal(h_all[T * k:], h_s) and torch.equal(y_all[T * k:], y_s), r
        a, b = int(offsets[e0]), int(offsets[e1])
        assert torch.equal(h_all[a:b], h_r[a:b]) and torch.equal(y_all[a:b], y_r[a:b]), r
        # rows of the other ranks' experts are not written
        assert not h_all[:a].any() and not h_all[b:T * k].any(), r


def test_partial_combine_full_range_is_the_combine_and_ranges_add_up():
    """moe_combine_partial over [0, E) with the shared output is moe_combine bit for bit (same
    fp32 order); over two complementary ranges (the second with S) the two results sum, in
    float64, to the combine up to the two bf16 roundings."""
    rng = np.random.default_rng(4)
    T, k, H, E = 50, 6, 512, 40
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    w = rng.random((T, k)).astype(np.float32)
    inv = rng.permutation(T * k).astype(np.int32)
    y = torch.from_numpy(rng.standard_normal((T * k, H)).astype(np.float32)).to(torch.bfloat16)
    S = torch.from_numpy(rng.standard_normal((T, H)).astype(np.float32)).to(torch.bfloat16)
    dev = lambda a: (a if torch.is_tensor(a) else torch.from_numpy(a)).to("cuda")
    y_d, S_d = dev(y.view(torch.int16)), dev(S.view(torch.int16))
    ids_d, w_d, inv_d = dev(ids), dev(w), dev(inv)
    full = moe.moe_combine(y_d, inv_d, w_d, S_d, T, k, H)
    whole = moe.moe_combine_partial(y_d, inv_d, ids_d, w_d, 0, E, S_d, T, k, H)
    lo = moe.moe_combine_partial(y_d, inv_d, ids_d, w_d, 0, 17, None, T, k, H)
    hi = moe.moe_combine_partial(y_d, inv_d, ids_d, w_d, 17, E, S_d, T, k, H)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(whole.cpu().numpy(), full.cpu().numpy())
    got = f(lo.cpu().numpy().view(np.uint16)) + f(hi.cpu().numpy().view(np.uint16))
    assert_rows_close("two ranges", got, f(full.cpu().numpy().view(np.uint16)))
