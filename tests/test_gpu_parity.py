"""GPU parity: libmoe (through the C ABI) against the CPU oracle on seeded synthetic layers.

Bars: routing ids, counts, offsets, perm and inv bit-exact; routing weights within 1e-6;
h, y, the shared expert's output and the layer output within 1e-2 relative L2 per row.
"""
import numpy as np
import pytest
import torch

import oracle
import routed_expert_grouped_amd as moe
import synth
from gpu_util import (DEV, assert_rows_close, compare_sampled, compare_with_oracle, layer_for, mid,
                      run_gpu)

pytestmark = pytest.mark.gpu

# ------------------------------------------------------------------ number formats and layouts


def test_fp8_decode_and_scale_layout_exhaustive():
    """Down projection with identity activations reads every weight back exactly:
    y[p][c] = Wd[c][p] * s[c/128][p/128].  All finite E4M3FN codes, power-of-two block scales."""
    H, I = 256, 256
    codes = (np.arange(H)[:, None] * 7 + np.arange(I)[None, :] * 3) % 256
    codes[(codes == 0x7F) | (codes == 0xFF)] = 0x00  # NaN codes would poison whole rows
    q = torch.from_numpy(codes.astype(np.uint8))[None].to(DEV)
    s = torch.tensor([[[1.0, 2.0 ** -3], [2.0 ** 5, 0.5]]], dtype=torch.float32, device=DEV)
    ew = synth.ExpertWeights("fp8", q.transpose(1, 2).contiguous(), q.transpose(1, 2).contiguous(),
                             q, s, s, s)
    w = moe.expert_weights(ew)
    eye = torch.eye(I, dtype=torch.float32).to(torch.bfloat16).view(torch.int16).to(DEV)
    y = moe.moe_expert_down(eye, I, 1, None, w)
    torch.cuda.synchronize()
    got = oracle.bf16_bits_to_float(y.cpu())  # [p][c]
    val = torch.from_numpy(codes.astype(np.uint8)).view(torch.float8_e4m3fn).double().numpy()
    sx = np.repeat(np.repeat(s[0].cpu().double().numpy(), 128, 0), 128, 1)
    np.testing.assert_array_equal(got, (val * sx).T)


def test_bf16_weight_layout_exhaustive():
    """Same identity read-back for bf16 weights (bit patterns of many magnitudes)."""
    H, I = 128, 256
    rng = np.random.default_rng(0)
    vals = (rng.standard_normal((H, I)) * np.exp2(rng.integers(-20, 20, (H, I)))).astype(np.float32)
    wd = torch.from_numpy(vals).to(torch.bfloat16).view(torch.int16)[None].to(DEV)
    g = torch.zeros((1, I, H), dtype=torch.int16, device=DEV)
    ew = synth.ExpertWeights("bf16", g, g, wd, None, None, None)
    eye = torch.eye(I, dtype=torch.float32).to(torch.bfloat16).view(torch.int16).to(DEV)
    y = moe.moe_expert_down(eye, I, 1, None, moe.expert_weights(ew))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(y.cpu().numpy().view(np.uint16), wd[0].cpu().numpy().view(np.uint16).T)


# ------------------------------------------------------------------ whole layer, small shapes


@pytest.mark.parametrize("cfg", ["tiny", "tiny_fp8"])
def test_tiny_layer(cfg):
    layer = layer_for(cfg)
    compare_with_oracle(layer, run_gpu(layer))


@pytest.mark.parametrize("over", [
    dict(),                                  # several m-tiles per expert, ragged tails
    dict(T=37, E=64, k=8),                   # mostly 1-row experts, some empty
    dict(T=300, E=4, k=1, score_fn="softmax"),  # few experts with many rows
    dict(T=1, E=24, k=4),                    # a single token
    dict(T=64, E=16, k=16, renorm=0),        # k = E (every expert), unnormalised sigmoid
    dict(T=96, E=40, k=3, score_fn="softmax", renorm=0, wdtype="bf16"),
    dict(T=160, H=640, E=8, k=2),            # H an odd multiple of 128: register-staged GEMM
    dict(T=48, H=16384, I=256, E=4, k=2),    # the largest H (MOE_MAX_DIM), GEMV path
    dict(T=24, H=640, E=16, k=2),            # GEMV gate/up with an odd count of 128-blocks:
    dict(T=24, H=768, E=16, k=2),            # K unsplit, and K in two parts (four elsewhere)
    dict(T=200, H=16384, I=256, E=4, k=2),   # the largest H, GEMM path (128 scale blocks)
    dict(T=150, H=256, I=16384, E=2, k=1),   # the largest I, GEMM path
    dict(T=300, I=512, E=8, k=4),            # 160 x 512 tiles in both phases; experts above
                                             # 160 rows take a second m-tile
    dict(T=600, I=512, E=8, k=4),            # 300 rows per expert: 256 x 256 tiles
])
def test_mid_layer(over):
    layer = layer_for(mid(**over), seed=1)
    compare_with_oracle(layer, run_gpu(layer))


def test_skewed_routing_one_hot_expert():
    """Zipf-skewed scores: a few experts take most tokens (deep m-tile stacks)."""
    layer = layer_for(mid(T=256, E=32, k=2, scores="zipf"), seed=2)
    g = run_gpu(layer)
    assert g["counts"].max() >= 200
    compare_with_oracle(layer, g)


@pytest.mark.parametrize("I,T,E", [(384, 200, 8), (512, 200, 8), (512, 400, 4)])
def test_block_scales_zero_and_wide_range(I, T, E):
    """Weight blocks with zero scales and scales spread over six decades, on the grouped-GEMM
    path (many rows per expert) of the routed and the shared experts (I = 384: phase 2 has an
    odd number of 128-long K blocks; I = 512: an even number; 50 rows per expert take the
    160 x 512 tiles where the shape allows, 200 the 256 x 256 ones).  A zero scale makes its
    whole block contribute nothing."""
    layer = synth.make_layer(mid(T=T, E=E, k=2, I=I), seed=5)
    rng = np.random.default_rng(5)
    for ew in (layer.experts, layer.shared):
        for name in ("s_gate", "s_up", "s_down"):
            s = getattr(ew, name)
            f = rng.choice(np.array([0.0, 1e-3, 1.0, 1e3], np.float32), size=tuple(s.shape))
            s.mul_(torch.from_numpy(f))
    layer = layer.to(DEV)
    g = run_gpu(layer)
    assert g["counts"].max() > 32  # the grouped GEMM runs (more than 32 rows per expert)
    compare_with_oracle(layer, g)


def test_repeat_runs_are_bit_identical():
    layer = layer_for(mid(), seed=1)
    a, b = run_gpu(layer), run_gpu(layer)
    for key in a:
        np.testing.assert_array_equal(a[key], b[key])


# ------------------------------------------------------------------ routing / grouping edges


@pytest.mark.parametrize("T,E,k,fn", [(64, 64, 8, "sigmoid"), (33, 1024, 32, "softmax"),
                                      (5, 1, 1, "softmax"), (17, 5, 5, "sigmoid"),
                                      (4096, 256, 8, "sigmoid"), (50, 384, 8, "softmax")])
def test_route_ties_and_limits(T, E, k, fn):
    rng = np.random.default_rng(T + E)
    s = (rng.integers(-3, 4, size=(T, E)) / 2.0).astype(np.float32)  # many exact ties
    zero = rng.random((T, E)) < 0.2
    s[zero] = np.where(rng.random(zero.sum()) < 0.5, np.float32(0.0), np.float32(-0.0))
    for renorm in (1, 0):
        ids, w = moe.moe_route(torch.from_numpy(s).to(DEV), k, fn, renorm)
        torch.cuda.synchronize()
        rid, rw = oracle.route(s, k, fn, renorm)
        np.testing.assert_array_equal(ids.cpu().numpy(), rid)
        assert np.max(np.abs(w.cpu().numpy().astype(np.float64) - rw)) <= 1e-6


@pytest.mark.parametrize("T,E,k,skew", [(32768, 256, 8, 0.0), (20000, 256, 8, 2.0),
                                        (3000, 1024, 4, 0.0), (1, 7, 7, 0.0), (999, 3, 1, 0.0),
                                        (256, 256, 8, 1.0), (2049, 64, 1, 0.0),
                                        # the smallest multi-block sizes at the most experts:
                                        # the per-block count table (B * E ints) just fits in inv
                                        (2049, 1024, 1, 0.0), (257, 1024, 8, 3.0),
                                        (4097, 1024, 1, 0.0)])
def test_permute_large_and_skewed(T, E, k, skew):
    ids = synth.random_topk_ids(T, E, k, seed=11, skew=skew)
    c, o, p, i = moe.moe_permute(ids.to(DEV), E)
    torch.cuda.synchronize()
    rc, ro, rp, ri = oracle.permute(ids.numpy(), E)
    for got, ref in ((c, rc), (o, ro), (p, rp), (i, ri)):
        np.testing.assert_array_equal(got.cpu().numpy(), ref)


@pytest.mark.parametrize("T,E,k,fn", [(16, 256, 8, "sigmoid"), (1, 7, 7, "softmax"),
                                      (33, 1024, 32, "softmax"), (256, 256, 8, "sigmoid"),
                                      (100, 64, 6, "sigmoid")])
def test_fused_route_permute_is_the_two_calls(T, E, k, fn):
    """moe_route_permute (one launch, T*k <= 2048) gives the outputs of moe_route followed by
    moe_permute bit for bit, up to the largest fused size (T*k = 2048)."""
    scores = torch.rand((T, E), generator=torch.Generator().manual_seed(T * E + k)).to(DEV)
    ids, w = moe.moe_route(scores, k, fn)
    sep = (ids, w) + tuple(moe.moe_permute(ids, E))
    fused = moe.moe_route_permute(scores, k, fn)
    torch.cuda.synchronize()
    for a, b in zip(sep, fused):
        assert torch.equal(a, b)


def test_permute_all_to_one_expert():
    ids = torch.full((5000, 1), 3, dtype=torch.int32)
    c, o, p, i = moe.moe_permute(ids.to(DEV), 8)
    torch.cuda.synchronize()
    assert c.cpu().tolist() == [0, 0, 0, 5000, 0, 0, 0, 0]
    assert o.cpu().tolist() == [0, 0, 0, 0, 5000, 5000, 5000, 5000, 5000]
    np.testing.assert_array_equal(p.cpu().numpy(), np.arange(5000))
    np.testing.assert_array_equal(i.cpu().numpy(), np.arange(5000))


def test_zero_tokens_enqueue_nothing():
    layer = layer_for("tiny_fp8")
    sentinel = torch.full((4, 8), 7, dtype=torch.int32, device=DEV)
    moe.moe_route(layer.scores[:0], 2, "softmax", 1, sentinel, torch.empty(4, 8, device=DEV))
    moe.moe_permute(torch.empty((0, 2), dtype=torch.int32, device=DEV), 16, sentinel[0], sentinel[1],
                    sentinel[2], sentinel[3])
    torch.cuda.synchronize()
    assert bool((sentinel == 7).all())


# ------------------------------------------------------------------ full-size layers


def test_dsv3_decode_full():
    """DeepSeek-V3 decode layer (T=16, 256 experts, top-8): every token against the oracle."""
    layer = layer_for("dsv3_decode")
    g = run_gpu(layer)
    assert (g["counts"] > 0).sum() > 80
    compare_sampled(layer, g, rows=list(range(layer.T)))


@pytest.mark.parametrize("cfg,over", [("tiny_fp8", {}), ("tiny", {}), ("dsv3_decode", {}),
                                      ("dsv3_decode", {"wdtype": "mxfp4"}),
                                      (mid(T=37, E=64, k=8), {}),            # GEMV: one grid
                                      (mid(T=24, H=640, E=16, k=2), {}),     # K unsplit
                                      (mid(), {})])                          # GEMMs: two launches
def test_shared_expert_in_the_routed_launches_is_the_separate_calls(cfg, over):
    """moe_expert_gate_up_shared / moe_expert_down_shared (the shared expert as an extra group
    of the routed launches at decode sizes) give the routed rows of the separate routed calls bit
    for bit, and the shared rows of the separate shared calls bit for bit where those run the
    same kernel (T <= 32, or many rows per expert); at T > 32 with few rows per expert the
    separate shared call runs a GEMM, and the rows agree to the parity bar."""
    layer = layer_for(cfg, **over) if isinstance(cfg, str) else layer_for(cfg, seed=1)
    T, k = layer.T, layer.k
    ids, _ = moe.moe_route(layer.scores, k, layer.score_fn, layer.renorm)
    _, offsets, perm, _ = moe.moe_permute(ids, layer.E)
    w, ws = moe.expert_weights(layer.experts), moe.expert_weights(layer.shared)
    h_all = moe.moe_expert_gate_up_shared(layer.x, k, perm, offsets, w, ws)
    y_all = moe.moe_expert_down_shared(h_all, T, k, offsets, w, ws)
    h_r = moe.moe_expert_gate_up(layer.x, k, perm, offsets, w)
    y_r = moe.moe_expert_down(h_r, T, k, offsets, w)
    h_s = moe.moe_expert_gate_up(layer.x, 1, None, None, ws)
    y_s = moe.moe_expert_down(h_s, T, 1, None, ws)
    torch.cuda.synchronize()
    assert torch.equal(h_all[:T * k], h_r) and torch.equal(y_all[:T * k], y_r)
    same_kernel = T <= 32 or T * k > 32 * layer.E
    for got, ref in ((h_all[T * k:], h_s), (y_all[T * k:], y_s)):
        if same_kernel:
            assert torch.equal(got, ref)
        else:
            g = oracle.bf16_bits_to_float(got.cpu())
            r = oracle.bf16_bits_to_float(ref.cpu())
            rel = np.linalg.norm(g - r, axis=1) / np.linalg.norm(r, axis=1)
            assert rel.max() <= 1e-2, rel.max()


@pytest.mark.parametrize("T,k,E", [(300, 8, 256), (4096, 8, 256), (8192, 8, 384)])
def test_permute_workspace_contents_do_not_matter(T, k, E):
    """The grouping above 2048 assignments keeps its count table in the caller's workspace;
    whatever the workspace holds on entry, the result is the oracle's, and nothing outside the
    queried size is written."""
    ids = synth.random_topk_ids(T, E, k, seed=T)
    need = moe.moe_permute_workspace_size(T, k, E)
    assert need == (0 if T * k <= 2048 else -(-T * k // 2048) * E * 4)
    ref = oracle.permute(ids.numpy(), E)
    for fill in (0x00, 0x7F, 0xFF):
        buf = torch.full((need + 2 * 4096,), fill, dtype=torch.uint8, device=DEV)
        ws = buf[4096:4096 + need] if need else None
        got = moe.moe_permute(ids.to(DEV), E, ws=ws)
        torch.cuda.synchronize()
        for a, b in zip(got, ref):
            np.testing.assert_array_equal(a.cpu().numpy(), b)
        assert bool((buf[:4096] == fill).all()) and bool((buf[4096 + need:] == fill).all())


@pytest.mark.parametrize("cfg", ["tiny", "tiny_fp8", mid(), mid(T=37, E=64, k=8),
                                 mid(wdtype="mxfp4")])
def test_expert_ffn_call_against_the_oracle(cfg):
    """moe_expert_ffn (both expert phases in one call, h in the caller's workspace) through the
    C ABI: h and y of every assignment against the oracle, and equal to the two phase calls bit
    for bit."""
    layer = layer_for(cfg, seed=2)
    T, k = layer.T, layer.k
    ids, w_ = moe.moe_route(layer.scores, k, layer.score_fn, layer.renorm)
    _, offsets, perm, inv = moe.moe_permute(ids, layer.E)
    w = moe.expert_weights(layer.experts)
    need = moe.moe_expert_ffn_workspace_size(T, k, w)
    assert need == T * k * layer.I * 2
    ws = torch.full((need,), 0x5A, dtype=torch.uint8, device=DEV)
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_expert_ffn(layer.x, k, perm, offsets, w, ws=ws[:need - 1])
    assert ei.value.status == moe.MOE_ERR_WORKSPACE
    y, _ = moe.moe_expert_ffn(layer.x, k, perm, offsets, w, ws=ws)
    h2 = moe.moe_expert_gate_up(layer.x, k, perm, offsets, w)
    y2 = moe.moe_expert_down(h2, T, k, offsets, w)
    torch.cuda.synchronize()
    h = ws.view(torch.int16).view(T * k, layer.I)
    assert torch.equal(h, h2) and torch.equal(y, y2)
    ref = oracle.moe_layer(layer, want_h=True, want_y=True)
    np.testing.assert_array_equal(ids.cpu().numpy(), ref["ids"])
    pos = inv.cpu().numpy()  # grouped row of flat assignment t*k+j
    f = oracle.bf16_bits_to_float
    assert_rows_close("h", f(h.cpu().numpy().view(np.uint16)[pos]), f(ref["h"]).reshape(-1, layer.I))
    assert_rows_close("y", f(y.cpu().numpy().view(np.uint16)[pos]), ref["y"].reshape(-1, layer.H))


@pytest.mark.parametrize("T,k,H,E", [(300, 8, 7168, 256), (77, 13, 512, 40), (16, 8, 7168, 256),
                                     (5, 32, 256, 64), (40, 1, 256, 8), (50, 2, 7168, 16),
                                     (33, 6, 1024, 64), (9, 8, 8200, 16), (12, 3, 40, 8)])
def test_combine_is_the_slot_ordered_fp32_fma_sum(T, k, H, E):
    """moe_combine and moe_combine_partial bit for bit against the sum they state: fp32 fused
    multiply-adds S + w_0 y_0 + ... + w_{k-1} y_{k-1} in slot order (skipping other ranks'
    experts in the partial form), rounded to bf16.  Emulated exactly in float64: each product
    of an fp32 weight and a bf16 value, plus the fp32 accumulator, is exact in double, so
    rounding it to fp32 is the fused operation.  The kernel reads y in groups of 8, then 4, then
    single rows: k = 1, 2, 6, 8, 13 and 32 take every mix of them, with and without a shared
    row.  A workgroup covers up to 8192 columns of a token: H = 8200 takes two per token, H = 40
    one partly filled wave."""
    rng = np.random.default_rng(T * k)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    w = rng.random((T, k)).astype(np.float32)
    inv = rng.permutation(T * k).astype(np.int32)
    y = torch.from_numpy(rng.standard_normal((T * k, H)).astype(np.float32)).to(torch.bfloat16)
    S = torch.from_numpy(rng.standard_normal((T, H)).astype(np.float32)).to(torch.bfloat16)
    d = lambda a: (a if torch.is_tensor(a) else torch.from_numpy(a)).to(DEV)
    yb, Sb = d(y.view(torch.int16)), d(S.view(torch.int16))
    out = moe.moe_combine(yb, d(inv), d(w), Sb, T, k, H)
    out0 = moe.moe_combine(yb, d(inv), d(w), None, T, k, H)
    e0, e1 = 3, E // 2
    part = moe.moe_combine_partial(yb, d(inv), d(ids), d(w), e0, e1, None, T, k, H)
    torch.cuda.synchronize()
    yf, Sf = y.double().numpy(), S.double().numpy()

    def fma_sum(acc, lo, hi):
        acc = acc.astype(np.float32)
        for j in range(k):
            sel = (ids[:, j] >= lo) & (ids[:, j] < hi)
            nxt = (w[:, j:j + 1].astype(np.float64) * yf[inv[np.arange(T) * k + j]]
                   + acc.astype(np.float64)).astype(np.float32)
            acc = np.where(sel[:, None], nxt, acc)
        return torch.from_numpy(acc).to(torch.bfloat16).view(torch.int16).numpy()

    np.testing.assert_array_equal(out.cpu().numpy(), fma_sum(Sf, 0, E))
    np.testing.assert_array_equal(out0.cpu().numpy(), fma_sum(np.zeros((T, H)), 0, E))
    np.testing.assert_array_equal(part.cpu().numpy(), fma_sum(np.zeros((T, H)), e0, e1))
