"""Pins of the CPU oracle against things other than itself (runs without a GPU).

* number formats: all 256 E4M3FN codes against torch's float8_e4m3fn and the OCP spec's closed
  forms; bf16 round-to-nearest-even against torch's cast and hand-made ties;
* routing: numpy's stable argsort (brute force over a full sort), argmax for k=1, torch/scipy
  softmax and logistic functions for the weights, invariants;
* grouping: numpy's stable argsort of the flat expert ids, bincount, inverse-permutation identity,
  and the lecture notes' worked answer for the mean number of tokens per expert;
* expert FFN + combine: a dense brute force (every expert on every token, masked by its gate
  weight, numpy float64 matrix products, torch's FP8 decode, numpy-expanded scale blocks);
  the E=1, k=1 textbook SwiGLU case; the identical-experts closed form; k=1 combine;
* FP8 activations (the FP8 MFMA mode): the E4M3FN encoder against torch's float8_e4m3fn cast
  (random values, exact ties, subnormals), the power-of-two block-scale exponent against exact
  rational arithmetic, the row quantiser against a numpy/torch re-implementation, and the
  quantised-activation layer against the dense brute force fed with torch-quantised activations.
"""
from fractions import Fraction
import numpy as np
import pytest
import scipy.special
import torch

import oracle
import synth

# ----------------------------------------------------------------------------- number formats


def test_fp8_all_codes_match_torch():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = np.array([oracle.fp8_e4m3fn_to_double(c) for c in range(256)])
    nan = np.isnan(ref)
    assert list(np.nonzero(nan)[0]) == [0x7F, 0xFF]
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # signed zero
    assert np.signbit(got[0x80]) and not np.signbit(got[0x00])


def test_fp8_closed_forms_from_the_ocp_spec():
    d = oracle.fp8_e4m3fn_to_double
    assert d(0x7E) == 448.0  # largest finite
    assert d(0x01) == 2.0 ** -9  # smallest subnormal
    assert d(0x07) == 7 * 2.0 ** -9  # largest subnormal
    assert d(0x08) == 2.0 ** -6  # smallest normal
    assert d(0x38) == 1.0  # exponent field 7 = bias
    assert d(0x3F) == 1.875
    assert d(0xC0) == -2.0


def test_bf16_round_to_nearest_even():
    r = oracle.double_to_bf16
    one = 0x3F80
    assert r(1.0) == one
    assert r(1.0 + 2.0 ** -8) == one  # tie -> even (1.0)
    assert r(1.0 + 3 * 2.0 ** -8) == one + 2  # tie -> even (1 + 2^-6)
    assert r(1.0 + 2.0 ** -8 + 2.0 ** -40) == one + 1  # just above a tie: up (no double rounding)
    assert r(2.0 ** -133) == 0x0001  # smallest subnormal
    assert r(2.0 ** -134) == 0x0000  # tie between 0 and the smallest subnormal -> 0
    assert r(3 * 2.0 ** -134) == 0x0002  # tie -> even
    assert r(-0.0) == 0x8000
    assert r((2 - 2.0 ** -7) * 2.0 ** 127) == 0x7F7F  # largest finite
    assert r((2 - 2.0 ** -8) * 2.0 ** 127) == 0x7F80  # rounds to +inf
    assert r(float("nan")) & 0x7F80 == 0x7F80
    # random fp32 values against torch's fp32 -> bf16 cast (a single rounding)
    rng = np.random.default_rng(1)
    v = np.concatenate([rng.standard_normal(3000).astype(np.float32),
                        (rng.standard_normal(1000) * 1e-38).astype(np.float32),
                        (rng.standard_normal(1000) * 1e30).astype(np.float32)])
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([r(float(a)) for a in v], dtype=np.uint16)
    assert np.array_equal(got, ref)


def test_bf16_decode():
    bits = np.arange(0, 65536, 97, dtype=np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = np.array([oracle.bf16_to_double(b) for b in bits])
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok]) and np.array_equal(np.isnan(got), ~ok)


# ----------------------------------------------------------------------------- routing


def _tied_scores(T, E, seed):
    """Scores on a coarse grid (many ties), with some +0.0 / -0.0 pairs."""
    rng = np.random.default_rng(seed)
    s = (rng.integers(-4, 5, size=(T, E)) / 4.0).astype(np.float32)
    zero = rng.random((T, E)) < 0.2
    s[zero] = np.where(rng.random(zero.sum()) < 0.5, np.float32(0.0), np.float32(-0.0))
    return s


@pytest.mark.parametrize("T,E,k", [(64, 16, 2), (40, 256, 8), (17, 384, 8), (9, 5, 5), (33, 7, 1)])
def test_route_ids_match_stable_full_sort(T, E, k):
    for s in (_tied_scores(T, E, T + E), np.random.default_rng(E).random((T, E), dtype=np.float32)):
        ids, w = oracle.route(s, k, "sigmoid")
        ref = np.argsort(-s, axis=1, kind="stable")[:, :k]
        assert np.array_equal(ids, ref)
        assert all(len(set(r)) == k for r in ids)
        if k == 1:
            assert np.array_equal(ids[:, 0], np.argmax(s, axis=1))


def test_route_weights_softmax_and_sigmoid():
    rng = np.random.default_rng(3)
    s = rng.standard_normal((50, 64)).astype(np.float32)
    k = 6
    ref_ids = np.argsort(-s, axis=1, kind="stable")[:, :k]
    g = np.take_along_axis(s, ref_ids, axis=1).astype(np.float64)
    # softmax over the selected logits
    ids, w = oracle.route(s, k, "softmax", renorm=1)
    assert np.array_equal(ids, ref_ids)
    ref = torch.softmax(torch.from_numpy(g), dim=1).numpy()
    np.testing.assert_allclose(w, ref, rtol=2e-7, atol=0)
    # softmax over all experts, then the selected probabilities
    _, w0 = oracle.route(s, k, "softmax", renorm=0)
    full = torch.softmax(torch.from_numpy(s.astype(np.float64)), dim=1).numpy()
    np.testing.assert_allclose(w0, np.take_along_axis(full, ref_ids, axis=1), rtol=2e-7, atol=0)
    # sigmoid, renormalised over the selected
    _, ws = oracle.route(s, k, "sigmoid", renorm=1)
    e = scipy.special.expit(g)
    np.testing.assert_allclose(ws, e / e.sum(axis=1, keepdims=True), rtol=2e-7, atol=0)
    _, ws0 = oracle.route(s, k, "sigmoid", renorm=0)
    np.testing.assert_allclose(ws0, e, rtol=2e-7, atol=0)
    for ww in (w, ws):
        np.testing.assert_allclose(ww.astype(np.float64).sum(axis=1), 1.0, atol=1e-6)
        assert np.all(np.diff(ww, axis=1) <= 0)  # descending with the scores


def test_route_rejects_bad_k():
    s = np.zeros((2, 4), np.float32)
    with pytest.raises(ValueError):
        oracle.route(s, 5, "softmax")
    with pytest.raises(ValueError):
        oracle.route(s, 0, "softmax")


# ----------------------------------------------------------------------------- grouping


@pytest.mark.parametrize("T,E,k,skew", [(64, 256, 8, 0.0), (333, 16, 2, 0.0), (200, 32, 4, 1.5),
                                        (1, 8, 8, 0.0), (128, 64, 1, 3.0)])
def test_permute_matches_stable_argsort(T, E, k, skew):
    ids = synth.random_topk_ids(T, E, k, seed=T, skew=skew).numpy()
    counts, offsets, perm, inv = oracle.permute(ids, E)
    flat = ids.ravel()
    assert np.array_equal(counts, np.bincount(flat, minlength=E))
    assert offsets[0] == 0 and offsets[-1] == T * k
    assert np.array_equal(np.diff(offsets), counts)
    assert np.array_equal(perm, np.argsort(flat, kind="stable"))
    assert np.array_equal(inv[perm], np.arange(T * k))
    for e in range(E):
        seg = perm[offsets[e]:offsets[e + 1]]
        assert np.all(flat[seg] == e) and np.all(np.diff(seg) > 0)


def test_permute_mean_tokens_per_expert_worked_answer():
    # CMU 11-868 appendix A2 notes, exercise 7 (worked answer): at batch 64, a DeepSeek-V3
    # routed expert (256 experts, 8 per token) is used by 64*8/256 = 2 tokens on average.
    ids = synth.random_topk_ids(64, 256, 8, seed=0).numpy()
    counts, offsets, _, _ = oracle.permute(ids, 256)
    assert counts.sum() / 256 == 2.0 and offsets[-1] == 512


def test_permute_rejects_out_of_range_ids():
    with pytest.raises(ValueError):
        oracle.permute(np.array([[0, 9]], np.int32), 4)


# ----------------------------------------------------------------------------- expert FFN


# The E2M1 magnitudes as the OCP microscaling spec tabulates them (codes 0..7; bit 3 is the sign)
OCP_E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def _dense_weights(ew, H, I):
    """float64 [n, rows, cols] dequantised weights via torch's FP8/bf16 decode, the OCP E2M1
    table for MXFP4, and numpy scale expansion."""
    def deq(q, s):
        if ew.wdtype == "bf16":
            return q.view(torch.bfloat16).to(torch.float64).numpy()
        if ew.wdtype == "mxfp4":
            b = q.numpy()
            codes = np.stack([b & 15, b >> 4], axis=-1).reshape(*b.shape[:-1], -1)
            v = np.where(codes & 8, -1.0, 1.0) * OCP_E2M1[codes & 7]
            return v * np.repeat(np.exp2(s.numpy().astype(np.float64) - 127), 32, axis=-1)
        v = q.view(torch.float8_e4m3fn).to(torch.float64).numpy()
        sx = np.repeat(np.repeat(s.numpy().astype(np.float64), 128, axis=1), 128, axis=2)
        return v * sx
    return deq(ew.gate, ew.s_gate), deq(ew.up, ew.s_up), deq(ew.down, ew.s_down)


def _to_bf16_f64(a):
    return torch.from_numpy(a.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()


def _dense_brute_force(layer, ids, w, act_fp8=False):
    """Every expert on every token (float64), masked by its gate weight, plus the shared expert.
    act_fp8: x and the bf16 h are quantised in 1x128 blocks first (_ref_quantize)."""
    x = torch.from_numpy(oracle._np(layer.x, np.uint16).view(np.int16)).view(torch.bfloat16)
    x = x.to(torch.float64).numpy()
    if act_fp8:
        x = _ref_quantize(x)
    Wg, Wu, Wd = _dense_weights(layer.experts, layer.H, layer.I)
    Sg, Su, Sd = _dense_weights(layer.shared, layer.H, layer.I)

    def ffn(g, u, d):
        G, U = x @ g.T, x @ u.T
        h = _to_bf16_f64(scipy.special.expit(G) * G * U)  # note: h is exact within fp32 first
        return h, (_ref_quantize(h) if act_fp8 else h) @ d.T

    hS, S = ffn(Sg[0], Su[0], Sd[0])
    gate = np.zeros((layer.T, layer.E))
    np.put_along_axis(gate, ids, w.astype(np.float64), axis=1)
    acc = S.copy()
    ys, hs = [], []
    for e in range(layer.E):
        h, y = ffn(Wg[e], Wu[e], Wd[e])
        acc += gate[:, e:e + 1] * y
        hs.append(h)
        ys.append(y)
    return acc, np.stack(hs, 1), np.stack(ys, 1), S, hS


def _check_layer_against_dense(layer, act_fp8=False, fn=None):
    fn = oracle.moe_layer if fn is None else fn
    res = fn(layer, want_h=True, want_y=True, act_fp8=act_fp8)
    acc, hs, ys, S, hS = _dense_brute_force(layer, res["ids"], res["w"], act_fp8)
    T = layer.T
    y_sel = ys[np.arange(T)[:, None], res["ids"]]  # [T, k, H]
    h_sel = hs[np.arange(T)[:, None], res["ids"]]
    hb = oracle.bf16_bits_to_float(res["h"])
    # h: identical bf16 values except where the dense path's fp32 detour (double rounding)
    # moves a value across a bf16 tie; those rows of y then differ by that one h ulp
    assert np.mean(hb == h_sel) > 0.999
    np.testing.assert_allclose(hb, h_sel, rtol=2.0 ** -7, atol=0)
    same_h = np.all(hb == h_sel, axis=-1)  # [T, k]
    np.testing.assert_allclose(res["y"][same_h], y_sel[same_h], rtol=1e-9, atol=1e-14)
    d = np.linalg.norm(res["y"] - y_sel, axis=-1) / np.linalg.norm(y_sel, axis=-1)
    assert d.max() < 1e-3
    # shared expert: same caveat
    hSb = oracle.bf16_bits_to_float(res["hS"])
    assert np.mean(hSb == hS) > 0.999
    np.testing.assert_allclose(hSb, hS, rtol=2.0 ** -7, atol=0)
    dS = np.linalg.norm(res["S"] - S, axis=-1) / np.linalg.norm(S, axis=-1)
    assert dS.max() < 1e-3 and np.mean(dS < 1e-12) > 0.8
    out = oracle.bf16_bits_to_float(res["out"])
    np.testing.assert_allclose(out, _to_bf16_f64(acc), rtol=2.0 ** -7, atol=1e-30)
    assert np.mean(out == _to_bf16_f64(acc)) > 0.99
    return res


def test_ffn_dense_brute_force_tiny_bf16():
    _check_layer_against_dense(synth.make_layer("tiny", seed=0))


def test_ffn_dense_brute_force_tiny_fp8():
    _check_layer_against_dense(synth.make_layer("tiny_fp8", seed=0))


@pytest.mark.parametrize("e_range", [(0, 4), (4, 9), (9, 16), (5, 5)])
def test_partial_reduction_dense_brute_force(e_range):
    """One rank's partial (experts [e0, e1) only, no shared expert) against the dense brute force
    with the gate weights of the other experts set to zero; inside the range y equals the full
    run's y bit for bit, outside it is zero."""
    e0, e1 = e_range
    layer = synth.make_layer("tiny_fp8", seed=0)
    full = oracle.moe_layer(layer, want_y=True)
    res = oracle.moe_layer(layer, with_shared=False, want_y=True, expert_range=e_range)
    np.testing.assert_array_equal(res["ids"], full["ids"])
    _, _, ys, _, _ = _dense_brute_force(layer, full["ids"], full["w"])
    local = (res["ids"] >= e0) & (res["ids"] < e1)  # [T, k]
    np.testing.assert_array_equal(res["y"][local], full["y"][local])
    assert not res["y"][~local].any()
    gate = np.zeros((layer.T, layer.E))
    np.put_along_axis(gate, res["ids"], np.where(local, res["w"], 0).astype(np.float64), axis=1)
    acc = np.einsum("te,teh->th", gate, ys)
    out = oracle.bf16_bits_to_float(res["out"])
    np.testing.assert_allclose(out, _to_bf16_f64(acc), rtol=2.0 ** -7, atol=1e-30)
    assert not out[~local.any(axis=1)].any()  # tokens with no local expert: exactly zero


def test_partial_reductions_partition_the_layer_at_k1():
    """With one expert per token, each token's output comes from exactly one of the ranks'
    expert ranges: that rank's partial equals the full output bit for bit, the others are 0."""
    layer = synth.make_layer(dict(T=40, H=256, I=128, E=12, k=1, score_fn="softmax",
                                  scores="normal", wdtype="fp8"), seed=2)
    full = oracle.moe_layer(layer, with_shared=False)
    bounds = [0, 3, 7, 12]
    owner = np.searchsorted(bounds, full["ids"][:, 0], side="right") - 1
    for r in range(3):
        part = oracle.moe_layer(layer, with_shared=False, expert_range=(bounds[r], bounds[r + 1]))
        mine = owner == r
        np.testing.assert_array_equal(part["out"][mine], full["out"][mine])
        assert not part["out"][~mine].any()


def test_ffn_dense_brute_force_rectangular_scale_grid():
    # H != I so that a transposed scale index or weight layout cannot go unnoticed; random
    # per-block scales so that every block's scale matters.
    layer = synth.make_layer(dict(T=24, H=384, I=256, E=6, k=3, score_fn="sigmoid", scores="uniform",
                                  wdtype="fp8"), seed=3)
    g = torch.Generator().manual_seed(5)
    for ew in (layer.experts, layer.shared):
        for s in (ew.s_gate, ew.s_up, ew.s_down):
            s.mul_(torch.rand(s.shape, generator=g) * 4 + 0.25)
    _check_layer_against_dense(layer)


def test_ffn_single_expert_is_textbook_swiglu():
    # E = 1, k = 1: softmax over one logit gives weight 1, so out = bf16(shared(x) + FFN(x)).
    layer = synth.make_layer(dict(T=8, H=256, I=128, E=1, k=1, score_fn="softmax", scores="normal",
                                  wdtype="fp8"), seed=2)
    res = oracle.moe_layer(layer, want_y=True, want_h=True)
    assert np.all(res["w"] == 1.0) and np.all(res["ids"] == 0)
    x = oracle.bf16_bits_to_float(layer.x)
    Wg, Wu, Wd = (a[0] for a in _dense_weights(layer.experts, 256, 128))
    g, u = x @ Wg.T, x @ Wu.T
    h = _to_bf16_f64(g / (1 + np.exp(-g)) * u)
    np.testing.assert_allclose(res["y"][:, 0], h @ Wd.T, rtol=1e-9, atol=1e-14)
    expect = _to_bf16_f64(res["S"] + res["y"][:, 0])
    got = oracle.bf16_bits_to_float(res["out"])
    np.testing.assert_allclose(got, expect, rtol=2.0 ** -8, atol=0)
    assert np.mean(got == expect) > 0.99


def test_ffn_identical_experts_closed_form():
    # All routed experts equal: sum_j w_j FFN(x) = FFN(x) since the renormalised weights sum to 1.
    base = dict(T=12, H=256, I=128, k=4, score_fn="sigmoid", scores="uniform", wdtype="fp8")
    many = synth.make_layer(dict(base, E=8), seed=4)
    one = synth.make_layer(dict(base, E=1, k=1), seed=4)
    for name in ("gate", "up", "down", "s_gate", "s_up", "s_down"):
        t = getattr(one.experts, name)
        setattr(many.experts, name, t.expand(8, *t.shape[1:]).contiguous())
    one.shared = many.shared
    one.x = many.x
    a = oracle.moe_layer(many, want_y=True)
    b = oracle.moe_layer(one, want_y=True)
    for j in range(4):
        np.testing.assert_array_equal(a["y"][:, j], b["y"][:, 0])
    fa, fb = oracle.bf16_bits_to_float(a["out"]), oracle.bf16_bits_to_float(b["out"])
    np.testing.assert_allclose(fa, fb, rtol=2.0 ** -8, atol=0)


def test_layer_row_subset_and_expert_slots_agree_with_full_run():
    layer = synth.make_layer("tiny_fp8", seed=1)
    full = oracle.moe_layer(layer, want_y=True, want_h=True)
    rows = [3, 0, 15, 7]
    used = sorted(set(full["ids"][rows].ravel().tolist()))
    slot = np.full(layer.E, -1, np.int32)
    slot[used] = np.arange(len(used))
    sub = oracle.moe_layer(layer, rows=rows, routed=layer.experts.select(used), expert_slot=slot,
                           want_y=True, want_h=True)
    for key in ("ids", "w", "out", "h", "y", "S"):
        np.testing.assert_array_equal(sub[key], full[key][rows])
    with pytest.raises(ValueError):  # an expert that was not provided
        slot2 = slot.copy()
        slot2[used[0]] = -1
        oracle.moe_layer(layer, rows=rows, routed=layer.experts.select(used), expert_slot=slot2)


# ----------------------------------------------------------------------------- FP8 activations


def _e4m3_grid():
    """All finite non-negative E4M3FN values (float64, ascending), from torch's decode."""
    v = torch.arange(0, 0x7F, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64)
    return np.unique(v.numpy())


def _torch_e4m3_codes(v32):
    return torch.from_numpy(np.ascontiguousarray(v32, dtype=np.float32)).to(
        torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3_encoder_matches_torch_cast():
    grid = _e4m3_grid()
    mids = (grid[:-1] + grid[1:]) / 2  # exact ties between neighbours
    rng = np.random.default_rng(0)
    vals = np.concatenate([grid, mids, rng.uniform(-448, 448, 4000),
                           rng.uniform(-1, 1, 2000) * 2.0 ** rng.integers(-12, 0, 2000),
                           -grid, -mids, [0.0, -0.0, 2.0 ** -10, 2.0 ** -11 * 3]]).astype(np.float32)
    vals = vals[np.abs(vals) <= 448]
    ours = np.array([oracle.float_to_e4m3fn(float(v)) for v in vals], np.uint8)
    np.testing.assert_array_equal(ours, _torch_e4m3_codes(vals))
    # ties go to the even code (the grid step halves at each binade, so check on the codes)
    t = np.array([oracle.float_to_e4m3fn(float(v)) for v in mids.astype(np.float32)], np.uint8)
    assert np.all(t % 2 == 0)


def _ref_scale_exp(amax):
    """Smallest integer e with amax <= 448 * 2^e, by exact rational comparison (clamped)."""
    if amax == 0:
        return 0
    a = Fraction(amax)
    e = -200
    while a > 448 * Fraction(2) ** e:
        e += 1
    return max(-127, min(127, e))


def test_activation_scale_exponent_exact():
    rng = np.random.default_rng(1)
    cases = [0.0, 448.0, 448.0 * 2 ** -20, 448.0 * 2 ** 30, 1.0, 1e-30, 1e-45, 3e38]
    cases += list(np.nextafter(np.float32(448.0), np.float32(1e9)) * 2.0 ** np.arange(-5, 5))
    cases += list(np.nextafter(np.float32(448.0), np.float32(0)) * 2.0 ** np.arange(-5, 5))
    cases += list(rng.uniform(0, 1, 300) * 10.0 ** rng.integers(-30, 30, 300))
    for a in cases:
        a = float(np.float32(a))
        assert oracle.act_scale_exp(a) == _ref_scale_exp(a), a


def _ref_quantize(x, codes_out=None, exps_out=None):
    """[rows][K] float64 (exact in bf16) -> dequantised values, one power-of-two scale per 1x128
    block, codes from torch's float8_e4m3fn cast of x * 2^-e computed in float32."""
    rows, K = x.shape
    out = np.empty_like(x)
    for r in range(rows):
        for b in range(K // 128):
            blk = x[r, b * 128:(b + 1) * 128]
            e = _ref_scale_exp(float(np.max(np.abs(blk))))
            v = np.ldexp(blk.astype(np.float32), np.int32(-e)).astype(np.float32)
            c = _torch_e4m3_codes(v)
            out[r, b * 128:(b + 1) * 128] = np.ldexp(
                torch.from_numpy(c).view(torch.float8_e4m3fn).to(torch.float64).numpy(), e)
            if codes_out is not None:
                codes_out[r, b * 128:(b + 1) * 128] = c
                exps_out[r, b] = e
    return out


def test_quantize_rows_matches_reference():
    rng = np.random.default_rng(2)
    rows, K = 6, 512
    x = rng.standard_normal((rows, K)) * 10.0 ** rng.integers(-8, 8, (rows, K // 128)).repeat(128, 1)
    x[1, 128:256] = 0.0                       # an all-zero block
    x[2, 256:384] = 0.0
    x[2, 300] = -3.5                          # a single nonzero
    x[3, :128] = 448.0 * 2.0 ** 3             # amax exactly at a scale boundary
    bits = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    xb = oracle.bf16_bits_to_float(bits)
    codes, exps = oracle.quantize_rows(bits, K)
    rc = np.zeros((rows, K), np.uint8)
    re = np.zeros((rows, K // 128), np.int64)
    deq = _ref_quantize(xb, rc, re)
    np.testing.assert_array_equal(codes, rc)
    np.testing.assert_array_equal(exps.astype(np.int64), re)
    # round to nearest: within half a grid step, i.e. 2^-4 relative for normal codes
    nz = np.abs(xb) >= 2.0 ** -6 * 2.0 ** re.repeat(128, 1)
    assert np.all(np.abs(deq - xb)[nz] <= 2.0 ** -4 * np.abs(xb)[nz])
    # every nonzero block's largest magnitude lands in (224, 448] after scaling
    for r in range(rows):
        for b in range(K // 128):
            m = np.max(np.abs(xb[r, b * 128:(b + 1) * 128]))
            if m > 0:
                assert 224 < m * 2.0 ** -re[r, b] <= 448


def test_ffn_fp8_activations_dense_brute_force():
    layer = synth.make_layer(dict(T=24, H=384, I=256, E=6, k=3, score_fn="sigmoid", scores="uniform",
                                  wdtype="fp8"), seed=4)
    res = _check_layer_against_dense(layer, act_fp8=True)
    # the quantisation changes the result (it is not silently skipped)
    plain = oracle.moe_layer(layer, act_fp8=False)
    assert np.any(plain["out"] != res["out"])


def test_expert_phases_dense_brute_force():
    """The single-phase entry points against numpy float64 matrix products: arbitrary (token,
    expert) lists, a rectangular H != I scale grid with random per-block scales."""
    layer = synth.make_layer(dict(T=20, H=384, I=256, E=5, k=2, score_fn="sigmoid",
                                  scores="uniform", wdtype="fp8"), seed=9)
    g = torch.Generator().manual_seed(9)
    for s in (layer.experts.s_gate, layer.experts.s_up, layer.experts.s_down):
        s.mul_(torch.rand(s.shape, generator=g) * 4 + 0.25)
    rng = np.random.default_rng(9)
    token = rng.integers(0, layer.T, 60)
    slot = rng.integers(0, layer.E, 60)
    h = oracle.expert_gate_up(layer.x, token, slot, layer.experts)
    Wg, Wu, Wd = _dense_weights(layer.experts, layer.H, layer.I)
    x = oracle.bf16_bits_to_float(oracle._np(layer.x, np.uint16))
    G = np.einsum("pnc,pc->pn", Wg[slot], x[token])
    U = np.einsum("pnc,pc->pn", Wu[slot], x[token])
    h_ref = _to_bf16_f64(scipy.special.expit(G) * G * U)
    hb = oracle.bf16_bits_to_float(h)
    assert np.mean(hb == h_ref) > 0.999  # (the dense path's fp32 detour may move a tie)
    np.testing.assert_allclose(hb, h_ref, rtol=2.0 ** -7, atol=0)
    # phase 2 on bf16 rows of every magnitude class, independent of phase 1
    hrand = torch.from_numpy(rng.standard_normal((60, layer.I)).astype(np.float32) *
                             np.exp2(rng.integers(-8, 8, (60, 1))).astype(np.float32))
    hbits = hrand.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    y = oracle.expert_down(hbits, slot, layer.experts)
    y_ref = np.einsum("pcn,pn->pc", Wd[slot], oracle.bf16_bits_to_float(hbits))
    np.testing.assert_allclose(y, y_ref, rtol=1e-12, atol=1e-300)


def test_expert_phases_reproduce_the_layer():
    """Phase 1 then phase 2 on the layer's own (token, expert) pairs give the layer's h and y."""
    layer = synth.make_layer("tiny_fp8", seed=4)
    res = oracle.moe_layer(layer, want_h=True, want_y=True)
    token = np.repeat(np.arange(layer.T), layer.k)
    slot = res["ids"].reshape(-1)
    h = oracle.expert_gate_up(layer.x, token, slot, layer.experts)
    np.testing.assert_array_equal(h, res["h"].reshape(-1, layer.I))
    y = oracle.expert_down(h, slot, layer.experts)
    np.testing.assert_array_equal(y, res["y"].reshape(-1, layer.H))


def test_fp4_e2m1_decode_matches_the_ocp_table():
    for c in range(16):
        want = (-1.0 if c & 8 else 1.0) * OCP_E2M1[c & 7]
        assert oracle.fp4_e2m1_to_double(c) == want, c


def test_e8m0_decode():
    assert oracle.e8m0_to_double(127) == 1.0
    assert np.isnan(oracle.e8m0_to_double(255))
    v = np.array([oracle.e8m0_to_double(s) for s in range(255)])
    m, e = np.frexp(v)
    assert np.all(m == 0.5) and np.all(np.diff(e) == 1)  # consecutive powers of two
    assert v[0] == 2.0 ** -127 and v[254] == 2.0 ** 127


def test_mxfp4_generator_round_to_nearest_even():
    """The synthetic 4-bit weights: every element is the nearest E2M1 value of w / 2^X (ties to
    the even code), X = floor(log2(max|w|)) - 2 per group of 32."""
    g = torch.Generator().manual_seed(3)
    w = torch.randn((8, 256), generator=g) * 0.02
    q, sc = synth.quantize_mxfp4(w)
    (deq,) = [_dense_weights(synth.ExpertWeights("mxfp4", q[None], q[None], q[None], sc[None],
                                                 sc[None], sc[None]), 256, 8)[0][0]]
    wd = w.double().numpy()
    X = np.floor(np.log2(np.abs(wd).reshape(8, 8, 32).max(-1))) - 2
    assert np.array_equal(sc.numpy().astype(np.int64), (X + 127).astype(np.int64))
    grid = np.concatenate([-OCP_E2M1[::-1], OCP_E2M1[1:]])
    p = (wd.reshape(8, 8, 32) / np.exp2(X)[..., None]).reshape(8, 256)
    err = np.abs(grid[None, None, :] - p[..., None])
    best = err.min(-1)
    got = (deq / np.repeat(np.exp2(X), 32, axis=1))
    assert np.all(np.abs(got - p) <= best + 1e-12)  # a nearest grid value (saturation aside)


def test_ffn_dense_brute_force_mxfp4():
    _check_layer_against_dense(synth.make_layer(dict(T=24, H=256, I=128, E=6, k=2,
                                                     score_fn="sigmoid", scores="uniform",
                                                     wdtype="mxfp4"), seed=2))


def test_ffn_mxfp4_fp8_activations_dense_brute_force():
    """W4A8: MXFP4 weights (OCP E2M1 table, numpy scale expansion) with the FP8-quantised
    activations of the dense brute force."""
    layer = synth.make_layer(dict(T=24, H=384, I=256, E=6, k=3, score_fn="sigmoid",
                                  scores="uniform", wdtype="mxfp4"), seed=6)
    res = _check_layer_against_dense(layer, act_fp8=True)
    plain = oracle.moe_layer(layer, act_fp8=False)
    assert np.any(plain["out"] != res["out"])


# ----------------------------------------------------------------------------- batched form
# oracle.moe_layer_batched evaluates the same definition expert by expert with float64 library
# matrix products (what makes the full-size layers cheap to check on every row).  It is pinned
# like the per-token form: against the dense brute force in every weight and activation mode,
# and against the per-token form itself up to the order of the float64 sums.

_MID = dict(T=24, H=384, I=256, E=6, k=3, score_fn="sigmoid", scores="uniform")


@pytest.mark.parametrize("cfg,act_fp8", [
    ("tiny", False), ("tiny_fp8", False),
    (dict(_MID, wdtype="fp8"), True),
    (dict(_MID, T=24, H=256, I=128, k=2, wdtype="mxfp4"), False),
    (dict(_MID, wdtype="mxfp4"), True)])
def test_batched_form_dense_brute_force(cfg, act_fp8):
    layer = synth.make_layer(cfg, seed=4)
    _check_layer_against_dense(layer, act_fp8=act_fp8, fn=oracle.moe_layer_batched)


def test_batched_form_rectangular_scale_grid():
    layer = synth.make_layer(dict(_MID, wdtype="fp8"), seed=3)
    g = torch.Generator().manual_seed(5)
    for ew in (layer.experts, layer.shared):
        for s in (ew.s_gate, ew.s_up, ew.s_down):
            s.mul_(torch.rand(s.shape, generator=g) * 4 + 0.25)
    _check_layer_against_dense(layer, fn=oracle.moe_layer_batched)


@pytest.mark.parametrize("act_fp8", [False, True])
def test_batched_form_agrees_with_per_token_form(act_fp8):
    """Many tokens per expert, a row subset in a scrambled order, and an expert range: the two
    forms route identically, give the same h bits except where the float64 sums land on the two
    sides of a bf16 tie (never more than one ulp), and y and out to float64 rounding."""
    layer = synth.make_layer(dict(T=96, H=384, I=256, E=8, k=3, score_fn="sigmoid",
                                  scores="uniform", wdtype="fp8"), seed=7)
    rows = np.random.default_rng(1).permutation(96)[:70]
    for er in (None, (2, 6)):
        a = oracle.moe_layer(layer, rows=rows, want_h=True, want_y=True, act_fp8=act_fp8,
                             expert_range=er)
        b = oracle.moe_layer_batched(layer, rows=rows, want_h=True, want_y=True,
                                     act_fp8=act_fp8, expert_range=er)
        np.testing.assert_array_equal(a["ids"], b["ids"])
        np.testing.assert_array_equal(a["w"], b["w"])
        for key in ("h", "hS"):
            ha, hb = oracle.bf16_bits_to_float(a[key]), oracle.bf16_bits_to_float(b[key])
            assert np.mean(ha == hb) > 0.9999
            np.testing.assert_allclose(hb, ha, rtol=2.0 ** -7, atol=0)
        same = np.all(a["h"] == b["h"], axis=-1)
        np.testing.assert_allclose(b["y"][same], a["y"][same], rtol=1e-9, atol=1e-13)
        np.testing.assert_allclose(b["S"], a["S"], rtol=1e-9, atol=1e-13)
        oa, ob = oracle.bf16_bits_to_float(a["out"]), oracle.bf16_bits_to_float(b["out"])
        np.testing.assert_allclose(ob, oa, rtol=2.0 ** -7, atol=0)
        assert np.mean(oa == ob) > 0.999
        if er is not None:  # outside the range: nothing
            local = (a["ids"] >= er[0]) & (a["ids"] < er[1])
            assert not b["y"][~local].any() and not b["h"][~local].any()


def test_batched_helpers():
    """The element-wise pieces: dequantisation equals the FP8 code times its block's scale;
    SiLU-times-up rounding and the double -> bf16 array rounding equal the scalar functions."""
    layer = synth.make_layer(dict(_MID, wdtype="fp8"), seed=2)
    one = layer.experts.select([3])
    Wg, Wu, Wd = _dense_weights(one, layer.H, layer.I)
    for which, ref in enumerate((Wg[0], Wu[0], Wd[0])):
        np.testing.assert_array_equal(oracle.dequantize(one, which), ref)
    rng = np.random.default_rng(3)
    g, u = rng.standard_normal(500) * 4, rng.standard_normal(500)
    h = oracle.silu_mul_bf16(g, u)
    assert all(h[i] == oracle.double_to_bf16(g[i] / (1 + np.exp(-g[i])) * u[i]) for i in range(500))
    v = rng.standard_normal(300) * np.exp2(rng.integers(-40, 40, 300))
    assert list(oracle.double_to_bf16_array(v)) == [oracle.double_to_bf16(t) for t in v]


@pytest.mark.parametrize("wdtype", ["fp8", "mxfp4"])
def test_batched_phases_agree_with_per_row_phases(wdtype):
    layer = synth.make_layer(dict(_MID, wdtype=wdtype), seed=5)
    rng = np.random.default_rng(5)
    token = rng.integers(0, layer.T, 80)
    slot = rng.integers(0, layer.E, 80)
    h = oracle.expert_gate_up(layer.x, token, slot, layer.experts)
    hb = oracle.expert_gate_up_batched(layer.x, token, slot, layer.experts)
    fa, fb = oracle.bf16_bits_to_float(h), oracle.bf16_bits_to_float(hb)
    assert np.mean(fa == fb) > 0.999
    np.testing.assert_allclose(fb, fa, rtol=2.0 ** -7, atol=0)
    y = oracle.expert_down(h, slot, layer.experts)
    yb = oracle.expert_down_batched(h, slot, layer.experts)
    np.testing.assert_allclose(yb, y, rtol=1e-9, atol=1e-13)
