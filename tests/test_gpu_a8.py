"""GPU parity of the FP8 activation mode (E4M3FN activations in 1x128 blocks with power-of-two
scales) against the oracle's model of the same arithmetic.

Bars: codes and block exponents bit-exact; h, y, the shared expert's output and the layer output
within the same 1e-2 relative L2 per row as the bf16 mode.
"""
import numpy as np
import pytest
import torch

import oracle
import routed_expert_grouped_amd as moe
import synth
from gpu_util import (DEV, assert_rows_close, compare_sampled, compare_with_oracle, layer_for, mid,
                      rel_l2_rows, run_gpu)

pytestmark = pytest.mark.gpu


def _bf16_bits(v):
    return torch.from_numpy(np.asarray(v, np.float32)).to(torch.bfloat16).view(torch.int16)


def _quant_inputs():
    """Rows of 512 values (4 blocks) that reach every branch of the quantiser."""
    rng = np.random.default_rng(7)
    rows = []
    # magnitudes over the whole bf16 range, one decade per row
    for p in range(-130, 128, 6):
        rows.append(rng.standard_normal(512) * 2.0 ** p)
    # heavy tails inside a block: small values become E4M3 subnormals or zero
    rows.append(rng.standard_normal(512) * np.exp2(rng.integers(-30, 4, 512)))
    b = np.zeros(512)  # an all-zero block, a single nonzero, signed zeros, the 448 boundary
    b[128] = 3.0
    b[256:384] = -0.0
    b[384], b[385], b[386] = 448.0, -1.0, 0.01
    rows.append(b)
    c = np.zeros(512)
    c[0:128] = 450.0  # just above 448: the next exponent
    c[128:256] = np.linspace(-448, 448, 128)
    c[256:384] = 2.0 ** -133  # bf16's smallest subnormal: the exponent clamps at -127
    c[384:512] = 3.0e38  # near bf16's largest finite value
    rows.append(c)
    # values halfway between two E4M3 codes (ties to even), of both signs
    m = rng.integers(0, 8, 512)
    e = rng.integers(-6, 9, 512)
    t = (1 + (2 * m + 1) / 16.0) * 2.0 ** e * rng.choice([-1.0, 1.0], 512)
    t[::128] = 448.0  # fixes the block scale at 2^0
    rows.append(t)
    return _bf16_bits(np.stack(rows))


def test_quantize_act_bit_exact():
    x = _quant_inputs()
    codes, exps = moe.moe_quantize_act(x.to(DEV))
    torch.cuda.synchronize()
    rc, re_ = oracle.quantize_rows(x.numpy().view(np.uint16), x.shape[1])
    np.testing.assert_array_equal(exps.cpu().numpy()[:, :x.shape[1] // 128], re_)
    np.testing.assert_array_equal(codes.cpu().numpy(), rc)
    assert re_.min() == -127 and (rc == 0x80).any()  # the clamp and a signed zero were reached


def test_quantize_act_ragged_row_counts():
    """Row counts that leave the last workgroup partly idle (4 blocks per workgroup)."""
    rng = np.random.default_rng(3)
    for rows, K in ((1, 128), (3, 384), (5, 7168), (37, 2048)):
        x = _bf16_bits(rng.standard_normal((rows, K)) * 10)
        codes, exps = moe.moe_quantize_act(x.to(DEV), pitch=K // 128)  # unpadded rows
        torch.cuda.synchronize()
        rc, re_ = oracle.quantize_rows(x.numpy().view(np.uint16), K)
        np.testing.assert_array_equal(exps.cpu().numpy(), re_)
        np.testing.assert_array_equal(codes.cpu().numpy(), rc)


@pytest.mark.parametrize("cfg", [
    "tiny_fp8",                                   # few rows per expert: dequantise + GEMV
    mid(),                                        # FP8-code GEMMs in both phases, ragged tails
    mid(T=37, E=64, k=8),                         # mostly 1-row experts, some empty
    mid(T=160, H=640, E=8, k=2),                  # phase 2 outside the FP8 GEMM's tiles
    mid(T=300, E=4, k=1, score_fn="softmax"),     # few experts with many rows (m-tile stacks)
    mid(T=200, H=2560, E=8, k=2),                 # 20 exponent blocks a row (32-byte pitch)
    mid(T=150, H=5120, E=6, k=2),                 # 40 blocks (48-byte pitch)
    mid(T=256, E=32, k=2, scores="zipf"),         # skewed routing
    mid(T=144, H=8192, I=256, E=2, k=2),          # K = 8192, the FP8-code GEMM's largest
    mid(T=200, H=16384, I=256, E=4, k=2),         # the largest H: phase 1 dequantises
    mid(T=150, H=256, I=16384, E=2, k=1),         # the largest I: phase 2 dequantises
    mid(T=600, I=512, E=8, k=2, scores="zipf"),   # 160 x 512 tiles (150 rows an expert on
                                                  # average), a hot expert's m-tile stack
    mid(T=120, H=640, I=768, E=4, k=2),           # 160 x 512 tiles in phase 1 with 5 blocks
])
def test_a8_layer(cfg):
    layer = layer_for(cfg, seed=1)
    g = run_gpu(layer, act="fp8")
    compare_with_oracle(layer, g, act_fp8=True)


def test_a8_block_scales_zero_and_wide_range():
    """Weight blocks with zero scales and scales over six decades, on the FP8-code GEMMs."""
    layer = synth.make_layer(mid(T=200, E=8, k=2, I=512), seed=5)
    rng = np.random.default_rng(5)
    for ew in (layer.experts, layer.shared):
        for name in ("s_gate", "s_up", "s_down"):
            s = getattr(ew, name)
            f = rng.choice(np.array([0.0, 1e-3, 1.0, 1e3], np.float32), size=tuple(s.shape))
            s.mul_(torch.from_numpy(f))
    layer = layer.to(DEV)
    g = run_gpu(layer, act="fp8")
    assert g["counts"].max() > 32
    compare_with_oracle(layer, g, act_fp8=True)


def test_a8_repeat_runs_are_bit_identical():
    layer = layer_for(mid(), seed=1)
    a, b = run_gpu(layer, act="fp8"), run_gpu(layer, act="fp8")
    for key in a:
        np.testing.assert_array_equal(a[key], b[key])


def test_a8_is_not_the_bf16_path():
    """The FP8 mode's outputs sit much closer to the oracle's FP8 model than to its bf16 one."""
    layer = layer_for(mid(), seed=1)
    g = run_gpu(layer, act="fp8")
    f = oracle.bf16_bits_to_float
    a8 = oracle.moe_layer(layer, act_fp8=True)
    bf = oracle.moe_layer(layer, act_fp8=False)
    d_a8 = np.median(rel_l2_rows(f(g["out"]), f(a8["out"])))
    d_bf = np.median(rel_l2_rows(f(g["out"]), f(bf["out"])))
    assert d_bf > 1e-2 and d_a8 < d_bf / 10, (d_a8, d_bf)


def test_a8_dsv3_decode_full():
    layer = layer_for("dsv3_decode")
    g = run_gpu(layer, act="fp8")
    compare_sampled(layer, g, rows=list(range(layer.T)), act_fp8=True)


def _dequant_bits(codes, exps):
    """bf16 bits of code * 2^e, exactly: the activations that quantised rows stand for."""
    v = codes.view(torch.float8_e4m3fn).to(torch.float32)
    v = v * torch.exp2(exps.to(torch.float32)).repeat_interleave(128, dim=1)
    return v.to(torch.bfloat16).view(torch.int16)


def _padded(exps, pitch):
    out = torch.zeros((exps.shape[0], pitch), dtype=torch.int8)
    out[:, :exps.shape[1]] = exps
    return out


@pytest.mark.parametrize("wdtype", ["fp8", "mxfp4"])
@pytest.mark.parametrize("cfg,rows", [
    (mid(T=200, E=8, k=2), None),                      # every row; ragged m-tiles
    (mid(T=300, H=2560, I=256, E=4, k=2), None),      # 32-byte exponent pitch, deep m-tile stacks
    (mid(T=120, H=256, I=1152, E=3, k=1), None),      # odd number of 128-blocks in phase 2
    ("dsv3_prefill", None),                             # full size, every assignment
])
def test_a8_phases_exact_inputs(cfg, rows, wdtype):
    """The FP8-code GEMMs (FP8 or MXFP4 weights) on quantised activations drawn directly (codes
    and exponents), against the oracle's phases on the values they stand for: no quantisation
    on either side.  Every assignment's row of h and y is compared."""
    layer = layer_for(cfg, wdtype=wdtype) if isinstance(cfg, str) else layer_for(dict(cfg, wdtype=wdtype))
    T, H, I, E, k = layer.T, layer.H, layer.I, layer.E, layer.k
    ids = synth.random_topk_ids(T, E, k, seed=21)
    counts, offsets, perm, inv = oracle.permute(ids.numpy(), E)
    got = moe.moe_permute(ids.to(DEV), E)
    for a, b in zip(got, (counts, offsets, perm, inv)):
        np.testing.assert_array_equal(a.cpu().numpy(), b)
    _, offsets_d, perm_d, _ = got
    w = moe.expert_weights(layer.experts)
    xc, xe = synth.random_fp8_activations(T, H, seed=22)
    hc, he = synth.random_fp8_activations(T * k, I, seed=23)
    h = moe.moe_expert_gate_up_a8(xc.to(DEV), _padded(xe, moe.exp_pitch(H)).to(DEV), k, perm_d,
                                  offsets_d, w)
    y = moe.moe_expert_down_a8(hc.to(DEV), _padded(he, moe.exp_pitch(I)).to(DEV), T, k,
                               offsets_d, w)
    torch.cuda.synchronize()
    flat = np.arange(T * k) if rows is None else np.array([t * k + j for t in rows for j in range(k)])
    experts = ids.numpy().reshape(-1)[flat]
    f = oracle.bf16_bits_to_float
    big = T * k > 4096  # the oracle's expert-by-expert form at full size (weights read in place)
    if big:
        gate_up, down = oracle.expert_gate_up_batched, oracle.expert_down_batched
        slot, sub = experts, layer.experts
    else:
        gate_up, down = oracle.expert_gate_up, oracle.expert_down
        used = sorted(set(experts.tolist()))
        slot = np.searchsorted(used, experts)
        sub = layer.experts.select(used)
    h_ref = gate_up(_dequant_bits(xc, xe), flat // k, slot, sub)
    assert_rows_close("h", f(h.cpu().numpy().view(np.uint16)[inv[flat]]), f(h_ref))
    p = inv[flat]  # grouped rows of the checked assignments
    y_ref = down(_dequant_bits(hc[torch.from_numpy(p)], he[torch.from_numpy(p)]), slot, sub)
    assert_rows_close("y", f(y.cpu().numpy().view(np.uint16)[p]), y_ref)


def test_a8_rejects_bf16_weights():
    layer = layer_for("tiny")
    with pytest.raises(moe.MoeError) as ei:
        run_gpu(layer, act="fp8")
    assert ei.value.status == moe.MOE_ERR_UNSUPPORTED
