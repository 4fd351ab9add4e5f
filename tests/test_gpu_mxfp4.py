"""GPU parity of the 4-bit MXFP4 weight format (OCP E2M1 codes with one E8M0 scale per 32 inputs)
against the oracle.  Bars as for the other weight formats."""
import numpy as np
import pytest
import torch

import oracle
import routed_expert_grouped_amd as moe
import synth
from gpu_util import DEV, compare_sampled, compare_with_oracle, layer_for, mid, run_gpu

pytestmark = pytest.mark.gpu

E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


@pytest.mark.parametrize("route", ["gemv", "gemm"])
@pytest.mark.parametrize("I", [
    128,    # one 128-block per row: the smallest scale window
    640,    # 5 blocks: a window of odd length, the last stage half used
    2048,   # 16 blocks
    8448,   # 66 blocks: two full 32-block windows of the four-group kernel, then one of 2
])
def test_mxfp4_decode_and_scale_layout_exhaustive(I, route):
    """Down projection with identity activations reads every weight back exactly:
    y[p][c] = code(Wd[c][p]) * 2^(s[c][p/32] - 127), over all 16 codes in both nibbles and scales
    from 2^-20 to 2^20.  "gemv": 32 rows a call (the decode kernel); "gemm": all I rows in one
    call (the 4-bit GEMM)."""
    H = 256
    rng = np.random.default_rng(I)
    codes = rng.integers(0, 16, size=(H, I))
    codes[:16, :16] = np.arange(16)[:, None]  # every code in both nibble positions
    scales = rng.integers(127 - 20, 127 + 21, size=(H, I // 32))
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    q = torch.from_numpy(packed)[None].to(DEV)
    s = torch.from_numpy(scales.astype(np.uint8))[None].to(DEV)
    g = torch.zeros((1, I, H // 2), dtype=torch.uint8, device=DEV)
    gs = torch.full((1, I, H // 32), 127, dtype=torch.uint8, device=DEV)
    ew = synth.ExpertWeights("mxfp4", g, g, q, gs, gs, s)
    eye = torch.eye(I, dtype=torch.float32).to(torch.bfloat16).view(torch.int16).to(DEV)
    w = moe.expert_weights(ew)
    if route == "gemm":
        y = moe.moe_expert_down(eye, I, 1, None, w)
    else:
        y = torch.cat([moe.moe_expert_down(eye[p:p + 32].contiguous(), 32, 1, None, w)
                       for p in range(0, I, 32)])
    torch.cuda.synchronize()
    got = oracle.bf16_bits_to_float(y.cpu())  # [p][c]
    want = np.where(codes & 8, -1.0, 1.0) * E2M1[codes & 7] * np.exp2(np.repeat(scales, 32, 1) - 127.0)
    np.testing.assert_array_equal(got, want.T)


@pytest.mark.parametrize("cfg", [
    dict(T=16, H=256, I=128, E=16, k=2, score_fn="softmax", scores="normal", wdtype="mxfp4"),
    mid(wdtype="mxfp4"),                       # many rows per expert: the 4-bit GEMM
    mid(T=37, E=64, k=8, wdtype="mxfp4"),
    mid(T=160, H=640, E=8, k=2, wdtype="mxfp4"),              # phase 2 (N = 640): 2.5 column
                                                              # tiles of the 4-bit GEMM
    mid(T=30, H=128, I=384, E=4, k=2, wdtype="mxfp4"),       # K = 128 in phase 1
    mid(T=60, H=16384, I=256, E=4, k=2, wdtype="mxfp4"),     # the largest H: two scale windows
    mid(T=40, H=256, I=8320, E=3, k=1, wdtype="mxfp4"),      # phase 2: 65 blocks (32 + 32 + 1)
    # phase 2 with H = 384 (not a multiple of 256): the two-group decode kernel, whose 64-block
    # scale window refills after the first 64 of the 66 blocks
    mid(T=40, H=384, I=8448, E=3, k=1, wdtype="mxfp4"),
    mid(T=300, E=4, k=1, score_fn="softmax", wdtype="mxfp4"),  # 4-bit GEMM: deep m-tile stacks
    mid(T=200, H=16384, I=256, E=4, k=2, wdtype="mxfp4"),    # 4-bit GEMM at K = 16384
    mid(T=200, H=256, I=8320, E=3, k=1, wdtype="mxfp4"),     # 4-bit GEMM phase 2: 65 slots (odd)
    mid(T=300, H=384, E=8, k=4, wdtype="mxfp4"),             # phase 2 N = 384: one whole and one
                                                              # half column tile, 150 rows/expert
])
def test_mxfp4_layer(cfg):
    layer = layer_for(cfg, seed=1)
    compare_with_oracle(layer, run_gpu(layer))


def test_mxfp4_dsv3_decode_full():
    layer = layer_for("dsv3_decode", wdtype="mxfp4")
    g = run_gpu(layer)
    compare_sampled(layer, g, rows=list(range(layer.T)))


@pytest.mark.parametrize("cfg", [
    mid(wdtype="mxfp4"),                                        # W4A8 GEMMs, ragged m-tiles
    mid(T=300, E=4, k=1, score_fn="softmax", wdtype="mxfp4"),   # phase 2: 384 = 1.5 weight slots
    mid(T=200, H=2560, E=8, k=2, wdtype="mxfp4"),               # 10 slots, 32-byte exponent rows
    mid(T=160, H=640, E=8, k=2, wdtype="mxfp4"),                # 2.5 slots; phase 2 dequantises
    mid(T=144, H=8192, I=256, E=2, k=2, wdtype="mxfp4"),        # K = 8192, the GEMM's largest
    mid(T=200, H=256, I=128, E=2, k=1, wdtype="mxfp4"),         # smallest K: 256 (one weight
                                                                # slot), 128 (two stages)
    mid(T=200, H=16384, I=256, E=4, k=2, wdtype="mxfp4"),       # phase 1 dequantises (K > 8192)
    mid(T=37, E=64, k=8, wdtype="mxfp4"),                       # few rows: dequantise + GEMV
])
def test_w4a8_layer(cfg):
    """MXFP4 weights with FP8 activations against the oracle's model of the same arithmetic."""
    layer = layer_for(cfg, seed=1)
    compare_with_oracle(layer, run_gpu(layer, act="fp8"), act_fp8=True)
