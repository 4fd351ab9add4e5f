"""The mid-size layer shapes of the other GPU tests again, drawn from further seeds and run in
both activation modes, every token row compared with the oracle (same bars as
test_gpu_parity.py).  Each seed draws new router scores (so new expert row counts and m-tile
tails), activations and weights.  MOE_TEST_SEEDS sets how many seeds run (default 3; a 30-seed
sweep, 930 layers, passed)."""
import os

import pytest

import synth
from gpu_util import DEV, compare_with_oracle, mid, run_gpu

pytestmark = pytest.mark.gpu

SEEDS = range(100, 100 + int(os.environ.get("MOE_TEST_SEEDS", "3")))

SHAPES = {
    "tiles_ragged": dict(),
    "one_row_experts": dict(T=37, E=64, k=8),
    "few_experts_softmax": dict(T=300, E=4, k=1, score_fn="softmax"),
    "one_token": dict(T=1, E=24, k=4),
    "k_equals_E": dict(T=64, E=16, k=16, renorm=0),
    "bf16_weights": dict(T=96, E=40, k=3, score_fn="softmax", renorm=0, wdtype="bf16"),
    "H_odd_blocks": dict(T=160, H=640, E=8, k=2),
    "gemv_odd_blocks": dict(T=24, H=640, E=16, k=2),
    "gemv_two_parts": dict(T=24, H=768, E=16, k=2),
    "tiles_160x512": dict(T=300, I=512, E=8, k=4),
    "tiles_256x256": dict(T=600, I=512, E=8, k=4),
    "zipf": dict(T=256, E=32, k=2, scores="zipf"),
    "mxfp4_160_rows": dict(T=300, I=512, E=8, k=4, wdtype="mxfp4"),
    "mxfp4_300_rows": dict(T=600, I=512, E=8, k=4, wdtype="mxfp4"),
    "mxfp4_gemv": dict(T=37, E=64, k=8, wdtype="mxfp4"),
    "mxfp4_smallest_K": dict(T=200, H=256, I=128, E=2, k=1, wdtype="mxfp4"),
}


# the FP8-activation mode takes FP8 or MXFP4 weights
CASES = [(s, a) for s in sorted(SHAPES) for a in ("bf16", "fp8")
         if not (a == "fp8" and SHAPES[s].get("wdtype") == "bf16")]


@pytest.mark.parametrize("seed", SEEDS)
@pytest.mark.parametrize("shape,act", CASES)
def test_mid_layers_further_seeds(shape, act, seed):
    layer = synth.make_layer(mid(**SHAPES[shape]), seed=seed).to(DEV)
    compare_with_oracle(layer, run_gpu(layer, act=act), act_fp8=act == "fp8")
