"""Whole layers at the limits of the grouped GEMMs, every token row against the oracle (same bars
as test_gpu_parity.py), in both activation modes:

- E = 1024 (MOE_MAX_EXPERTS) with 8 assignments a token and 64 rows an expert on average: the
  GEMM path's tile search over 1024 groups (16 a lane), FP8 and MXFP4 weights;
- k = 32 (the largest top-k) over 64 experts;
- H = 16384 and I = 16384 in the FP8-activation mode (K above the FP8-code GEMM's 8192: that
  phase dequantises to bf16);
- two experts with 2500 rows each at K = 128: ten-deep m-tile stacks and the smallest K.
"""
import pytest

import synth
from gpu_util import DEV, compare_with_oracle, mid, run_gpu

pytestmark = pytest.mark.gpu

CASES = [
    (dict(T=8192, H=256, I=256, E=1024, k=8), "bf16"),
    (dict(T=8192, H=256, I=256, E=1024, k=8), "fp8"),
    (dict(T=8192, H=256, I=256, E=1024, k=8, wdtype="mxfp4"), "bf16"),
    (dict(T=8192, H=256, I=256, E=1024, k=8, wdtype="mxfp4"), "fp8"),
    (dict(T=2048, H=256, I=256, E=64, k=32), "bf16"),
    (dict(T=2048, H=256, I=256, E=64, k=32), "fp8"),
    (dict(T=600, H=16384, I=256, E=4, k=2), "fp8"),
    (dict(T=600, H=256, I=16384, E=4, k=2), "fp8"),
    (dict(T=5000, H=128, I=128, E=2, k=1, score_fn="softmax"), "bf16"),
    (dict(T=5000, H=128, I=128, E=2, k=1, score_fn="softmax"), "fp8"),
]


@pytest.mark.parametrize("over,act", CASES,
                         ids=[f"{'-'.join(f'{k}{v}' for k, v in o.items())}-{a}" for o, a in CASES])
def test_layer_at_limits(over, act):
    layer = synth.make_layer(mid(**over), seed=7).to(DEV)
    compare_with_oracle(layer, run_gpu(layer, act=act), act_fp8=act == "fp8", n_threads=16)
