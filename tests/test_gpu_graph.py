"""The layer captured into a HIP graph: every replay equals the eager forward, bit for bit, also
after the inputs change in place and with other GPU work and synchronisations in between."""
import dataclasses

import pytest
import torch

import routed_expert_grouped_amd as moe
from gpu_util import DEV, layer_for, mid

pytestmark = pytest.mark.gpu


def _eager(layer, act):
    L = moe.MoeLayer(layer.T, layer.H, layer.I, layer.E, layer.k, layer.experts, layer.shared,
                     layer.score_fn, layer.renorm, act=act)
    out = L.forward(layer.scores, layer.x).clone()
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("cfg,act", [("tiny_fp8", "bf16"), (mid(), "bf16"), (mid(), "fp8"),
                                     ("dsv3_decode", "bf16")])
def test_graph_replays_match_eager(cfg, act):
    layer = layer_for(cfg)
    scores, x = layer.scores.clone(), layer.x.clone()  # the captured input buffers
    L = moe.MoeLayer(layer.T, layer.H, layer.I, layer.E, layer.k, layer.experts, layer.shared,
                     layer.score_fn, layer.renorm, act=act)
    L.capture(scores, x)
    want = _eager(layer, act)
    for rep in range(3):
        torch.cuda.synchronize()
        junk = torch.randn(1 << 20, device=DEV).sum()  # unrelated eager work between replays
        got = L.replay().clone()
        torch.cuda.synchronize()
        assert torch.equal(got, want), f"replay {rep} differs from the eager forward"
        del junk
    # new inputs (the tokens rotated by one), copied into the captured buffers
    layer2 = dataclasses.replace(layer, scores=torch.roll(layer.scores, 1, 0),
                                 x=torch.roll(layer.x, 1, 0))
    scores.copy_(layer2.scores)
    x.copy_(layer2.x)
    got = L.replay().clone()
    torch.cuda.synchronize()
    assert torch.equal(got, _eager(layer2, act))
