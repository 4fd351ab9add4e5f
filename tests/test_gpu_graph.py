"""The layer captured into a HIP graph: every replay equals the eager forward, bit for bit, also
after the inputs change in place and with other GPU work and synchronisations in between; and
the replayed output meets the oracle's bars by itself."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import routed_expert_grouped_amd as moe
from gpu_util import DEV, assert_rows_close, layer_for, mid

pytestmark = pytest.mark.gpu


def _eager(layer, act, fuse="auto"):
    L = moe.MoeLayer(layer.T, layer.H, layer.I, layer.E, layer.k, layer.experts, layer.shared,
                     layer.score_fn, layer.renorm, act=act, fuse_shared=fuse)
    out = L.forward(layer.scores, layer.x).clone()
    torch.cuda.synchronize()
    return out


# fuse: the shared expert inside the routed launches ("auto" at decode sizes) or on the side
# stream (False)
@pytest.mark.parametrize("cfg,act,fuse", [("tiny_fp8", "bf16", "auto"), (mid(), "bf16", "auto"),
                                          (mid(), "fp8", "auto"), ("dsv3_decode", "bf16", "auto"),
                                          ("dsv3_decode", "bf16", False)])
def test_graph_replays_match_eager(cfg, act, fuse):
    layer = layer_for(cfg)
    scores, x = layer.scores.clone(), layer.x.clone()  # the captured input buffers
    L = moe.MoeLayer(layer.T, layer.H, layer.I, layer.E, layer.k, layer.experts, layer.shared,
                     layer.score_fn, layer.renorm, act=act, fuse_shared=fuse)
    L.capture(scores, x)
    want = _eager(layer, act, fuse)
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
    assert torch.equal(got, _eager(layer2, act, fuse))


@pytest.mark.parametrize("cfg,fuse", [("tiny", "auto"), ("tiny_fp8", "auto"),
                                      ("dsv3_decode", "auto"), ("dsv3_decode", False)])
def test_graph_replay_against_the_oracle(cfg, fuse):
    """Replays of the captured layer (the shared expert inside the routed launches, and for the
    DeepSeek-V3 decode layer also on the side stream) against the oracle: routing ids bit-exact,
    the layer output within 1e-2 relative L2 per row, on each of three replays and after the
    inputs change in place."""
    layer = layer_for(cfg)
    scores, x = layer.scores.clone(), layer.x.clone()
    L = moe.MoeLayer(layer.T, layer.H, layer.I, layer.E, layer.k, layer.experts, layer.shared,
                     layer.score_fn, layer.renorm, fuse_shared=fuse)
    L.capture(scores, x)
    f = oracle.bf16_bits_to_float
    for rep, shift in enumerate((0, 0, 0, 3)):
        lay = dataclasses.replace(layer, scores=torch.roll(layer.scores, shift, 0),
                                  x=torch.roll(layer.x, shift, 0))
        scores.copy_(lay.scores)
        x.copy_(lay.x)
        out = L.replay().clone()
        torch.cuda.synchronize()
        ref = oracle.moe_layer_batched(lay) if layer.H > 1024 else oracle.moe_layer(lay)
        np.testing.assert_array_equal(L.topk_ids.cpu().numpy(), ref["ids"])
        assert_rows_close(f"replay {rep} out", f(out.cpu().numpy().view(np.uint16)), f(ref["out"]))
