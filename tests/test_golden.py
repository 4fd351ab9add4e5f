"""The layer shapes (synth/) and the byte accounting that bench.py reports against, pinned to
the numbers the pages print (tests/golden/page_figures.json, each with its citation).

A wrong shape, a transposed dimension or a byte formula that drops the scales or counts a
matrix twice moves at least one of these figures outside the rounding of the printed value.
"""
import json
import os

import bench
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_figures.json")
MOE_LAYERS = 58  # DeepSeek-V3 MoE layers (the pages' count)


def figures():
    return {f["name"]: f for f in json.load(open(GOLDEN))["figures"]}


def close(name, got):
    f = figures()[name]
    want, tol = f["value"], f["rel_tol"]
    assert abs(got - want) <= tol * abs(want), f"{name}: {got} vs printed {want} ({f['cite']})"


def test_every_figure_has_a_citation():
    for f in figures().values():
        assert f["cite"] and f["value"] > 0


def test_deepseek_v3_expert_sizes():
    c = synth.CONFIGS["dsv3_decode"]
    H, I, E, k = c["H"], c["I"], c["E"], c["k"]
    params_per_expert = 3 * H * I
    close("dsv3_routed_params", MOE_LAYERS * E * params_per_expert)
    close("dsv3_routed_params_per_token", MOE_LAYERS * k * params_per_expert)
    close("dsv3_routed_gb_per_token_at_4p5_bit", MOE_LAYERS * k * params_per_expert * 4.5 / 8 / 1e9)
    close("dsv3_expert_weight_tensors", MOE_LAYERS * E * 3)
    # one FP8 matrix: bench's per-expert bytes less the scales, over the three matrices
    one_matrix = (bench.expert_bytes(H, I, "fp8") - 3 * (H // 128) * (I // 128) * 4) // 3
    close("fp8_matrix_mb_from_gemv", one_matrix / 1e6)
    close("dsv3_layer_expert_gb", E * bench.expert_bytes(H, I, "fp8") / 1e9)


def test_kimi_k2_layer_size():
    c = synth.CONFIGS["kimi_k2"]
    close("kimi_k2_layer_expert_gb", c["E"] * bench.expert_bytes(c["H"], c["I"], "fp8") / 1e9)


def test_tokens_per_expert():
    c = synth.CONFIGS["dsv3_decode"]
    close("tokens_per_routed_expert_at_batch_64", 64 * c["k"] / c["E"])


def test_layer_bytes_count_every_touched_expert_once():
    """bench.layer_bytes = touched experts' weights + the shared expert + activations."""
    c = synth.CONFIGS["dsv3_decode"]
    H, I, E, k, T = c["H"], c["I"], c["E"], c["k"], c["T"]
    per = bench.expert_bytes(H, I, "fp8")
    lb = bench.layer_bytes(T, H, I, E, k, touched=100)
    assert 101 * per <= lb <= 101 * per + 8 * T * k * (H + I) + 8 * T * H
