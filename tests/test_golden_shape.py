"""Page-stated constants of the layer (tests/golden/flint_moe_shape.txt)."""

import os

import synth


def load(repo_root):
    vals = {}
    with open(os.path.join(repo_root, "tests", "golden", "flint_moe_shape.txt")) as fh:
        for line in fh:
            if line.strip() and not line.startswith("#"):
                key, val = line.split()[:2]
                vals[key] = float(val)
    return vals


def test_nvfp4_bytes_per_weight_match_the_page(repo_root):
    g = load(repo_root)
    H, I = 2048, 768
    per_weight = synth.expert_bytes(synth.FMT_NVFP4, H, I) / (3 * H * I)
    assert abs(per_weight - 0.5625) < 1e-5
    assert round(per_weight, 2) == g["bytes_per_param_4bit"]
    assert synth.expert_bytes(synth.FMT_NVFP4, H, I) == 2654220
    assert synth.expert_bytes(synth.FMT_INT4_G64, H, I) == 2580480


def test_layer_constants(repo_root):
    g = load(repo_root)
    assert (g["routed_experts"], g["experts_per_token"], g["shared_experts"], g["moe_layers"]) == (256, 6, 1, 47)
    assert g["int4_group"] == 64
