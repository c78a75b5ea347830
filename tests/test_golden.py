"""The shape bookkeeping reproduces the parameter counts the pages print (tests/golden/param_counts.txt).

The per-block count E*3*d*I + 3*d*Is + d*E (bias-free SwiGLU experts plus a d x E router) is what
the bench's algorithmic bytes are built from; the pages' tables pin it at the Qwen3.8-Max shape."""
import os

import pytest

from sparse_mixture_experts_softmax_amd import workload as wl

HERE = os.path.dirname(os.path.abspath(__file__))

# Qwen3.8-Max shapes from the config.json listing on the Architecture page
D, LAYERS, E, K, I, IS, VOCAB = 8192, 92, 512, 10, 2048, 2048, 248320
# per-layer counts of the other layer kinds, as printed in the parameter table (not derived here)
DELTANET_LAYER, DELTANET_LAYERS = 438.4e6, 69
ATTN_LAYER, ATTN_LAYERS = 419.4e6, 23


def golden():
    out = {}
    for line in open(os.path.join(HERE, "golden", "param_counts.txt")):
        if line.startswith("#") or not line.strip():
            continue
        key, printed, value, cite = [f.strip() for f in line.split("|")]
        out[key] = (printed, float(value), cite)
    return out


def computed():
    block = wl.block_params(D, E, I, IS)
    moe_total = LAYERS * block
    emb = VOCAB * D
    head = D * VOCAB
    norms = 185 * D
    total = moe_total + DELTANET_LAYERS * DELTANET_LAYER + ATTN_LAYERS * ATTN_LAYER + emb + head + norms
    active_moe = LAYERS * wl.active_params_per_token(D, E, K, I, IS)
    active_total = active_moe + DELTANET_LAYERS * DELTANET_LAYER + ATTN_LAYERS * ATTN_LAYER + emb + head
    return {
        "moe_block_params": block,
        "moe_blocks_total": moe_total,
        "moe_blocks_share": moe_total / total,
        "model_total": total,
        "attention_layer_params": ATTN_LAYER,
        "mtp_layer_params": block + ATTN_LAYER,
        "moe_active_per_token": active_moe,
        "moe_active_share": active_moe / active_total,
        "active_total": active_total,
    }


def printed_resolution(printed):
    """Half a unit of the last printed digit, in the value's own unit."""
    p = printed.replace(" ", " ").split()[-2] if printed.split()[-1] in ("G", "M", "%") else printed
    scale = {"G": 1e9, "M": 1e6, "%": 1e-2}[printed.split()[-1]]
    decimals = len(p.split(",")[1]) if "," in p else 0
    return 0.5 * 10 ** (-decimals) * scale


@pytest.mark.parametrize("key", sorted(golden()))
def test_parameter_counts_match_the_pages(key):
    printed, value, cite = golden()[key]
    got = computed()[key]
    assert abs(got - value) <= printed_resolution(printed) + 1e-12 * abs(value), (key, got, value, cite)


def test_block_count_pins_bias_free_experts_and_a_router():
    block = wl.block_params(D, E, I, IS)
    assert block == 25_824_329_728
    # without the router, or with expert biases (2I + d per expert), the printed 25,82 G would not round right
    assert round((block - D * E) / 1e9, 2) != 25.82 or round((LAYERS * (block - D * E)) / 1e9, 1) != 2375.8
    with_bias = block + (E + 1) * (2 * I + D)
    assert round(LAYERS * with_bias / 1e9, 1) != 2375.8
