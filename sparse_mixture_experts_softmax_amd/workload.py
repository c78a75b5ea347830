"""Shape bookkeeping for one MoE block: parameter counts, algorithmic bytes and FLOPs.

The per-block count E*3*d*I + 3*d*Is + d*E (three bias-free d x I matrices per expert plus a d x E
router) is the one the Qwen3.8-Max overview page's parameter table implies: with hidden_size 8192,
512 routed experts plus one shared, moe_intermediate_size 2048, it gives the printed 25.82 G per
block. Algorithmic work counts only what the method itself must move or compute.
"""

# MI355X published peaks
HBM_PEAK_BPS = 8.0e12
BF16_MFMA_PEAK_FLOPS = 2.5e15
FP32_VECTOR_PEAK_FLOPS = 157.3e12
FP32_MFMA_PEAK_FLOPS = 157.3e12


def expert_params(d, I):
    return 3 * d * I


def block_params(d, E, I, Is):
    return E * expert_params(d, I) + (expert_params(d, Is) if Is else 0) + d * E


def active_params_per_token(d, E, k, I, Is):
    return k * expert_params(d, I) + (expert_params(d, Is) if Is else 0) + d * E


def elem_bytes(dtype):
    """0 = fp32, 1 = bf16."""
    return 4 if dtype == 0 else 2


def algorithmic_bytes(T, d, E, I, Is, dtype, touched):
    """Bytes one forward pass must move: the touched experts' and the shared expert's weights,
    the fp32 router weight, x in and out."""
    s = elem_bytes(dtype)
    return touched * expert_params(d, I) * s + (expert_params(d, Is) * s if Is else 0) + 4 * d * E + 2 * T * d * s


def ffn1_algorithmic_bytes(T, d, I, Is, dtype, touched, k=None):
    """Gate/up step: W_g and W_u of the touched experts and of the shared expert, and x read once.
    The intermediate H it writes is implementation traffic (a fused block would keep it on chip)
    and is not counted."""
    s = elem_bytes(dtype)
    return (touched * 2 * d * I + (2 * d * Is if Is else 0)) * s + T * d * s


def algorithmic_bytes_fp8(T, d, E, I, Is, touched):
    """As algorithmic_bytes with e4m3 expert weights (1 byte each) and their fp32 column scales
    (I + I + d per expert); activations bf16."""
    w = touched * (expert_params(d, I) + 4 * (2 * I + d)) + ((expert_params(d, Is) + 4 * (2 * Is + d)) if Is else 0)
    return w + 4 * d * E + 2 * T * d * 2


def ffn1_algorithmic_bytes_fp8(T, d, I, Is, touched, k=None):
    """Gate/up step with e4m3 weights: codes and column scales of W_g and W_u (touched experts and
    the shared expert) and x read once (bf16); H is not counted."""
    return (touched * 2 * (d * I + 4 * I) + ((2 * (d * Is + 4 * Is)) if Is else 0)) + T * d * 2


def expert_flops(T, d, k, I, Is):
    """Multiply-adds x2 of the routed and shared SwiGLU experts."""
    return 6 * d * (T * k * I + T * Is)


def ffn1_flops(T, d, k, I, Is):
    return 4 * d * (T * k * I + T * Is)


def router_flops(T, d, E):
    return 2 * T * d * E


def touched_experts(topk_idx, E):
    import numpy as np
    return int(np.unique(np.asarray(topk_idx).reshape(-1)).size)
