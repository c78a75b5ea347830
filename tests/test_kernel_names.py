"""moe_kernel_name (host only, no GPU): the kernels the forward launches for the workloads' shapes.

Pins the plan's choices at the measured shapes -- the dominant kernel that bench.py labels and
that the committed traces name -- and the query's refusals."""
import pytest

import synthetic as syn

moe = pytest.importorskip("sparse_mixture_experts_softmax_amd")


def _dims(cfg, T=None):
    return moe.MoeDims(T=cfg.T if T is None else T, d=cfg.d, E=cfg.E, k=cfg.k, I=cfg.I, I_shared=cfg.Is,
                       dtype=cfg.dtype, renormalize=cfg.renorm)


@pytest.fixture(scope="module")
def lib():
    try:
        return moe.load_library()
    except OSError as e:  # not built
        pytest.skip(str(e))


EXPECTED = {
    # workload: (gate/up, down)
    "tiny": ("ffn_f32_kernel<true>", "ffn_f32_kernel<false>"),
    "mid": ("ffn_mfma_tall_kernel<true, 3>", "ffn_mfma_tall_kernel<false, 3>"),
    "decode": ("ffn_mfma_stream_kernel<true, 4, 4>", "ffn_mfma_stream_kernel<false, 2, 3>"),
    "prefill": ("ffn_mfma_tall_kernel<true, 3>", "ffn_mfma_tall_kernel<false, 3>"),
    "skew": ("ffn_mfma_tall_kernel<true, 3>", "ffn_mfma_tall_kernel<false, 3>"),
}


@pytest.mark.parametrize("name", sorted(EXPECTED))
def test_grouped_gemm_kernels_of_the_workloads(lib, name):
    cfg = syn.CONFIGS[name]
    gu, dn = EXPECTED[name]
    assert moe.moe_kernel_name(_dims(cfg), moe.KERNEL_FFN_GATE_UP) == gu
    assert moe.moe_kernel_name(_dims(cfg), moe.KERNEL_FFN_DOWN) == dn


def test_few_token_and_fp8_kernels(lib):
    cfg = syn.CONFIGS["decode"]
    assert moe.moe_kernel_name(_dims(cfg, T=1), moe.KERNEL_FFN_GATE_UP) == "ffn_skinny_kernel<true, 1>"
    assert moe.moe_kernel_name(_dims(cfg, T=2), moe.KERNEL_FFN_DOWN) == "ffn_skinny_kernel<false, 2>"
    assert moe.moe_kernel_name(_dims(cfg), moe.KERNEL_FFN_GATE_UP, fp8=True) == "ffn_fp8_stream_kernel<true, 4, 32>"
    assert moe.moe_kernel_name(_dims(cfg, T=1), moe.KERNEL_FFN_GATE_UP, fp8=True) == "ffn_fp8_skinny_kernel<true, 1>"
    assert moe.moe_kernel_name(_dims(cfg, T=2), moe.KERNEL_FFN_DOWN, fp8=True) == "ffn_fp8_skinny_kernel<false, 2>"
    pre = syn.CONFIGS["prefill"]
    assert moe.moe_kernel_name(_dims(pre), moe.KERNEL_FFN_DOWN, fp8=True) == "ffn_fp8_stream_kernel<false, 5, 128>"
    assert moe.moe_kernel_name(_dims(pre), moe.KERNEL_ROUTER) == "router_mfma_kernel<4>"
    assert moe.moe_kernel_name(_dims(cfg), moe.KERNEL_ROUTER) == "router_small_kernel"
    assert moe.moe_kernel_name(_dims(cfg), moe.KERNEL_PERMUTE) == "permute_one_chunk_kernel"
    # up to four tokens (E > 64): top-k and dispatch in one launch
    assert moe.moe_kernel_name(_dims(cfg, T=1), moe.KERNEL_PERMUTE) == "route_dispatch_kernel"
    assert moe.moe_kernel_name(_dims(cfg, T=4), moe.KERNEL_PERMUTE) == "route_dispatch_kernel"
    assert moe.moe_kernel_name(_dims(cfg, T=5), moe.KERNEL_PERMUTE) == "permute_one_chunk_kernel"
    assert moe.moe_kernel_name(_dims(pre), moe.KERNEL_COMBINE) == "combine_kernel"


def test_refusals(lib):
    cfg = syn.CONFIGS["mid"]
    with pytest.raises(ValueError):
        moe.moe_kernel_name(_dims(cfg), 0)
    with pytest.raises(ValueError):
        moe.moe_kernel_name(_dims(cfg), 6)
    with pytest.raises(ValueError):  # fp32 dims: no FP8 path
        moe.moe_kernel_name(_dims(syn.CONFIGS["tiny"]), moe.KERNEL_FFN_GATE_UP, fp8=True)
    bad = _dims(cfg)
    bad.k = bad.E + 1
    with pytest.raises(ValueError):
        moe.moe_kernel_name(bad, moe.KERNEL_FFN_GATE_UP)
