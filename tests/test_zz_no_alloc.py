"""moe_forward_noalloc (no allocation: the library's per-GPU scratch array in place of a caller's
workspace) against moe_forward with a workspace, through the C ABI: two calls in a row on the
same GPU, the second with fewer tokens, each equal to the workspace entry point's result."""
import numpy as np
import pytest

import synthetic as syn
from moe_testlib import compare, device_from_host, host_inputs, oracle_full, run_forward, to_host

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("shape", [
    # name, T first, T second, d, E, k, I, Is
    ("mid_width", 300, 37, 2048, 64, 8, 512, 512),
    ("few_tokens", 5, 1, 2048, 32, 6, 512, 256),  # split-K MFMA, then the skinny kernels
])
def test_noalloc_forward_matches_workspace_forward(shape):
    import torch
    import sparse_mixture_experts_softmax_amd as moe
    name, T1, T2, d, E, k, I, Is = shape
    assert torch.cuda.is_available()
    moe.load_library()
    cfg = syn.MoEConfig("noalloc_" + name, T=T1, d=d, E=E, k=k, I=I, Is=Is, dtype=syn.BF16, seed=81)
    print("case", cfg, "then T =", T2, flush=True)
    h = host_inputs(cfg)
    dev = device_from_host(h, cfg)
    for T in (T1, T2):
        x = dev["x"][:T].contiguous()
        out = torch.empty_like(x)
        idx = torch.empty(T, k, dtype=torch.int32, device="cuda")
        w = torch.empty(T, k, dtype=torch.float32, device="cuda")
        gap = torch.empty(T, dtype=torch.float32, device="cuda")
        moe.moe_forward_noalloc(x, dev["w_router"], dev["wg"], dev["wu"], dev["wd"], dev["wg_s"], dev["wu_s"],
                                dev["wd_s"], k, out, router_bias=dev["bias"], topk_idx=idx, topk_w=w, topk_gap=gap)
        dref = dict(dev, x=x)
        ref, ridx, rw, rgap = run_forward(dref, cfg.with_(T=T))
        torch.cuda.synchronize()
        # the same kernels on the same inputs: identical results
        assert torch.equal(out, ref) and torch.equal(idx, ridx) and torch.equal(w, rw) and torch.equal(gap, rgap)
        # and the oracle's bar on every token
        hT = dict(h, x=h["x"][:T])
        r_out, r_idx, r_w, r_gap = oracle_full(hT, cfg.with_(T=T))
        st = compare(cfg.with_(T=T), to_host(out), to_host(idx), to_host(w), r_out, r_idx, r_w, r_gap, name)
        print(name, "T =", T, st, flush=True)
