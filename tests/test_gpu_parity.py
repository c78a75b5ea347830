"""GPU parity: the HIP path through the C ABI against the CPU oracle on the same seeded inputs."""
import numpy as np
import pytest

import oracle
import synthetic as syn
from moe_testlib import (compare, coverage_tokens, device_from_host, host_inputs, oracle_full, oracle_tokens, run_forward,
                         to_host, torch_dtype)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    import torch as _t
    assert _t.cuda.is_available(), "GPU tests need a GPU"
    import sparse_mixture_experts_softmax_amd as moe
    moe.load_library()
    return _t


def _say(*a):
    print(*a, flush=True)


# --------------------------------------------------------------------------------------------
# input generator: device fill equals host fill bit for bit
# --------------------------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", [syn.F32, syn.BF16])
def test_device_generator_matches_host(torch, dtype):
    n, off = 3 * 1000003, 123457
    tdt = torch.float32 if dtype == syn.F32 else torch.bfloat16
    t = torch.empty(n, dtype=tdt, device="cuda")
    syn.device_fill(t, 7, syn.TID_WG, 0.0123, offset=off)
    h = syn.host_fill(n, dtype, 7, syn.TID_WG, 0.0123, offset=off)
    g = t.view(torch.int32 if dtype == syn.F32 else torch.int16).cpu().numpy()
    assert np.array_equal(g.view(h.dtype), h)


# --------------------------------------------------------------------------------------------
# whole block on small shapes, every token against the oracle
# --------------------------------------------------------------------------------------------
def _full_check(torch, cfg, label):
    _say("case", label, cfg)
    h = host_inputs(cfg)
    dev = device_from_host(h, cfg)
    out, idx, w, gap = run_forward(dev, cfg)
    torch.cuda.synchronize()
    ref_out, ref_idx, ref_w, ref_gap = oracle_full(h, cfg)
    st = compare(cfg, to_host(out), to_host(idx), to_host(w), ref_out, ref_idx, ref_w, ref_gap, label)
    # the GPU gap agrees with the oracle's where it matters
    g = to_host(gap)
    fin = np.isfinite(ref_gap)
    assert np.all(np.isinf(g[~fin]))
    assert np.max(np.abs(g[fin] - ref_gap[fin]), initial=0.0) < 1e-4
    _say(label, st)
    return st


def test_tiny_fp32_config(torch):
    st = _full_check(torch, syn.CONFIGS["tiny"], "tiny")
    assert st["rel"] <= 1e-5


SMALL_CASES = [
    # name, T, d, E, k, I, Is, dtype, renorm, zipf
    ("e1k1_dense", 37, 64, 1, 1, 32, 32, syn.BF16, 1, 0.0),
    ("k_eq_E", 50, 128, 4, 4, 64, 0, syn.BF16, 1, 0.0),
    ("ragged_bf16", 300, 264, 40, 3, 136, 72, syn.BF16, 1, 0.0),
    ("ragged_f32", 300, 264, 40, 3, 136, 72, syn.F32, 1, 0.0),
    ("no_renorm", 129, 256, 64, 6, 128, 128, syn.BF16, 0, 0.0),
    ("no_shared_f32", 77, 96, 13, 5, 40, 0, syn.F32, 0, 0.0),
    ("one_token", 1, 512, 32, 4, 256, 256, syn.BF16, 1, 0.0),
    ("many_tiles", 700, 512, 16, 4, 384, 256, syn.BF16, 1, 0.0),
    ("skewed_small", 512, 128, 64, 8, 64, 64, syn.BF16, 1, 1.2),
    ("E65_k16", 200, 64, 65, 16, 24, 8, syn.F32, 1, 0.0),
    ("wide_E", 96, 64, 1024, 16, 16, 16, syn.BF16, 1, 0.0),
    ("router_mfma", 300, 256, 256, 8, 128, 128, syn.BF16, 1, 0.0),
    ("router_mfma_E512", 520, 512, 512, 10, 128, 0, syn.BF16, 0, 0.0),
    ("rows_ragged", 1000, 256, 8, 2, 128, 128, syn.BF16, 1, 0.0),
    ("narrow_shared_smaller", 333, 1024, 16, 4, 512, 256, syn.BF16, 1, 0.0),
    # 128 x 512 streaming tiles: gate/up at d >= 4096 (shared expert wider than the routed ones),
    # down at I >= 2048 with >= 64 rows per expert
    ("wide_gate_up", 200, 4096, 8, 2, 256, 512, syn.BF16, 1, 0.0),
    ("wide_down", 300, 512, 8, 2, 2048, 0, syn.BF16, 1, 0.0),
    # T <= 2: the skinny kernels (one or two rows per group; K splits with the last-arriver sum,
    # empty splits and unused column blocks; shared expert as wide as, wider than, narrower than
    # the routed ones, or absent)
    ("skinny_T1", 1, 2048, 64, 4, 1024, 1024, syn.BF16, 1, 0.0),
    ("skinny_T1_narrow_shared", 1, 768, 6, 3, 512, 256, syn.BF16, 0, 0.0),
    ("skinny_T2_wide_shared", 2, 512, 4, 2, 256, 512, syn.BF16, 1, 0.0),
    ("skinny_T2_no_shared", 2, 1024, 8, 2, 256, 0, syn.BF16, 1, 0.0),
    # a few more tokens: the MFMA gate/up product's K split over workgroups (2 ways on 128 x 256
    # tiles; 4 or 8 ways on 128 x 512 tiles with a shared expert narrower than the routed ones)
    ("split_k_T3", 3, 4096, 32, 6, 512, 256, syn.BF16, 1, 0.0),
    ("split_k_T4_narrow_shared", 4, 768, 6, 3, 512, 256, syn.BF16, 0, 0.0),
    ("split_k_T4_no_shared", 4, 1024, 8, 2, 256, 0, syn.BF16, 1, 0.0),
    ("split_k_T6", 6, 2048, 64, 4, 1024, 1024, syn.BF16, 1, 0.0),
    ("split_k_T5", 5, 4096, 32, 6, 512, 256, syn.BF16, 1, 0.0),
    # the most experts and the largest k on the streaming GEMMs and the MFMA router (1025 groups)
    ("stream_E1024_k16", 300, 512, 1024, 16, 128, 128, syn.BF16, 1, 0.0),
    # few tokens with E > 64: top-k on four wavefronts per token (E not a multiple of 256, k = 16
    # with 68 merge candidates, no renormalisation, fp32)
    ("topk_wide_no_renorm", 5, 256, 300, 7, 128, 0, syn.BF16, 0, 0.0),
    ("topk_wide_k16", 60, 512, 1024, 16, 64, 64, syn.BF16, 1, 0.0),
    ("topk_wide_f32", 20, 64, 130, 4, 32, 32, syn.F32, 1, 0.0),
    # equal row tiles (<= 192 rows per expert on average) under Zipf-skewed loads of ~50 .. ~650 rows
    ("balanced_tiles_skewed", 700, 512, 16, 4, 256, 128, syn.BF16, 1, 0.8),
    # one or two tokens with more than 64 experts (top-k on four wavefronts per token, skinny
    # GEMMs); a shared expert wider than the routed ones (three column blocks of 256 against two)
    ("skinny_many_experts_T1", 1, 1024, 128, 6, 512, 512, syn.BF16, 1, 0.0),
    ("skinny_many_experts_T2", 2, 2048, 96, 8, 512, 768, syn.BF16, 0, 0.0),
    # 160-row tall tiles (96 .. 256 rows per expert on average): ~200-row experts as two row tiles
    # of 3 and 4 sub-tiles and the 400 shared rows as three (4, 4, 5); ~100-row experts in one row
    # tile of four sub-tiles (the last one partial); Zipf-skewed loads from ~500 rows down to a few
    # (one partial sub-tile)
    ("tall_tiles", 400, 512, 8, 4, 256, 256, syn.BF16, 1, 0.0),
    ("tall_tiles_one_row_tile", 200, 512, 8, 4, 256, 256, syn.BF16, 0, 0.0),
    ("tall_tiles_skewed", 700, 512, 16, 4, 256, 0, syn.BF16, 0, 1.2),
    # 192-row tiles, taken per group where they need fewer row tiles than 160-row ones (here
    # ~350-row experts as two 192-row tiles, larger ones as three 160-row tiles, both in one
    # launch); a shared expert wider than the routed ones; Zipf-skewed loads from every token down
    # to a few rows; k = E, so that every group holds T rows: 576 as three full 192-row tiles, 161
    # as one (six sub-tiles, one row in the last), 384 as two full ones
    ("wide_tiles", 700, 512, 8, 4, 256, 256, syn.BF16, 1, 0.0),
    ("wide_tiles_wide_shared", 513, 1024, 4, 2, 256, 512, syn.BF16, 1, 0.0),
    ("wide_tiles_skewed", 2000, 512, 16, 4, 256, 0, syn.BF16, 0, 1.2),
    ("wide_tiles_576", 576, 512, 4, 4, 256, 256, syn.BF16, 1, 0.0),
    ("wide_tiles_161", 161, 512, 4, 4, 256, 512, syn.BF16, 1, 0.0),
    ("wide_tiles_384", 384, 1024, 4, 4, 512, 256, syn.BF16, 0, 0.0),
    # T <= 4 with E > 64: top-k and dispatch in one launch (four wavefronts per token, the T*k
    # picks scattered from LDS): 1024 experts (four logits per lane) with k = 16 and three tokens;
    # 65 experts (wavefronts holding one expert or none) with 4 * 16 = 64 pairs, fp32; four tokens
    # on the MFMA gate/up product's K split
    ("fused_route_E1024_T3", 3, 256, 1024, 16, 64, 64, syn.BF16, 1, 0.0),
    ("fused_route_E65_T4_f32", 4, 128, 65, 16, 32, 0, syn.F32, 0, 0.0),
    ("fused_route_E200_T4", 4, 1024, 200, 8, 256, 256, syn.BF16, 1, 0.0),
]


@pytest.mark.parametrize("case", SMALL_CASES, ids=[c[0] for c in SMALL_CASES])
def test_small_shapes(torch, case):
    name, T, d, E, k, I, Is, dt, rn, za = case
    cfg = syn.MoEConfig(name, T=T, d=d, E=E, k=k, I=I, Is=Is, dtype=dt, renorm=rn, seed=11, zipf_alpha=za)
    _full_check(torch, cfg, name)


# Every token routed to the same k experts: a router bias of +32 on them lies far above the
# synthetic logits' spread (under 8), so k groups hold all T rows and every other group is empty --
# the largest groups the grouped GEMMs meet, next to empty ones; one-workgroup and chunked dispatch,
# 128 x 256 and 128 x 512 tiles. Bias +32 keeps the fp32 logits' rounding (ulp 3.8e-6) within the
# routing-weight bound.
@pytest.mark.parametrize("T,d,E,k,Is", [(200, 512, 64, 4, 128), (1100, 512, 64, 4, 128), (300, 4096, 16, 2, 512)])
def test_all_tokens_to_the_same_experts(torch, T, d, E, k, Is):
    cfg = syn.MoEConfig("same_experts", T=T, d=d, E=E, k=k, I=256, Is=Is, dtype=syn.BF16, renorm=1, seed=5)
    label = "same_experts_T%d_d%d" % (T, d)
    _say("case", label, cfg)
    h = host_inputs(cfg)
    chosen = [5, E - 1, 2, 11][:k]
    bias = np.zeros(E, np.float32)
    bias[chosen] = 32.0
    h["bias"] = bias
    dev = device_from_host(h, cfg)
    out, idx, w, gap = run_forward(dev, cfg)
    torch.cuda.synchronize()
    ref_out, ref_idx, ref_w, ref_gap = oracle_full(h, cfg)
    assert sorted(set(ref_idx.ravel().tolist())) == sorted(chosen)  # the bias does force the routing
    st = compare(cfg, to_host(out), to_host(idx), to_host(w), ref_out, ref_idx, ref_w, ref_gap, label)
    assert st["flagged"] == 0
    _say(label, st)


def test_zero_tokens_is_a_no_op(torch):
    import sparse_mixture_experts_softmax_amd as moe
    cfg = syn.CONFIGS["tiny"].with_(T=3)
    dev = device_from_host(host_inputs(cfg), cfg)
    x0 = dev["x"][:0]
    out = torch.full((0, cfg.d), 7.0, device="cuda")
    res = moe.moe_forward(x0, dev["w_router"], dev["wg"], dev["wu"], dev["wd"], dev["wg_s"], dev["wu_s"], dev["wd_s"],
                          cfg.k, out=out)
    torch.cuda.synchronize()
    assert res.shape == (0, cfg.d)


# --------------------------------------------------------------------------------------------
# dispatch alone, on skewed indices with out-of-range entries; several 256-token chunks and a
# ragged tail, and single chunks (T <= 256: the one-workgroup dispatch)
# --------------------------------------------------------------------------------------------
@pytest.mark.parametrize("E,T", [(300, 2500), (700, 2500), (300, 200), (1024, 256), (64, 1)])
def test_permute_skewed_with_invalid_indices(torch, E, T):
    import sparse_mixture_experts_softmax_amd as moe
    k = 5
    rng = np.random.default_rng(E + T)
    # k distinct experts per token (as top-k selection gives), drawn with Zipf(1.2) weights
    p = 1.0 / np.arange(1, E + 1) ** 1.2
    p /= p.sum()
    idx = np.stack([rng.choice(E, size=k, replace=False, p=p) for _ in range(T)]).astype(np.int32)
    bad = rng.random((T, k))
    idx[bad < 0.01] = -1
    idx[(bad >= 0.01) & (bad < 0.02)] = E
    dims = moe.MoeDims(T, 64, E, k, 64, 0, syn.BF16, 1)
    d_idx = torch.from_numpy(idx).to("cuda")
    offs, sorted_token, slot_of = moe.moe_permute(dims, d_idx)
    torch.cuda.synchronize()

    flat_e = idx.reshape(-1).astype(np.int64)
    flat_t = np.repeat(np.arange(T), k)
    valid = (flat_e >= 0) & (flat_e < E)
    order = np.lexsort((flat_t[valid], flat_e[valid]))  # expert major, token ascending
    counts = np.bincount(flat_e[valid], minlength=E)
    n = int(valid.sum())
    exp_slot = np.full(T * k, -1, np.int64)
    exp_slot[np.flatnonzero(valid)[order]] = np.arange(n)
    assert np.array_equal(to_host(offs), np.concatenate([[0], np.cumsum(counts)]))
    assert np.array_equal(to_host(sorted_token)[:n], flat_t[valid][order])
    assert np.array_equal(to_host(slot_of), exp_slot)


# --------------------------------------------------------------------------------------------
# the four step entry points compose to moe_forward, bit for bit; permute is a stable sort
# --------------------------------------------------------------------------------------------
# the grouped GEMMs' three bf16 paths: MFMA tiles (T = 600), MFMA with K split (T = 5), skinny (T = 2);
# with E > 64 and T <= 4 the forward runs top-k and dispatch as one launch, the steps as two
@pytest.mark.parametrize("T,d,I,Is,E", [(600, 256, 128, 64, 48), (5, 2048, 512, 512, 48), (2, 512, 256, 256, 48),
                                        (2, 512, 256, 256, 96), (4, 1024, 256, 128, 300)])
def test_steps_compose_and_permute_is_stable_sort(torch, T, d, I, Is, E):
    import sparse_mixture_experts_softmax_amd as moe
    cfg = syn.MoEConfig("steps", T=T, d=d, E=E, k=6, I=I, Is=Is, dtype=syn.BF16, seed=3)
    h = host_inputs(cfg)
    dev = device_from_host(h, cfg)
    dims = moe.dims_for(dev["x"], dev["w_router"], dev["wg"], dev["wg_s"], cfg.k, True)
    ws = moe.workspace(dims, "cuda")
    idx, w, gap = moe.moe_router_topk(dims, dev["x"], dev["w_router"], None, ws)
    offs, sorted_token, slot_of = moe.moe_permute(dims, idx, ws)
    y = moe.moe_grouped_ffn(dims, dev["x"], offs, sorted_token, dev["wg"], dev["wu"], dev["wd"], dev["wg_s"],
                            dev["wu_s"], dev["wd_s"], ws)
    out = moe.moe_combine(dims, y, slot_of, w)
    out2, idx2, w2, gap2 = run_forward(dev, cfg)
    torch.cuda.synchronize()
    assert torch.equal(out, out2) and torch.equal(idx, idx2) and torch.equal(w, w2)

    # dispatch against a host stable sort by (expert, token)
    ih = to_host(idx).astype(np.int64)
    flat_e = ih.reshape(-1)
    flat_t = np.repeat(np.arange(cfg.T), cfg.k)
    order = np.lexsort((flat_t, flat_e))  # expert major, token ascending
    counts = np.bincount(flat_e, minlength=cfg.E)
    exp_offs = np.concatenate([[0], np.cumsum(counts)])
    exp_sorted = flat_t[order]
    exp_slot = np.empty(cfg.T * cfg.k, np.int64)
    exp_slot[order] = np.arange(cfg.T * cfg.k)
    assert np.array_equal(to_host(offs), exp_offs)
    assert np.array_equal(to_host(sorted_token), exp_sorted)
    assert np.array_equal(to_host(slot_of), exp_slot)


def test_deterministic_and_token_permutation_equivariant(torch):
    cfg = syn.MoEConfig("perm", T=333, d=192, E=24, k=4, I=96, Is=64, dtype=syn.BF16, seed=5)
    h = host_inputs(cfg)
    dev = device_from_host(h, cfg)
    out1, idx1, w1, _ = run_forward(dev, cfg)
    out2, idx2, w2, _ = run_forward(dev, cfg)
    torch.cuda.synchronize()
    assert torch.equal(out1, out2) and torch.equal(idx1, idx2)
    perm = torch.from_numpy(np.random.default_rng(0).permutation(cfg.T)).cuda()
    dev_p = dict(dev)
    dev_p["x"] = dev["x"][perm].contiguous()
    out_p, idx_p, w_p, _ = run_forward(dev_p, cfg)
    torch.cuda.synchronize()
    assert torch.equal(out_p, out1[perm]) and torch.equal(idx_p, idx1[perm])


# --------------------------------------------------------------------------------------------
# the full-size configurations, in the launch configuration the benchmark times
# --------------------------------------------------------------------------------------------
def _device_inputs(cfg, cache={}):
    """Device inputs; the three d=8192 configurations share identical weights (same seed and shapes)."""
    key = (cfg.d, cfg.E, cfg.I, cfg.Is, cfg.dtype, cfg.seed)
    if cache.get("key") != key:
        cache.clear()
        cache["key"] = key
        cache["w"] = syn.device_inputs(cfg, with_x=False)
    import torch
    dev = dict(cache["w"])
    dev["x"] = syn.device_fill(torch.empty(cfg.T, cfg.d, dtype=torch_dtype(cfg), device="cuda"), cfg.seed, syn.TID_X,
                               1.0)
    b = syn.router_bias(cfg)
    dev["bias"] = None if b is None else torch.from_numpy(b).cuda()
    return dev


def _full_size_check(torch, name, n_min, budget, T=None):
    cfg = syn.CONFIGS[name] if T is None else syn.CONFIGS[name].with_(T=T)
    _say("config", cfg)
    dev = _device_inputs(cfg)
    out, idx, w, gap = run_forward(dev, cfg)
    torch.cuda.synchronize()
    idx_h, w_h, out_h = to_host(idx), to_host(w), to_host(out)
    # properties on every token
    assert idx_h.min() >= 0 and idx_h.max() < cfg.E
    s = np.sort(idx_h, axis=1)
    assert np.all(s[:, 1:] != s[:, :-1]), "repeated expert within a token"
    np.testing.assert_allclose(w_h.sum(axis=1), 1.0, atol=1e-5)
    assert np.all(np.isfinite(out_h))
    # the oracle on every token, or on tokens covering every row band of every group
    if n_min >= cfg.T:
        tokens, cov = np.arange(cfg.T), 1.0
    else:
        tokens, cov = coverage_tokens(idx_h, cfg.E, n_min, budget, seed=1234)
    _say(name, "checking", len(tokens), "tokens against the oracle; 64-row band coverage %.4f" % cov)
    ref_out, ref_idx, ref_w, ref_gap = oracle_tokens(cfg, tokens)
    st = compare(cfg, out_h[tokens], idx_h[tokens], w_h[tokens], ref_out, ref_idx, ref_w, ref_gap, name)
    load = np.bincount(idx_h.ravel(), minlength=cfg.E)
    _say(name, st, "max rel err %.3e" % st["rel"], "touched experts", int((load > 0).sum()), "max load",
         int(load.max()))
    return cfg, idx_h, load, cov


def test_mid_config_router_all_tokens_and_covering_outputs(torch):
    cfg, idx_h, load, cov = _full_size_check(torch, "mid", 384, 1024)
    assert cov == 1.0
    # router + top-k on every token against the oracle
    x = syn.host_x(cfg)
    ref_idx, _, ref_gap, _ = oracle.router(x, syn.host_router(cfg), cfg.k)
    ok = ~oracle.flagged(ref_gap)
    assert np.array_equal(np.sort(idx_h[ok], axis=1), np.sort(ref_idx[ok], axis=1))
    _say("mid flagged tokens", int((~ok).sum()))


def test_decode_config_every_token(torch):
    cfg, idx_h, load, cov = _full_size_check(torch, "decode", 32, 32)
    assert (load > 0).sum() > 150


@pytest.mark.parametrize("T", [1, 2, 3])
def test_decode_shape_few_tokens(torch, T):
    # the large shape at T <= 2 runs the skinny kernels, at T = 3 the MFMA kernels with K split;
    # every token against the oracle
    _full_size_check(torch, "decode", T, T, T=T)


def test_prefill_config_covering_every_row_band(torch):
    cfg, idx_h, load, cov = _full_size_check(torch, "prefill", 256, 640)
    assert cov == 1.0


def test_skew_config_covering_every_row_band(torch):
    cfg, idx_h, load, cov = _full_size_check(torch, "skew", 256, 640)
    assert cov == 1.0
    L = syn.zipf_targets(cfg.T, cfg.E, cfg.k, cfg.zipf_alpha)
    # the two heaviest experts take (almost) every token; popularity bands follow the Zipf targets
    assert load[0] >= 0.99 * cfg.T and load[1] >= 0.99 * cfg.T
    for a, b in [(0, 10), (10, 50), (50, 200), (200, cfg.E)]:
        assert abs(load[a:b].sum() / L[a:b].sum() - 1) < 0.05, (a, b)
    assert np.corrcoef(np.log(load + 1), np.log(L + 1))[0, 1] > 0.97


# --------------------------------------------------------------------------------------------
# steps either side of the block: zero-centred RMSNorm in front, the residual add after
# --------------------------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", [syn.F32, syn.BF16])
def test_rmsnorm_matches_oracle_bit_for_bit(torch, dtype):
    # both sides compute in fp64 and round once; the rows the router ranks on must be identical
    import sparse_mixture_experts_softmax_amd as moe
    cfg = syn.MoEConfig("norm", T=777, d=2048 + 8 * 3, E=8, k=2, I=64, Is=0, dtype=dtype, seed=4)
    x = syn.host_x(cfg)
    g = syn.host_gamma(cfg)
    ref = oracle.rmsnorm(x, g)
    dims = moe.MoeDims(cfg.T, cfg.d, cfg.E, cfg.k, cfg.I, 0, dtype, 1)
    dt = torch_dtype(cfg)
    from moe_testlib import to_device
    h = moe.moe_rmsnorm(dims, to_device(x, dt), to_device(g, dt))
    torch.cuda.synchronize()
    hb = h.view(torch.int32 if dtype == syn.F32 else torch.int16).cpu().numpy().view(ref.dtype)
    assert np.array_equal(hb, ref)


BLOCK_CASES = [
    syn.CONFIGS["tiny"],
    syn.MoEConfig("block_ragged", T=300, d=264, E=40, k=3, I=136, Is=72, dtype=syn.BF16, seed=12),
    syn.MoEConfig("block_mid_shape", T=700, d=2048, E=256, k=8, I=512, Is=512, dtype=syn.BF16, seed=13),
    # one and two tokens: the skinny products, the residual added by the down product's last workgroups
    syn.MoEConfig("block_one_token", T=1, d=2048, E=128, k=8, I=512, Is=512, dtype=syn.BF16, seed=17),
    syn.MoEConfig("block_two_tokens", T=2, d=1024, E=40, k=5, I=768, Is=256, dtype=syn.BF16, seed=18),
]


@pytest.mark.parametrize("cfg", BLOCK_CASES, ids=[c.name for c in BLOCK_CASES])
def test_block_forward_matches_oracle(torch, cfg):
    import sparse_mixture_experts_softmax_amd as moe
    from moe_testlib import to_device
    _say("case", cfg)
    h = host_inputs(cfg)
    dev = device_from_host(h, cfg)
    g = syn.host_gamma(cfg)
    dg = to_device(g, torch_dtype(cfg))
    out, idx, w, gap = moe.moe_forward_block(dev["x"], dg, dev["w_router"], dev["wg"], dev["wu"], dev["wd"],
                                             dev["wg_s"], dev["wu_s"], dev["wd_s"], cfg.k,
                                             renormalize=bool(cfg.renorm), router_bias=dev["bias"],
                                             return_routing=True)
    torch.cuda.synchronize()
    ref_out, ref_idx, ref_w, ref_gap, _ = oracle.block_forward(h["x"], g, h["w_router"], h["wg"], h["wu"], h["wd"],
                                                               h["wg_s"], h["wu_s"], h["wd_s"], cfg.k,
                                                               renorm=bool(cfg.renorm), bias=h["bias"])
    st = compare(cfg, to_host(out), to_host(idx), to_host(w), ref_out, ref_idx, ref_w, ref_gap, cfg.name,
                 residual=oracle.widen(h["x"]))
    _say(cfg.name, st)


# one and two tokens: the skinny down product writes the block's output itself (the combine with
# the residual folded into its last workgroup per column block)
@pytest.mark.parametrize("cfg", [
    syn.MoEConfig("block_steps", T=333, d=512, E=24, k=4, I=256, Is=128, dtype=syn.BF16, seed=14),
    syn.MoEConfig("block_steps_T1", T=1, d=2048, E=96, k=6, I=512, Is=512, dtype=syn.BF16, seed=15),
    syn.MoEConfig("block_steps_T2", T=2, d=1024, E=48, k=8, I=256, Is=768, dtype=syn.BF16, seed=16),
], ids=lambda c: c.name)
def test_block_steps_compose_bit_for_bit(torch, cfg):
    # rmsnorm -> router -> dispatch -> experts -> combine with the residual == the one-call block
    import sparse_mixture_experts_softmax_amd as moe
    from moe_testlib import to_device
    h = host_inputs(cfg)
    dev = device_from_host(h, cfg)
    dg = to_device(syn.host_gamma(cfg), torch_dtype(cfg))
    dims = moe.dims_for(dev["x"], dev["w_router"], dev["wg"], dev["wg_s"], cfg.k, True)
    ws = moe.workspace(dims, "cuda")
    hn = moe.moe_rmsnorm(dims, dev["x"], dg)
    idx, w, _ = moe.moe_router_topk(dims, hn, dev["w_router"], None, ws)
    offs, sorted_token, slot_of = moe.moe_permute(dims, idx, ws)
    y = moe.moe_grouped_ffn(dims, hn, offs, sorted_token, dev["wg"], dev["wu"], dev["wd"], dev["wg_s"],
                            dev["wu_s"], dev["wd_s"], ws)
    out = moe.moe_combine_residual(dims, y, slot_of, w, dev["x"])
    out2, idx2, w2, _ = moe.moe_forward_block(dev["x"], dg, dev["w_router"], dev["wg"], dev["wu"], dev["wd"],
                                              dev["wg_s"], dev["wu_s"], dev["wd_s"], cfg.k, return_routing=True)
    torch.cuda.synchronize()
    assert torch.equal(out, out2) and torch.equal(idx, idx2) and torch.equal(w, w2)


# --------------------------------------------------------------------------------------------
# router statistics for load balancing
# --------------------------------------------------------------------------------------------
STAT_CASES = [
    syn.CONFIGS["tiny"],
    syn.MoEConfig("stats_mid_shape", T=1500, d=2048, E=256, k=8, I=64, Is=0, dtype=syn.BF16, seed=31),
    syn.MoEConfig("stats_E512_skew", T=700, d=512, E=512, k=10, I=64, Is=0, dtype=syn.BF16, seed=32,
                  zipf_alpha=1.2),
    syn.MoEConfig("stats_E1024_one", T=1, d=256, E=1024, k=16, I=64, Is=0, dtype=syn.BF16, seed=33),
]


@pytest.mark.parametrize("cfg", STAT_CASES, ids=[c.name for c in STAT_CASES])
def test_router_stats_match_oracle(torch, cfg):
    import sparse_mixture_experts_softmax_amd as moe
    from moe_testlib import to_device
    _say("case", cfg)
    x = syn.host_x(cfg)
    wr = syn.host_router(cfg)
    bias = syn.router_bias(cfg)
    dx = to_device(x, torch_dtype(cfg))
    dwr = to_device(wr, torch.float32)
    db = None if bias is None else to_device(bias, torch.float32)
    dims = moe.MoeDims(cfg.T, cfg.d, cfg.E, cfg.k, cfg.I, 0, cfg.dtype, 1)
    idx, w, gap, counts, pm = moe.moe_router_topk_stats(dims, dx, dwr, db)
    torch.cuda.synchronize()
    ridx, rw, rgap, logits = oracle.router(x, wr, cfg.k, bias=bias)
    rcounts, rpm = oracle.router_stats(logits, ridx, cfg.E)
    gi = to_host(idx)
    # counts: exactly the GPU's own selections; those equal the oracle's off the tie band
    assert np.array_equal(to_host(counts), np.bincount(gi.reshape(-1), minlength=cfg.E))
    ok = ~oracle.flagged(rgap)
    assert np.array_equal(np.sort(gi[ok], axis=1), np.sort(ridx[ok], axis=1))
    if ok.all():
        assert np.array_equal(to_host(counts), rcounts)
    # mean probabilities: fp32 logits agree to ~1e-6, so do the probabilities
    g = to_host(pm).astype(np.float64)
    assert abs(g.sum() - 1.0) < 1e-5
    err = np.max(np.abs(g - rpm))
    assert err <= 1e-5 * rpm.max(), (err, rpm.max())
    _say(cfg.name, "flagged", int((~ok).sum()), "prob_mean max err", err)


# --------------------------------------------------------------------------------------------
# exact ties: a zero router makes the logits the bias itself, bias[e] = -(e % 64) / 4, so experts
# 64 apart tie and every tie class spans all four wavefronts of the few-token top-k. The pages'
# rule as read (largest logit, the lower expert index among equals, kept in that order) fixes
# the indices, their order and the weights even where the k-th and (k+1)-th logits are equal.
# Few-token top-k (T <= 64, E > 64; k = 16 with 68 merge candidates) and one wavefront per token.
# --------------------------------------------------------------------------------------------
@pytest.mark.parametrize("T,E,k,renorm", [(3, 300, 7, 1), (2, 1024, 16, 0), (1, 512, 10, 1), (70, 300, 7, 1),
                                          (40, 64, 8, 0)])
def test_router_exact_ties_lower_index_first(torch, T, E, k, renorm):
    import sparse_mixture_experts_softmax_amd as moe
    from moe_testlib import to_device
    cfg = syn.MoEConfig("ties", T=T, d=256, E=E, k=k, I=64, Is=0, dtype=syn.BF16, renorm=renorm, seed=41)
    _say("case", "ties", T, E, k, renorm)
    x = syn.host_x(cfg)
    wr = np.zeros((cfg.d, E), np.float32)
    bias = (-(np.arange(E) % 64) * 0.25).astype(np.float32)
    dims = moe.MoeDims(T, cfg.d, E, k, cfg.I, 0, cfg.dtype, renorm)
    idx, w, gap = moe.moe_router_topk(dims, to_device(x, torch_dtype(cfg)), to_device(wr, torch.float32),
                                      to_device(bias, torch.float32))
    torch.cuda.synchronize()
    ridx, rw, rgap, _ = oracle.router(x, wr, k, renorm=bool(renorm), bias=bias)
    # the tie rule by brute force: by descending bias, then ascending index
    order = np.lexsort((np.arange(E), -bias.astype(np.float64)))[:k]
    assert np.array_equal(ridx, np.tile(order, (T, 1)))
    assert np.array_equal(to_host(idx), ridx)
    assert np.max(np.abs(to_host(w).astype(np.float64) - rw)) <= 1e-6
    assert np.array_equal(to_host(gap).astype(np.float64), rgap)


# --------------------------------------------------------------------------------------------
# FP8 expert weights: the quantiser bit for bit, the block on the codes against the oracle on
# the weights they stand for (each side quantises its own copy)
# --------------------------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", [syn.F32, syn.BF16])
def test_fp8_quantiser_matches_oracle_bit_for_bit(torch, dtype):
    import sparse_mixture_experts_softmax_amd as moe
    from moe_testlib import to_device, fp8_untile
    rng = np.random.default_rng(51 + dtype)
    B, K, N = 3, 352, 384  # 11 K tiles x 3 column tiles
    w = (rng.standard_normal((B, K, N)) * np.exp2(rng.integers(-14, 6, size=(B, 1, N)))).astype(np.float32)
    w[1, :, 5] = 0.0
    w[2, 7, 9] = 1e-30  # a column whose maximum is tiny
    if dtype == syn.BF16:
        w = (w.view(np.uint32) >> 16).astype(np.uint16)  # truncation: any bf16 values will do
    q_ref, s_ref = oracle.quantize_fp8(w)
    dw = to_device(w, torch.float32 if dtype == syn.F32 else torch.bfloat16)
    q, s = moe.moe_quantize_fp8(dw)
    torch.cuda.synchronize()
    assert np.array_equal(s.cpu().numpy(), s_ref)
    assert q.shape == (B, N // 128, K // 32, 4096)
    assert np.array_equal(fp8_untile(q.cpu().numpy(), N, K), q_ref)


def _fp8_host_experts(h, cfg):
    """The oracle's view of FP8 experts: its own quantisation of the bf16 weights, dequantised
    (exact in bf16)."""
    def rt(w):
        if w is None:
            return None
        q, s = oracle.quantize_fp8(w)
        return oracle.dequantize_fp8(q, s)
    return {key: rt(h[key]) for key in ("wg", "wu", "wd", "wg_s", "wu_s", "wd_s")}


FP8_CASES = [
    syn.MoEConfig("fp8_ragged", T=300, d=512, E=24, k=4, I=256, Is=128, dtype=syn.BF16, seed=61),
    syn.MoEConfig("fp8_mid_width", T=400, d=2048, E=32, k=8, I=512, Is=512, dtype=syn.BF16, seed=62),
    syn.MoEConfig("fp8_one_token", T=1, d=2048, E=64, k=4, I=512, Is=256, dtype=syn.BF16, seed=63),
    syn.MoEConfig("fp8_no_shared", T=129, d=768, E=16, k=3, I=384, Is=0, dtype=syn.BF16, seed=64),
    # few tokens: 32-row tiles (T <= 32; the shared expert fills one) and 64-row tiles (T <= 64)
    syn.MoEConfig("fp8_T32", T=32, d=2048, E=64, k=6, I=512, Is=512, dtype=syn.BF16, seed=65),
    syn.MoEConfig("fp8_T48", T=48, d=1024, E=32, k=4, I=256, Is=384, dtype=syn.BF16, seed=66),
    # row counts at which the bf16 GEMMs take 160-row (~150 per expert) and 192-row (~350) tiles:
    # the FP8 GEMMs keep their own 128-row tile list
    # one or two tokens: the skinny code streams (gate/up split over K at d = 4096 and finished by
    # the follow-up kernel; 384-wide experts beside a 640-wide shared one)
    syn.MoEConfig("fp8_two_tokens", T=2, d=1024, E=96, k=6, I=384, Is=640, dtype=syn.BF16, seed=69),
    syn.MoEConfig("fp8_one_token_split", T=1, d=4096, E=32, k=4, I=512, Is=512, dtype=syn.BF16, seed=70),
    syn.MoEConfig("fp8_tall_rows", T=300, d=512, E=8, k=4, I=256, Is=256, dtype=syn.BF16, seed=67),
    syn.MoEConfig("fp8_wide_rows", T=700, d=512, E=8, k=4, I=256, Is=256, dtype=syn.BF16, seed=68),
]


@pytest.mark.parametrize("cfg", FP8_CASES, ids=[c.name for c in FP8_CASES])
def test_fp8_forward_matches_oracle(torch, cfg):
    import sparse_mixture_experts_softmax_amd as moe
    _say("case", cfg)
    h = host_inputs(cfg)
    dev = device_from_host(h, cfg)
    experts = moe.Fp8Experts(dev["wg"], dev["wu"], dev["wd"], dev["wg_s"], dev["wu_s"], dev["wd_s"])
    out, idx, w, gap = moe.moe_forward_fp8(dev["x"], dev["w_router"], experts, cfg.k,
                                           renormalize=bool(cfg.renorm), router_bias=dev["bias"],
                                           return_routing=True)
    out16 = run_forward(dev, cfg)[0]
    torch.cuda.synchronize()
    hq = _fp8_host_experts(h, cfg)
    ref_out, ref_idx, ref_w, ref_gap = oracle.forward(h["x"], h["w_router"], hq["wg"], hq["wu"], hq["wd"], hq["wg_s"],
                                                      hq["wu_s"], hq["wd_s"], cfg.k, renorm=bool(cfg.renorm),
                                                      bias=h["bias"])
    st = compare(cfg, to_host(out), to_host(idx), to_host(w), ref_out, ref_idx, ref_w, ref_gap, cfg.name)
    # what the format costs (reported, loosely bounded): the FP8 block against the bf16 one
    o8, o16 = to_host(out).astype(np.float64), to_host(out16).astype(np.float64)
    qerr = float(np.max(np.abs(o8 - o16)) / np.max(np.abs(o16)))
    _say(cfg.name, st, "fp8 vs bf16 max rel", qerr)
    assert qerr < 0.15


# --------------------------------------------------------------------------------------------
# HIP graphs: the forward enqueues kernels only (no allocation, copy, memset or sync), so it can
# be captured once and replayed; each replay must equal an eager call on the same input
# --------------------------------------------------------------------------------------------
GRAPH_CASES = [
    ("bf16_split_k", syn.MoEConfig("graph_split_k", T=3, d=2048, E=32, k=6, I=512, Is=256, dtype=syn.BF16, seed=71)),
    ("bf16_skinny", syn.MoEConfig("graph_skinny", T=1, d=2048, E=32, k=6, I=512, Is=512, dtype=syn.BF16, seed=75)),
    ("bf16_skinny_many_experts", syn.MoEConfig("graph_skinny_e96", T=2, d=2048, E=96, k=6, I=512, Is=512,
                                               dtype=syn.BF16, seed=76)),
    # ~350 rows per expert: the tall kernel with 160- and 192-row tiles in one launch
    ("bf16_tall_tiles", syn.MoEConfig("graph_tall", T=700, d=512, E=8, k=4, I=256, Is=256, dtype=syn.BF16,
                                      seed=77)),
    ("bf16_mid_width", syn.MoEConfig("graph_mid", T=300, d=2048, E=64, k=8, I=512, Is=512, dtype=syn.BF16, seed=72)),
    ("fp8", syn.MoEConfig("graph_fp8", T=40, d=1024, E=32, k=4, I=256, Is=256, dtype=syn.BF16, seed=73)),
    ("block", syn.MoEConfig("graph_block", T=200, d=512, E=24, k=4, I=256, Is=128, dtype=syn.BF16, seed=74)),
    ("block_one_token", syn.MoEConfig("graph_block_T1", T=1, d=2048, E=64, k=8, I=512, Is=512, dtype=syn.BF16,
                                      seed=78)),
]


@pytest.mark.parametrize("kind,cfg", GRAPH_CASES, ids=[c[0] for c in GRAPH_CASES])
def test_forward_replays_in_a_hip_graph(torch, kind, cfg):
    import sparse_mixture_experts_softmax_amd as moe
    from moe_testlib import to_device
    _say("case", kind, cfg)
    h = host_inputs(cfg)
    dev = device_from_host(h, cfg)
    dims = moe.dims_for(dev["x"], dev["w_router"], dev["wg"], dev["wg_s"], cfg.k, True)
    gamma = to_device(syn.host_gamma(cfg), torch_dtype(cfg)) if kind.startswith("block") else None
    experts = moe.Fp8Experts(dev["wg"], dev["wu"], dev["wd"], dev["wg_s"], dev["wu_s"], dev["wd_s"]) \
        if kind == "fp8" else None

    def call(x, ws):
        if kind == "fp8":
            return moe.moe_forward_fp8(x, dev["w_router"], experts, cfg.k, router_bias=dev["bias"], ws=ws, dims=dims)
        if kind.startswith("block"):
            return moe.moe_forward_block(x, gamma, dev["w_router"], dev["wg"], dev["wu"], dev["wd"], dev["wg_s"],
                                         dev["wu_s"], dev["wd_s"], cfg.k, ws=ws, dims=dims)
        return moe.moe_forward(x, dev["w_router"], dev["wg"], dev["wu"], dev["wd"], dev["wg_s"], dev["wu_s"],
                               dev["wd_s"], cfg.k, router_bias=dev["bias"], ws=ws, dims=dims)

    ws_graph, ws_eager = moe.workspace(dims, "cuda"), moe.workspace(dims, "cuda")
    x_static = dev["x"].clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(x_static, ws_graph)  # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out_g = call(x_static, ws_graph)
    inputs = [dev["x"], torch.flip(dev["x"], dims=[0]).contiguous(), (dev["x"] * 0.5).contiguous()]
    for rep, xi in enumerate(inputs + inputs[:1]):
        x_static.copy_(xi)
        g.replay()
        ref = call(xi, ws_eager)
        torch.cuda.synchronize()
        assert torch.equal(out_g, ref), (kind, rep)
