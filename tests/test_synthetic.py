"""The seeded input generator: determinism, slicing, distribution, bf16 rounding, Zipf targets."""
import math

import numpy as np

import synthetic as syn


def test_deterministic_and_seed_dependent():
    a = syn.host_fill(1000, syn.F32, 0, syn.TID_X, 1.0)
    b = syn.host_fill(1000, syn.F32, 0, syn.TID_X, 1.0)
    c = syn.host_fill(1000, syn.F32, 1, syn.TID_X, 1.0)
    d = syn.host_fill(1000, syn.F32, 0, syn.TID_WR, 1.0)
    assert np.array_equal(a, b)
    assert not np.array_equal(a, c) and not np.array_equal(a, d)


def test_offsets_and_rows_match_full_tensor():
    full = syn.host_fill(40 * 24, syn.BF16, 3, syn.TID_WG, 0.1).reshape(40, 24)
    part = syn.host_fill(5 * 24, syn.BF16, 3, syn.TID_WG, 0.1, offset=7 * 24).reshape(5, 24)
    assert np.array_equal(part, full[7:12])
    rows = [39, 0, 17, 17]
    assert np.array_equal(syn.host_rows(rows, 24, syn.BF16, 3, syn.TID_WG, 0.1), full[rows])


def test_expert_slice_is_slice_of_full_tensor():
    cfg = syn.CONFIGS["tiny"]
    wg, wu, wd = syn.host_all_experts(cfg)
    g5, u5, d5 = syn.host_expert(cfg, 5)
    assert np.array_equal(g5, wg[5]) and np.array_equal(u5, wu[5]) and np.array_equal(d5, wd[5])


def test_distribution_is_close_to_normal():
    from scipy import stats
    z = syn.host_fill(1 << 20, syn.F32, 0, syn.TID_X, 1.0).astype(np.float64)
    assert abs(z.mean()) < 5e-3 and abs(z.std() - 1) < 5e-3
    assert stats.kstest(z[:100000], "norm").pvalue > 1e-3
    s = syn.host_fill(1 << 18, syn.F32, 0, syn.TID_WG, 1 / math.sqrt(8192)).astype(np.float64)
    assert abs(s.std() * math.sqrt(8192) - 1) < 1e-2


def test_bf16_is_round_to_nearest_even_of_fp32():
    f = syn.host_fill(1 << 16, syn.F32, 2, syn.TID_WU, 0.05)
    b = syn.host_fill(1 << 16, syn.BF16, 2, syn.TID_WU, 0.05)
    bits = f.view(np.uint32).astype(np.uint64)
    lower = (bits & 0xFFFF)
    trunc = (bits >> 16)
    up = (lower > 0x8000) | ((lower == 0x8000) & ((trunc & 1) == 1))
    assert np.array_equal(b.astype(np.uint64), trunc + up)


def test_quantile_table_is_antisymmetric_normal():
    from scipy.stats import norm
    q = syn.quantile_table()
    assert len(q) == 65537 and q[32768] == 0.0
    assert np.array_equal(q, -q[::-1])
    j = np.arange(1, 65536, 97)
    np.testing.assert_allclose(q[j], norm.ppf(j / 65536.0), rtol=1e-10, atol=1e-12)


def test_zipf_targets_water_filled():
    L = syn.zipf_targets(8192, 512, 10, 1.2)
    assert abs(L.sum() - 81920) < 1e-6
    assert L.max() <= 8192 + 1e-9
    assert np.all(np.diff(L) <= 1e-9)
    free = L < 8192 - 1e-9
    r = np.arange(1, 513)[free]
    ratio = L[free] * r ** 1.2
    np.testing.assert_allclose(ratio, ratio[0], rtol=1e-12)


def test_coverage_tokens_cover_every_row_band():
    # the token selection of the full-size parity tests: on a routing shaped like the prefill and
    # skew workloads, every 64-row band of every expert's slots and of the shared expert's rows
    # holds a selected token, and at least n_min tokens are selected
    from moe_testlib import coverage_tokens
    rng = np.random.default_rng(0)
    for T, E, k, skew in [(4096, 128, 6, False), (2048, 128, 6, True)]:
        logits = rng.standard_normal((T, E))
        if skew:
            logits += 2.0 * np.log(1.0 / np.arange(1, E + 1))
        idx = np.argsort(-logits, axis=1)[:, :k].astype(np.int32)
        tokens, cov = coverage_tokens(idx, E, 300, 2000, seed=1)
        assert cov == 1.0 and len(tokens) >= 300 and len(set(tokens.tolist())) == len(tokens)
        # brute-force check of the claim
        flat_e, flat_t = idx.reshape(-1), np.repeat(np.arange(T), k)
        sel = set(tokens.tolist())
        for e in range(E):
            toks = np.sort(flat_t[flat_e == e])
            for b0 in range(0, len(toks), 64):
                assert sel & set(toks[b0:b0 + 64].tolist()), (e, b0)
        for b0 in range(0, T, 64):
            assert sel & set(range(b0, min(T, b0 + 64)))
