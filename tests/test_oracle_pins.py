"""Pins of the CPU oracle to facts that do not come from the oracle itself.

Each test checks the oracle against a library routine used independently (numpy float64 dense
algebra, scipy's softmax), a brute-force enumeration, a closed form worked by hand, or an
invariant the definition implies. A plausible mistake in the oracle (a dropped term, a wrong sign,
a swapped index or operand, softmax over the wrong set, a wrong tie rule) fails at least one.
"""
import itertools
import math

import numpy as np
import pytest
from scipy.special import softmax

import oracle
import synthetic as syn


def rand_layer(rng, T, d, E, I, Is, scale_r=None):
    x = rng.standard_normal((T, d)).astype(np.float32)
    wr = (rng.standard_normal((d, E)) * (scale_r or 1 / math.sqrt(d))).astype(np.float32)
    wg = (rng.standard_normal((E, d, I)) / math.sqrt(d)).astype(np.float32)
    wu = (rng.standard_normal((E, d, I)) / math.sqrt(d)).astype(np.float32)
    wd = (rng.standard_normal((E, I, d)) / math.sqrt(I)).astype(np.float32)
    if Is:
        wgs = (rng.standard_normal((d, Is)) / math.sqrt(d)).astype(np.float32)
        wus = (rng.standard_normal((d, Is)) / math.sqrt(d)).astype(np.float32)
        wds = (rng.standard_normal((Is, d)) / math.sqrt(Is)).astype(np.float32)
    else:
        wgs = wus = wds = None
    return x, wr, wg, wu, wd, wgs, wus, wds


def dense_swiglu(x, wg, wu, wd):
    """numpy float64 dense SwiGLU FFN, (silu(x Wg) * (x Wu)) Wd."""
    x = x.astype(np.float64)
    g = x @ wg.astype(np.float64)
    u = x @ wu.astype(np.float64)
    h = g / (1.0 + np.exp(-g)) * u
    return h @ wd.astype(np.float64)


# --------------------------------------------------------------------------------------------
# router
# --------------------------------------------------------------------------------------------
def test_logits_match_numpy_float64():
    rng = np.random.default_rng(1)
    x, wr, *_ = rand_layer(rng, 33, 96, 24, 8, 0)
    bias = rng.standard_normal(24).astype(np.float32)
    idx, w, gap, logits = oracle.router(x, wr, 3, bias=bias)
    ref = (x.astype(np.float64) @ wr.astype(np.float64) + bias.astype(np.float64)).astype(np.float32)
    # both sum in double and round once; only the summation order may differ
    ulp = np.spacing(np.abs(ref))
    assert np.all(np.abs(logits.astype(np.float64) - ref) <= ulp)
    assert np.mean(logits == ref) > 0.99


def brute_force_topk(l, k):
    """Exhaustive search over all k-subsets: the selected set is the one whose logits, sorted
    descending, are lexicographically largest; among equal logit multisets the one with the
    lexicographically smallest sorted index tuple."""
    E = len(l)
    best = None
    for S in itertools.combinations(range(E), k):
        key = (tuple(sorted((float(l[e]) for e in S), reverse=True)), tuple(-e for e in S))
        if best is None or key > best[0]:
            best = (key, S)
    return set(best[1])


@pytest.mark.parametrize("E,k", [(1, 1), (2, 1), (4, 2), (6, 3), (8, 3), (8, 8), (5, 4)])
def test_topk_matches_brute_force(E, k):
    rng = np.random.default_rng(100 + E * 10 + k)
    x, wr, *_ = rand_layer(rng, 16, 8, E, 4, 0)
    idx, w, gap, logits = oracle.router(x, wr, k)
    for t in range(16):
        assert set(idx[t].tolist()) == brute_force_topk(logits[t], k)
        # listed by descending logit
        assert np.all(np.diff(logits[t][idx[t]]) <= 0)
        if k < E:
            rest = np.delete(logits[t], idx[t])
            assert gap[t] == pytest.approx(float(logits[t][idx[t][-1]]) - float(rest.max()), abs=0)
        else:
            assert math.isinf(gap[t])


def test_topk_ties_go_to_lower_index():
    # duplicate router columns give exactly equal logits
    rng = np.random.default_rng(7)
    d, E = 8, 6
    base = rng.standard_normal((d, 3)).astype(np.float32)
    wr = np.concatenate([base, base], axis=1)  # expert e and e+3 tie exactly
    x = rng.standard_normal((20, d)).astype(np.float32)
    for k in (1, 2, 3, 4, 5):
        idx, w, gap, logits = oracle.router(x, wr, k)
        for t in range(20):
            assert set(idx[t].tolist()) == brute_force_topk(logits[t], k)
    idx, w, gap, logits = oracle.router(x, wr, 1)
    assert np.all(idx[:, 0] < 3)  # the lower of each tied pair wins
    assert np.all(gap == 0.0)  # and the runner-up ties it exactly


def test_weights_sum_to_one_with_renorm():
    rng = np.random.default_rng(2)
    x, wr, *_ = rand_layer(rng, 50, 32, 16, 4, 0)
    idx, w, gap, logits = oracle.router(x, wr, 4, renorm=True)
    np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-12)
    assert np.all(w > 0)
    assert np.all(np.diff(w, axis=1) <= 0)  # weights follow the descending logits


def test_weights_equal_softmax_of_kept_logits():
    rng = np.random.default_rng(3)
    x, wr, *_ = rand_layer(rng, 40, 32, 16, 4, 0)
    idx, w, gap, logits = oracle.router(x, wr, 5, renorm=True)
    kept = np.take_along_axis(logits.astype(np.float64), idx, axis=1)
    np.testing.assert_allclose(w, softmax(kept, axis=1), rtol=1e-12, atol=0)


def test_k_equals_E_is_full_softmax():
    rng = np.random.default_rng(4)
    x, wr, *_ = rand_layer(rng, 30, 16, 7, 4, 0)
    idx, w, gap, logits = oracle.router(x, wr, 7, renorm=True)
    p = softmax(logits.astype(np.float64), axis=1)
    np.testing.assert_allclose(w, np.take_along_axis(p, idx, axis=1), rtol=1e-12)
    assert np.all(np.isinf(gap))


def test_no_renorm_gives_full_softmax_probabilities():
    rng = np.random.default_rng(5)
    x, wr, *_ = rand_layer(rng, 30, 16, 12, 4, 0, scale_r=1.0)
    idx, w, gap, logits = oracle.router(x, wr, 3, renorm=False)
    p = softmax(logits.astype(np.float64), axis=1)
    np.testing.assert_allclose(w, np.take_along_axis(p, idx, axis=1), rtol=1e-12)
    assert np.all(w.sum(axis=1) < 1.0)


def test_indices_distinct_and_in_range():
    cfg = syn.CONFIGS["tiny"]
    x, wr = syn.host_x(cfg), syn.host_router(cfg)
    idx, w, gap, logits = oracle.router(x, wr, cfg.k)
    assert idx.min() >= 0 and idx.max() < cfg.E
    assert all(len(set(r.tolist())) == cfg.k for r in idx)


def test_constant_bias_changes_nothing_material():
    rng = np.random.default_rng(6)
    x, wr, *_ = rand_layer(rng, 64, 32, 16, 4, 0)
    idx0, w0, gap0, _ = oracle.router(x, wr, 3)
    idx1, w1, gap1, _ = oracle.router(x, wr, 3, bias=np.full(16, 0.375, np.float32))
    ok = ~oracle.flagged(gap0)
    assert ok.sum() > 50
    np.testing.assert_array_equal(idx0[ok], idx1[ok])
    np.testing.assert_allclose(w0[ok], w1[ok], rtol=1e-5)


# --------------------------------------------------------------------------------------------
# experts, shared expert, combine
# --------------------------------------------------------------------------------------------
def test_single_expert_is_dense_swiglu_plus_shared():
    rng = np.random.default_rng(8)
    x, wr, wg, wu, wd, wgs, wus, wds = rand_layer(rng, 12, 40, 1, 24, 16)
    out, idx, w, gap = oracle.forward(x, wr, wg, wu, wd, wgs, wus, wds, k=1)
    ref = dense_swiglu(x, wg[0], wu[0], wd[0]) + dense_swiglu(x, wgs, wus, wds)
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)
    assert np.all(idx == 0) and np.all(w == 1.0)


def test_routed_part_matches_per_token_numpy():
    rng = np.random.default_rng(9)
    T, d, E, k, I = 10, 24, 6, 2, 16
    x, wr, wg, wu, wd, *_ = rand_layer(rng, T, d, E, I, 0)
    out, idx, w, gap = oracle.forward(x, wr, wg, wu, wd, None, None, None, k=k)
    for t in range(T):
        ref = sum(w[t, j] * dense_swiglu(x[t:t + 1], wg[idx[t, j]], wu[idx[t, j]], wd[idx[t, j]])[0]
                  for j in range(k))
        np.testing.assert_allclose(out[t], ref, rtol=1e-12, atol=1e-13)


def test_identical_experts_ignore_routing():
    rng = np.random.default_rng(10)
    T, d, E, I, Is = 9, 16, 5, 8, 8
    x, wr, wg, wu, wd, wgs, wus, wds = rand_layer(rng, T, d, E, I, Is)
    wg[:] = wg[0]
    wu[:] = wu[0]
    wd[:] = wd[0]
    out, *_ = oracle.forward(x, wr, wg, wu, wd, wgs, wus, wds, k=3)
    ref = dense_swiglu(x, wg[0], wu[0], wd[0]) + dense_swiglu(x, wgs, wus, wds)
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)


def test_zero_down_projections():
    rng = np.random.default_rng(11)
    T, d, E, I, Is = 7, 16, 4, 8, 12
    x, wr, wg, wu, wd, wgs, wus, wds = rand_layer(rng, T, d, E, I, Is)
    out, *_ = oracle.forward(x, wr, wg, wu, np.zeros_like(wd), wgs, wus, wds, k=2)
    np.testing.assert_allclose(out, dense_swiglu(x, wgs, wus, wds), rtol=1e-12, atol=1e-14)
    out_routed, *_ = oracle.forward(x, wr, wg, wu, wd, None, None, None, k=2)
    out_zero_shared, *_ = oracle.forward(x, wr, wg, wu, wd, wgs, wus, np.zeros_like(wds), k=2)
    np.testing.assert_allclose(out_zero_shared, out_routed, rtol=1e-14, atol=0)


def test_linear_in_down_projections():
    rng = np.random.default_rng(12)
    T, d, E, I, Is = 7, 16, 4, 8, 8
    x, wr, wg, wu, wd, wgs, wus, wds = rand_layer(rng, T, d, E, I, Is)
    out1, *_ = oracle.forward(x, wr, wg, wu, wd, wgs, wus, wds, k=2)
    out2, *_ = oracle.forward(x, wr, wg, wu, 2 * wd, wgs, wus, 2 * wds, k=2)
    np.testing.assert_allclose(out2, 2 * out1, rtol=1e-13, atol=1e-15)


def test_hand_worked_example():
    """d=2, E=2, k=1, I=1, shared I=1, all by hand.
    x = (1, 0); W_r = [[2, 0], [0, 0]] gives logits (2, 0), so expert 0 with weight 1.
    Expert 0: W_g = (1, 0)^T, W_u = (3, 0)^T, W_d = (1, -1): g = 1, u = 3,
      h = silu(1) * 3 = 3 / (1 + e^-1), y = (h, -h).
    Shared: W_g = (0, 0)^T gives g = 0 and silu(0) = 0, so it adds nothing.
    Without renormalisation the weight is softmax(2, 0)[0] = 1 / (1 + e^-2)."""
    x = np.array([[1.0, 0.0]], np.float32)
    wr = np.array([[2.0, 0.0], [0.0, 0.0]], np.float32)
    wg = np.array([[[1.0], [0.0]], [[5.0], [5.0]]], np.float32)
    wu = np.array([[[3.0], [0.0]], [[5.0], [5.0]]], np.float32)
    wd = np.array([[[1.0, -1.0]], [[7.0, 7.0]]], np.float32)
    wgs = np.zeros((2, 1), np.float32)
    wus = np.ones((2, 1), np.float32)
    wds = np.ones((1, 2), np.float32)
    h = 3.0 / (1.0 + math.exp(-1.0))
    out, idx, w, gap = oracle.forward(x, wr, wg, wu, wd, wgs, wus, wds, k=1, renorm=True)
    assert idx[0, 0] == 0 and w[0, 0] == 1.0 and gap[0] == 2.0
    np.testing.assert_allclose(out[0], [h, -h], rtol=1e-15)
    out, idx, w, gap = oracle.forward(x, wr, wg, wu, wd, wgs, wus, wds, k=1, renorm=False)
    p0 = 1.0 / (1.0 + math.exp(-2.0))
    np.testing.assert_allclose(w[0, 0], p0, rtol=1e-15)
    np.testing.assert_allclose(out[0], [p0 * h, -p0 * h], rtol=1e-15)


# --------------------------------------------------------------------------------------------
# whole-block invariants
# --------------------------------------------------------------------------------------------
def test_token_permutation_equivariance_bitwise():
    cfg = syn.CONFIGS["tiny"]
    x = syn.host_x(cfg)
    wr = syn.host_router(cfg)
    wg, wu, wd = syn.host_all_experts(cfg)
    wgs, wus, wds = syn.host_shared(cfg)
    out, idx, w, gap = oracle.forward(x, wr, wg, wu, wd, wgs, wus, wds, k=cfg.k)
    perm = np.random.default_rng(13).permutation(cfg.T)
    out_p, idx_p, w_p, gap_p = oracle.forward(x[perm], wr, wg, wu, wd, wgs, wus, wds, k=cfg.k)
    assert np.array_equal(out_p, out[perm])
    assert np.array_equal(idx_p, idx[perm])


def test_expert_relabelling_invariance():
    rng = np.random.default_rng(14)
    T, d, E, I, Is = 20, 16, 8, 8, 8
    x, wr, wg, wu, wd, wgs, wus, wds = rand_layer(rng, T, d, E, I, Is)
    out, idx, w, gap = oracle.forward(x, wr, wg, wu, wd, wgs, wus, wds, k=3)
    pi = rng.permutation(E)  # new expert e' holds old expert pi[e']
    out2, idx2, w2, gap2 = oracle.forward(x, wr[:, pi], wg[pi], wu[pi], wd[pi], wgs, wus, wds, k=3)
    ok = ~oracle.flagged(gap)
    assert np.array_equal(pi[idx2[ok]], idx[ok])
    # the softmax denominator is summed in expert order, so only rounding may differ
    np.testing.assert_allclose(out2[ok], out[ok], rtol=1e-13, atol=1e-14)


def test_zero_token_gives_zero_output():
    rng = np.random.default_rng(15)
    x, wr, wg, wu, wd, wgs, wus, wds = rand_layer(rng, 4, 16, 6, 8, 8)
    x[2] = 0.0
    out, idx, w, gap = oracle.forward(x, wr, wg, wu, wd, wgs, wus, wds, k=2)
    assert np.all(out[2] == 0.0)
    assert gap[2] == 0.0 and oracle.flagged(gap)[2]  # every logit is 0: all tie
    assert list(idx[2]) == [0, 1]


def test_bf16_inputs_equal_widened_fp32():
    cfg = syn.CONFIGS["tiny"].with_(dtype=syn.BF16, T=16)
    x = syn.host_x(cfg)
    wr = syn.host_router(cfg)
    wg, wu, wd = syn.host_all_experts(cfg)
    wgs, wus, wds = syn.host_shared(cfg)
    w = syn.bf16_bits_to_f32
    a = oracle.forward(x, wr, wg, wu, wd, wgs, wus, wds, k=cfg.k)
    b = oracle.forward(w(x), wr, w(wg), w(wu), w(wd), w(wgs), w(wus), w(wds), k=cfg.k)
    for u, v in zip(a, b):
        assert np.array_equal(u, v)


def test_per_expert_pointers_allow_missing_unselected_experts():
    cfg = syn.CONFIGS["tiny"]
    x = syn.host_x(cfg)[:5]
    wr = syn.host_router(cfg)
    wg, wu, wd = syn.host_all_experts(cfg)
    wgs, wus, wds = syn.host_shared(cfg)
    full, idx, *_ = oracle.forward(x, wr, wg, wu, wd, wgs, wus, wds, k=cfg.k)
    used = set(idx.ravel().tolist())
    sel = lambda a: [a[e] if e in used else None for e in range(cfg.E)]  # noqa: E731
    part, *_ = oracle.forward(x, wr, sel(wg), sel(wu), sel(wd), wgs, wus, wds, k=cfg.k)
    assert np.array_equal(part, full)
    missing = [None] * cfg.E
    missing[0] = wg[0]
    with pytest.raises(RuntimeError):
        oracle.forward(x, wr, missing, missing, missing, wgs, wus, wds, k=cfg.k)


def test_expert_rows_match_numpy_per_pair():
    # the per-pair expert output against the dense numpy SwiGLU, for pairs that repeat rows and
    # experts in any order (fp32 and bf16 inputs)
    rng = np.random.default_rng(21)
    x, wr, wg, wu, wd, *_ = rand_layer(rng, 9, 40, 5, 24, 0)
    rows = np.array([3, 0, 3, 8, 1, 1])
    es = [4, 2, 2, 0, 4, 1]
    y = oracle.expert_rows(x, rows, [(wg[e], wu[e], wd[e]) for e in es])
    for p, (r, e) in enumerate(zip(rows, es)):
        np.testing.assert_allclose(y[p], dense_swiglu(x[r:r + 1], wg[e], wu[e], wd[e])[0], rtol=1e-12, atol=1e-13)
    xb = (x.view(np.uint32) >> 16).astype(np.uint16)
    bits = lambda a: (a.view(np.uint32) >> 16).astype(np.uint16)  # noqa: E731
    yb = oracle.expert_rows(xb, rows, [(bits(wg[e]), bits(wu[e]), bits(wd[e])) for e in es])
    xw = oracle.widen(xb)
    for p, (r, e) in enumerate(zip(rows, es)):
        ref = dense_swiglu(xw[r:r + 1], oracle.widen(bits(wg[e])), oracle.widen(bits(wu[e])), oracle.widen(bits(wd[e])))
        np.testing.assert_allclose(yb[p], ref[0], rtol=1e-12, atol=1e-13)
    assert oracle.expert_rows(x, np.zeros(0, np.int64), []).shape == (0, 40)


@pytest.mark.parametrize("renorm,shared,batch", [(True, True, 3), (False, True, 1), (True, False, 64)])
def test_forward_by_expert_equals_forward(renorm, shared, batch):
    # the expert-major visit order (bounded host memory for the large shapes) gives the per-token
    # definition's result up to the order of a k-term double sum, and the same routing
    rng = np.random.default_rng(22)
    T, d, E, k, I, Is = 40, 48, 12, 3, 32, 24
    x, wr, wg, wu, wd, wgs, wus, wds = rand_layer(rng, T, d, E, I, Is if shared else 0)
    bias = rng.standard_normal(E).astype(np.float32) * 0.3
    ref, ridx, rw, rgap = oracle.forward(x, wr, wg, wu, wd, wgs, wus, wds, k=k, renorm=renorm, bias=bias)
    loaded = []

    def load(e):
        loaded.append(e)
        return wg[e], wu[e], wd[e]

    out, idx, w, gap = oracle.forward_by_expert(x, wr, k, load, shared=(wgs, wus, wds) if shared else None,
                                                renorm=renorm, bias=bias, batch=batch)
    assert np.array_equal(idx, ridx) and np.array_equal(w, rw) and np.array_equal(gap, rgap)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-13 * np.abs(ref).max())
    assert sorted(loaded) == sorted(set(ridx.ravel().tolist()))  # each selected expert loaded once


# --------------------------------------------------------------------------------------------
# zero-centred RMSNorm in front of the block, and the residual add around it
# --------------------------------------------------------------------------------------------
def bf16_bits_of(v):
    """bf16 bit pattern of a value that bf16 holds exactly."""
    b = np.float32(v).view(np.uint32)
    assert b & 0xFFFF == 0, v
    return np.uint16(b >> 16)


def test_rmsnorm_constant_row_closed_form():
    # a row of d equal values c: mean(x^2) = c^2, so h = c / sqrt(c^2 + eps) * (1 + gamma). A sum
    # in place of the mean gives 1/sqrt(d); eps outside the root, or dropped, moves h at small c.
    d = 64
    for c, eps in ((0.5, 1e-6), (1e-3, 1e-6), (-2.0, 0.0), (3e-4, 1e-6)):
        x = np.full((1, d), c, np.float32)
        h = oracle.rmsnorm(x, np.zeros(d, np.float32), eps)
        cf = float(np.float32(c))
        expect = cf / math.sqrt(cf * cf + eps)  # in double; the oracle rounds once to fp32
        assert np.allclose(h.astype(np.float64), expect, rtol=2 ** -23, atol=0), (c, eps, h[0, 0], expect)
    # c = 1e-3, eps = 1e-6: h = 1/sqrt(2) exactly in the definition
    h = oracle.rmsnorm(np.full((1, d), 1e-3, np.float64).astype(np.float32), np.zeros(d, np.float32), 1e-6)
    assert abs(float(h[0, 0]) - 1 / math.sqrt(2)) < 1e-6


def test_rmsnorm_scale_is_one_plus_gamma():
    # gamma = 0 is the identity scale (zero-centred); gamma = -1 zeroes the element; gamma = 1
    # doubles it. A plain-gamma scale would zero everything at gamma = 0.
    rng = np.random.default_rng(5)
    d = 48
    x = rng.standard_normal((3, d)).astype(np.float32)
    base = oracle.rmsnorm(x, np.zeros(d, np.float32), 1e-6).astype(np.float64)
    gamma = np.zeros(d, np.float32)
    gamma[::3] = -1.0
    gamma[1::3] = 1.0
    h = oracle.rmsnorm(x, gamma, 1e-6).astype(np.float64)
    assert np.all(h[:, ::3] == 0.0)
    assert np.allclose(h[:, 1::3], 2 * base[:, 1::3], rtol=2 ** -23, atol=0)
    assert np.array_equal(h[:, 2::3], base[:, 2::3])
    # rows have unit mean square before the scale (eps small against it)
    assert np.allclose((base ** 2).mean(axis=1), 1.0, rtol=1e-5)


def test_rmsnorm_scale_invariance_without_eps():
    # with eps = 0 the norm is invariant to scaling a row by a power of two (exact in fp32)
    rng = np.random.default_rng(6)
    x = rng.standard_normal((4, 40)).astype(np.float32)
    g = (rng.standard_normal(40) * 0.1).astype(np.float32)
    assert np.array_equal(oracle.rmsnorm(x, g, 0.0), oracle.rmsnorm(x * np.float32(8.0), g, 0.0))


def test_rmsnorm_bf16_rounds_to_nearest_even():
    # rows of ones (h = 1 + gamma exactly with eps = 0): gamma = 2^-8 puts h halfway between bf16
    # 1.0 and 1.0078125 (ties to the even 1.0); 3 * 2^-8 is halfway between 1.0078125 and
    # 1.015625 (ties to the even 1.015625); 2^-8 + 2^-12 is above halfway (rounds up).
    # Truncation or round-half-up fails one of them.
    gam = [2 ** -8, 3 * 2 ** -8, 2 ** -8 + 2 ** -12, -(2 ** -9)]
    want = [1.0, 1.015625, 1.0078125, 1.0]  # 1 - 2^-9 is halfway below 1.0 (bf16 step 2^-8 there)
    d = len(gam)
    x = np.full((1, d), bf16_bits_of(1.0), np.uint16)
    g = np.array([bf16_bits_of(v) for v in gam], np.uint16)
    h = oracle.rmsnorm(x, g, 0.0)
    assert [int(b) for b in h[0]] == [int(bf16_bits_of(v)) for v in want]


def test_block_forward_zero_experts_is_the_residual_and_composes():
    # with every expert (and the shared one) zero, the block passes x through unchanged; in
    # general it is x plus the block applied to the normalised rows
    rng = np.random.default_rng(8)
    T, d, E, k, I, Is = 5, 32, 6, 2, 16, 8
    x, wr, wg, wu, wd, wgs, wus, wds = rand_layer(rng, T, d, E, I, Is)
    gamma = (rng.standard_normal(d) * 0.1).astype(np.float32)
    z = np.zeros_like
    out, idx, _, _, h = oracle.block_forward(x, gamma, wr, z(wg), z(wu), z(wd), z(wgs), z(wus), z(wds), k)
    assert np.array_equal(out, x.astype(np.float64))
    out, idx, w, gap, h = oracle.block_forward(x, gamma, wr, wg, wu, wd, wgs, wus, wds, k)
    ref = x.astype(np.float64)
    hh = h.astype(np.float64)
    for t in range(T):
        acc = dense_swiglu(hh[t:t + 1], wgs, wus, wds)[0]
        for j in range(k):
            e = idx[t, j]
            acc = acc + w[t, j] * dense_swiglu(hh[t:t + 1], wg[e], wu[e], wd[e])[0]
        ref[t] += acc
    assert np.allclose(out, ref, rtol=1e-10, atol=1e-12)


# --------------------------------------------------------------------------------------------
# router statistics (per-expert counts, mean probability)
# --------------------------------------------------------------------------------------------
def test_router_stats_invariants_and_closed_forms():
    rng = np.random.default_rng(21)
    T, d, E, k = 57, 24, 11, 3
    x = rng.standard_normal((T, d)).astype(np.float32)
    wr = (rng.standard_normal((d, E)) / math.sqrt(d)).astype(np.float32)
    idx, w, gap, logits = oracle.router(x, wr, k)
    counts, pm = oracle.router_stats(logits, idx, E)
    # every token contributes k selections and a probability vector that sums to one
    assert counts.sum() == T * k and np.all(counts >= 0)
    assert abs(pm.sum() - 1.0) < 1e-12
    # counts equal a brute-force tally of the selections
    assert np.array_equal(counts, [sum(int(e in idx[t]) for t in range(T)) for e in range(E)])
    # a zero router weight gives equal logits: every expert has mean probability 1/E
    _, _, _, lz = oracle.router(x, np.zeros_like(wr), k)
    _, pz = oracle.router_stats(lz, idx, E)
    assert np.allclose(pz, 1.0 / E, rtol=1e-12, atol=0)
    # one token repeated: the mean is that token's own softmax (scipy, independent)
    xr = np.repeat(x[:1], 9, axis=0)
    i1, _, _, l1 = oracle.router(xr, wr, k)
    _, p1 = oracle.router_stats(l1, i1, E)
    assert np.allclose(p1, softmax(l1[0].astype(np.float64)), rtol=1e-12, atol=1e-15)
    # the mean is over tokens, not over selections: doubling every logit's spread of one token
    # changes only its own contribution
    l2 = logits.astype(np.float64).copy()
    l2[0] *= 2
    _, pm2 = oracle.router_stats(l2, idx, E)
    assert np.allclose(pm2 - pm, (softmax(l2[0]) - softmax(logits[0].astype(np.float64))) / T, atol=1e-15)


# --------------------------------------------------------------------------------------------
# FP8 expert weights: OCP e4m3 codes, round to nearest even, power-of-two column scales
# --------------------------------------------------------------------------------------------
def test_e4m3_code_table_closed_forms():
    # values fixed by the format: bias 7, 3 mantissa bits, subnormals below 2^-6, 448 the largest
    # finite value, S.1111.111 the NaN codes, sign-magnitude
    v = oracle.e4m3_value(np.arange(256))
    assert v[0x00] == 0.0 and v[0x01] == 2.0 ** -9 and v[0x07] == 7 * 2.0 ** -9
    assert v[0x08] == 2.0 ** -6 and v[0x38] == 1.0 and v[0x39] == 1.125 and v[0x7E] == 448.0
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF]) and np.sum(np.isnan(v)) == 2
    assert np.array_equal(v[0x80:0xFF], -v[0x00:0x7F])
    assert np.all(np.diff(v[:0x7F]) > 0)  # codes 0 .. 126 ascend


def test_e4m3_round_to_nearest_even():
    pos = oracle.e4m3_value(np.arange(127))
    # every finite value rounds to its own code
    assert np.array_equal(oracle.e4m3_round(pos), np.arange(127, dtype=np.uint8))
    assert np.array_equal(oracle.e4m3_round(-pos[1:]), (np.arange(1, 127) | 0x80).astype(np.uint8))
    # halfway points go to the even code; just off halfway goes to the nearer one
    cases = [(1.0625, 0x38), (1.1875, 0x3A), (1.0625 + 2 ** -20, 0x39), (2.0 ** -10, 0x00),
             (1.5 * 2.0 ** -9, 0x02), (2.5 * 2.0 ** -9, 0x02), (432.0, 0x7E), (416.0, 0x7D), (-1.0625, 0xB8)]
    for val, code in cases:
        assert int(oracle.e4m3_round(np.array([val]))[0]) == code, (val, hex(code))
    # against brute force: the code whose value is nearest, ties to the even code
    rng = np.random.default_rng(41)
    x = rng.uniform(-448, 448, 4000) * rng.choice([1, 2.0 ** -6, 2.0 ** -9], 4000)
    got = oracle.e4m3_round(x)
    d = np.abs(np.abs(x)[:, None] - pos[None, :])
    best = d.min(axis=1, keepdims=True)
    near = d == best
    want = np.where(near.sum(axis=1) == 2, np.argmax(near & (np.arange(127) % 2 == 0), axis=1), np.argmax(near, axis=1))
    want = np.where((x < 0) & (want != 0), want | 0x80, want)
    assert np.array_equal(got, want.astype(np.uint8))


def test_fp8_quantisation_scales_layout_and_error():
    rng = np.random.default_rng(42)
    K, N = 96, 40
    w = (rng.standard_normal((2, K, N)) * np.exp2(rng.integers(-12, 4, size=(2, 1, N)))).astype(np.float32)
    w[1, :, 7] = 0.0
    q, s = oracle.quantize_fp8(w)
    assert q.shape == (2, N, K) and s.shape == (2, N)
    amax = np.abs(w).max(axis=1)
    # power-of-two scales, the smallest with amax / s <= 448
    e = np.log2(s.astype(np.float64))
    assert np.array_equal(e, np.round(e))
    nz = amax > 0
    assert np.all(amax[nz] / s[nz] <= 448) and np.all(amax[nz] / s[nz] > 224)
    assert s[1, 7] == 1.0 and np.all(q[1, 7] == 0)
    # q[n, k] encodes w[k, n] (the transposed, K-contiguous layout), each within half a step
    d = oracle.dequantize_fp8(q, s, np.float32).astype(np.float64)
    wf = w.astype(np.float64)
    step = np.where(np.abs(wf) / s[:, None, :] < 2.0 ** -6, 2.0 ** -9, 2.0 ** (np.floor(np.log2(np.maximum(np.abs(wf) / s[:, None, :], 2.0 ** -6))) - 3))
    assert np.all(np.abs(d - wf) <= 0.5 * step * s[:, None, :] * (1 + 1e-12))
    # values already on the grid come back exactly
    g = oracle.dequantize_fp8(q, s, np.float32)
    q2, s2 = oracle.quantize_fp8(g)
    assert np.array_equal(q2, q) and np.array_equal(s2, s)
