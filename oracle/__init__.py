"""CPU oracle for the sparse MoE block forward pass -- TEST INFRASTRUCTURE ONLY.

Only the test suite, ``__graft_entry__.smoke()`` and the benchmark's ``cpu_baseline`` leg may
import this package. It is the plain per-token definition in C with double accumulation
(``moe_oracle.c`` states each step and the passage it follows) behind a ctypes wrapper, and it
shares no code with the GPU library.

Arrays are numpy: float32 for fp32 data, uint16 bf16 bit patterns for bf16 data.
"""
import ctypes
import os

import numpy as np

from . import build as _build

F32, BF16 = 0, 1

_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        lib = ctypes.CDLL(_build.LIB)
        p, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
        lib.moe_oracle_router.argtypes = [i64, i32, i32, i32, i32, i32, p, p, p, p, p, p, p]
        lib.moe_oracle_router.restype = ctypes.c_int
        lib.moe_oracle_forward.argtypes = [i64, i32, i32, i32, i32, i32, i32, i32, p, p, p,
                                           p, p, p, p, p, p, p, p, p, p]
        lib.moe_oracle_forward.restype = ctypes.c_int
        lib.moe_oracle_rmsnorm.argtypes = [i64, i32, i32, p, p, ctypes.c_double, p]
        lib.moe_oracle_rmsnorm.restype = ctypes.c_int
        lib.moe_oracle_expert_rows.argtypes = [i64, i32, i32, i32, p, p, p, p, p, p]
        lib.moe_oracle_expert_rows.restype = ctypes.c_int
        lib.moe_oracle_threads.argtypes = []
        lib.moe_oracle_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def _dtype_of(a):
    a = np.asarray(a)
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    raise TypeError("oracle arrays are float32 or uint16 (bf16 bits), got %s" % a.dtype)


def _c(a, dt):
    return np.ascontiguousarray(a, dtype=dt)


def router(x, w_router, k, renorm=True, bias=None):
    """Router, top-k and routing weights.

    Returns (topk_idx int32 [T,k] by descending logit, topk_w float64 [T,k], gap float64 [T],
    logits float32 [T,E])."""
    dt = _dtype_of(x)
    x = _c(x, np.float32 if dt == F32 else np.uint16)
    w_router = _c(w_router, np.float32)
    T, d = x.shape
    E = w_router.shape[1]
    assert w_router.shape == (d, E)
    b = None if bias is None else _c(bias, np.float32)
    idx = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float64)
    gap = np.empty(T, np.float64)
    logits = np.empty((T, E), np.float32)
    rc = _load().moe_oracle_router(T, d, E, k, int(bool(renorm)), dt, x.ctypes.data, w_router.ctypes.data,
                                   None if b is None else b.ctypes.data, logits.ctypes.data, idx.ctypes.data,
                                   w.ctypes.data, gap.ctypes.data)
    if rc != 0:
        raise RuntimeError("moe_oracle_router failed: %d" % rc)
    return idx, w, gap, logits


def forward(x, w_router, wg, wu, wd, wg_s, wu_s, wd_s, k, renorm=True, bias=None):
    """Whole MoE block for every row of x.

    wg, wu, wd: either full arrays [E,d,I] / [E,I,d] or sequences of E per-expert 2-D arrays where
    an entry may be None when no token of x selects that expert. wg_s/wu_s/wd_s: shared expert
    ([d,Is], [d,Is], [Is,d]) or None for no shared expert.

    Returns (out float64 [T,d], topk_idx, topk_w, gap)."""
    dt = _dtype_of(x)
    npdt = np.float32 if dt == F32 else np.uint16
    x = _c(x, npdt)
    w_router = _c(w_router, np.float32)
    T, d = x.shape
    E = w_router.shape[1]
    keep = []

    def per_expert(w):
        ptrs = (ctypes.c_void_p * E)()
        for e in range(E):
            m = w[e]
            if m is None:
                ptrs[e] = None
            else:
                m = _c(m, npdt)
                keep.append(m)
                ptrs[e] = m.ctypes.data
        return ptrs

    I = next(m for m in wg if m is not None).shape[1]
    pg, pu, pd = per_expert(wg), per_expert(wu), per_expert(wd)
    if wg_s is None:
        Is, sg, su, sd = 0, None, None, None
    else:
        wg_s, wu_s, wd_s = _c(wg_s, npdt), _c(wu_s, npdt), _c(wd_s, npdt)
        Is = wg_s.shape[1]
        assert wg_s.shape == (d, Is) and wu_s.shape == (d, Is) and wd_s.shape == (Is, d)
        sg, su, sd = wg_s.ctypes.data, wu_s.ctypes.data, wd_s.ctypes.data
    b = None if bias is None else _c(bias, np.float32)
    out = np.empty((T, d), np.float64)
    idx = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float64)
    gap = np.empty(T, np.float64)
    rc = _load().moe_oracle_forward(T, d, E, k, I, Is, int(bool(renorm)), dt, x.ctypes.data, w_router.ctypes.data,
                                    None if b is None else b.ctypes.data, pg, pu, pd, sg, su, sd,
                                    out.ctypes.data, idx.ctypes.data, w.ctypes.data, gap.ctypes.data)
    if rc != 0:
        raise RuntimeError("moe_oracle_forward failed: %d" % rc)
    return out, idx, w, gap


def expert_rows(x, rows, experts):
    """One expert output per (row, expert) pair, unweighted: y[p] = (silu(x_r Wg) * (x_r Wu)) Wd for
    r = rows[p] and experts[p] = (Wg [d,n], Wu [d,n], Wd [n,d]). Returns float64 [len(rows), d]."""
    dt = _dtype_of(x)
    npdt = np.float32 if dt == F32 else np.uint16
    x = _c(x, npdt)
    T, d = x.shape
    rows = _c(rows, np.int64)
    npairs = len(rows)
    y = np.empty((npairs, d), np.float64)
    if npairs == 0:
        return y
    assert rows.min() >= 0 and rows.max() < T
    keep = {}

    def ptrs(which):
        arr = (ctypes.c_void_p * npairs)()
        for i, ex in enumerate(experts):
            m = ex[which]
            key = (id(m), which)
            if key not in keep:
                keep[key] = _c(m, npdt)
            arr[i] = keep[key].ctypes.data
        return arr

    n = experts[0][0].shape[1]
    for ex in experts:
        assert ex[0].shape == (d, n) and ex[1].shape == (d, n) and ex[2].shape == (n, d)
    rc = _load().moe_oracle_expert_rows(npairs, d, n, dt, x.ctypes.data, rows.ctypes.data, ptrs(0), ptrs(1), ptrs(2),
                                        y.ctypes.data)
    if rc != 0:
        raise RuntimeError("moe_oracle_expert_rows failed: %d" % rc)
    return y


def forward_by_expert(x, w_router, k, load_expert, shared=None, renorm=True, bias=None, batch=16):
    """The whole block, as forward() defines it, for inputs whose expert weights need not all be in
    host memory at once: out_t = sum over the token's kept experts j of w_tj y_j(x_t), plus the
    shared expert's output s(x_t). The routing is router()'s; the experts the tokens select are
    visited `batch` at a time in ascending index, load_expert(e) returning (Wg [d,I], Wu [d,I],
    Wd [I,d]), and each adds its weighted outputs to its tokens' rows (so a token's k terms are summed
    in ascending expert index rather than in descending logit; the sum is in double either way).
    shared: (Wg_s, Wu_s, Wd_s) or None.

    Returns (out float64 [T,d], topk_idx, topk_w, gap) like forward()."""
    idx, w, gap, _ = router(x, w_router, k, renorm=renorm, bias=bias)
    T, d = np.asarray(x).shape
    out = np.zeros((T, d), np.float64)
    needed = np.unique(idx)
    for b0 in range(0, len(needed), batch):
        group = needed[b0:b0 + batch]
        weights = {int(e): load_expert(int(e)) for e in group}
        tt, jj = np.nonzero(np.isin(idx, group))
        y = expert_rows(x, tt, [weights[int(e)] for e in idx[tt, jj]])
        np.add.at(out, tt, w[tt, jj][:, None] * y)
        del weights
    if shared is not None:
        out += expert_rows(x, np.arange(T), [shared] * T)
    return out, idx, w, gap


def router_stats(logits, topk_idx, E):
    """Router statistics for load balancing, per expert e (the configuration listing on the
    Qwen3.8-Max architecture page sets router_aux_loss_coef; the loss itself is not on the
    pages): the number of tokens that select e, and the mean over tokens of e's probability
    under the softmax over all E fp32 logits (the explorer page's router section: one
    probability per expert), in double.

    logits float32 [T,E] (from router(), bias included); topk_idx int32 [T,k].
    Returns (counts int64 [E], prob_mean float64 [E])."""
    lg = np.asarray(logits, dtype=np.float64)
    T = lg.shape[0]
    counts = np.bincount(np.asarray(topk_idx, dtype=np.int64).reshape(-1), minlength=E)
    if T == 0:
        return counts, np.zeros(E)
    p = np.exp(lg - lg.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    return counts, p.sum(axis=0) / T


# ----------------------------------------------------------------------------------------------
# FP8 expert weights (the Fondations page names FP8 among the formats; no scheme is given, so the
# chosen one is stated here): OCP e4m3 (4 exponent bits, bias 7, 3 mantissa bits, no infinities,
# largest finite 448), one power-of-two scale per output column, round to nearest even.
# ----------------------------------------------------------------------------------------------
E4M3_MAX = 448.0


def e4m3_value(code):
    """Value of an OCP e4m3 byte (float64; NaN for the two NaN codes)."""
    c = np.asarray(code, dtype=np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 15
    m = (c & 7).astype(np.float64)
    v = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    v = np.where((e == 15) & ((c & 7) == 7), np.nan, v)
    return s * v


def e4m3_round(v):
    """Nearest e4m3 code of each value (|v| <= 448), ties to the even code, found by search over
    the 127 non-negative finite values in double."""
    v = np.asarray(v, dtype=np.float64)
    assert np.all(np.abs(v) <= E4M3_MAX), "outside the e4m3 range"
    pos = e4m3_value(np.arange(127))          # codes 0 .. 126, ascending values
    a = np.abs(v)
    hi = np.searchsorted(pos, a, side="left")  # first code with value >= a
    hi = np.minimum(hi, 126)
    lo = np.maximum(hi - 1, 0)
    dlo = a - pos[lo]
    dhi = pos[hi] - a
    pick = np.where(dlo < dhi, lo, np.where(dhi < dlo, hi, np.where(lo % 2 == 0, lo, hi)))
    pick = np.where(a == pos[hi], hi, pick)
    return (pick | np.where((v < 0) & (pick != 0), 0x80, 0)).astype(np.uint8)


def quantize_fp8(w):
    """Quantise weights w [..., K, N] (float32, or bf16 bits as uint16) stored N-contiguous.

    Per output column n: scale s_n = 2^ceil(log2(max_k |w[k, n]| / 448)) (1 for an all-zero
    column), q = e4m3_round(w / s_n) -- the division by a power of two is exact. Returns
    (q uint8 [..., N, K] with K contiguous, s float32 [..., N])."""
    wf = widen(w)
    amax = np.abs(wf).max(axis=-2)                            # [..., N]
    ex = np.ceil(np.log2(np.where(amax > 0, amax, 1.0) / E4M3_MAX))
    # exact guard: the smallest power of two with amax / s <= 448
    ex = np.where(amax / np.exp2(ex) > E4M3_MAX, ex + 1, ex)
    ex = np.where(amax / np.exp2(ex - 1) <= E4M3_MAX, ex - 1, ex)
    scale = np.where(amax > 0, np.exp2(ex), 1.0)
    q = e4m3_round(wf / scale[..., None, :])
    return np.ascontiguousarray(np.swapaxes(q, -1, -2)), scale.astype(np.float32)


def dequantize_fp8(q, s, dtype=np.uint16):
    """The weights q, s stand for, back in the N-contiguous [..., K, N] layout: exact in bf16
    (4 significant bits times a power of two), returned as bf16 bits (or float32)."""
    v = e4m3_value(q) * np.asarray(s, dtype=np.float64)[..., :, None]   # [..., N, K]
    v = np.ascontiguousarray(np.swapaxes(v, -1, -2)).astype(np.float32)
    if dtype == np.float32:
        return v
    b = v.view(np.uint32)
    assert np.all(b & 0xFFFF == 0), "dequantised weight not exact in bf16"
    return (b >> 16).astype(np.uint16)


RMS_NORM_EPS = 1e-6


def rmsnorm(x, gamma, eps=RMS_NORM_EPS):
    """Zero-centred RMSNorm of each row: x / sqrt(mean(x^2) + eps) * (1 + gamma), in double,
    rounded once to the element type of x (float32, or bf16 bits by round-to-nearest-even)."""
    dt = _dtype_of(x)
    npdt = np.float32 if dt == F32 else np.uint16
    x = _c(x, npdt)
    gamma = _c(gamma, npdt)
    T, d = x.shape
    assert gamma.shape == (d,)
    h = np.empty((T, d), npdt)
    rc = _load().moe_oracle_rmsnorm(T, d, dt, x.ctypes.data, gamma.ctypes.data, float(eps), h.ctypes.data)
    if rc != 0:
        raise RuntimeError("moe_oracle_rmsnorm failed: %d" % rc)
    return h


def widen(a):
    """float32 or bf16-bit array as float64."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def block_forward(x, gamma, w_router, wg, wu, wd, wg_s, wu_s, wd_s, k, renorm=True, bias=None,
                  eps=RMS_NORM_EPS):
    """The MoE block between its neighbours: out = x + MoE(rmsnorm(x)); the router and the
    experts both see the normalised rows, stored in the element type of x.

    Returns (out float64 [T,d], topk_idx, topk_w, gap, h)."""
    h = rmsnorm(x, gamma, eps)
    moe_out, idx, w, gap = forward(h, w_router, wg, wu, wd, wg_s, wu_s, wd_s, k, renorm=renorm, bias=bias)
    return widen(x) + moe_out, idx, w, gap, h


def threads():
    """Host threads the oracle's parallel loops use."""
    return int(_load().moe_oracle_threads())


TIE_BAND = 1e-5


def flagged(gap):
    """Tokens whose k-th and (k+1)-th fp32 logits are closer than the tie band; their expert set
    is not unique to within rounding, so they are excluded from index and output comparisons."""
    return np.asarray(gap) < TIE_BAND
