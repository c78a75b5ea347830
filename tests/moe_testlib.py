"""Helpers for the GPU parity tests: inputs, oracle references on token samples, comparisons.

The comparison rule: expert index sets must match exactly except for tokens the oracle flags
(k-th and (k+1)-th fp32 logits closer than 1e-5); outputs must satisfy
max|out - ref| <= tol * max|ref| over the non-flagged tokens, tol = 2e-2 for bf16 and 1e-5 for fp32.
"""
import numpy as np

import oracle
import synthetic as syn

TOL = {syn.F32: 1e-5, syn.BF16: 2e-2}
WEIGHT_ATOL = 1e-5
RESULTS = []  # (label, max relative error, tokens checked, tokens flagged) of every comparison


def torch_dtype(cfg):
    import torch
    return torch.float32 if cfg.dtype == syn.F32 else torch.bfloat16


def to_device(a, dtype, device="cuda"):
    """numpy float32 or uint16 (bf16 bits) -> device tensor of the given torch dtype."""
    import torch
    if a is None:
        return None
    if a.dtype == np.uint16:
        assert dtype == torch.bfloat16
        return torch.from_numpy(a.view(np.int16).copy()).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device).to(dtype)


def to_host(t):
    """Device tensor -> numpy (bf16 returned as float32 values)."""
    import torch
    t = t.detach()
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.cpu().numpy()


def fp8_untile(q, N, K):
    """FP8 code tiles (moe.h layout: tile (n // 128) * (K // 32) + k // 32 of 4096 bytes; in a tile
    Q[n, k] at byte 32 r + 16 (h ^ ((r // 8) % 2)) + k % 16 with r = n % 128, h = (k % 32) // 16)
    back to plain codes [..., N, K]."""
    q = np.asarray(q).reshape(q.shape[:-3] + (-1,)) if q.ndim >= 3 else np.asarray(q)
    n = np.arange(N)[:, None]
    k = np.arange(K)[None, :]
    r, h = n % 128, (k % 32) // 16
    at = ((n // 128) * (K // 32) + k // 32) * 4096 + 32 * r + 16 * (h ^ ((r // 8) % 2)) + k % 16
    return q[..., at]


def host_inputs(cfg):
    """All inputs on the host (small configs): dict of numpy arrays in the config's dtype."""
    wg, wu, wd = syn.host_all_experts(cfg)
    wgs, wus, wds = syn.host_shared(cfg)
    return dict(x=syn.host_x(cfg), w_router=syn.host_router(cfg), bias=syn.router_bias(cfg), wg=wg, wu=wu, wd=wd,
                wg_s=wgs, wu_s=wus, wd_s=wds)


def device_from_host(h, cfg, device="cuda"):
    import torch
    dt = torch_dtype(cfg)
    out = {}
    for key, a in h.items():
        if a is None:
            out[key] = None
        elif key in ("w_router", "bias"):
            out[key] = to_device(a, torch.float32, device)
        else:
            out[key] = to_device(a, dt, device)
    return out


def run_forward(dev, cfg, ws=None):
    import sparse_mixture_experts_softmax_amd as moe
    return moe.moe_forward(dev["x"], dev["w_router"], dev["wg"], dev["wu"], dev["wd"], dev["wg_s"], dev["wu_s"],
                           dev["wd_s"], cfg.k, renormalize=bool(cfg.renorm), router_bias=dev["bias"],
                           return_routing=True, ws=ws)


def oracle_full(h, cfg):
    return oracle.forward(h["x"], h["w_router"], h["wg"], h["wu"], h["wd"], h["wg_s"], h["wu_s"], h["wd_s"], cfg.k,
                          renorm=bool(cfg.renorm), bias=h["bias"])


def coverage_tokens(idx, E, n_min, budget, seed, band=64):
    """Tokens to check against the oracle so that every 64-row band of every group's rows in the
    grouped GEMMs -- each routed expert's slots (tokens ascending, as the dispatch orders them)
    and the shared expert's T rows -- holds at least one checked row: every row tile, its first,
    middle and last (partial) ones alike, and every 32-row sub-tile pair of the waves in it.
    Greedy maximum coverage (each step takes the token adding the most uncovered bands; seeded
    tie-break), then seeded random tokens up to n_min. Returns (sorted tokens, covered fraction)."""
    T, k = idx.shape
    flat_e = idx.reshape(-1).astype(np.int64)
    flat_t = np.repeat(np.arange(T), k)
    order = np.lexsort((flat_t, flat_e))
    counts = np.bincount(flat_e, minlength=E)
    offs = np.concatenate([[0], np.cumsum(counts)])
    rank = np.empty(T * k, np.int64)
    rank[order] = np.arange(T * k) - offs[flat_e[order]]
    nb = (counts + band - 1) // band
    boff = np.concatenate([[0], np.cumsum(nb)])
    pid = np.concatenate([(boff[flat_e] + rank // band).reshape(T, k), (boff[E] + np.arange(T) // band)[:, None]],
                         axis=1)
    covered = np.zeros(boff[E] + (T + band - 1) // band, bool)
    rng = np.random.default_rng(seed)
    tie = rng.random(T) * 1e-3
    chosen = np.zeros(T, bool)
    while chosen.sum() < budget:
        gain = (~covered[pid]).sum(axis=1) + tie
        gain[chosen] = -1.0
        t = int(np.argmax(gain))
        if gain[t] < 1.0:
            break
        chosen[t] = True
        covered[pid[t]] = True
    rest = np.flatnonzero(~chosen)
    extra = max(0, min(n_min, T) - int(chosen.sum()))
    chosen[rng.choice(rest, size=extra, replace=False)] = True
    return np.flatnonzero(chosen), float(covered.mean())


def oracle_tokens(cfg, tokens):
    """The oracle on the given token rows of a configuration, visiting the selected experts a few at
    a time (each generated on the host when its turn comes), so that host memory stays bounded at
    the large shapes."""
    x = syn.host_x(cfg, rows=tokens)
    return oracle.forward_by_expert(x, syn.host_router(cfg), cfg.k, lambda e: syn.host_expert(cfg, e),
                                    shared=syn.host_shared(cfg) if cfg.Is else None, renorm=bool(cfg.renorm),
                                    bias=syn.router_bias(cfg), batch=16)


# final rounding of an output row to the element type, relative (half an ulp at bf16 / fp32)
OUT_ROUND = {syn.F32: 2.0 ** -24, syn.BF16: 2.0 ** -9}


def compare(cfg, out, idx, w, ref_out, ref_idx, ref_w, ref_gap, label="", residual=None):
    """Checks one set of GPU rows against the oracle's. Returns a stats dict.

    residual: the block's input rows (float64) when out = residual + MoE(...). The MoE part keeps
    its bound, tol * max|ref - residual|, and each element also gets the rounding of its own
    magnitude once the residual is added, OUT_ROUND * |ref|."""
    out = np.asarray(out, dtype=np.float64)
    idx = np.asarray(idx)
    w = np.asarray(w, dtype=np.float64)
    T, k = ref_idx.shape
    flagged = oracle.flagged(ref_gap)
    ok = ~flagged
    # validity everywhere
    assert idx.min() >= 0 and idx.max() < cfg.E, label
    assert all(len(set(r.tolist())) == k for r in idx), label + ": repeated expert in a token"
    if cfg.renorm:
        np.testing.assert_allclose(w.sum(axis=1), 1.0, atol=1e-5, err_msg=label)
    # exact expert sets on non-flagged tokens
    gi = np.sort(idx[ok], axis=1)
    ri = np.sort(ref_idx[ok], axis=1)
    bad = np.nonzero(np.any(gi != ri, axis=1))[0]
    assert bad.size == 0, "%s: %d token(s) with a different expert set, first %s" % (label, bad.size, bad[:5])
    # weights, matched by expert
    go = np.argsort(idx[ok], axis=1)
    ro = np.argsort(ref_idx[ok], axis=1)
    gw = np.take_along_axis(w[ok], go, axis=1)
    rw = np.take_along_axis(ref_w[ok], ro, axis=1)
    werr = float(np.max(np.abs(gw - rw))) if gw.size else 0.0
    assert werr <= WEIGHT_ATOL, "%s: routing weight error %g" % (label, werr)
    # outputs
    tol = TOL[cfg.dtype]
    if residual is None:
        ref_max = float(np.max(np.abs(ref_out[ok]))) if ok.any() else 0.0
        err = float(np.max(np.abs(out[ok] - ref_out[ok]))) if ok.any() else 0.0
        assert err <= tol * ref_max, "%s: max|out-ref| = %g > %g * max|ref| = %g" % (label, err, tol, tol * ref_max)
    else:
        moe_ref = ref_out[ok] - np.asarray(residual, dtype=np.float64)[ok]
        ref_max = float(np.max(np.abs(moe_ref))) if ok.any() else 0.0
        diff = np.abs(out[ok] - ref_out[ok])
        bound = tol * ref_max + OUT_ROUND[cfg.dtype] * np.abs(ref_out[ok])
        err = float(np.max(diff)) if ok.any() else 0.0
        worst = float(np.max(diff - bound)) if ok.any() else 0.0
        assert worst <= 0.0, "%s: |out-ref| exceeds tol*max|moe ref| + rounding by %g" % (label, worst)
    RESULTS.append((label, err / ref_max if ref_max else 0.0, int(T), int(flagged.sum())))
    return dict(flagged=int(flagged.sum()), max_err=err, max_ref=ref_max, rel=err / ref_max if ref_max else 0.0,
                weight_err=werr)
