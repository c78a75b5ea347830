"""Seeded synthetic inputs for the sparse MoE block, shared by the CPU oracle and the GPU path.

This module holds no arithmetic of the MoE block itself. It provides:

* the five workload presets (shapes, dtypes, seeds) the tests and the benchmark use;
* host and device fills of any tensor (or any expert's slice of one) from the counter-based
  generator defined in ``synth_core.h`` -- the host fill (C) and the device fill (HIP) are
  bit-identical, so the oracle never needs data copied back from the GPU;
* the per-expert router bias that skews expert loads towards a Zipf law (skew workload).

Tensor ids: x 0, router W_r 1, W_g 2, W_u 3, W_d 4, shared W_g 5, W_u 6, W_d 7.
Standard deviations: x 1; every weight 1/sqrt(fan_in) with fan_in = d for W_r, W_g, W_u and the
shared W_g, W_u, and fan_in = I (resp. I_shared) for W_d (resp. shared W_d).
"""
import ctypes
import dataclasses
import math
import os

import numpy as np

from . import build as _build

HERE = os.path.dirname(os.path.abspath(__file__))

TID_X, TID_WR, TID_WG, TID_WU, TID_WD, TID_WGS, TID_WUS, TID_WDS, TID_GAMMA = range(9)

F32, BF16 = 0, 1


@dataclasses.dataclass(frozen=True)
class MoEConfig:
    """One MoE-layer workload. Field names follow the model configuration's vocabulary."""

    name: str
    T: int  # tokens in the batch
    d: int  # hidden_size
    E: int  # num_experts
    k: int  # num_experts_per_tok
    I: int  # moe_intermediate_size
    Is: int  # shared_expert_intermediate_size (0 = no shared expert)
    dtype: int  # F32 or BF16 for x, expert weights and out; the router is always fp32
    renorm: int = 1
    seed: int = 0
    zipf_alpha: float = 0.0  # > 0: add a per-expert router bias so loads follow Zipf(alpha)

    def with_(self, **kw):
        return dataclasses.replace(self, **kw)

    @property
    def dtype_name(self):
        return "f32" if self.dtype == F32 else "bf16"


CONFIGS = {
    "tiny": MoEConfig("tiny", T=64, d=256, E=16, k=2, I=128, Is=128, dtype=F32),
    "mid": MoEConfig("mid", T=4096, d=2048, E=256, k=8, I=512, Is=512, dtype=BF16),
    "decode": MoEConfig("decode", T=32, d=8192, E=512, k=10, I=2048, Is=2048, dtype=BF16),
    "prefill": MoEConfig("prefill", T=16384, d=8192, E=512, k=10, I=2048, Is=2048, dtype=BF16),
    "skew": MoEConfig("skew", T=8192, d=8192, E=512, k=10, I=2048, Is=2048, dtype=BF16,
                      zipf_alpha=1.2),
}


def sigma_of(cfg, tid):
    if tid == TID_X:
        return 1.0
    if tid in (TID_WR, TID_WG, TID_WU, TID_WGS, TID_WUS):
        return 1.0 / math.sqrt(cfg.d)
    if tid == TID_WD:
        return 1.0 / math.sqrt(cfg.I)
    if tid == TID_WDS:
        return 1.0 / math.sqrt(cfg.Is)
    if tid == TID_GAMMA:
        return GAMMA_SIGMA
    raise ValueError(tid)


# zero-centred norm scale gamma (the scale is 1 + gamma): small spread around its zero start
GAMMA_SIGMA = 0.1


def host_gamma(cfg):
    """The norm scale parameter gamma [d] in the config's dtype."""
    return host_fill(cfg.d, cfg.dtype, cfg.seed, TID_GAMMA, GAMMA_SIGMA)


def device_gamma(cfg, device="cuda"):
    import torch
    tdt = torch.float32 if cfg.dtype == F32 else torch.bfloat16
    return device_fill(torch.empty(cfg.d, dtype=tdt, device=device), cfg.seed, TID_GAMMA, GAMMA_SIGMA)


# ----------------------------------------------------------------------------------------------
# native libraries
# ----------------------------------------------------------------------------------------------
_host = None
_dev = None
_table = None
_dev_tables = {}


def _load_host():
    global _host
    if _host is None:
        if not os.path.exists(_build.HOST_LIB):
            _build.build_host()
        lib = ctypes.CDLL(_build.HOST_LIB)
        lib.synth_build_table.argtypes = [ctypes.c_void_p]
        lib.synth_build_table.restype = None
        lib.synth_fill_host.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_uint64, ctypes.c_uint64,
                                        ctypes.c_uint64, ctypes.c_uint32, ctypes.c_double, ctypes.c_void_p]
        lib.synth_fill_host.restype = None
        lib.synth_fill_rows_host.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_int64,
                                             ctypes.c_int64, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint32,
                                             ctypes.c_double, ctypes.c_void_p]
        lib.synth_fill_rows_host.restype = None
        _host = lib
    return _host


def _load_dev():
    global _dev
    if _dev is None:
        if not os.path.exists(_build.DEV_LIB):
            _build.build_device()
        lib = ctypes.CDLL(_build.DEV_LIB)
        lib.synth_fill_device.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_uint64, ctypes.c_uint64,
                                          ctypes.c_uint64, ctypes.c_uint32, ctypes.c_double, ctypes.c_void_p,
                                          ctypes.c_void_p]
        lib.synth_fill_device.restype = ctypes.c_int
        _dev = lib
    return _dev


def quantile_table():
    """The 65537-entry standard-normal quantile table (float64), built once per process."""
    global _table
    if _table is None:
        t = np.empty(65537, dtype=np.float64)
        _load_host().synth_build_table(t.ctypes.data)
        _table = t
    return _table


# ----------------------------------------------------------------------------------------------
# host fills
# ----------------------------------------------------------------------------------------------
def host_fill(n, dtype, seed, tid, sigma, offset=0):
    """Elements [offset, offset+n) of tensor (seed, tid): float32 array, or uint16 bf16 bits."""
    out = np.empty(n, dtype=np.float32 if dtype == F32 else np.uint16)
    if n:
        _load_host().synth_fill_host(out.ctypes.data, dtype, n, offset, seed, tid, sigma,
                                     quantile_table().ctypes.data)
    return out


def host_rows(rows, ncols, dtype, seed, tid, sigma, base=0):
    """Rows `rows` (any order) of a row-major [*, ncols] tensor starting at flat index base."""
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    out = np.empty((len(rows), ncols), dtype=np.float32 if dtype == F32 else np.uint16)
    if len(rows):
        _load_host().synth_fill_rows_host(out.ctypes.data, dtype, rows.ctypes.data, len(rows), ncols, base,
                                          seed, tid, sigma, quantile_table().ctypes.data)
    return out


def bf16_bits_to_f32(a):
    """Exact widening of bf16 bit patterns (uint16) to float32."""
    return (np.asarray(a, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def host_x(cfg, rows=None):
    """x [T, d] (or the given token rows) in the config's dtype."""
    if rows is None:
        return host_fill(cfg.T * cfg.d, cfg.dtype, cfg.seed, TID_X, 1.0).reshape(cfg.T, cfg.d)
    return host_rows(rows, cfg.d, cfg.dtype, cfg.seed, TID_X, 1.0)


def host_router(cfg):
    """Router weight W_r [d, E], always fp32."""
    return host_fill(cfg.d * cfg.E, F32, cfg.seed, TID_WR, sigma_of(cfg, TID_WR)).reshape(cfg.d, cfg.E)


def host_expert(cfg, e):
    """(W_g[e] [d, I], W_u[e] [d, I], W_d[e] [I, d]) in the config's dtype."""
    n = cfg.d * cfg.I
    wg = host_fill(n, cfg.dtype, cfg.seed, TID_WG, sigma_of(cfg, TID_WG), offset=e * n).reshape(cfg.d, cfg.I)
    wu = host_fill(n, cfg.dtype, cfg.seed, TID_WU, sigma_of(cfg, TID_WU), offset=e * n).reshape(cfg.d, cfg.I)
    wd = host_fill(n, cfg.dtype, cfg.seed, TID_WD, sigma_of(cfg, TID_WD), offset=e * n).reshape(cfg.I, cfg.d)
    return wg, wu, wd


def host_shared(cfg):
    """(W_g_s [d, Is], W_u_s [d, Is], W_d_s [Is, d]) in the config's dtype, or Nones if Is == 0."""
    if cfg.Is == 0:
        return None, None, None
    n = cfg.d * cfg.Is
    wg = host_fill(n, cfg.dtype, cfg.seed, TID_WGS, sigma_of(cfg, TID_WGS)).reshape(cfg.d, cfg.Is)
    wu = host_fill(n, cfg.dtype, cfg.seed, TID_WUS, sigma_of(cfg, TID_WUS)).reshape(cfg.d, cfg.Is)
    wd = host_fill(n, cfg.dtype, cfg.seed, TID_WDS, sigma_of(cfg, TID_WDS)).reshape(cfg.Is, cfg.d)
    return wg, wu, wd


def host_all_experts(cfg):
    """Full W_g, W_u [E, d, I] and W_d [E, I, d] (small configs only)."""
    n = cfg.E * cfg.d * cfg.I
    wg = host_fill(n, cfg.dtype, cfg.seed, TID_WG, sigma_of(cfg, TID_WG)).reshape(cfg.E, cfg.d, cfg.I)
    wu = host_fill(n, cfg.dtype, cfg.seed, TID_WU, sigma_of(cfg, TID_WU)).reshape(cfg.E, cfg.d, cfg.I)
    wd = host_fill(n, cfg.dtype, cfg.seed, TID_WD, sigma_of(cfg, TID_WD)).reshape(cfg.E, cfg.I, cfg.d)
    return wg, wu, wd


# ----------------------------------------------------------------------------------------------
# device fills (torch tensors are used only as device memory)
# ----------------------------------------------------------------------------------------------
def _dev_table(device):
    import torch
    key = str(device)
    if key not in _dev_tables:
        _dev_tables[key] = torch.from_numpy(quantile_table()).to(device)
    return _dev_tables[key]


def device_fill(t, seed, tid, sigma, offset=0):
    """Fill a contiguous float32 or bfloat16 CUDA tensor with elements [offset, offset+numel)."""
    import torch
    assert t.is_cuda and t.is_contiguous()
    if t.dtype == torch.float32:
        dt = F32
    elif t.dtype == torch.bfloat16:
        dt = BF16
    else:
        raise TypeError(t.dtype)
    q = _dev_table(t.device)
    stream = torch.cuda.current_stream(t.device).cuda_stream
    rc = _load_dev().synth_fill_device(t.data_ptr(), dt, t.numel(), offset, seed, tid, sigma, q.data_ptr(),
                                       stream)
    if rc != 0:
        raise RuntimeError("synth_fill_device failed with hip error %d" % rc)
    return t


def device_inputs(cfg, device="cuda", with_x=True):
    """All layer inputs as device tensors: dict with x, w_router, bias, wg, wu, wd, wg_s, wu_s, wd_s."""
    import torch
    tdt = torch.float32 if cfg.dtype == F32 else torch.bfloat16
    d, E, I, Is = cfg.d, cfg.E, cfg.I, cfg.Is
    out = {}
    if with_x:
        out["x"] = device_fill(torch.empty(cfg.T, d, dtype=tdt, device=device), cfg.seed, TID_X, 1.0)
    out["w_router"] = device_fill(torch.empty(d, E, dtype=torch.float32, device=device), cfg.seed, TID_WR,
                                  sigma_of(cfg, TID_WR))
    out["wg"] = device_fill(torch.empty(E, d, I, dtype=tdt, device=device), cfg.seed, TID_WG, sigma_of(cfg, TID_WG))
    out["wu"] = device_fill(torch.empty(E, d, I, dtype=tdt, device=device), cfg.seed, TID_WU, sigma_of(cfg, TID_WU))
    out["wd"] = device_fill(torch.empty(E, I, d, dtype=tdt, device=device), cfg.seed, TID_WD, sigma_of(cfg, TID_WD))
    if Is > 0:
        out["wg_s"] = device_fill(torch.empty(d, Is, dtype=tdt, device=device), cfg.seed, TID_WGS,
                                  sigma_of(cfg, TID_WGS))
        out["wu_s"] = device_fill(torch.empty(d, Is, dtype=tdt, device=device), cfg.seed, TID_WUS,
                                  sigma_of(cfg, TID_WUS))
        out["wd_s"] = device_fill(torch.empty(Is, d, dtype=tdt, device=device), cfg.seed, TID_WDS,
                                  sigma_of(cfg, TID_WDS))
    else:
        out["wg_s"] = out["wu_s"] = out["wd_s"] = None
    b = router_bias(cfg)
    out["bias"] = None if b is None else torch.from_numpy(b).to(device)
    return out


# ----------------------------------------------------------------------------------------------
# skewed routing: per-expert router bias giving Zipf expert loads
# ----------------------------------------------------------------------------------------------
def zipf_targets(T, E, k, alpha):
    """Expected load of the expert of popularity rank r (= index + 1): proportional to r^-alpha,
    water-filled so that no expert exceeds T tokens and the loads sum to T*k."""
    w = np.arange(1, E + 1, dtype=np.float64) ** (-alpha)
    capped = np.zeros(E, dtype=bool)
    L = np.zeros(E)
    while True:
        free = ~capped
        rem = T * k - T * capped.sum()
        L[free] = rem * w[free] / w[free].sum()
        L[capped] = T
        over = free & (L > T)
        if not over.any():
            return L
        capped |= over


_bias_cache = {}


def router_bias(cfg, iters=30, mc_seed=20240601):
    """Per-expert fp32 router bias for Zipf-skewed loads, or None when cfg.zipf_alpha == 0.

    Model of the synthetic inputs: a token's logit for expert e is s_t * sigma_e * z with z ~ N(0, 1)
    independent across experts and tokens, sigma_e = |W_r[:, e]| (the generated router column's
    norm) and s_t = |x_t| / sqrt(d). If every token kept exactly the experts above one common
    threshold tau, expert e's share of tokens would be Q(tau - b_e), so the bias starts at
    b_e = Phi^-1(L_e / T) for target load L_e; experts whose target is every token get +10.
    Monte Carlo refinement on 4*T model tokens then moves each bias by the log-ratio of target to
    simulated load divided by the local sensitivity d ln(load)/d b (the normal hazard rate), damped."""
    if cfg.zipf_alpha <= 0:
        return None
    key = (cfg.T, cfg.d, cfg.E, cfg.k, cfg.zipf_alpha, cfg.seed)
    if key in _bias_cache:
        return _bias_cache[key]
    from scipy.stats import norm

    T, E, k = cfg.T, cfg.E, cfg.k
    L = zipf_targets(T, E, k, cfg.zipf_alpha)
    capped = L >= T * (1 - 1e-12)
    p = np.clip(L / T, 1e-9, 1 - 1e-9)
    b = norm.ppf(p)
    b[capped] = 10.0
    sigma = np.sqrt((host_router(cfg).astype(np.float64) ** 2).sum(axis=0))
    rng = np.random.default_rng(mc_seed)
    M = 4 * T
    s = np.sqrt(rng.chisquare(cfg.d, size=(M, 1)) / cfg.d)
    Z = (rng.standard_normal((M, E)) * sigma[None, :] * s).astype(np.float32)
    for _ in range(iters):
        sel = np.argpartition(-(Z + b.astype(np.float32)), k - 1, axis=1)[:, :k]
        load = np.bincount(sel.ravel(), minlength=E) * (T / M)
        q = np.clip(load / T, 1e-6, 1 - 1e-6)
        zq = norm.isf(q)
        hazard = norm.pdf(zq) / q
        step = 0.7 * np.log(L / np.maximum(load, 0.25)) / np.maximum(hazard, 0.2)
        b[~capped] += step[~capped]
    out = b.astype(np.float32)
    _bias_cache[key] = out
    return out
