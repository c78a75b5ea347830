"""Seeded small-shape fuzz of the whole block against the CPU oracle, through the C ABI.

A fixed list of cases drawn once from a seeded generator: T in [0, 300], E in [1, 64],
k in [1, min(E, 16)], d and I multiples of 8 or of 64, a shared expert or none, renormalisation
on or off, a router bias or none, bf16 or fp32. Every token is compared (the comparison rule of
moe_testlib); pytest -x stops at the first failing case, whose id and shape are printed first.
"""
import numpy as np
import pytest

import synthetic as syn
from moe_testlib import compare, device_from_host, host_inputs, oracle_full, run_forward, to_host

pytestmark = pytest.mark.gpu


def fuzz_cases(n=48, seed=20261203):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        T = int(rng.integers(0, 301)) if i % 16 else 0 if i == 0 else int(rng.integers(1, 4))
        E = int(rng.integers(1, 65))
        k = int(rng.integers(1, min(E, 16) + 1))
        unit = 8 if rng.random() < 0.5 else 64
        d = unit * int(rng.integers(1, 1024 // unit + 1))
        I = unit * int(rng.integers(1, 512 // unit + 1))
        Is = 0 if rng.random() < 0.25 else unit * int(rng.integers(1, 512 // unit + 1))
        dtype = syn.F32 if rng.random() < 0.2 else syn.BF16
        renorm = int(rng.random() < 0.7)
        bias = bool(rng.random() < 0.4)
        cases.append(("fuzz_%02d" % i, T, d, E, k, I, Is, dtype, renorm, bias, 100 + i))
    return cases


CASES = fuzz_cases()


def test_fuzz_list_spans_the_stated_ranges():
    T = [c[1] for c in CASES]
    assert min(T) == 0 and max(T) <= 300
    assert {c[3] for c in CASES} >= {1} or min(c[3] for c in CASES) <= 4
    assert all(1 <= c[4] <= min(c[3], 16) for c in CASES)
    assert all(c[2] % 8 == 0 and c[5] % 8 == 0 and c[6] % 8 == 0 for c in CASES)
    assert {c[7] for c in CASES} == {syn.F32, syn.BF16} and {c[8] for c in CASES} == {0, 1}
    assert {c[9] for c in CASES} == {False, True} and any(c[6] == 0 for c in CASES)


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_fuzz_case(case):
    import torch
    import sparse_mixture_experts_softmax_amd as moe
    name, T, d, E, k, I, Is, dtype, renorm, with_bias, seed = case
    cfg = syn.MoEConfig(name, T=T, d=d, E=E, k=k, I=I, Is=Is, dtype=dtype, renorm=renorm, seed=seed)
    print("case", name, cfg, "bias", with_bias, flush=True)
    assert torch.cuda.is_available()
    moe.load_library()
    h = host_inputs(cfg)
    if with_bias:
        h["bias"] = (np.random.default_rng(seed).standard_normal(E) * 0.5).astype(np.float32)
    dev = device_from_host(h, cfg)
    out, idx, w, gap = run_forward(dev, cfg)
    torch.cuda.synchronize()
    if T == 0:
        assert out.shape == (0, d)
        return
    ref_out, ref_idx, ref_w, ref_gap = oracle_full(h, cfg)
    st = compare(cfg, to_host(out), to_host(idx), to_host(w), ref_out, ref_idx, ref_w, ref_gap, name)
    print(name, st, flush=True)
