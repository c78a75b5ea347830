"""The C-ABI library loads on a machine without a GPU, exports every entry point include/moe.h
declares, and rejects bad arguments on the host before any HIP call."""
import ctypes
import os
import re

import pytest

import sparse_mixture_experts_softmax_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OK, INVALID, UNSUPPORTED, WORKSPACE = 0, 1, 2, 3


def declared_functions():
    src = open(os.path.join(ROOT, "include", "moe.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:moe_status|const char\s*\*)\s+(moe_\w+)\s*\(", src, flags=re.M)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("moe_router_topk", "moe_permute", "moe_grouped_ffn", "moe_combine", "moe_forward",
              "moe_workspace_size", "moe_status_string", "moe_last_error"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = moe.load_library()
    for n in declared_functions():
        assert hasattr(lib, n), n


def dims(**kw):
    base = dict(T=64, d=256, E=16, k=2, I=128, I_shared=128, dtype=moe.MOE_F32, renormalize=1)
    base.update(kw)
    return moe.MoeDims(**base)


def ws_status(dm):
    lib = moe.load_library()
    n = ctypes.c_size_t(0)
    st = lib.moe_workspace_size(ctypes.byref(dm), ctypes.byref(n))
    return st, n.value, lib.moe_last_error().decode()


@pytest.mark.parametrize("kw,status,needle", [
    (dict(T=-1), INVALID, "T"),
    (dict(E=0), INVALID, "E"),
    (dict(E=1025, k=2), UNSUPPORTED, "E"),
    (dict(k=0), INVALID, "k"),
    (dict(k=17, E=32), UNSUPPORTED, "k"),
    (dict(k=20, E=16), INVALID, "k"),
    (dict(d=12), INVALID, "d"),
    (dict(d=0), INVALID, "d"),
    (dict(I=100), INVALID, "I"),
    (dict(I_shared=4), INVALID, "I_shared"),
    (dict(dtype=2), INVALID, "dtype"),
    (dict(renormalize=2), INVALID, "renormalize"),
    (dict(T=(1 << 31) // 3 + 1, k=2), UNSUPPORTED, "int32"),
])
def test_dims_validation(kw, status, needle):
    st, _, msg = ws_status(dims(**kw))
    assert st == status
    assert needle in msg


def test_workspace_size_grows_with_tokens():
    sizes = [ws_status(dims(T=t))[1] for t in (0, 1, 64, 1000)]
    assert all(a < b for a, b in zip(sizes, sizes[1:]))
    assert ws_status(dims(T=0))[0] == OK
    # the large prefill shape: intermediates H and Y dominate
    st, n, _ = ws_status(dims(T=16384, d=8192, E=512, k=10, I=2048, I_shared=2048, dtype=moe.MOE_BF16))
    assert st == OK
    rows = 16384 * 11
    assert n >= rows * 2048 * 2 + rows * 8192 * 2


FAKE = 0x100000  # never dereferenced: every call below fails validation first


def forward_status(dm, **ptrs):
    lib = moe.load_library()
    p = dict(x=FAKE, w_router=FAKE, bias=None, wg=FAKE, wu=FAKE, wd=FAKE, wg_s=FAKE, wu_s=FAKE, wd_s=FAKE, out=FAKE,
             idx=None, w=None, gap=None, ws=FAKE, ws_bytes=1 << 40)
    p.update(ptrs)
    st = lib.moe_forward(ctypes.byref(dm), p["x"], p["w_router"], p["bias"], p["wg"], p["wu"], p["wd"], p["wg_s"],
                         p["wu_s"], p["wd_s"], p["out"], p["idx"], p["w"], p["gap"], p["ws"], p["ws_bytes"], None)
    return st, lib.moe_last_error().decode()


def test_forward_rejects_bad_pointers_and_workspace():
    dm = dims()
    assert forward_status(dm, x=None) == (INVALID, "x is NULL")
    st, msg = forward_status(dm, x=FAKE + 8)
    assert st == INVALID and "aligned" in msg
    st, msg = forward_status(dm, wd_s=None)
    assert st == INVALID and "wd_s" in msg
    st, msg = forward_status(dm, ws=None)
    assert st == WORKSPACE
    st, msg = forward_status(dm, ws_bytes=16)
    assert st == WORKSPACE and "needs" in msg
    st, msg = forward_status(dm, ws=FAKE + 64)
    assert st == WORKSPACE and "256" in msg


def test_forward_without_shared_expert_accepts_null_shared_weights():
    dm = dims(I_shared=0)
    st, msg = forward_status(dm, wg_s=None, wu_s=None, wd_s=None, ws=None)
    assert st == WORKSPACE  # got past the shared-weight checks


def test_zero_tokens_is_a_no_op():
    dm = dims(T=0)
    assert forward_status(dm, x=None, ws=None)[0] == OK


def test_status_strings():
    lib = moe.load_library()
    assert lib.moe_status_string(0) == b"MOE_OK"
    assert lib.moe_status_string(3) == b"MOE_ERR_WORKSPACE"


def test_python_binding_raises_with_detail():
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_workspace_size(dims(k=0))
    assert "MOE_ERR_INVALID_ARG" in str(ei.value)


@pytest.mark.parametrize("eps", [-1e-6, float("nan"), float("inf")])
def test_rmsnorm_and_block_reject_bad_eps(eps):
    import sparse_mixture_experts_softmax_amd as moe
    lib = moe.load_library()
    dims = moe.MoeDims(4, 64, 8, 2, 32, 0, moe.MOE_BF16, 1)
    rc = lib.moe_rmsnorm(ctypes.byref(dims), None, None, eps, None, None)
    assert rc == 1 and b"eps" in lib.moe_last_error()  # MOE_ERR_INVALID_ARG
    rc = lib.moe_forward_block(ctypes.byref(dims), None, None, eps, None, None, None, None, None, None, None, None,
                               None, None, None, None, None, 0, None)
    assert rc == 1 and b"eps" in lib.moe_last_error()  # MOE_ERR_INVALID_ARG


def test_rmsnorm_rejects_null_gamma():
    import sparse_mixture_experts_softmax_amd as moe
    lib = moe.load_library()
    dims = moe.MoeDims(4, 64, 8, 2, 32, 0, moe.MOE_BF16, 1)
    rc = lib.moe_rmsnorm(ctypes.byref(dims), ctypes.c_void_p(4096), None, 1e-6, ctypes.c_void_p(4096), None)
    assert rc == 1 and b"gamma" in lib.moe_last_error()  # MOE_ERR_INVALID_ARG


def test_fp8_forward_rejects_unsupported_shapes():
    import sparse_mixture_experts_softmax_amd as moe
    lib = moe.load_library()
    args = [None] * 20 + [0, None]
    for dims in (moe.MoeDims(4, 512, 8, 2, 256, 0, moe.MOE_F32, 1),    # fp32 activations
                 moe.MoeDims(4, 264, 8, 2, 256, 0, moe.MOE_BF16, 1),   # d % 256 != 0
                 moe.MoeDims(4, 512, 8, 2, 200, 0, moe.MOE_BF16, 1)):  # I % 128 != 0
        rc = lib.moe_forward_fp8(ctypes.byref(dims), *args)
        assert rc == 2 and b"FP8" in lib.moe_last_error()  # MOE_ERR_UNSUPPORTED


def test_fp8_quantiser_rejects_bad_arguments():
    import sparse_mixture_experts_softmax_amd as moe
    lib = moe.load_library()
    assert lib.moe_quantize_fp8(None, 7, 1, 16, 16, None, None, None) == 1
    assert lib.moe_quantize_fp8(None, moe.MOE_BF16, 1, 0, 16, None, None, None) == 1
    assert lib.moe_quantize_fp8(None, moe.MOE_BF16, 1, 16, 16, None, None, None) == 1  # null w
    assert lib.moe_quantize_fp8(None, moe.MOE_BF16, 0, 16, 16, None, None, None) == 0  # empty batch
    p = ctypes.c_void_p(FAKE)  # never dereferenced: the shape check fails first
    assert lib.moe_quantize_fp8(p, moe.MOE_BF16, 1, 48, 128, p, p, None) == UNSUPPORTED  # K % 32
    assert lib.moe_quantize_fp8(p, moe.MOE_BF16, 1, 64, 192, p, p, None) == UNSUPPORTED  # N % 128
    assert lib.moe_quantize_fp8(p, moe.MOE_BF16, 1, 64, 128, ctypes.c_void_p(FAKE + 8), p, None) == INVALID  # q align


def test_fp8_untile_is_a_permutation():
    from moe_testlib import fp8_untile
    import numpy as np
    N, K = 256, 96
    flat = np.arange(N * K, dtype=np.int64)
    u = fp8_untile(flat.reshape(N // 128, K // 32, 4096), N, K)
    assert u.shape == (N, K) and np.array_equal(np.sort(u.ravel()), flat)
    # each tile's column run is 32 contiguous bytes; within a tile, columns follow each other
    assert np.array_equal(np.sort(u[5, :32]), np.arange(5 * 32, 6 * 32))
    assert u[130, 40] // 4096 == 1 * (K // 32) + 1


def test_binding_argument_lists_match_the_header():
    # every ctypes argument list has as many entries as the C declaration has parameters
    import sparse_mixture_experts_softmax_amd as moe
    lib = moe.load_library()
    src = open(os.path.join(ROOT, "include", "moe.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    decls = re.findall(r"(?:moe_status|const char\s*\*)\s+(moe_\w+)\s*\(([^)]*)\)\s*;", src)
    assert decls
    for name, params in decls:
        params = params.strip()
        n = 0 if params in ("", "void") else len(params.split(","))
        at = getattr(lib, name).argtypes
        assert at is not None and len(at) == n, (name, n, at)


def test_noalloc_forward_rejects_dims_beyond_its_scratch():
    # checked on the host before the scratch buffer is looked up or anything is enqueued
    import sparse_mixture_experts_softmax_amd as moe
    lib = moe.load_library()
    big = moe.MoeDims(4096, 8192, 512, 10, 2048, 2048, moe.MOE_BF16, 1)
    p = ctypes.c_void_p(FAKE)
    args = [p] * 10 + [None, None, None, None]
    assert moe.moe_workspace_size(big) > moe.MOE_NOALLOC_SCRATCH_BYTES
    assert lib.moe_forward_noalloc(ctypes.byref(big), *args) == UNSUPPORTED
    assert b"scratch" in lib.moe_last_error()
    zero = moe.MoeDims(0, 8192, 512, 10, 2048, 2048, moe.MOE_BF16, 1)
    assert lib.moe_forward_noalloc(ctypes.byref(zero), *([None] * 14)) == OK
    # the decode-sized layer fits
    assert moe.moe_workspace_size(moe.MoeDims(64, 8192, 512, 10, 2048, 2048, moe.MOE_BF16, 1)) <= \
        moe.MOE_NOALLOC_SCRATCH_BYTES
