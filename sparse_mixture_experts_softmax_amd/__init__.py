"""MI355X (gfx950) sparse Mixture-of-Experts block: Python binding of libmoe.so.

The functions below carry the C ABI's names (``include/moe.h``) and only marshal arguments:
torch tensors provide device memory and the current HIP stream; every step of the block runs in
the library's HIP kernels. There is no fallback: if libmoe.so cannot be loaded the call raises.
"""
import ctypes
import os

from . import build as _build

__all__ = [
    "MOE_F32", "MOE_BF16", "MoeDims", "MoeError", "dims_for", "load_library", "moe_workspace_size",
    "workspace", "moe_router_topk", "moe_permute", "moe_grouped_ffn", "moe_combine", "moe_forward",
]

MOE_F32, MOE_BF16 = 0, 1
_STATUS = {0: "MOE_OK", 1: "MOE_ERR_INVALID_ARG", 2: "MOE_ERR_UNSUPPORTED", 3: "MOE_ERR_WORKSPACE", 4: "MOE_ERR_HIP"}


class MoeDims(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("d", ctypes.c_int32), ("E", ctypes.c_int32), ("k", ctypes.c_int32),
                ("I", ctypes.c_int32), ("I_shared", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("renormalize", ctypes.c_int32)]

    def __repr__(self):
        return "MoeDims(%s)" % ", ".join("%s=%s" % (f, getattr(self, f)) for f, _ in self._fields_)


class MoeError(RuntimeError):
    def __init__(self, status, detail):
        super().__init__("%s: %s" % (_STATUS.get(status, status), detail))
        self.status = status


_lib = None
_P = ctypes.c_void_p


def load_library(path=None):
    """Load libmoe.so (built in-tree; built first if absent). Raises if it cannot be loaded."""
    global _lib
    if _lib is not None:
        return _lib
    path = path or _build.LIB
    if not os.path.exists(path):
        _build.build()
    lib = ctypes.CDLL(path)
    D = ctypes.POINTER(MoeDims)
    st = ctypes.c_int
    lib.moe_workspace_size.argtypes = [D, ctypes.POINTER(ctypes.c_size_t)]
    lib.moe_workspace_size.restype = st
    lib.moe_router_topk.argtypes = [D, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]
    lib.moe_router_topk.restype = st
    lib.moe_permute.argtypes = [D, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]
    lib.moe_permute.restype = st
    lib.moe_grouped_ffn.argtypes = [D, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]
    lib.moe_grouped_ffn.restype = st
    lib.moe_combine.argtypes = [D, _P, _P, _P, _P, _P]
    lib.moe_combine.restype = st
    lib.moe_forward.argtypes = [D, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]
    lib.moe_forward.restype = st
    lib.moe_router_topk_stats.argtypes = [D, _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]
    lib.moe_router_topk_stats.restype = st
    lib.moe_quantize_fp8.argtypes = [_P, ctypes.c_int32, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, _P, _P, _P]
    lib.moe_quantize_fp8.restype = st
    # dims; x, w_router, router_bias, 6 code arrays and 6 scale arrays, out, topk_idx, topk_w, topk_gap, ws;
    # ws_bytes; stream
    lib.moe_forward_fp8.argtypes = [D] + [_P] * 20 + [ctypes.c_size_t, _P]
    lib.moe_forward_fp8.restype = st
    lib.moe_rmsnorm.argtypes = [D, _P, _P, ctypes.c_double, _P, _P]
    lib.moe_rmsnorm.restype = st
    lib.moe_combine_residual.argtypes = [D, _P, _P, _P, _P, _P, _P]
    lib.moe_combine_residual.restype = st
    lib.moe_forward_block.argtypes = [D, _P, _P, ctypes.c_double, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                      _P, ctypes.c_size_t, _P]
    lib.moe_forward_block.restype = st
    lib.moe_forward_noalloc.argtypes = [D, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P]
    lib.moe_forward_noalloc.restype = st
    lib.moe_profile_next_forward.argtypes = [ctypes.c_int32, _P, _P]
    lib.moe_profile_next_forward.restype = st
    lib.moe_kernel_name.argtypes = [D, ctypes.c_int32, ctypes.c_int32]
    lib.moe_kernel_name.restype = ctypes.c_char_p
    lib.moe_status_string.argtypes = [ctypes.c_int]
    lib.moe_status_string.restype = ctypes.c_char_p
    lib.moe_last_error.argtypes = []
    lib.moe_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(status):
    if status != 0:
        raise MoeError(status, _lib.moe_last_error().decode())


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(t):
    import torch
    return torch.cuda.current_stream(t.device).cuda_stream


def _dtype_code(t):
    import torch
    if t.dtype == torch.float32:
        return MOE_F32
    if t.dtype == torch.bfloat16:
        return MOE_BF16
    raise TypeError("x and expert weights must be float32 or bfloat16, got %s" % t.dtype)


# ---------------------------------------------------------------------------------------------
# Argument checks. The C ABI sees only raw device pointers, so a tensor of the wrong element type,
# shape, layout or device would reach the kernels unnoticed; every function below checks its
# tensors here first and raises TypeError (element type) or ValueError (anything else).
# ---------------------------------------------------------------------------------------------
def _torch_dtype(code):
    import torch
    if code == MOE_F32:
        return torch.float32
    if code == MOE_BF16:
        return torch.bfloat16
    raise ValueError("dims.dtype must be MOE_F32 (0) or MOE_BF16 (1), got %r" % (code,))


def _need(t, name, dtype, shape):
    """t must be a dense row-major tensor of the given element type and shape."""
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor, got %s" % (name, type(t).__name__))
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if tuple(t.shape) != tuple(int(v) for v in shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(int(v) for v in shape), tuple(t.shape)))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous (row-major, densely packed)" % name)


def _need_ws(ws):
    import torch
    if not isinstance(ws, torch.Tensor) or ws.dtype != torch.uint8 or ws.dim() != 1 or not ws.is_contiguous():
        raise TypeError("ws must be a contiguous 1-D torch.uint8 tensor (see workspace())")


def _one_device(**named):
    """Every given tensor on the same HIP device."""
    dev = None
    for name, t in named.items():
        if t is None:
            continue
        if t.device.type != "cuda":
            raise ValueError("%s is on %s, not on a GPU" % (name, t.device))
        if dev is None:
            dev, first = t.device, name
        elif t.device != dev:
            raise ValueError("%s is on %s but %s is on %s" % (name, t.device, first, dev))


def _need_dims(dims):
    if not isinstance(dims, MoeDims):
        raise TypeError("dims must be a MoeDims, got %s" % type(dims).__name__)
    return _torch_dtype(dims.dtype)


def _need_experts(dims, dt, wg, wu, wd, wg_s, wu_s, wd_s):
    _need(wg, "wg", dt, (dims.E, dims.d, dims.I))
    _need(wu, "wu", dt, (dims.E, dims.d, dims.I))
    _need(wd, "wd", dt, (dims.E, dims.I, dims.d))
    shared = (wg_s, wu_s, wd_s)
    if dims.I_shared == 0:
        if any(w is not None for w in shared):
            raise ValueError("dims.I_shared = 0 (no shared expert) but shared expert weights were given")
        return
    _need(wg_s, "wg_s", dt, (dims.d, dims.I_shared))
    _need(wu_s, "wu_s", dt, (dims.d, dims.I_shared))
    _need(wd_s, "wd_s", dt, (dims.I_shared, dims.d))


def _need_router(dims, dt, x, w_router, router_bias):
    import torch
    _need(x, "x", dt, (dims.T, dims.d))
    _need(w_router, "w_router", torch.float32, (dims.d, dims.E))
    if router_bias is not None:
        _need(router_bias, "router_bias", torch.float32, (dims.E,))


def _block_dims(x, w_router, wg, wu, wd, wg_s, wu_s, wd_s, k, renormalize, dims):
    """The dims of a whole-block call, from the tensors (or checked against the given dims)."""
    import torch
    if not isinstance(x, torch.Tensor) or x.dim() != 2:
        raise ValueError("x must be a 2-D tensor [T, d]")
    if not isinstance(w_router, torch.Tensor) or w_router.dim() != 2:
        raise ValueError("w_router must be a 2-D tensor [d, E]")
    if not isinstance(wg, torch.Tensor) or wg.dim() != 3:
        raise ValueError("wg must be a 3-D tensor [E, d, I]")
    if (wg_s is None) != (wu_s is None) or (wg_s is None) != (wd_s is None):
        raise ValueError("the shared expert needs all of wg_s, wu_s, wd_s (or none of them)")
    if wg_s is not None and (not isinstance(wg_s, torch.Tensor) or wg_s.dim() != 2):
        raise ValueError("wg_s must be a 2-D tensor [d, I_shared]")
    got = dims_for(x, w_router, wg, wg_s, k, renormalize)
    if dims is None:
        return got
    _need_dims(dims)
    for f, _ in MoeDims._fields_:
        if f != "renormalize" and getattr(dims, f) != getattr(got, f):
            raise ValueError("dims.%s = %s does not match the tensors (%s)" % (f, getattr(dims, f), getattr(got, f)))
    return dims


def dims_for(x, w_router, wg, wg_s, k, renormalize=True):
    """MoeDims from tensor shapes: x [T,d], w_router [d,E], wg [E,d,I], wg_s [d,Is] or None."""
    T, d = x.shape
    E = w_router.shape[1]
    I = wg.shape[2]
    Is = 0 if wg_s is None else wg_s.shape[1]
    return MoeDims(T, d, E, k, I, Is, _dtype_code(x), int(bool(renormalize)))


def moe_workspace_size(dims):
    n = ctypes.c_size_t(0)
    _check(load_library().moe_workspace_size(ctypes.byref(dims), ctypes.byref(n)))
    return n.value


KERNEL_ROUTER, KERNEL_PERMUTE, KERNEL_FFN_GATE_UP, KERNEL_FFN_DOWN, KERNEL_COMBINE = 1, 2, 3, 4, 5


def moe_kernel_name(dims, kernel, fp8=False):
    """Name of the kernel the forward launches for one step with these dims (moe_kernel_name)."""
    _need_dims(dims)
    name = load_library().moe_kernel_name(ctypes.byref(dims), int(kernel), 1 if fp8 else 0)
    if name is None:
        raise ValueError("no kernel name for kernel id %r with these dims" % (kernel,))
    return name.decode()


def workspace(dims, device):
    """A device workspace of moe_workspace_size(dims) bytes (torch's allocator aligns to 512 B)."""
    import torch
    return torch.empty(max(moe_workspace_size(dims), 1), dtype=torch.uint8, device=device)


def moe_router_topk(dims, x, w_router, router_bias=None, ws=None, with_gap=True):
    """Returns (topk_idx int32 [T,k], topk_w float32 [T,k], topk_gap float32 [T] or None)."""
    import torch
    dt = _need_dims(dims)
    _need_router(dims, dt, x, w_router, router_bias)
    if ws is not None:
        _need_ws(ws)
    _one_device(x=x, w_router=w_router, router_bias=router_bias, ws=ws)
    lib = load_library()
    ws = workspace(dims, x.device) if ws is None else ws
    idx = torch.empty(dims.T, dims.k, dtype=torch.int32, device=x.device)
    w = torch.empty(dims.T, dims.k, dtype=torch.float32, device=x.device)
    gap = torch.empty(dims.T, dtype=torch.float32, device=x.device) if with_gap else None
    _check(lib.moe_router_topk(ctypes.byref(dims), _ptr(x), _ptr(w_router), _ptr(router_bias), _ptr(idx), _ptr(w),
                               _ptr(gap), _ptr(ws), ws.numel(), _stream(x)))
    return idx, w, gap


def moe_permute(dims, topk_idx, ws=None):
    """Returns (expert_offsets int32 [E+1], sorted_token int32 [T*k], slot_of int32 [T*k])."""
    import torch
    _need_dims(dims)
    _need(topk_idx, "topk_idx", torch.int32, (dims.T, dims.k))
    if ws is not None:
        _need_ws(ws)
    _one_device(topk_idx=topk_idx, ws=ws)
    lib = load_library()
    dev = topk_idx.device
    ws = workspace(dims, dev) if ws is None else ws
    offs = torch.empty(dims.E + 1, dtype=torch.int32, device=dev)
    sorted_token = torch.empty(dims.T * dims.k, dtype=torch.int32, device=dev)
    slot_of = torch.empty(dims.T * dims.k, dtype=torch.int32, device=dev)
    _check(lib.moe_permute(ctypes.byref(dims), _ptr(topk_idx), _ptr(offs), _ptr(sorted_token), _ptr(slot_of),
                           _ptr(ws), ws.numel(), _stream(topk_idx)))
    return offs, sorted_token, slot_of


def _y_rows(dims):
    return dims.T * dims.k + (dims.T if dims.I_shared > 0 else 0)


def moe_grouped_ffn(dims, x, expert_offsets, sorted_token, wg, wu, wd, wg_s=None, wu_s=None, wd_s=None, ws=None):
    """Returns y [T*k + T, d] (T*k rows without a shared expert) in x's dtype."""
    import torch
    dt = _need_dims(dims)
    _need(x, "x", dt, (dims.T, dims.d))
    _need(expert_offsets, "expert_offsets", torch.int32, (dims.E + 1,))
    _need(sorted_token, "sorted_token", torch.int32, (dims.T * dims.k,))
    _need_experts(dims, dt, wg, wu, wd, wg_s, wu_s, wd_s)
    if ws is not None:
        _need_ws(ws)
    _one_device(x=x, expert_offsets=expert_offsets, sorted_token=sorted_token, wg=wg, wu=wu, wd=wd, wg_s=wg_s,
                wu_s=wu_s, wd_s=wd_s, ws=ws)
    lib = load_library()
    ws = workspace(dims, x.device) if ws is None else ws
    y = torch.empty(_y_rows(dims), dims.d, dtype=x.dtype, device=x.device)
    _check(lib.moe_grouped_ffn(ctypes.byref(dims), _ptr(x), _ptr(expert_offsets), _ptr(sorted_token), _ptr(wg),
                               _ptr(wu), _ptr(wd), _ptr(wg_s), _ptr(wu_s), _ptr(wd_s), _ptr(y), _ptr(ws), ws.numel(),
                               _stream(x)))
    return y


def _need_combine(dims, dt, y, slot_of, topk_w, out):
    import torch
    _need(y, "y", dt, (_y_rows(dims), dims.d))
    _need(slot_of, "slot_of", torch.int32, (dims.T * dims.k,))
    _need(topk_w, "topk_w", torch.float32, (dims.T, dims.k))
    if out is not None:
        _need(out, "out", dt, (dims.T, dims.d))


def moe_combine(dims, y, slot_of, topk_w, out=None):
    """Returns out [T, d] in y's dtype."""
    import torch
    dt = _need_dims(dims)
    _need_combine(dims, dt, y, slot_of, topk_w, out)
    _one_device(y=y, slot_of=slot_of, topk_w=topk_w, out=out)
    lib = load_library()
    out = torch.empty(dims.T, dims.d, dtype=y.dtype, device=y.device) if out is None else out
    _check(lib.moe_combine(ctypes.byref(dims), _ptr(y), _ptr(slot_of), _ptr(topk_w), _ptr(out), _stream(y)))
    return out


def _routing_outputs(dims, device, return_routing):
    import torch
    if not return_routing:
        return None, None, None
    return (torch.empty(dims.T, dims.k, dtype=torch.int32, device=device),
            torch.empty(dims.T, dims.k, dtype=torch.float32, device=device),
            torch.empty(dims.T, dtype=torch.float32, device=device))


def moe_forward(x, w_router, wg, wu, wd, wg_s, wu_s, wd_s, k, renormalize=True, router_bias=None,
                return_routing=False, ws=None, out=None, dims=None):
    """The whole MoE block. Returns out [T, d], or (out, topk_idx, topk_w, topk_gap) with return_routing."""
    import torch
    dims = _block_dims(x, w_router, wg, wu, wd, wg_s, wu_s, wd_s, k, renormalize, dims)
    dt = _torch_dtype(dims.dtype)
    _need_router(dims, dt, x, w_router, router_bias)
    _need_experts(dims, dt, wg, wu, wd, wg_s, wu_s, wd_s)
    if out is not None:
        _need(out, "out", dt, (dims.T, dims.d))
    if ws is not None:
        _need_ws(ws)
    _one_device(x=x, w_router=w_router, router_bias=router_bias, wg=wg, wu=wu, wd=wd, wg_s=wg_s, wu_s=wu_s, wd_s=wd_s,
                out=out, ws=ws)
    lib = load_library()
    ws = workspace(dims, x.device) if ws is None else ws
    out = torch.empty_like(x) if out is None else out
    idx, w, gap = _routing_outputs(dims, x.device, return_routing)
    _check(lib.moe_forward(ctypes.byref(dims), _ptr(x), _ptr(w_router), _ptr(router_bias), _ptr(wg), _ptr(wu),
                           _ptr(wd), _ptr(wg_s), _ptr(wu_s), _ptr(wd_s), _ptr(out), _ptr(idx), _ptr(w), _ptr(gap),
                           _ptr(ws), ws.numel(), _stream(x)))
    if return_routing:
        return out, idx, w, gap
    return out


MOE_NOALLOC_SCRATCH_BYTES = 64 << 20


def moe_forward_noalloc(x, w_router, wg, wu, wd, wg_s, wu_s, wd_s, k, out, renormalize=True, router_bias=None,
                        topk_idx=None, topk_w=None, topk_gap=None, dims=None):
    """moe_forward with the library's own per-GPU scratch buffer (MOE_NOALLOC_SCRATCH_BYTES) in place
    of a workspace, for callers that cannot allocate: it allocates nothing, so the caller passes
    out [T, d] and, optionally, the routing outputs. Returns out."""
    import torch
    dims = _block_dims(x, w_router, wg, wu, wd, wg_s, wu_s, wd_s, k, renormalize, dims)
    dt = _torch_dtype(dims.dtype)
    _need_router(dims, dt, x, w_router, router_bias)
    _need_experts(dims, dt, wg, wu, wd, wg_s, wu_s, wd_s)
    _need(out, "out", dt, (dims.T, dims.d))
    if topk_idx is not None:
        _need(topk_idx, "topk_idx", torch.int32, (dims.T, dims.k))
    if topk_w is not None:
        _need(topk_w, "topk_w", torch.float32, (dims.T, dims.k))
    if topk_gap is not None:
        _need(topk_gap, "topk_gap", torch.float32, (dims.T,))
    _one_device(x=x, w_router=w_router, router_bias=router_bias, wg=wg, wu=wu, wd=wd, wg_s=wg_s, wu_s=wu_s, wd_s=wd_s,
                out=out, topk_idx=topk_idx, topk_w=topk_w, topk_gap=topk_gap)
    lib = load_library()
    _check(lib.moe_forward_noalloc(ctypes.byref(dims), _ptr(x), _ptr(w_router), _ptr(router_bias), _ptr(wg),
                                   _ptr(wu), _ptr(wd), _ptr(wg_s), _ptr(wu_s), _ptr(wd_s), _ptr(out), _ptr(topk_idx),
                                   _ptr(topk_w), _ptr(topk_gap), _stream(x)))
    return out


RMS_NORM_EPS = 1e-6


def moe_rmsnorm(dims, x, gamma, eps=RMS_NORM_EPS, h=None):
    """Zero-centred RMSNorm of the rows of x: returns h [T, d] in x's dtype."""
    import torch
    dt = _need_dims(dims)
    _need(x, "x", dt, (dims.T, dims.d))
    _need(gamma, "gamma", dt, (dims.d,))
    if h is not None:
        _need(h, "h", dt, (dims.T, dims.d))
    _one_device(x=x, gamma=gamma, h=h)
    lib = load_library()
    h = torch.empty_like(x) if h is None else h
    _check(lib.moe_rmsnorm(ctypes.byref(dims), _ptr(x), _ptr(gamma), float(eps), _ptr(h), _stream(x)))
    return h


def moe_combine_residual(dims, y, slot_of, topk_w, residual, out=None):
    """moe_combine plus the residual rows; returns out [T, d] in y's dtype."""
    import torch
    dt = _need_dims(dims)
    _need_combine(dims, dt, y, slot_of, topk_w, out)
    _need(residual, "residual", dt, (dims.T, dims.d))
    _one_device(y=y, slot_of=slot_of, topk_w=topk_w, residual=residual, out=out)
    lib = load_library()
    out = torch.empty(dims.T, dims.d, dtype=y.dtype, device=y.device) if out is None else out
    _check(lib.moe_combine_residual(ctypes.byref(dims), _ptr(y), _ptr(slot_of), _ptr(topk_w), _ptr(residual),
                                    _ptr(out), _stream(y)))
    return out


def moe_forward_block(x, gamma, w_router, wg, wu, wd, wg_s, wu_s, wd_s, k, renormalize=True, router_bias=None,
                      eps=RMS_NORM_EPS, return_routing=False, ws=None, out=None, dims=None):
    """out = x + MoE(rmsnorm(x)). Returns out [T, d], or (out, topk_idx, topk_w, topk_gap) with
    return_routing."""
    import torch
    dims = _block_dims(x, w_router, wg, wu, wd, wg_s, wu_s, wd_s, k, renormalize, dims)
    dt = _torch_dtype(dims.dtype)
    _need_router(dims, dt, x, w_router, router_bias)
    _need(gamma, "gamma", dt, (dims.d,))
    _need_experts(dims, dt, wg, wu, wd, wg_s, wu_s, wd_s)
    if out is not None:
        _need(out, "out", dt, (dims.T, dims.d))
    if ws is not None:
        _need_ws(ws)
    _one_device(x=x, gamma=gamma, w_router=w_router, router_bias=router_bias, wg=wg, wu=wu, wd=wd, wg_s=wg_s,
                wu_s=wu_s, wd_s=wd_s, out=out, ws=ws)
    lib = load_library()
    ws = workspace(dims, x.device) if ws is None else ws
    out = torch.empty_like(x) if out is None else out
    idx, w, gap = _routing_outputs(dims, x.device, return_routing)
    _check(lib.moe_forward_block(ctypes.byref(dims), _ptr(x), _ptr(gamma), float(eps), _ptr(w_router),
                                 _ptr(router_bias), _ptr(wg), _ptr(wu), _ptr(wd), _ptr(wg_s), _ptr(wu_s), _ptr(wd_s),
                                 _ptr(out), _ptr(idx), _ptr(w), _ptr(gap), _ptr(ws), ws.numel(), _stream(x)))
    if return_routing:
        return out, idx, w, gap
    return out


def moe_router_topk_stats(dims, x, w_router, router_bias=None, ws=None):
    """Router and top-k plus statistics. Returns (topk_idx [T,k], topk_w [T,k], topk_gap [T],
    expert_counts int32 [E], prob_mean float32 [E])."""
    import torch
    dt = _need_dims(dims)
    _need_router(dims, dt, x, w_router, router_bias)
    if ws is not None:
        _need_ws(ws)
    _one_device(x=x, w_router=w_router, router_bias=router_bias, ws=ws)
    lib = load_library()
    ws = workspace(dims, x.device) if ws is None else ws
    idx = torch.empty(dims.T, dims.k, dtype=torch.int32, device=x.device)
    w = torch.empty(dims.T, dims.k, dtype=torch.float32, device=x.device)
    gap = torch.empty(dims.T, dtype=torch.float32, device=x.device)
    counts = torch.empty(dims.E, dtype=torch.int32, device=x.device)
    pm = torch.empty(dims.E, dtype=torch.float32, device=x.device)
    _check(lib.moe_router_topk_stats(ctypes.byref(dims), _ptr(x), _ptr(w_router), _ptr(router_bias), _ptr(idx),
                                     _ptr(w), _ptr(gap), _ptr(counts), _ptr(pm), _ptr(ws), ws.numel(), _stream(x)))
    return idx, w, gap, counts, pm


def moe_quantize_fp8(w):
    """FP8 (e4m3) codes and column scales of w [..., K, N] (float32 or bfloat16, N-contiguous;
    K % 32 == 0, N % 128 == 0). Returns (q uint8 [..., N // 128, K // 32, 4096]: the code tiles of
    moe.h, scale float32 [..., N])."""
    import torch
    if not isinstance(w, torch.Tensor) or w.dim() < 2:
        raise ValueError("w must be a tensor [..., K, N]")
    _dtype_code(w)
    if not w.is_contiguous():
        raise ValueError("w must be contiguous (row-major, densely packed)")
    _one_device(w=w)
    lib = load_library()
    K, N = w.shape[-2], w.shape[-1]
    batch = w.numel() // (K * N) if w.numel() else 0
    q = torch.empty(w.shape[:-2] + (N // 128, K // 32, 4096), dtype=torch.uint8, device=w.device)
    s = torch.empty(w.shape[:-2] + (N,), dtype=torch.float32, device=w.device)
    _check(lib.moe_quantize_fp8(_ptr(w), _dtype_code(w), batch, K, N, _ptr(q), _ptr(s), _stream(w)))
    return q, s


class Fp8Experts:
    """Expert weights in FP8 (moe_quantize_fp8 of the bf16 wg, wu, wd and the shared expert)."""

    def __init__(self, wg, wu, wd, wg_s=None, wu_s=None, wd_s=None):
        self.wg, self.sg = moe_quantize_fp8(wg)
        self.wu, self.su = moe_quantize_fp8(wu)
        self.wd, self.sd = moe_quantize_fp8(wd)
        if wg_s is not None:
            self.wg_s, self.sg_s = moe_quantize_fp8(wg_s)
            self.wu_s, self.su_s = moe_quantize_fp8(wu_s)
            self.wd_s, self.sd_s = moe_quantize_fp8(wd_s)
        else:
            self.wg_s = self.sg_s = self.wu_s = self.su_s = self.wd_s = self.sd_s = None
        self.E, self.d, self.I = wg.shape
        self.I_shared = 0 if wg_s is None else wg_s.shape[1]

    def check(self, dims):
        """The codes and scales have the layout moe.h fixes for these dims."""
        import torch
        u8, f32 = torch.uint8, torch.float32
        if (self.E, self.d, self.I, self.I_shared) != (dims.E, dims.d, dims.I, dims.I_shared):
            raise ValueError("FP8 experts are for E=%d, d=%d, I=%d, I_shared=%d, dims say E=%d, d=%d, I=%d, "
                             "I_shared=%d" % (self.E, self.d, self.I, self.I_shared, dims.E, dims.d, dims.I,
                                              dims.I_shared))
        E, d, I, Is = dims.E, dims.d, dims.I, dims.I_shared
        _need(self.wg, "wg codes", u8, (E, I // 128, d // 32, 4096))
        _need(self.wu, "wu codes", u8, (E, I // 128, d // 32, 4096))
        _need(self.wd, "wd codes", u8, (E, d // 128, I // 32, 4096))
        _need(self.sg, "sg", f32, (E, I))
        _need(self.su, "su", f32, (E, I))
        _need(self.sd, "sd", f32, (E, d))
        if Is:
            _need(self.wg_s, "wg_s codes", u8, (Is // 128, d // 32, 4096))
            _need(self.wu_s, "wu_s codes", u8, (Is // 128, d // 32, 4096))
            _need(self.wd_s, "wd_s codes", u8, (d // 128, Is // 32, 4096))
            _need(self.sg_s, "sg_s", f32, (Is,))
            _need(self.su_s, "su_s", f32, (Is,))
            _need(self.sd_s, "sd_s", f32, (d,))

    def tensors(self):
        return dict(wg=self.wg, wu=self.wu, wd=self.wd, sg=self.sg, su=self.su, sd=self.sd, wg_s=self.wg_s,
                    wu_s=self.wu_s, wd_s=self.wd_s, sg_s=self.sg_s, su_s=self.su_s, sd_s=self.sd_s)


def moe_forward_fp8(x, w_router, experts, k, renormalize=True, router_bias=None, return_routing=False, ws=None,
                    out=None, dims=None):
    """The MoE block with FP8 expert weights (an Fp8Experts). Returns out [T, d], or
    (out, topk_idx, topk_w, topk_gap) with return_routing."""
    import torch
    f = experts
    if not isinstance(f, Fp8Experts):
        raise TypeError("experts must be an Fp8Experts")
    if not isinstance(x, torch.Tensor) or x.dim() != 2:
        raise ValueError("x must be a 2-D tensor [T, d]")
    if dims is None:
        T, d = x.shape
        dims = MoeDims(T, d, w_router.shape[1], k, f.I, f.I_shared, _dtype_code(x), int(bool(renormalize)))
    dt = _need_dims(dims)
    if dt != torch.bfloat16:
        raise TypeError("FP8 experts take bfloat16 activations")
    _need_router(dims, dt, x, w_router, router_bias)
    f.check(dims)
    if out is not None:
        _need(out, "out", dt, (dims.T, dims.d))
    if ws is not None:
        _need_ws(ws)
    _one_device(x=x, w_router=w_router, router_bias=router_bias, out=out, ws=ws,
                **{k_: v for k_, v in f.tensors().items()})
    lib = load_library()
    ws = workspace(dims, x.device) if ws is None else ws
    out = torch.empty_like(x) if out is None else out
    idx, w, gap = _routing_outputs(dims, x.device, return_routing)
    _check(lib.moe_forward_fp8(ctypes.byref(dims), _ptr(x), _ptr(w_router), _ptr(router_bias), _ptr(f.wg),
                               _ptr(f.wu), _ptr(f.wd), _ptr(f.sg), _ptr(f.su), _ptr(f.sd), _ptr(f.wg_s), _ptr(f.wu_s),
                               _ptr(f.wd_s), _ptr(f.sg_s), _ptr(f.su_s), _ptr(f.sd_s), _ptr(out), _ptr(idx), _ptr(w),
                               _ptr(gap), _ptr(ws), ws.numel(), _stream(x)))
    if return_routing:
        return out, idx, w, gap
    return out
