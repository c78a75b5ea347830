"""The Python binding checks every tensor argument (element type, shape, layout, device) before it
hands raw pointers to the C ABI, which cannot tell a wrong tensor from a right one. CPU only: the
tensors here live on the host, so a call with every argument right stops at the device check,
and one with any argument wrong stops earlier, naming it."""
import pytest
import torch

import sparse_mixture_experts_softmax_amd as moe

T, D, E, K, I, IS = 6, 64, 8, 2, 32, 16


def block_args(dtype=torch.bfloat16, shared=True):
    a = dict(x=torch.zeros(T, D, dtype=dtype), w_router=torch.zeros(D, E), wg=torch.zeros(E, D, I, dtype=dtype),
             wu=torch.zeros(E, D, I, dtype=dtype), wd=torch.zeros(E, I, D, dtype=dtype))
    if shared:
        a.update(wg_s=torch.zeros(D, IS, dtype=dtype), wu_s=torch.zeros(D, IS, dtype=dtype),
                 wd_s=torch.zeros(IS, D, dtype=dtype))
    else:
        a.update(wg_s=None, wu_s=None, wd_s=None)
    return a


def call_forward(a, **kw):
    return moe.moe_forward(a["x"], a["w_router"], a["wg"], a["wu"], a["wd"], a["wg_s"], a["wu_s"], a["wd_s"], K, **kw)


def test_forward_with_right_arguments_stops_at_the_device_check():
    with pytest.raises(ValueError, match="not on a GPU"):
        call_forward(block_args())
    with pytest.raises(ValueError, match="not on a GPU"):
        call_forward(block_args(torch.float32, shared=False))


BAD = [
    # (argument, replacement, exception, message fragment)
    ("w_router", lambda: torch.zeros(D, E, dtype=torch.bfloat16), TypeError, "w_router"),
    ("w_router", lambda: torch.zeros(D + 8, E), ValueError, "dims.d|w_router"),
    ("wg", lambda: torch.zeros(E, D, I), TypeError, "wg"),
    ("wu", lambda: torch.zeros(E, D, I + 8, dtype=torch.bfloat16), ValueError, "wu"),
    ("wd", lambda: torch.zeros(E, D, I, dtype=torch.bfloat16), ValueError, "wd"),
    ("wd", lambda: torch.zeros(E, D, I, dtype=torch.bfloat16).transpose(1, 2), ValueError, "wd must be contiguous"),
    ("wd_s", lambda: torch.zeros(IS, D), TypeError, "wd_s"),
    ("wu_s", lambda: torch.zeros(D, IS + 8, dtype=torch.bfloat16), ValueError, "wu_s"),
    ("wg_s", lambda: None, ValueError, "shared expert"),
    ("x", lambda: torch.zeros(T, D, dtype=torch.float16), TypeError, "float32 or bfloat16"),
    ("x", lambda: torch.zeros(D, T, dtype=torch.bfloat16).t(), ValueError, "x must be contiguous"),
    ("x", lambda: torch.zeros(T * D, dtype=torch.bfloat16), ValueError, "2-D"),
]


@pytest.mark.parametrize("arg,make,exc,msg", BAD, ids=["%s-%d" % (b[0], i) for i, b in enumerate(BAD)])
def test_forward_rejects_a_wrong_tensor(arg, make, exc, msg):
    a = block_args()
    a[arg] = make()
    with pytest.raises(exc, match=msg):
        call_forward(a)


def test_forward_rejects_wrong_optional_tensors():
    a = block_args()
    with pytest.raises(TypeError, match="router_bias"):
        call_forward(a, router_bias=torch.zeros(E, dtype=torch.float64))
    with pytest.raises(ValueError, match="router_bias"):
        call_forward(a, router_bias=torch.zeros(E + 1))
    with pytest.raises(ValueError, match="out"):
        call_forward(a, out=torch.zeros(T - 1, D, dtype=torch.bfloat16))
    with pytest.raises(TypeError, match="out"):
        call_forward(a, out=torch.zeros(T, D))
    with pytest.raises(TypeError, match="ws"):
        call_forward(a, ws=torch.zeros(100, dtype=torch.float32))
    with pytest.raises(ValueError, match="dims.I "):
        call_forward(a, dims=moe.MoeDims(T, D, E, K, I + 8, IS, moe.MOE_BF16, 1))


def test_step_entry_points_check_their_tensors():
    dm = moe.MoeDims(T, D, E, K, I, IS, moe.MOE_BF16, 1)
    a = block_args()
    with pytest.raises(TypeError, match="x must be torch.bfloat16"):
        moe.moe_router_topk(dm, a["x"].float(), a["w_router"])
    with pytest.raises(TypeError, match="topk_idx"):
        moe.moe_permute(dm, torch.zeros(T, K, dtype=torch.int64))
    with pytest.raises(ValueError, match="topk_idx"):
        moe.moe_permute(dm, torch.zeros(T, K + 1, dtype=torch.int32))
    offs = torch.zeros(E + 1, dtype=torch.int32)
    st = torch.zeros(T * K, dtype=torch.int32)
    with pytest.raises(ValueError, match="sorted_token"):
        moe.moe_grouped_ffn(dm, a["x"], offs, st[:-1], a["wg"], a["wu"], a["wd"], a["wg_s"], a["wu_s"], a["wd_s"])
    with pytest.raises(ValueError, match="I_shared = 0"):
        moe.moe_grouped_ffn(moe.MoeDims(T, D, E, K, I, 0, moe.MOE_BF16, 1), a["x"], offs, st, a["wg"], a["wu"],
                            a["wd"], a["wg_s"], a["wu_s"], a["wd_s"])
    y = torch.zeros(T * K + T, D, dtype=torch.bfloat16)
    w = torch.zeros(T, K)
    with pytest.raises(ValueError, match="y must have shape"):
        moe.moe_combine(dm, y[:-1], st, w)
    with pytest.raises(TypeError, match="topk_w"):
        moe.moe_combine(dm, y, st, w.double())
    with pytest.raises(ValueError, match="residual"):
        moe.moe_combine_residual(dm, y, st, w, torch.zeros(T, D + 8, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="gamma"):
        moe.moe_rmsnorm(dm, a["x"], torch.zeros(D - 8, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="not on a GPU"):
        moe.moe_combine(dm, y, st, w)
    with pytest.raises(TypeError, match="dims must be a MoeDims"):
        moe.moe_permute((T, D, E, K), torch.zeros(T, K, dtype=torch.int32))


def test_block_and_fp8_entry_points_check_their_tensors():
    a = block_args()
    with pytest.raises(ValueError, match="gamma"):
        moe.moe_forward_block(a["x"], torch.zeros(D + 8, dtype=torch.bfloat16), a["w_router"], a["wg"], a["wu"],
                              a["wd"], a["wg_s"], a["wu_s"], a["wd_s"], K)
    with pytest.raises(ValueError, match="not contiguous|must be contiguous"):
        moe.moe_quantize_fp8(torch.zeros(64, 256).t())
    with pytest.raises(TypeError, match="float32 or bfloat16"):
        moe.moe_quantize_fp8(torch.zeros(32, 128, dtype=torch.float16))
    with pytest.raises(TypeError, match="Fp8Experts"):
        moe.moe_forward_fp8(a["x"], a["w_router"], object(), K)
