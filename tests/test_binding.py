"""The Python binding's own checks, host side only (no GPU, no kernel).

The C ABI receives bare pointers, so it cannot see a tensor's size: a tensor of
the wrong shape, dtype or device would let a kernel read or write past it. The
binding therefore checks every tensor before the call. These tests replace the
library with a recorder and accept CPU tensors in place of GPU ones, then show
that each malformed argument raises MoeError with no call made, and that
well-formed ones reach the library. The last tests keep the real device check,
which rejects CPU tensors outright.
"""
import pytest
import torch

import combine_ep_recv_amd as moe

W, BS, EPR, H, K = 4, 3, 2, 32, 2
N, ROWS = W * BS, W * BS * K


class _Recorder:
    """Stands in for libmoe_ep.so: workspace queries go to the real library (they run
    on the host), launches are only counted."""

    def __init__(self, real):
        self.real = real
        self.calls = []
        self.moe_dispatch_workspace_size = real.moe_dispatch_workspace_size
        self.moe_combine_workspace_size = real.moe_combine_workspace_size
        self.moe_status_str = real.moe_status_str

    def moe_dispatch(self, *args):
        self.calls.append("moe_dispatch")
        return moe.MOE_OK

    def moe_combine(self, *args):
        self.calls.append("moe_combine")
        return moe.MOE_OK


@pytest.fixture
def rec(monkeypatch):
    r = _Recorder(moe.library())
    monkeypatch.setattr(moe, "library", lambda: r)
    monkeypatch.setattr(moe, "_gpu_device", lambda name, t: t.device)
    monkeypatch.setattr(moe, "_stream_ptr", lambda device: 0)
    return r


def _dispatch_args(dtype=torch.bfloat16, quant_mode=0):
    buf = moe.DispatchBuffers(W, BS, EPR, H, K, dtype, quant_mode, "cpu")
    x = torch.zeros((N, H), dtype=dtype)
    ids = torch.zeros((N, K), dtype=torch.int32)
    return buf, x, ids


def _combine_args(dtype=torch.bfloat16):
    return dict(x_out=torch.empty((N, H), dtype=dtype), expand_x=torch.zeros((ROWS, H), dtype=dtype),
                assist_info=torch.zeros((ROWS, 3), dtype=torch.int32),
                ep_recv_count=torch.zeros((W, EPR * W), dtype=torch.int32),
                expert_ids=torch.zeros((N, K), dtype=torch.int32),
                expert_scales=torch.zeros((N, K), dtype=torch.float32), ep_world=W, experts_per_rank=EPR)


def test_well_formed_calls_reach_the_library(rec):
    buf, x, ids = _dispatch_args()
    moe.dispatch_into(buf, x, ids)
    moe.dispatch_into(buf, x, ids, expert_scales=torch.zeros((N, K), dtype=torch.float32))
    moe.combine_into(**_combine_args())
    moe.combine_into(**_combine_args(), workspace=moe.combine_workspace(W, BS, EPR, H, K, torch.bfloat16, "cpu"))
    assert rec.calls == ["moe_dispatch", "moe_dispatch", "moe_combine", "moe_combine"]


@pytest.mark.parametrize("bad", [
    "x_rows", "x_dtype", "x_noncontig", "ids_dtype", "ids_shape", "scales_shape", "scales_8_bytes",
    "buf_expand_x_small", "buf_expand_x_dtype", "buf_assist_small", "buf_erc_shape", "buf_workspace_dtype",
])
def test_dispatch_into_rejects_before_the_call(rec, bad):
    buf, x, ids = _dispatch_args()
    kw = {}
    if bad == "x_rows":
        x = torch.zeros((N - 1, H), dtype=torch.bfloat16)
    elif bad == "x_dtype":
        x = torch.zeros((N, H), dtype=torch.float16)
    elif bad == "x_noncontig":
        x = torch.zeros((H, N), dtype=torch.bfloat16).t()
    elif bad == "ids_dtype":
        ids = torch.zeros((N, K), dtype=torch.int64)
    elif bad == "ids_shape":
        ids = torch.zeros((N, K + 1), dtype=torch.int32)
    elif bad == "scales_shape":
        kw["expert_scales"] = torch.zeros((N, K - 1), dtype=torch.float32)
    elif bad == "scales_8_bytes":
        kw["expert_scales"] = torch.zeros((N, K), dtype=torch.float64)
    elif bad == "buf_expand_x_small":
        buf.expand_x = torch.empty((ROWS - 1, H), dtype=torch.bfloat16)
    elif bad == "buf_expand_x_dtype":
        buf.expand_x = torch.empty((ROWS, H), dtype=torch.float32)
    elif bad == "buf_assist_small":
        buf.assist_info = torch.empty((ROWS, 2), dtype=torch.int32)
    elif bad == "buf_erc_shape":
        buf.ep_recv_count = torch.empty((W, EPR), dtype=torch.int32)
    elif bad == "buf_workspace_dtype":
        buf.workspace = torch.empty(buf.workspace.numel(), dtype=torch.int32)
    with pytest.raises(moe.MoeError):
        moe.dispatch_into(buf, x, ids, **kw)
    assert rec.calls == []


def test_replaced_buffers_are_checked_again(rec):
    buf, x, ids = _dispatch_args(quant_mode=moe.MOE_QUANT_DYN_TOKEN)
    moe.dispatch_into(buf, x, ids)
    buf.dynamic_scales = torch.empty((ROWS - 1,), dtype=torch.float32)     # after a good call
    with pytest.raises(moe.MoeError):
        moe.dispatch_into(buf, x, ids)
    buf.dynamic_scales = torch.empty((ROWS,), dtype=torch.float32)
    moe.dispatch_into(buf, x, ids)
    assert rec.calls == ["moe_dispatch", "moe_dispatch"]


@pytest.mark.parametrize("field,value", [
    ("x_out", torch.empty((N - 1, H), dtype=torch.bfloat16)),
    ("x_out", torch.empty((N, H), dtype=torch.float16)),
    ("expand_x", torch.zeros((ROWS - 1, H), dtype=torch.bfloat16)),
    ("assist_info", torch.zeros((ROWS, 3), dtype=torch.int64)),
    ("assist_info", torch.zeros((ROWS - 1, 3), dtype=torch.int32)),
    ("ep_recv_count", torch.zeros((W, EPR), dtype=torch.int32)),
    ("expert_ids", torch.zeros((N, K), dtype=torch.int64)),
    ("expert_scales", torch.zeros((N, K), dtype=torch.int32)),
    ("expert_scales", torch.zeros((N, K + 1), dtype=torch.float32)),
    ("workspace", torch.empty((64,), dtype=torch.float32)),
    ("expand_x", torch.zeros(ROWS * H, dtype=torch.bfloat16)),
], ids=["x_out_rows", "x_out_dtype", "expand_x_rows", "assist_dtype", "assist_rows", "erc_shape", "ids_dtype",
        "scales_dtype", "scales_shape", "workspace_dtype", "expand_x_1d"])
def test_combine_into_rejects_before_the_call(rec, field, value):
    args = _combine_args()
    args[field] = value
    with pytest.raises(moe.MoeError):
        moe.combine_into(**args)
    assert rec.calls == []


def test_copy_experts_need_a_fitting_ori_x(rec):
    args = _combine_args()
    with pytest.raises(moe.MoeError):
        moe.combine_into(**args, copy_experts=1)
    with pytest.raises(moe.MoeError):
        moe.combine_into(**args, copy_experts=1, ori_x=torch.zeros((N, H - 1), dtype=torch.bfloat16))
    moe.combine_into(**args, copy_experts=1, ori_x=torch.zeros((N, H), dtype=torch.bfloat16))
    assert rec.calls == ["moe_combine"]


def test_cpu_tensors_are_rejected_without_a_call(monkeypatch):
    r = _Recorder(moe.library())
    monkeypatch.setattr(moe, "library", lambda: r)
    buf, x, ids = _dispatch_args()
    with pytest.raises(moe.MoeError):
        moe.dispatch_into(buf, x, ids)
    with pytest.raises(moe.MoeError):
        moe.dispatch(x, ids, W, EPR)
    with pytest.raises(moe.MoeError):
        moe.combine_into(**_combine_args())
    args = _combine_args()
    del args["x_out"]
    with pytest.raises(moe.MoeError):
        moe.combine(**args)
    assert r.calls == []
