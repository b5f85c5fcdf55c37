"""MoE token dispatch / combine on MI355X: thin Python binding over libmoe_ep.so.

Every step of the path runs in the HIP kernels of ``csrc/moe_ep.hip``; this
module only allocates outputs with torch (device memory + the current stream)
and marshals pointers to the C ABI of ``include/moe_ep.h``. There is no CPU
fallback: importing works without the library, but any call raises when
``libmoe_ep.so`` has not been built (``python -m combine_ep_recv_amd._build``
or ``__graft_entry__.build()``).

    expand_x, dynamic_scales, assist_info, ep_recv_count = dispatch(
        x, expert_ids, ep_world, experts_per_rank, quant_mode=0)
    x_out = combine(expand_x, assist_info, ep_recv_count, expert_ids,
                    expert_scales, ep_world, experts_per_rank)
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe_ep.so")

MOE_OK = 0
(MOE_ERR_NULLPTR, MOE_ERR_SHAPE, MOE_ERR_DTYPE, MOE_ERR_QUANT, MOE_ERR_WORKSPACE, MOE_ERR_LAUNCH, MOE_ERR_SCHEDULE,
 MOE_ERR_ALIGN, MOE_ERR_MASK) = range(1, 10)
MOE_INT32, MOE_FP16, MOE_BF16 = 0, 1, 2
MOE_QUANT_NONE, MOE_QUANT_STATIC, MOE_QUANT_DYN_TOKEN, MOE_QUANT_DYN_GROUP, MOE_QUANT_MX = 0, 1, 2, 3, 4
MOE_SCHED_TOKEN, MOE_SCHED_SEGMENT, MOE_SCHED_ADAPTIVE = 0, 1, 2
MOE_MASK_NONE, MOE_MASK_TOKEN, MOE_MASK_PAIR = 0, 1, 2

EXPORTS = ("moe_dispatch_workspace_size", "moe_dispatch", "moe_dispatch_noalloc", "moe_combine_workspace_size",
           "moe_combine", "moe_status_str")
NOALLOC_SCRATCH_BYTES = 32 << 20      # MOE_NOALLOC_SCRATCH_BYTES


class MoeError(RuntimeError):
    def __init__(self, fn, status, msg):
        super().__init__("%s failed: status %d (%s)" % (fn, status, msg))
        self.status = status


class MoeSpecialExperts(ctypes.Structure):
    _fields_ = [("zero_expert_num", ctypes.c_int32), ("copy_expert_num", ctypes.c_int32),
                ("const_expert_num", ctypes.c_int32), ("reserved", ctypes.c_int32), ("ori_x", ctypes.c_void_p),
                ("const_x", ctypes.c_void_p)]


def _special(zero_experts: int, copy_experts: int, ori_x: Optional[torch.Tensor] = None, const_experts: int = 0,
             const_x: Optional[torch.Tensor] = None):
    """byref(moe_special_experts) or None when there are no special experts."""
    if not zero_experts and not copy_experts and not const_experts:
        return None
    sp = MoeSpecialExperts(zero_expert_num=int(zero_experts), copy_expert_num=int(copy_experts),
                           const_expert_num=int(const_experts),
                           ori_x=None if ori_x is None else ori_x.data_ptr(),
                           const_x=None if const_x is None else const_x.data_ptr())
    return ctypes.byref(sp)


class MoeSchedule(ctypes.Structure):
    """moe_schedule; by default the adaptive mode with the README's 2 MiB threshold (what a NULL schedule
    selects)."""
    _fields_ = [("mode", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("large_segment_bytes", ctypes.c_int64), ("segment_is_large", ctypes.c_void_p)]

    def __init__(self, mode=MOE_SCHED_ADAPTIVE, large_segment_bytes=-1, segment_is_large=None, reserved=0):
        super().__init__(mode, reserved, large_segment_bytes, segment_is_large)


_lib = None


def library() -> ctypes.CDLL:
    """Load libmoe_ep.so (raises if it was not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("libmoe_ep.so is not built (%s); build it with __graft_entry__.build()" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    P, I, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    lib.moe_dispatch_workspace_size.argtypes = [I, I, I, I, I, I, I, ctypes.POINTER(SZ)]
    lib.moe_dispatch_workspace_size.restype = I
    lib.moe_dispatch.argtypes = [P, P, P, P, I, ctypes.POINTER(MoeSpecialExperts), I, I, I, I, I, I, I, P,
                                 ctypes.c_int64, P, P, P, P, P, ctypes.POINTER(MoeSchedule), P, SZ, P]
    lib.moe_dispatch.restype = I
    lib.moe_dispatch_noalloc.argtypes = [P, P, P, P, I, ctypes.POINTER(MoeSpecialExperts), I, I, I, I, I, I, I, P,
                                         ctypes.c_int64, P, P, P, P, P, ctypes.POINTER(MoeSchedule), P]
    lib.moe_dispatch_noalloc.restype = I
    lib.moe_combine_workspace_size.argtypes = [I, I, I, I, I, I, ctypes.POINTER(SZ)]
    lib.moe_combine_workspace_size.restype = I
    lib.moe_combine.argtypes = [P, P, P, P, P, P, I, ctypes.POINTER(MoeSpecialExperts), I, I, I, I, I, I, P, P,
                                SZ, P]
    lib.moe_combine.restype = I
    lib.moe_status_str.argtypes = [I]
    lib.moe_status_str.restype = ctypes.c_char_p
    _lib = lib
    return lib


def status_str(status: int) -> str:
    return library().moe_status_str(int(status)).decode()


def _check(fn, status):
    if status != MOE_OK:
        raise MoeError(fn, status, status_str(status))


def dtype_code(dt: torch.dtype) -> int:
    if dt == torch.int32:
        return MOE_INT32
    if dt == torch.float16:
        return MOE_FP16
    if dt == torch.bfloat16:
        return MOE_BF16
    raise MoeError("dtype", MOE_ERR_DTYPE, "unsupported token dtype %s" % dt)


def _check_tensor(name, t, dtype, shape, device):
    """A contiguous tensor of this dtype and shape (a tuple) on this device, else MoeError before
    any launch. Callers first make sure that the device is a GPU. About 0.3 us per tensor."""
    try:
        ok = t.dtype == dtype and t.shape == shape and t.device == device and t.is_contiguous()
    except AttributeError:
        ok = False
    if not ok:
        raise MoeError(name, MOE_ERR_SHAPE, "%s must be a contiguous %s tensor of shape %s on %s; got %r"
                       % (name, dtype, tuple(shape), device, t if not isinstance(t, torch.Tensor)
                          else "%s %s on %s" % (t.dtype, tuple(t.shape), t.device)))


def _gpu_device(name, t):
    """The device of t, which must be a GPU tensor."""
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise MoeError(name, MOE_ERR_SHAPE, "%s must be a tensor on a GPU" % name)
    return t.device


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream_ptr(device) -> int:
    """torch's current HIP stream on this GPU, as the raw handle: torch's own accessor when this build
    has it (0.07 us per call), else the public one (1.8 us)."""
    if _raw_stream is not None:
        return _raw_stream(device.index)
    return torch.cuda.current_stream(device).cuda_stream


def _mask_args(mask: Optional[torch.Tensor], N: int, K: int, device):
    """(pointer, kind) for a token mask: None, bool/uint8 [N] (per token) or [N, K] (per pair)."""
    if mask is None:
        return None, MOE_MASK_NONE
    if mask.dtype not in (torch.bool, torch.uint8) or not mask.is_contiguous() or mask.device != device:
        raise MoeError("x_active_mask", MOE_ERR_MASK, "mask must be a contiguous bool or uint8 tensor on %s" % device)
    if tuple(mask.shape) == (N,):
        return _ptr(mask), MOE_MASK_TOKEN
    if tuple(mask.shape) == (N, K):
        return _ptr(mask), MOE_MASK_PAIR
    raise MoeError("x_active_mask", MOE_ERR_MASK,
                   "mask shape %s is neither (%d,) nor (%d, %d)" % (tuple(mask.shape), N, N, K))


def dispatch_workspace_size(ep_world, bs, experts_per_rank, h, topk, dtype, quant_mode=0) -> int:
    n = ctypes.c_size_t(0)
    _check("moe_dispatch_workspace_size",
           library().moe_dispatch_workspace_size(ep_world, bs, experts_per_rank, h, topk, dtype, quant_mode,
                                                 ctypes.byref(n)))
    return n.value


def combine_workspace_size(ep_world, bs, experts_per_rank, h, topk, dtype) -> int:
    n = ctypes.c_size_t(0)
    _check("moe_combine_workspace_size",
           library().moe_combine_workspace_size(ep_world, bs, experts_per_rank, h, topk, dtype, ctypes.byref(n)))
    return n.value


def _out_dtype(quant_mode, dtype):
    """expand_x's element type: int8 codes (quantMode 1, 2), E4M3 codes (3, 4), else the token dtype."""
    return {MOE_QUANT_STATIC: torch.int8, MOE_QUANT_DYN_TOKEN: torch.int8, MOE_QUANT_DYN_GROUP: torch.float8_e4m3fn,
            MOE_QUANT_MX: torch.float8_e4m3fn}.get(quant_mode, dtype)


class DispatchBuffers:
    """Preallocated outputs + workspace for repeated dispatch calls of one shape."""

    def __init__(self, ep_world, bs, experts_per_rank, h, topk, dtype: torch.dtype, quant_mode=0,
                 device="cuda", with_expand_scales=False):
        rows = ep_world * bs * topk
        self.shape = (ep_world, bs, experts_per_rank, h, topk)
        self.dtype, self.quant_mode = dtype, quant_mode
        self.expand_x = torch.empty((rows, h), dtype=_out_dtype(quant_mode, dtype), device=device)
        if quant_mode == MOE_QUANT_DYN_TOKEN:
            self.dynamic_scales = torch.empty((rows,), dtype=torch.float32, device=device)
        elif quant_mode == MOE_QUANT_DYN_GROUP:          # one scale per 128-element group
            self.dynamic_scales = torch.empty((rows, (h + 127) // 128), dtype=torch.float32, device=device)
        elif quant_mode == MOE_QUANT_MX:                 # one E8M0 byte per 32-element block
            self.dynamic_scales = torch.empty((rows, (h + 31) // 32), dtype=torch.uint8, device=device)
        else:
            self.dynamic_scales = None
        self.assist_info = torch.empty((rows, 3), dtype=torch.int32, device=device)
        self.ep_recv_count = torch.empty((ep_world, experts_per_rank * ep_world), dtype=torch.int32,
                                         device=device)
        self.expand_scales = (torch.empty((rows,), dtype=torch.float32 if dtype != torch.int32 else torch.int32,
                                          device=device) if with_expand_scales else None)
        ws = dispatch_workspace_size(ep_world, bs, experts_per_rank, h, topk, dtype_code(dtype), quant_mode)
        self.workspace = torch.empty((max(ws, 16),), dtype=torch.uint8, device=device)
        self._checked = None

    def check(self):
        """Check the buffers against the shape (once per set of tensor objects: the attributes are
        public, and a replaced tensor must fit before a kernel writes it). Returns the device."""
        now = (self.expand_x, self.dynamic_scales, self.assist_info, self.ep_recv_count, self.expand_scales,
               self.workspace)
        if self._checked is not None and all(a is b for a, b in zip(now, self._checked)):
            return self.expand_x.device
        W, bs, epr, h, K = self.shape
        rows = W * bs * K
        dev = _gpu_device("expand_x", self.expand_x)
        _check_tensor("expand_x", self.expand_x, _out_dtype(self.quant_mode, self.dtype), (rows, h), dev)
        if self.quant_mode == MOE_QUANT_DYN_TOKEN:
            _check_tensor("dynamic_scales", self.dynamic_scales, torch.float32, (rows,), dev)
        elif self.quant_mode == MOE_QUANT_DYN_GROUP:
            _check_tensor("dynamic_scales", self.dynamic_scales, torch.float32, (rows, (h + 127) // 128), dev)
        elif self.quant_mode == MOE_QUANT_MX:
            _check_tensor("dynamic_scales", self.dynamic_scales, torch.uint8, (rows, (h + 31) // 32), dev)
        _check_tensor("assist_info", self.assist_info, torch.int32, (rows, 3), dev)
        _check_tensor("ep_recv_count", self.ep_recv_count, torch.int32, (W, epr * W), dev)
        if self.expand_scales is not None:
            _check_tensor("expand_scales", self.expand_scales,
                          torch.int32 if self.expand_scales.dtype == torch.int32 else torch.float32, (rows,), dev)
        _check_tensor("workspace", self.workspace, torch.uint8, (self.workspace.numel(),), dev)
        self._checked = now          # held, so the objects compared by identity stay these ones
        return dev


def _quant_scales_args(qs: Optional[torch.Tensor], device):
    """(pointer, count) for quantMode 1's fp32 coefficients: 1, h or E*h values."""
    if qs is None:
        return None, 0
    if qs.dtype != torch.float32 or not qs.is_contiguous() or qs.device != device:
        raise MoeError("quant_scales", MOE_ERR_QUANT,
                       "quant_scales must be a contiguous float32 tensor on %s" % device)
    return _ptr(qs), qs.numel()


def dispatch_into(buf: DispatchBuffers, x: torch.Tensor, expert_ids: torch.Tensor,
                  expert_scales: Optional[torch.Tensor] = None, schedule: Optional[MoeSchedule] = None,
                  x_active_mask: Optional[torch.Tensor] = None, zero_experts: int = 0, copy_experts: int = 0,
                  quant_scales: Optional[torch.Tensor] = None, const_experts: int = 0):
    """moe_dispatch into preallocated buffers on the current stream. quant_scales: the static
    quantiser's coefficients (quantMode 1 only): 1, h or E*h fp32 values. The C ABI sees only
    pointers, so the tensors' shapes, dtypes and device are checked here against buf."""
    W, bs, epr, h, K = buf.shape
    dev = buf.check()
    _check_tensor("x", x, buf.dtype, (W * bs, h), dev)
    _check_tensor("expert_ids", expert_ids, torch.int32, (W * bs, K), dev)
    if expert_scales is not None:
        _check_tensor("expert_scales", expert_scales,
                      torch.int32 if getattr(expert_scales, "dtype", None) == torch.int32 else torch.float32,
                      (W * bs, K), dev)
    mp, mk = _mask_args(x_active_mask, W * bs, K, dev)
    qp, qn = _quant_scales_args(quant_scales, dev)
    rc = library().moe_dispatch(
        _ptr(x), _ptr(expert_ids), _ptr(expert_scales), mp, mk, _special(zero_experts, copy_experts, None,
                                                                         const_experts), W, bs, epr,
        h, K, dtype_code(buf.dtype),
        buf.quant_mode, qp, ctypes.c_int64(qn),
        _ptr(buf.expand_x), _ptr(buf.dynamic_scales), _ptr(buf.assist_info), _ptr(buf.ep_recv_count),
        _ptr(buf.expand_scales), ctypes.byref(schedule) if schedule is not None else None,
        _ptr(buf.workspace), buf.workspace.numel(), _stream_ptr(dev))
    _check("moe_dispatch", rc)
    return buf


def dispatch_noalloc_into(buf: DispatchBuffers, x: torch.Tensor, expert_ids: torch.Tensor,
                          expert_scales: Optional[torch.Tensor] = None, schedule: Optional[MoeSchedule] = None,
                          x_active_mask: Optional[torch.Tensor] = None, zero_experts: int = 0,
                          copy_experts: int = 0, quant_scales: Optional[torch.Tensor] = None,
                          const_experts: int = 0):
    """moe_dispatch_noalloc into preallocated buffers on the current stream: the same outputs as
    dispatch_into, with the library's own per-GPU scratch in place of buf.workspace (which is not
    used). The same checks run first."""
    W, bs, epr, h, K = buf.shape
    dev = buf.check()
    _check_tensor("x", x, buf.dtype, (W * bs, h), dev)
    _check_tensor("expert_ids", expert_ids, torch.int32, (W * bs, K), dev)
    if expert_scales is not None:
        _check_tensor("expert_scales", expert_scales,
                      torch.int32 if getattr(expert_scales, "dtype", None) == torch.int32 else torch.float32,
                      (W * bs, K), dev)
    mp, mk = _mask_args(x_active_mask, W * bs, K, dev)
    qp, qn = _quant_scales_args(quant_scales, dev)
    rc = library().moe_dispatch_noalloc(
        _ptr(x), _ptr(expert_ids), _ptr(expert_scales), mp, mk, _special(zero_experts, copy_experts, None,
                                                                         const_experts), W, bs, epr,
        h, K, dtype_code(buf.dtype), buf.quant_mode, qp, ctypes.c_int64(qn),
        _ptr(buf.expand_x), _ptr(buf.dynamic_scales), _ptr(buf.assist_info), _ptr(buf.ep_recv_count),
        _ptr(buf.expand_scales), ctypes.byref(schedule) if schedule is not None else None, _stream_ptr(dev))
    _check("moe_dispatch_noalloc", rc)
    return buf


def dispatch(x: torch.Tensor, expert_ids: torch.Tensor, ep_world: int, experts_per_rank: int,
             quant_mode: int = MOE_QUANT_NONE, expert_scales: Optional[torch.Tensor] = None,
             schedule: Optional[MoeSchedule] = None, x_active_mask: Optional[torch.Tensor] = None,
             zero_experts: int = 0, copy_experts: int = 0, quant_scales: Optional[torch.Tensor] = None,
             const_experts: int = 0):
    """Dispatch tokens into expert-grouped rows.

    x: [ep_world*bs, h] int32/fp16/bf16 on a GPU; expert_ids: [ep_world*bs, topk]
    int32. Returns (expand_x, dynamic_scales or None, assist_info, ep_recv_count)
    and, when expert_scales is given, a fifth item expand_scales. With a token
    mask (bool/uint8 [N] or [N, topk]) only the first ep_recv_count[:, -1].sum()
    rows of the row-indexed outputs are written; the same holds with special
    experts (ids E.. for zero_experts, then copy_experts, then const_experts), whose
    pairs get no row.
    quant_mode 1 (static int8) takes its coefficients in quant_scales (fp32, 1, h or
    E*h values) and returns no dynamic scales. quant_mode 3 returns float8_e4m3fn
    codes and fp32 scales per 128-element group; quant_mode 4 (MXFP8) returns
    float8_e4m3fn codes and uint8 E8M0 bytes per 32-element block (the scale
    2^(byte - 127)).
    """
    dev = _gpu_device("x", x)
    _gpu_device("expert_ids", expert_ids)
    if x.dim() != 2 or expert_ids.dim() != 2:
        raise MoeError("moe_dispatch", MOE_ERR_SHAPE, "x and expert_ids must be 2-D")
    N, h = x.shape
    K = expert_ids.shape[1]
    if N % ep_world:
        raise MoeError("moe_dispatch", MOE_ERR_SHAPE,
                       "token count %d is not a multiple of ep_world %d" % (N, ep_world))
    _check_tensor("expert_ids", expert_ids, torch.int32, (N, K), dev)
    buf = DispatchBuffers(ep_world, N // ep_world, experts_per_rank, h, K, x.dtype, quant_mode, dev,
                          with_expand_scales=expert_scales is not None)
    if expert_scales is not None:            # expand_scales takes the dtype of the scales given
        buf.expand_scales = torch.empty((N * K,), dtype=getattr(expert_scales, "dtype", torch.float32),
                                        device=dev)
    dispatch_into(buf, x, expert_ids, expert_scales, schedule, x_active_mask, zero_experts, copy_experts,
                  quant_scales, const_experts)
    out = (buf.expand_x, buf.dynamic_scales, buf.assist_info, buf.ep_recv_count)
    return out + (buf.expand_scales,) if expert_scales is not None else out


def combine_into(x_out: torch.Tensor, expand_x: torch.Tensor, assist_info: torch.Tensor,
                 ep_recv_count: torch.Tensor, expert_ids: torch.Tensor, expert_scales: torch.Tensor,
                 ep_world: int, experts_per_rank: int, workspace: Optional[torch.Tensor] = None,
                 x_active_mask: Optional[torch.Tensor] = None, zero_experts: int = 0, copy_experts: int = 0,
                 ori_x: Optional[torch.Tensor] = None, const_experts: int = 0,
                 const_x: Optional[torch.Tensor] = None):
    """moe_combine into a preallocated x_out on the current stream. Copy experts need ori_x,
    the tokens given to dispatch, and const experts const_x [const_experts, h], their fixed
    outputs, both in expand_x's dtype. The C ABI sees only pointers, so the tensors' shapes,
    dtypes and device are checked here."""
    dev = _gpu_device("expand_x", expand_x)
    _gpu_device("expert_ids", expert_ids)
    if expand_x.dim() != 2 or expert_ids.dim() != 2:
        raise MoeError("moe_combine", MOE_ERR_SHAPE, "expand_x and expert_ids must be 2-D")
    N, K = expert_ids.shape
    rows, h = expand_x.shape
    if N % ep_world or rows != N * K:
        raise MoeError("moe_combine", MOE_ERR_SHAPE, "expand_x must have ep_world*bs*topk rows")
    _check_tensor("expand_x", expand_x, expand_x.dtype, (rows, h), dev)
    _check_tensor("x_out", x_out, expand_x.dtype, (N, h), dev)
    _check_tensor("assist_info", assist_info, torch.int32, (rows, 3), dev)
    _check_tensor("ep_recv_count", ep_recv_count, torch.int32, (ep_world, experts_per_rank * ep_world), dev)
    _check_tensor("expert_ids", expert_ids, torch.int32, (N, K), dev)
    sdt = torch.int32 if expand_x.dtype == torch.int32 else torch.float32
    _check_tensor("expert_scales", expert_scales, sdt, (N, K), dev)
    mp, mk = _mask_args(x_active_mask, N, K, dev)
    if copy_experts:
        if ori_x is None:
            raise MoeError("moe_combine", MOE_ERR_NULLPTR, "copy experts need ori_x, the tokens given to dispatch")
        _check_tensor("ori_x", ori_x, expand_x.dtype, (N, h), dev)
    if const_experts:
        if const_x is None:
            raise MoeError("moe_combine", MOE_ERR_NULLPTR, "const experts need const_x, their outputs")
        _check_tensor("const_x", const_x, expand_x.dtype, (int(const_experts), h), dev)
    dt = dtype_code(expand_x.dtype)
    if workspace is None:
        workspace = combine_workspace(ep_world, N // ep_world, experts_per_rank, h, K, expand_x.dtype, dev)
    else:
        _check_tensor("workspace", workspace, torch.uint8, (workspace.numel(),), dev)
    rc = library().moe_combine(
        _ptr(expand_x), _ptr(assist_info), _ptr(ep_recv_count), _ptr(expert_ids), _ptr(expert_scales), mp, mk,
        _special(zero_experts, copy_experts, ori_x, const_experts, const_x), ep_world, N // ep_world,
        experts_per_rank, h, K, dt,
        _ptr(x_out), _ptr(workspace), workspace.numel(), _stream_ptr(dev))
    _check("moe_combine", rc)
    return x_out


def combine_workspace(ep_world, bs, experts_per_rank, h, topk, dtype: torch.dtype, device="cuda"):
    """Workspace tensor for moe_combine of this shape."""
    n = combine_workspace_size(ep_world, bs, experts_per_rank, h, topk, dtype_code(dtype))
    return torch.empty((max(n, 16),), dtype=torch.uint8, device=device)


def combine(expand_x: torch.Tensor, assist_info: torch.Tensor, ep_recv_count: torch.Tensor,
            expert_ids: torch.Tensor, expert_scales: torch.Tensor, ep_world: int, experts_per_rank: int,
            x_active_mask: Optional[torch.Tensor] = None, zero_experts: int = 0, copy_experts: int = 0,
            ori_x: Optional[torch.Tensor] = None, const_experts: int = 0, const_x: Optional[torch.Tensor] = None):
    """x_out[t] = sum over active k of expand_x[row(t,k)] * expert_scales[t,k] (fp32 accumulation);
    x_active_mask: the dispatch's."""
    dev = _gpu_device("expand_x", expand_x)
    _gpu_device("expert_ids", expert_ids)
    if expand_x.dim() != 2 or expert_ids.dim() != 2:
        raise MoeError("moe_combine", MOE_ERR_SHAPE, "expand_x and expert_ids must be 2-D")
    x_out = torch.empty((expert_ids.shape[0], expand_x.shape[1]), dtype=expand_x.dtype, device=dev)
    return combine_into(x_out, expand_x, assist_info, ep_recv_count, expert_ids, expert_scales, ep_world,
                        experts_per_rank, x_active_mask=x_active_mask, zero_experts=zero_experts,
                        copy_experts=copy_experts, ori_x=ori_x, const_experts=const_experts, const_x=const_x)
