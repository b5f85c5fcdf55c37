"""CPU oracle for MoE token dispatch and combine -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package. The product path (``combine_ep_recv_amd``)
never imports it and fails loudly when its own HIP library is missing.

The arithmetic lives in ``moe_oracle.c`` (plain C, gcc ``-O2
-ffp-contract=off``, no fast-math); this module only builds it and marshals
numpy arrays. bf16 arrays are carried as ``numpy.uint16`` bit patterns.

Sources, readings and pins are listed in the C file's header. Parity pins live
in ``tests/test_oracle.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB = os.path.join(_HERE, "libmoe_oracle.so")

INT32, FP16, BF16 = 0, 1, 2
_CFLAGS = ["-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", "-Wall"]


def build(force: bool = False) -> str:
    """Compile the oracle with gcc into ``oracle/libmoe_oracle.so``."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *_CFLAGS, "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        _lib = bind(ctypes.CDLL(build()))
    return _lib


def bind(lib):
    """Declare the C signatures on a loaded oracle library (the tests also bind
    copies of it built from altered sources, to show that the pins catch them)."""
    P, I, LL = ctypes.c_void_p, ctypes.c_int, ctypes.c_longlong
    lib.oracle_dispatch.argtypes = [P, P, P, I, I, I, I, I, I, I, P, LL, P, I, I, I, I, P, P, P, P, P]
    lib.oracle_dispatch.restype = I
    lib.oracle_combine.argtypes = [P, P, P, P, P, I, I, I, I, I, I, P, I, I, I, I, P, P, P]
    lib.oracle_combine.restype = I
    lib.oracle_large_segments.argtypes = [P, I, I, I, I, LL, P]
    lib.oracle_large_segments.restype = I
    lib.oracle_identity_expert_dequant.argtypes = [P, P, LL, I, P]
    lib.oracle_identity_expert_dequant.restype = None
    lib.oracle_identity_expert_dequant_fp8.argtypes = [P, P, LL, I, P]
    lib.oracle_identity_expert_dequant_fp8.restype = None
    lib.oracle_identity_expert_dequant_mx.argtypes = [P, P, LL, I, P]
    lib.oracle_identity_expert_dequant_mx.restype = None
    lib.oracle_e4m3_to_f32.argtypes = [ctypes.c_uint8]
    lib.oracle_e4m3_to_f32.restype = ctypes.c_float
    lib.oracle_f32_to_e4m3.argtypes = [ctypes.c_float]
    lib.oracle_f32_to_e4m3.restype = ctypes.c_uint8
    lib.oracle_f16_to_f32.argtypes = [ctypes.c_uint16]
    lib.oracle_f16_to_f32.restype = ctypes.c_float
    lib.oracle_f32_to_f16.argtypes = [ctypes.c_float]
    lib.oracle_f32_to_f16.restype = ctypes.c_uint16
    lib.oracle_bf16_to_f32.argtypes = [ctypes.c_uint16]
    lib.oracle_bf16_to_f32.restype = ctypes.c_float
    lib.oracle_f32_to_bf16.argtypes = [ctypes.c_float]
    lib.oracle_f32_to_bf16.restype = ctypes.c_uint16
    return lib


class OracleError(RuntimeError):
    pass


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def dtype_code(arr: np.ndarray, bf16: bool = False) -> int:
    if arr.dtype == np.int32:
        return INT32
    if arr.dtype == np.float16:
        return FP16
    if arr.dtype == np.uint16 and bf16:
        return BF16
    raise OracleError("unsupported token dtype %s (bf16 must be passed as uint16 bits with bf16=True)" % arr.dtype)


def _mask(mask, N, K):
    """(uint8 array or None, mask_kind): 1 for a per-token mask [N], 2 for a per-pair mask [N, K]."""
    if mask is None:
        return None, 0
    m = np.ascontiguousarray(mask).astype(np.uint8)
    if m.shape == (N,):
        return m, 1
    if m.shape == (N, K):
        return m, 2
    raise ValueError("mask must have shape (N,) or (N, K), got %s" % (m.shape,))


def dispatch(x, ids, ep_world, experts_per_rank, quant_mode=0, expert_scales=None, bf16=False, mask=None,
             zero_experts=0, copy_experts=0, quant_scales=None, const_experts=0):
    """Counting-sort dispatch. Returns dict with expand_x, dynamic_scales,
    assist_info, ep_recv_count, rows (the number of rows written: N*K, or the
    active pairs under a mask) and (when scales are given) expand_scales.
    mask: None, per-token [N] or per-pair [N, K] (nonzero = active).
    zero_experts / copy_experts / const_experts: special expert ids E.. (zero), E+zero..
    (copy) and E+zero+copy.. (const); their pairs are not exchanged.
    quant_scales: quantMode 1's fp32 coefficients, 1, h or E*h values (q = sat8(rint(x * c)), the
    exact product rounded once)."""
    x = np.ascontiguousarray(x)
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    N, h = x.shape
    K = ids.shape[1]
    W, epr = int(ep_world), int(experts_per_rank)
    assert N % W == 0 and ids.shape[0] == N
    bs = N // W
    dt = dtype_code(x, bf16)
    rows = N * K
    qs = None
    if quant_mode == 1:
        qs = np.ascontiguousarray(quant_scales, dtype=np.float32).reshape(-1)
        expand_x = np.zeros((rows, h), np.int8)
        dyn = None
    elif quant_mode == 2:
        expand_x = np.zeros((rows, h), np.int8)
        dyn = np.zeros((rows,), np.float32)
    elif quant_mode == 3:                     # E4M3 codes, ceil(h/128) group scales per row
        expand_x = np.zeros((rows, h), np.uint8)
        dyn = np.zeros((rows, (h + 127) // 128), np.float32)
    elif quant_mode == 4:                     # MXFP8: E4M3 codes, ceil(h/32) E8M0 scale bytes per row
        expand_x = np.zeros((rows, h), np.uint8)
        dyn = np.zeros((rows, (h + 31) // 32), np.uint8)
    else:
        expand_x = np.zeros((rows, h), x.dtype)
        dyn = None
    assist = np.zeros((rows, 3), np.int32)
    erc = np.zeros((W, epr * W), np.int32)
    esc = None
    if expert_scales is not None:
        expert_scales = np.ascontiguousarray(expert_scales)
        assert expert_scales.dtype.itemsize == 4 and expert_scales.shape == (N, K)
        esc = np.zeros((rows,), expert_scales.dtype)
    m, mk = _mask(mask, N, K)
    rc = _load().oracle_dispatch(_ptr(x), _ptr(ids), _ptr(expert_scales), W, bs, epr, h, K, dt,
                                 int(quant_mode), _ptr(qs), 0 if qs is None else qs.size, _ptr(m), mk,
                                 int(zero_experts), int(copy_experts), int(const_experts),
                                 _ptr(expand_x), _ptr(dyn), _ptr(assist),
                                 _ptr(erc), _ptr(esc))
    if rc != 0:
        raise OracleError("oracle_dispatch returned %d" % rc)
    out = dict(expand_x=expand_x, dynamic_scales=dyn, assist_info=assist, ep_recv_count=erc,
               rows=int(erc[:, -1].astype(np.int64).sum()) if erc.size else 0)
    if esc is not None:
        out["expand_scales"] = esc
    return out


def combine(expand_x, assist_info, ep_recv_count, ids, expert_scales, ep_world, experts_per_rank,
            bf16=False, mask=None, zero_experts=0, copy_experts=0, ori_x=None, const_experts=0, const_x=None):
    """Push-style combine: x_out[t] = sum over active k of expand_x[row(t,k)] * scales[t,k]
    (0 for a token with no active pair); mask as for dispatch. A copy expert adds
    ori_x[t] * weight (ori_x: the dispatch's x, same dtype as expand_x); const expert j
    adds const_x[j] * weight (const_x [const_experts, h], same dtype); a zero expert adds
    nothing."""
    expand_x = np.ascontiguousarray(expand_x)
    assist_info = np.ascontiguousarray(assist_info, dtype=np.int32)
    ep_recv_count = np.ascontiguousarray(ep_recv_count, dtype=np.int32)
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    expert_scales = np.ascontiguousarray(expert_scales)
    N, K = ids.shape
    W, epr = int(ep_world), int(experts_per_rank)
    bs = N // W
    h = expand_x.shape[1]
    dt = dtype_code(expand_x, bf16)
    want = np.int32 if dt == INT32 else np.float32
    if expert_scales.dtype != want:
        raise OracleError("scales must be %s for this dtype" % np.dtype(want))
    x_out = np.zeros((N, h), expand_x.dtype)
    m, mk = _mask(mask, N, K)
    ox = None if ori_x is None else np.ascontiguousarray(ori_x)   # kept alive across the call
    if ox is not None:
        assert ox.shape == (N, h) and ox.dtype.itemsize == expand_x.dtype.itemsize
    cx = None if const_x is None else np.ascontiguousarray(const_x)
    if cx is not None:
        assert cx.shape == (int(const_experts), h) and cx.dtype.itemsize == expand_x.dtype.itemsize
    rc = _load().oracle_combine(_ptr(expand_x), _ptr(assist_info), _ptr(ep_recv_count), _ptr(ids),
                                _ptr(expert_scales), W, bs, epr, h, K, dt, _ptr(m), mk, int(zero_experts),
                                int(copy_experts), int(const_experts), _ptr(ox), _ptr(cx), _ptr(x_out))
    if rc != 0:
        raise OracleError("oracle_combine returned %d" % rc)
    return x_out


def large_segments(ep_recv_count, ep_world, experts_per_rank, h, elem_bytes, threshold_bytes):
    """Flags [W, epr*W] (uint8) of the segments the large-segment predicate selects."""
    erc = np.ascontiguousarray(ep_recv_count, dtype=np.int32)
    W, epr = int(ep_world), int(experts_per_rank)
    flags = np.zeros((W, epr * W), np.uint8)
    _load().oracle_large_segments(_ptr(erc), W, epr, int(h), int(elem_bytes), int(threshold_bytes),
                                  _ptr(flags))
    return flags


def f16_to_f32(bits: int) -> float:
    return _load().oracle_f16_to_f32(bits)


def f32_to_f16(v: float) -> int:
    return _load().oracle_f32_to_f16(v)


def bf16_to_f32(bits: int) -> float:
    return _load().oracle_bf16_to_f32(bits)


def f32_to_bf16(v: float) -> int:
    return _load().oracle_f32_to_bf16(v)


def identity_expert(expand_x, dynamic_scales=None):
    """The harness's identity expert (not part of the method): returns expand_x
    unchanged, or the dequantised rows bf16(f32(q) * scale) as uint16 bits (one
    fp32 product, one rounding): int8 rows with one scale per row, E4M3 rows
    (uint8) with one fp32 scale per 128-element group, or E4M3 rows with one
    E8M0 byte (uint8, the scale 2^(byte - 127)) per 32-element block."""
    if dynamic_scales is None:
        return expand_x
    if np.asarray(dynamic_scales).dtype == np.uint8:
        q = np.ascontiguousarray(expand_x, dtype=np.uint8)
        sc = np.ascontiguousarray(dynamic_scales)
        assert sc.shape == (q.shape[0], (q.shape[1] + 31) // 32)
        y = np.zeros(q.shape, np.uint16)
        _load().oracle_identity_expert_dequant_mx(_ptr(q), _ptr(sc), q.shape[0], q.shape[1], _ptr(y))
        return y
    if np.asarray(dynamic_scales).ndim == 2:
        q = np.ascontiguousarray(expand_x, dtype=np.uint8)
        sc = np.ascontiguousarray(dynamic_scales, dtype=np.float32)
        y = np.zeros(q.shape, np.uint16)
        _load().oracle_identity_expert_dequant_fp8(_ptr(q), _ptr(sc), q.shape[0], q.shape[1], _ptr(y))
        return y
    q = np.ascontiguousarray(expand_x, dtype=np.int8)
    sc = np.ascontiguousarray(dynamic_scales, dtype=np.float32)
    y = np.zeros(q.shape, np.uint16)
    _load().oracle_identity_expert_dequant(_ptr(q), _ptr(sc), q.shape[0], q.shape[1], _ptr(y))
    return y


def e4m3_to_f32(code: int) -> float:
    return _load().oracle_e4m3_to_f32(code)


def f32_to_e4m3(v: float) -> int:
    """Nearest E4M3 code (ties to even) of a float with |v| <= 448."""
    return _load().oracle_f32_to_e4m3(v)
