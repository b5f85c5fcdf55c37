"""The all-cores CPU baseline (``moe_cpu_threads.c``): NOT the oracle.

Only the ``cpu_baseline`` leg of ``bench.py`` times it, beside the single-
threaded oracle, and ``tests/test_cpu_threads.py`` checks it against the oracle
bit for bit. Built with gcc like the oracle (``-O2 -ffp-contract=off``, no
fast-math) plus ``-pthread``. Covers the benchmark's plain shapes: copies and
per-token int8 (quantMode 2), no masks and no special experts.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

from . import _CFLAGS, _ptr, dtype_code

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_cpu_threads.c")
_LIB = os.path.join(_HERE, "libmoe_cpu_threads.so")
_lib = None


def build(force: bool = False) -> str:
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *_CFLAGS, "-pthread", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        lib = ctypes.CDLL(build())
        P, I = ctypes.c_void_p, ctypes.c_int
        lib.cpu_dispatch_threads.argtypes = [P, P, I, I, I, I, I, I, I, P, P, P, P, I]
        lib.cpu_dispatch_threads.restype = I
        lib.cpu_combine_threads.argtypes = [P, P, P, I, I, I, I, I, P, I]
        lib.cpu_combine_threads.restype = I
        _lib = lib
    return _lib


def default_threads() -> int:
    """The host cores this process may use, at most 16 (a host's share for one GPU)."""
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def dispatch(x, ids, ep_world, experts_per_rank, quant_mode=0, bf16=False, threads=None):
    """Same outputs as oracle.dispatch for copies and quantMode 2 (dict with expand_x,
    dynamic_scales, assist_info, ep_recv_count)."""
    x = np.ascontiguousarray(x)
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    N, h = x.shape
    K = ids.shape[1]
    W, epr = int(ep_world), int(experts_per_rank)
    bs = N // W
    rows = N * K
    if quant_mode == 2:
        expand_x, dyn = np.zeros((rows, h), np.int8), np.zeros((rows,), np.float32)
    elif quant_mode == 0:
        expand_x, dyn = np.zeros((rows, h), x.dtype), None
    else:
        raise ValueError("the threaded baseline takes quant modes 0 and 2")
    assist = np.zeros((rows, 3), np.int32)
    erc = np.zeros((W, epr * W), np.int32)
    rc = _load().cpu_dispatch_threads(_ptr(x), _ptr(ids), W, bs, epr, h, K, dtype_code(x, bf16), int(quant_mode),
                                      _ptr(expand_x), _ptr(dyn), _ptr(assist), _ptr(erc),
                                      int(threads or default_threads()))
    if rc != 0:
        raise RuntimeError("cpu_dispatch_threads returned %d" % rc)
    return dict(expand_x=expand_x, dynamic_scales=dyn, assist_info=assist, ep_recv_count=erc)


def combine(expand_x, assist_info, expert_scales, ep_world, bf16=False, threads=None):
    """Same x_out as oracle.combine for a full dispatch (every pair has a row)."""
    expand_x = np.ascontiguousarray(expand_x)
    assist_info = np.ascontiguousarray(assist_info, dtype=np.int32)
    expert_scales = np.ascontiguousarray(expert_scales)
    N, K = expert_scales.shape
    h = expand_x.shape[1]
    x_out = np.zeros((N, h), expand_x.dtype)
    rc = _load().cpu_combine_threads(_ptr(expand_x), _ptr(assist_info), _ptr(expert_scales), int(ep_world),
                                     N // int(ep_world), h, K, dtype_code(expand_x, bf16), _ptr(x_out),
                                     int(threads or default_threads()))
    if rc != 0:
        raise RuntimeError("cpu_combine_threads returned %d" % rc)
    return x_out
