"""moe_dispatch_noalloc: the allocation-free dispatch (the library's own per-GPU scratch in
place of a workspace) gives moe_dispatch's outputs bit for bit, on consecutive calls that
leave the scratch holding the previous call's contents (the second call smaller than the
first), in a fresh process or after the other tests. A shape whose workspace exceeds the
scratch is refused before anything runs (host only)."""
import ctypes

import numpy as np
import pytest
import torch

import combine_ep_recv_amd as moe
import workloads as wl

DEV = "cuda"


def _bufs(w, esc):
    tdt = {"int32": torch.int32, "fp16": torch.float16, "bf16": torch.bfloat16}[w.dtype]
    b = moe.DispatchBuffers(w.ep_world, w.bs, w.experts_per_rank, w.h, w.topk, tdt, w.quant_mode, DEV,
                            with_expand_scales=esc)
    for t in (b.expand_x, b.dynamic_scales, b.assist_info, b.ep_recv_count, b.expand_scales):
        if t is not None:
            t.view(torch.uint8).fill_(0xA5)           # untouched rows must agree too
    return b


def _np(t):
    return None if t is None else t.detach().cpu().view(torch.uint8).numpy()


CASES = [
    # the 16-rank int8 workload: route + per-token quantiser (chunk prefixes in the scratch)
    (wl.BY_NAME["w16_h7168_bf16_q8"], None),
    # smaller, through the segment schedule (plan and offsets in the scratch)
    (wl.custom(4, 300, 1024, 4, 3, "fp16", "zipf_topk", name="fp16_segment_schedule"),
     dict(mode=moe.MOE_SCHED_SEGMENT, large_segment_bytes=0)),
    # smaller still, with a token mask and more than 64 route chunks (the single-block scan)
    (wl.custom(80, 260, 64, 4, 2, "bf16", "gauss_topk", quant_mode=2, name="bf16_scan_path"), "mask"),
    # MXFP8 (uint8 scale bytes), smaller again
    (wl.custom(8, 40, 2048, 8, 4, "fp16", "zipf_topk", quant_mode=4, name="fp16_mx"), None),
    # the adaptive schedule with its large-segment pass engaged (row flags in the scratch)
    (wl.custom(4, 64, 1024, 8, 4, "bf16", "zipf_topk", quant_mode=2, name="bf16_adaptive_T0"),
     dict(mode=moe.MOE_SCHED_ADAPTIVE, large_segment_bytes=0)),
]


@pytest.mark.gpu
def test_noalloc_dispatch_matches_dispatch_on_consecutive_calls():
    for w, extra in CASES:
        print("no-alloc case %s W=%d bs=%d h=%d K=%d q%d" % (w.name, w.ep_world, w.bs, w.h, w.topk, w.quant_mode),
              flush=True)
        inp = wl.make_inputs(w)
        bf = w.dtype == "bf16"
        x = torch.from_numpy(inp["x"].view(np.int16) if bf else inp["x"]).to(DEV)
        x = x.view(torch.bfloat16) if bf else x
        ids = torch.from_numpy(inp["ids"]).to(DEV)
        sc = torch.from_numpy(inp["scales"]).to(DEV)
        kw = dict(expert_scales=sc)
        if isinstance(extra, dict):
            kw["schedule"] = moe.MoeSchedule(**extra)
        elif extra == "mask":
            kw["x_active_mask"] = torch.from_numpy(np.random.default_rng(5).random(w.num_tokens) < 0.7).to(DEV)
        a, b = _bufs(w, True), _bufs(w, True)
        moe.dispatch_into(a, x, ids, **kw)
        moe.dispatch_noalloc_into(b, x, ids, **kw)
        torch.cuda.synchronize()
        for name in ("expand_x", "dynamic_scales", "assist_info", "ep_recv_count", "expand_scales"):
            ga, gb = _np(getattr(a, name)), _np(getattr(b, name))
            assert (ga is None) == (gb is None), name
            if ga is not None:
                assert ga.tobytes() == gb.tobytes(), (w.name, name)


def test_noalloc_refuses_shapes_beyond_its_scratch():
    # 16 ranks x 65536 tokens, top-8: the per-pair ranks alone take 32 MiB
    n = ctypes.c_size_t(0)
    lib = moe.library()
    assert lib.moe_dispatch_workspace_size(16, 65536, 16, 64, 8, 2, 0, ctypes.byref(n)) == moe.MOE_OK
    assert n.value > moe.NOALLOC_SCRATCH_BYTES
    A = 1 << 20
    P = ctypes.c_void_p
    rc = lib.moe_dispatch_noalloc(P(A), P(2 * A), None, None, 0, None, 16, 65536, 16, 64, 8, 2, 0, None,
                                  ctypes.c_int64(0), P(3 * A), None, P(4 * A), P(5 * A), None, None, None)
    assert rc == moe.MOE_ERR_WORKSPACE, moe.status_str(rc)
    # and invalid scalars are reported as by moe_dispatch
    rc = lib.moe_dispatch_noalloc(P(A), P(2 * A), None, None, 0, None, 1, 4, 2, 16, 1, 1, 0, None,
                                  ctypes.c_int64(0), P(3 * A), None, P(4 * A), P(5 * A), None, None, None)
    assert rc == moe.MOE_ERR_SHAPE
