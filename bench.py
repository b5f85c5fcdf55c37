#!/usr/bin/env python3
"""Dispatch + combine throughput on one MI355X.

One step = moe_dispatch (rows and payload, with per-token int8 quantisation
on the default workload) + moe_combine (rows, gather and fp32 weighted
reduce) over one batch of synthetic tokens, inputs resident in HBM. The
expert between them is the identity expert; its output (bf16(q * scale) for
int8 rows) is produced once, before timing, as an input of combine.

Timing (the measurement protocol of the pages' perf runs: warm-up, then
timed loops): --warmup untimed steps, then exactly --steps timed steps. Before
each timed step an untimed 1 GiB read evicts L2 and the 256 MB Infinity
Cache; each step is bracketed by two HIP events on the stream the kernels run
on (launch gaps included), and the loop is synchronised before and after.
`value` is the algorithmic bytes over the median step. Reported beside it:
the minimum, the same steps back to back without eviction (warm), each call
alone back to back, the steps replayed from a HIP graph, and a 1 GiB
device-to-device copy measured in the same process, as the practical
ceiling. The combine is the dominant launch and gives the roofline figure.

    python bench.py [--steps 50] [--warmup 5] [--workload w16_h7168_bf16_q8]

Prints ONE JSON line.
"""
from __future__ import annotations

import argparse
import dataclasses
import json
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads as wl  # noqa: E402

METRIC = "dispatch+combine effective HBM GB/s (and % roofline), tokens/s at h=7168"
HBM_PEAK_GBPS = 8000.0


def algorithmic_bytes(w: wl.Workload, inp=None):
    """Bytes the method must move, each array once.

    dispatch: read x once (tokens with a row) + ids (+ the mask); write
              expand_x, assist_info, ep_recv_count (+ dynamic_scales when
              quantising dynamically; + the static coefficients read once for
              quantMode 1)
    combine:  read expand_x (expert output), scales, assist_info,
              ep_recv_count, ids (+ the mask, + the token of each copy-expert
              pair); write x_out

    Only pairs that get a row move a row: with a token mask or special experts
    the counts come from the inputs (made here when not given).
    """
    N, K, h, rows = w.num_tokens, w.topk, w.h, w.rows
    sx = 4 if w.dtype == "int32" else 2
    s_exp = 1 if w.quant_mode else sx             # int8 or E4M3 codes
    s_y = 2 if w.quant_mode else sx               # identity-expert output for quantised rows is bf16
    erc = w.ep_world * w.num_experts * 4
    toks, copies, mask_b = N, 0, 0
    if w.mask != "none" or w.zero_experts or w.copy_experts or w.const_experts:
        inp = inp if inp is not None else wl.make_inputs(w)
        ids, E = inp["ids"], w.num_experts
        act = np.ones((N, K), bool)
        if "mask" in inp:
            m = inp["mask"].astype(bool)
            act = np.broadcast_to(m[:, None], (N, K)) if m.ndim == 1 else m
            mask_b = inp["mask"].size
        real = act & (ids < E)
        rows, toks = int(real.sum()), int(real.any(axis=1).sum())
        copies = int((act & (ids >= E + w.zero_experts) & (ids < E + w.zero_experts + w.copy_experts)).sum())
    n_scales = {2: rows, 3: rows * ((h + 127) // 128)}.get(w.quant_mode, 0)   # fp32 dynamic scales
    if w.quant_mode == 1:                         # fp32 static coefficients, read
        n_scales = {"scalar": 1, "column": h, "expert": w.num_experts * h}[w.static_scales]
    scale_b = n_scales * 4
    if w.quant_mode == 4:                         # one E8M0 byte per 32-element block
        scale_b = rows * ((h + 31) // 32)
    disp = toks * h * sx + N * K * 4 + mask_b + rows * h * s_exp + rows * 12 + erc + scale_b
    consts = w.const_experts * h * s_y           # the const experts' outputs, read once
    comb = (rows * h * s_y + copies * h * s_y + consts + N * K * 4 + mask_b + rows * 12 + erc + N * K * 4
            + N * h * s_y)
    return disp, comb


def _device_inputs(w, torch):
    inp = wl.make_inputs(w)
    bf = w.dtype == "bf16"
    x = torch.from_numpy(inp["x"].view(np.int16) if bf else inp["x"]).cuda()
    if bf:
        x = x.view(torch.bfloat16)
    return inp, x, torch.from_numpy(inp["ids"]).cuda(), torch.from_numpy(inp["scales"]).cuda()


class StepEvents:
    """Timing events for the per-step samples: HIP events created with hipEventDisableSystemFence,
    recorded on torch's current stream. The timestamps are the same device clock as torch's events;
    without the system-scope fence a pair around nothing reads 1.5 us less (5.4 against 3.9 us on
    an MI355X), overhead that would otherwise sit in every sample. `n` pairs; pairs(i) -> (a, b)."""
    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self, torch, n):
        import ctypes
        self.torch, self.ct = torch, ctypes
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.ev = []
        for _ in range(2 * n):
            e = ctypes.c_void_p()
            if self.hip.hipEventCreateWithFlags(ctypes.byref(e), ctypes.c_uint(self.DISABLE_SYSTEM_FENCE)) != 0:
                raise RuntimeError("hipEventCreateWithFlags failed")
            self.ev.append(e)

    def record(self, i, which):
        stream = self.ct.c_void_p(self.torch.cuda.current_stream().cuda_stream)
        if self.hip.hipEventRecord(self.ev[2 * i + which], stream) != 0:
            raise RuntimeError("hipEventRecord failed")

    def ms(self, i):
        out = self.ct.c_float()
        if self.hip.hipEventElapsedTime(self.ct.byref(out), self.ev[2 * i], self.ev[2 * i + 1]) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return out.value

    def close(self):
        for e in self.ev:
            self.hip.hipEventDestroy(e)
        self.ev = []


QUANT_LABELS = {1: "static int8, one coefficient per %s", 2: "per-token dynamic int8",
                3: "per-group (128) dynamic fp8 e4m3", 4: "mx: e4m3 codes, one e8m0 scale byte per 32"}


def quant_label(w):
    lab = QUANT_LABELS.get(w.quant_mode, "none")
    if w.quant_mode == 1:
        lab %= {"scalar": "dispatch", "column": "column", "expert": "expert and column"}[w.static_scales]
    return lab


def measure(w, steps, warmup, flush, torch, moe, schedule=None):
    inp, x, ids, sc = _device_inputs(w, torch)
    tdt = {"int32": torch.int32, "fp16": torch.float16, "bf16": torch.bfloat16}[w.dtype]
    W, epr = w.ep_world, w.experts_per_rank
    qs = torch.from_numpy(inp["quant_scales"]).cuda() if w.quant_mode == 1 else None
    buf = moe.DispatchBuffers(W, w.bs, epr, w.h, w.topk, tdt, w.quant_mode, "cuda")
    # token mask and special experts (the copy experts' tokens: x itself, bf16 like the expert output;
    # the const experts' outputs in the combine's dtype)
    extra = dict(x_active_mask=torch.from_numpy(inp["mask"]).cuda() if "mask" in inp else None,
                 zero_experts=w.zero_experts, copy_experts=w.copy_experts, const_experts=w.const_experts)
    ori = dict(ori_x=x) if w.copy_experts else {}
    if w.const_experts:
        cx = torch.from_numpy(inp["const_x"].view(np.int16) if inp["const_x"].dtype == np.uint16
                              else inp["const_x"]).cuda()
        ori["const_x"] = cx.view(torch.bfloat16) if inp["const_x"].dtype == np.uint16 else cx
    dx = dict(extra, schedule=schedule) if schedule is not None else extra     # dispatch only
    moe.dispatch_into(buf, x, ids, quant_scales=qs, **dx)
    if w.quant_mode == 1:                      # static codes: the expert sees bf16(q)
        y = buf.expand_x.to(torch.bfloat16)
    elif w.quant_mode == 2:
        y = (buf.expand_x.float() * buf.dynamic_scales[:, None]).to(torch.bfloat16)
    elif w.quant_mode == 3:                    # one scale per 128-element group
        sc_full = buf.dynamic_scales.repeat_interleave(128, dim=1)[:, :w.h]
        y = (buf.expand_x.float() * sc_full).to(torch.bfloat16)
        del sc_full
    elif w.quant_mode == 4:                    # 2^(byte - 127) per 32-element block, from its bits
        b = buf.dynamic_scales.to(torch.int32)
        s32 = torch.where(b > 0, (b << 23).view(torch.float32), torch.full(b.shape, 2.0 ** -127, device="cuda"))
        y = (buf.expand_x.float() * s32.repeat_interleave(32, dim=1)[:, :w.h]).to(torch.bfloat16)
        del b, s32
    else:
        y = buf.expand_x                       # identity expert: combine reads dispatch's rows
    x_out = torch.empty((w.num_tokens, w.h), dtype=y.dtype, device="cuda")
    cws = moe.combine_workspace(W, w.bs, epr, w.h, w.topk, y.dtype)

    def step():
        moe.dispatch_into(buf, x, ids, quant_scales=qs, **dx)
        moe.combine_into(x_out, y, buf.assist_info, buf.ep_recv_count, ids, sc, W, epr, cws, **extra, **ori)

    def b2b(fn, n):
        """mean ms of n back-to-back calls between two events (one event bubble amortised over n)"""
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    # the timed region: exactly `steps` steps, each after an untimed eviction of L2 and the
    # Infinity Cache (a 1 GiB read) and bracketed by its own events; synchronised on both sides
    ev = StepEvents(torch, steps)
    torch.cuda.synchronize()
    for i in range(steps):
        flush.max()
        ev.record(i, 0)
        step()
        ev.record(i, 1)
    torch.cuda.synchronize()
    cold = [ev.ms(i) for i in range(steps)]
    # the same events around nothing after the same eviction: the overhead inside each sample
    for i in range(steps):
        flush.max()
        ev.record(i, 0)
        ev.record(i, 1)
    torch.cuda.synchronize()
    empty = statistics.median(ev.ms(i) for i in range(steps))
    ev.close()
    # warm: the same steps back to back between two events
    ms_step = b2b(step, steps)
    # each half alone, back to back (the combine is the dominant launch)
    ms_disp = b2b(lambda: moe.dispatch_into(buf, x, ids, quant_scales=qs, **dx), steps)
    ms_comb = b2b(lambda: moe.combine_into(x_out, y, buf.assist_info, buf.ep_recv_count, ids, sc, W, epr, cws,
                                           **extra, **ori),
                  steps)
    # the same steps captured once in a HIP graph and replayed (no host work per launch); reported
    # beside the eager figure, which stays the headline
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(steps):
            step()
    graph.replay()                        # the first replays of a fresh graph run slower: warm up twice
    graph.replay()
    ms_graph = b2b(graph.replay, 3) / steps
    del graph
    return dict(step=ms_step, disp=ms_disp, comb=ms_comb, cold=cold, graph=ms_graph, empty=empty)


def code_hash(path):
    """sha256 of a C/C++/HIP source with its comments removed and whitespace collapsed:
    it changes whenever the code can change, and not for an edited comment."""
    import hashlib

    text, out, i = open(path, encoding="utf-8").read(), [], 0
    n = len(text)
    while i < n:
        c = text[i]
        if c in "\"'":                                  # string or character literal, kept verbatim
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            i = text.find("\n", i)
            i = n if i < 0 else i
        elif text.startswith("/*", i):
            i = text.find("*/", i + 2)
            i = n if i < 0 else i + 2
            out.append(" ")
        else:
            out.append(c)
            i += 1
    code = " ".join("".join(out).split())
    return hashlib.sha256(code.encode("utf-8")).hexdigest()


def counted_traffic(w):
    """HBM bytes per moe_combine launch from the committed rocprofv3 FETCH_SIZE / WRITE_SIZE
    runs (profiles/), or None when the kernel code has changed since they were taken."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic_%s.json" % w.name)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if code_hash(os.path.join(ROOT, rec["source"])) != rec["source_code_sha256"]:
        return None
    return rec["per_launch_bytes"]["moe_combine"]


def combine_kernel(w) -> str:
    """The kernel(s) one moe_combine call launches for this workload's shape: the one-launch
    combine up to 2^16 pairs and 1024 pairs per source rank (rows in 16-byte pieces, topk <= 16),
    else the slot pass and the gather."""
    dt = "BF16" if (w.dtype == "bf16" or w.quant_mode != 0) else ("F16" if w.dtype == "fp16" else "int")
    es = 4 if dt == "int" else 2
    if (w.h * es) % 16 == 0 and w.topk <= 16 and w.rows <= 65535 and w.bs * w.topk <= 1024:
        pre = w.ep_world * w.num_experts <= 2048
        return "combine_fused_kernel<%s,%d,%s>" % (dt, 8 if w.topk <= 8 else 16, "true" if pre else "false")
    vec = (w.h * es) % 16 == 0
    gather = ("combine_gather_i32_kernel<%s>" % ("true" if vec else "false") if dt == "int"
              else "combine_gather_half_kernel<%s,%s>" % (dt, "true" if vec else "false"))
    return "combine_slots_kernel + " + gather


def cpu_model() -> str:
    """The host CPU's model name from /proc/cpuinfo ("unknown" when absent)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, reps=5):
    """The oracle as it stands (single-threaded C), timed on the host: 1 warm-up + the median
    of `reps` full steps; beside it the all-cores C baseline (oracle/moe_cpu_threads.c, whose
    outputs a CPU test checks against the oracle) on the same inputs, where it covers the
    workload (copies and per-token int8)."""
    import oracle
    from oracle import cpu_threads

    inp = wl.make_inputs(w)
    bf = w.dtype == "bf16"
    qs = inp.get("quant_scales")
    d = oracle.dispatch(inp["x"], inp["ids"], w.ep_world, w.experts_per_rank, w.quant_mode, bf16=bf,
                        quant_scales=qs)
    y = oracle.identity_expert(d["expand_x"], d["dynamic_scales"] if w.quant_mode != 1
                               else np.ones(w.rows, np.float32))
    out_bf = bf or w.quant_mode != 0

    def one():
        d = oracle.dispatch(inp["x"], inp["ids"], w.ep_world, w.experts_per_rank, w.quant_mode, bf16=bf,
                            quant_scales=qs)
        oracle.combine(y, d["assist_info"], d["ep_recv_count"], inp["ids"], inp["scales"], w.ep_world,
                       w.experts_per_rank, bf16=out_bf)

    def med(fn):
        fn()
        times = []
        for _ in range(reps):
            t0 = time.perf_counter()
            fn()
            times.append(time.perf_counter() - t0)
        return statistics.median(times)

    disp_b, comb_b = algorithmic_bytes(w)
    t1 = med(one)
    out = {"value": round((disp_b + comb_b) / t1 / 1e9, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
           "sample": "one full %s step (dispatch + combine, %d tokens), 1 warm-up + median of %d, single-threaded "
                     "C oracle (gcc -O2), identity-expert dequantisation untimed; %.3f s/step"
                     % (w.name, w.num_tokens, reps, t1),
           "cpu_model": cpu_model(), "cpu_count": os.cpu_count()}
    if w.quant_mode in (0, 2) and w.mask == "none" and not (w.zero_experts or w.copy_experts or w.const_experts):
        n = cpu_threads.default_threads()

        def many():
            c = cpu_threads.dispatch(inp["x"], inp["ids"], w.ep_world, w.experts_per_rank, w.quant_mode, bf16=bf,
                                     threads=n)
            cpu_threads.combine(y, c["assist_info"], inp["scales"], w.ep_world, bf16=out_bf, threads=n)

        tn = med(many)
        out["all_cores"] = {"value": round((disp_b + comb_b) / tn / 1e9, 3), "unit": "GB/s", "cores": n,
                            "kind": "threaded C baseline (same arithmetic, checked against the oracle)",
                            "sample": "the same step, payload and sums split over %d threads; %.3f s/step"
                                      % (n, tn)}
    return out


def copy_ceiling(torch, n_bytes=1 << 30, reps=5):
    """GB/s of a plain device-to-device copy of n_bytes (read + write counted), best of reps after
    one warm-up copy: the practical ceiling that streaming kernels meet on this GPU."""
    src = torch.empty(n_bytes, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    dst.copy_(src)
    best = None
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        best = ms if best is None else min(best, ms)
    del src, dst
    return 2 * n_bytes / (best * 1e-3) / 1e9


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="w16_h7168_bf16_q8", choices=sorted(wl.BY_NAME))
    ap.add_argument("--bs", type=int, default=None,
                    help="tokens per rank for the main workload (same seed and recipe; default: the workload's)")
    ap.add_argument("--schedule", choices=["adaptive", "token", "segment"], default="adaptive",
                    help="dispatch schedule of the main workload: adaptive (the library's default: token-major, "
                         "with whole workgroups for the large segments), token-major only, or segment-major "
                         "(the last two large-segment forms take copies and per-token int8 only)")
    ap.add_argument("--large-bytes", type=int, default=-1,
                    help="large-segment threshold T in bytes for the main workload (default: the README's 2 MiB)")
    ap.add_argument("--h", type=int, default=None,
                    help="hidden size for the main workload (same seed and recipe; default: the workload's)")
    ap.add_argument("--also", default="w8_h7168_fp16_uniform,w8_h7168_fp16_zipf,w16_h7168_bf16_fp8g128,"
                                      "w16_h7168_bf16_mxfp8,w16_h7168_bf16_static_q8,w16_h7168_bf16_q8_pair_mask,"
                                      "w16_h7168_bf16_q8_special",
                    help="comma-separated extra workloads reported under 'also' ('' for none)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 256 MiB device-to-device copy 5 times (HBM counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the expert-parallel ranks are emulated as partitions of one GPU's "
              "HBM, so --gpus %d is not offered (use --gpus 1)." % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch

    import combine_ep_recv_amd as moe

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.calibrate_copy:
        n = 256 << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(7)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibration": "device-to-device copy", "bytes_read": n, "bytes_written": n,
                          "launches": 5}), flush=True)
        return
    moe.library()
    flush = torch.empty(1 << 27, dtype=torch.int64, device="cuda").fill_(1)   # 1 GiB

    w = wl.BY_NAME[args.workload]
    if args.bs is not None and args.bs != w.bs:
        w = dataclasses.replace(w, bs=args.bs, name="%s_bs%d" % (w.name, args.bs))
    if args.h is not None and args.h != w.h:
        w = dataclasses.replace(w, h=args.h, name="%s_h%d" % (w.name, args.h))
    sched = None
    if args.schedule == "segment" and w.quant_mode in (1, 3, 4):
        print("the segment schedule takes copies and per-token int8 only", file=sys.stderr)
        sys.exit(2)
    if args.schedule != "adaptive" or args.large_bytes >= 0:
        mode = {"adaptive": moe.MOE_SCHED_ADAPTIVE, "token": moe.MOE_SCHED_TOKEN,
                "segment": moe.MOE_SCHED_SEGMENT}[args.schedule]
        sched = moe.MoeSchedule(mode=mode, large_segment_bytes=args.large_bytes)
        w = dataclasses.replace(w, name="%s_%s_schedule%s" % (
            w.name, args.schedule, "" if args.large_bytes < 0 else "_T%d" % args.large_bytes))
    r = measure(w, args.steps, args.warmup, flush, torch, moe, sched)
    disp_b, comb_b = algorithmic_bytes(w)
    ms = statistics.median(r["cold"])                 # the protocol's figure: median of the timed steps
    gbps = (disp_b + comb_b) / (ms * 1e-3) / 1e9
    comb_ms = r["comb"]
    comb_gbps = comb_b / (comb_ms * 1e-3) / 1e9

    also = {}
    for name in [n for n in args.also.split(",") if n]:
        wa = wl.BY_NAME[name]
        ra = measure(wa, args.steps, args.warmup, flush, torch, moe)
        da, ca = algorithmic_bytes(wa)
        msa = statistics.median(ra["cold"])
        also[name] = {"ms_per_step": round(msa, 5), "GB/s": round((da + ca) / (msa * 1e-3) / 1e9, 1),
                      "frac_of_hbm_peak": round((da + ca) / (msa * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                      "tokens_per_s": round(wa.num_tokens / (msa * 1e-3), 1),
                      "min_ms": round(min(ra["cold"]), 5),
                      "empty_event_pair_ms": round(ra["empty"], 5),
                      "warm_b2b_ms": round(ra["step"], 5),
                      "warm_b2b_GB/s": round((da + ca) / (ra["step"] * 1e-3) / 1e9, 1),
                      "dispatch_ms": round(ra["disp"], 5), "combine_ms": round(ra["comb"], 5),
                      "graph_ms_per_step": round(ra["graph"], 5),
                      "algorithmic_bytes": da + ca,
                      "quant": quant_label(wa)}
        if wa.mask != "none":
            also[name]["mask"] = {"pair": "per pair, 3/4 active",
                                  "token_prefix": "per token, each rank's first 3/4"}[wa.mask]
        if wa.zero_experts or wa.copy_experts or wa.const_experts:
            also[name]["special_experts"] = {"zero": wa.zero_experts, "copy": wa.copy_experts,
                                             "const": wa.const_experts}
    ceiling = copy_ceiling(torch)

    line = {
        "metric": METRIC, "value": round(gbps, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic, seeded: %s" % ("bf16 N(0,1) tokens, top-8 of N(0,1) router logits, softmax weights"
                                           if w.routing == "gauss_topk" else w.routing),
        "config": {"workload": w.name, "ep_world": w.ep_world, "bs": w.bs, "h": w.h, "topk": w.topk,
                   "experts_per_rank": w.experts_per_rank, "experts": w.num_experts, "tokens": w.num_tokens,
                   "quant": quant_label(w),
                   "combine_input": "bf16 identity-expert output" if w.quant_mode != 0 else w.dtype,
                   "working_set_MB": round((disp_b + comb_b) / 1e6),
                   "algorithmic_bytes": disp_b + comb_b},
        "tokens_per_s": round(w.num_tokens / (ms * 1e-3), 1),
        "frac_of_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4),
        "frac_of_copy_ceiling": round(gbps / ceiling, 4),
        "roofline": {"bound": "hbm", "achieved": round(comb_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(comb_gbps / HBM_PEAK_GBPS, 4), "traffic": counted_traffic(w),
                     "kernel": combine_kernel(w), "scope": "one moe_combine call (the dominant launch), "
                                                           "timed back to back",
                     "bytes_per_launch": comb_b, "avg_launch_ms": round(comb_ms, 5)},
        "timing": {"protocol": "%d warm-up steps, then %d timed steps, each after an untimed 1 GiB read that "
                               "evicts L2 and the Infinity Cache and bracketed by two HIP events on the kernels' "
                               "stream; synchronised before and after; value = median" % (args.warmup, args.steps),
                   "median_ms": round(ms, 5), "min_ms": round(min(r["cold"]), 5),
                   "empty_event_pair_ms": round(r["empty"], 5),
                   "event_note": "HIP events without the system-scope fence; empty_event_pair_ms is the median of "
                                 "the same event pair around nothing after the same eviction, included in every "
                                 "sample",
                   "warm_b2b_ms": round(r["step"], 5),
                   "warm_b2b_GB/s": round((disp_b + comb_b) / (r["step"] * 1e-3) / 1e9, 1),
                   "warm_note": "the same steps back to back between two events, no eviction",
                   "dispatch_ms": round(r["disp"], 5), "combine_ms": round(comb_ms, 5),
                   "graph_ms_per_step": round(r["graph"], 5),
                   "graph_note": "the same %d steps captured once in a HIP graph, replayed twice untimed, then "
                                 "3 timed replays (mean; no host work per launch)" % args.steps,
                   "copy_ceiling_GB/s": round(ceiling, 1),
                   "copy_note": "1 GiB device-to-device copy (read + write), best of 5"},
        "also": also,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
