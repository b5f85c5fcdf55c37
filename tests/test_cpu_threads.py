"""The all-cores CPU baseline (oracle/moe_cpu_threads.c) gives the oracle's outputs bit for bit
(CPU only). It is what the benchmark times on all host cores beside the single-threaded oracle."""
import numpy as np
import pytest

import oracle
from oracle import cpu_threads
import workloads as wl

CASES = [
    wl.WORKLOADS[0], wl.WORKLOADS[1],
    wl.custom(8, 8, 512, 8, 8, "fp16", "gauss_topk", name="fp16_w8"),
    wl.custom(4, 12, 256, 8, 4, "bf16", "zipf_topk", quant_mode=2, name="bf16_q8_zipf"),
    wl.custom(3, 5, 40, 3, 2, "fp16", "gauss_topk", quant_mode=2, name="fp16_q8_ragged"),
]


@pytest.mark.parametrize("threads", [1, 3, 8])
@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
def test_threaded_baseline_matches_the_oracle(w, threads):
    inp = wl.make_inputs(w)
    bf = w.dtype == "bf16"
    d = oracle.dispatch(inp["x"], inp["ids"], w.ep_world, w.experts_per_rank, w.quant_mode, bf16=bf)
    c = cpu_threads.dispatch(inp["x"], inp["ids"], w.ep_world, w.experts_per_rank, w.quant_mode, bf16=bf,
                             threads=threads)
    for key in ("expand_x", "assist_info", "ep_recv_count"):
        assert d[key].tobytes() == c[key].tobytes(), key
    if w.quant_mode:
        assert d["dynamic_scales"].tobytes() == c["dynamic_scales"].tobytes()
    y = oracle.identity_expert(d["expand_x"], d["dynamic_scales"])
    out_bf = bf or w.quant_mode != 0
    want = oracle.combine(y, d["assist_info"], d["ep_recv_count"], inp["ids"], inp["scales"], w.ep_world,
                          w.experts_per_rank, bf16=out_bf)
    got = cpu_threads.combine(y, c["assist_info"], inp["scales"], w.ep_world, bf16=out_bf, threads=threads)
    assert got.tobytes() == want.tobytes()
