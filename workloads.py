"""Seeded synthetic inputs for MoE dispatch/combine.

This module is the only thing the oracle side and the HIP side share. It
draws tokens, routings and routing weights; it holds none of the dispatch or
combine arithmetic.

Workloads (shapes and value distributions of the pages' runs):
  * ``w2_h16_int32``  -- 2 ranks, 8 tokens/rank, h=16, top-2, 2 experts/rank,
    int32 tokens in [-100, 100], distinct uniform expert ids, int32 weights in
    [1, 4] (the 2-card functional run of the combine_doubleplane README, 运行).
  * ``w8_h16_int32``  -- 8 ranks, 8 tokens/rank, h=16, top-2, 8 experts/rank
    (64 experts), int32 tokens in [-1000, 1000], as above (the 8-card,
    64-expert functional run).
  * ``w8_h7168_fp16_uniform`` -- 8 ranks, 32 tokens/rank, h=7168, top-8, 8
    experts/rank; fp16 N(0,1) tokens; ids = top-8 of N(0,1) router logits;
    fp32 weights = softmax over the chosen 8 logits (the README's perf shape,
    如何选择使用, with fp16 data).
  * ``w8_h7168_fp16_zipf`` -- as above with expert popularity Zipf(s=1.2):
    logits = z + ln p_e, p_e proportional to (e+1)^-1.2, so expert 0 is the
    most popular and rank 0 the hottest destination.
  * ``w16_h7168_bf16_q8`` -- 16 ranks, 256 tokens/rank, h=7168, top-8, 16
    experts/rank (256 experts); bf16 N(0,1) tokens; per-token dynamic int8
    quantisation in dispatch; combine on bf16 expert outputs; softmax weights.

Static quantisation (quantMode 1) draws its coefficients from a generator of
their own (seed 4321 + index), so a workload keeps its tokens and routing when
only the quantiser changes: c = (127 / 4) * 2^u with u uniform in [-1, 1], one
value, one per column (h) or one per expert and column (E*h). For N(0,1)
tokens 127 / 4 maps |x| = 4 to the edge of the int8 range, so a few codes of a
7168-wide row saturate.

Routing rule for the logit-driven workloads: each token's experts are its 8
largest logits in descending order, ties to the lower id (stable argsort of
-logits); weights are the softmax of those 8 logits in fp32 after subtracting
their max.

Tokens are seeded with ``numpy.random.default_rng(1234 + index)``. bf16 tokens
are fp32 draws rounded to nearest-even by torch's CPU conversion and carried as
uint16 bit patterns (numpy has no bfloat16).
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    index: int
    ep_world: int
    bs: int
    h: int
    topk: int
    experts_per_rank: int
    dtype: str              # "int32" | "fp16" | "bf16"
    routing: str            # "uniform_distinct" | "gauss_topk" | "zipf_topk"
    quant_mode: int = 0
    x_lo: int = 0           # int32 token range (inclusive)
    x_hi: int = 0
    zipf_s: float = 1.2
    zero_experts: int = 0   # special experts after the E real ones: ids E .. E+zero-1
    copy_experts: int = 0   # then E+zero .. E+zero+copy-1
    const_experts: int = 0  # then E+zero+copy .. E+zero+copy+const-1
    static_scales: str = "expert"   # quantMode 1 coefficients: "scalar" | "column" | "expert"
    mask: str = "none"      # token mask: "none" | "token_prefix" (each rank's first 3/4 of its tokens)
                            # | "pair" (each pair active with probability 3/4)

    @property
    def num_experts(self) -> int:
        return self.ep_world * self.experts_per_rank

    @property
    def num_tokens(self) -> int:
        return self.ep_world * self.bs

    @property
    def rows(self) -> int:
        return self.num_tokens * self.topk


WORKLOADS = [
    Workload("w2_h16_int32", 0, 2, 8, 16, 2, 2, "int32", "uniform_distinct", x_lo=-100, x_hi=100),
    Workload("w8_h16_int32", 1, 8, 8, 16, 2, 8, "int32", "uniform_distinct", x_lo=-1000, x_hi=1000),
    Workload("w8_h7168_fp16_uniform", 2, 8, 32, 7168, 8, 8, "fp16", "gauss_topk"),
    Workload("w8_h7168_fp16_zipf", 3, 8, 32, 7168, 8, 8, "fp16", "zipf_topk"),
    Workload("w16_h7168_bf16_q8", 4, 16, 256, 7168, 8, 16, "bf16", "gauss_topk", quant_mode=2),
]
# Not a page workload: the 16-rank one (same seed, so the same tokens and routing)
# with per-group FP8 E4M3 quantisation (quantMode 3) instead of per-token int8.
EXTRA_WORKLOADS = [
    Workload("w16_h7168_bf16_fp8g128", 4, 16, 256, 7168, 8, 16, "bf16", "gauss_topk", quant_mode=3),
    # and with MX quantisation (quantMode 4: MXFP8, E4M3 codes and one E8M0 byte per 32 elements)
    Workload("w16_h7168_bf16_mxfp8", 4, 16, 256, 7168, 8, 16, "bf16", "gauss_topk", quant_mode=4),
    # and with static int8 quantisation (quantMode 1), one coefficient per expert and column
    Workload("w16_h7168_bf16_static_q8", 4, 16, 256, 7168, 8, 16, "bf16", "gauss_topk", quant_mode=1),
    # per-token int8 with a per-pair token mask (3/4 of the pairs active)
    Workload("w16_h7168_bf16_q8_pair_mask", 4, 16, 256, 7168, 8, 16, "bf16", "gauss_topk", quant_mode=2,
             mask="pair"),
    # per-token int8 with 16 zero, 16 copy and 16 const experts beside the 256 real ones (the router
    # picks among 304)
    Workload("w16_h7168_bf16_q8_special", 4, 16, 256, 7168, 8, 16, "bf16", "gauss_topk", quant_mode=2,
             zero_experts=16, copy_experts=16, const_experts=16),
]
BY_NAME = {w.name: w for w in WORKLOADS + EXTRA_WORKLOADS}


def custom(ep_world, bs, h, topk, experts_per_rank, dtype="int32", routing="uniform_distinct",
           quant_mode=0, x_lo=-1000, x_hi=1000, name="custom", index=100, zero_experts=0, copy_experts=0,
           static_scales="expert", const_experts=0):
    """A workload of arbitrary shape, for edge-case tests. zero_experts / copy_experts /
    const_experts add special expert ids after the E real ones, drawn by the routing like
    any other."""
    return Workload(name, index, ep_world, bs, h, topk, experts_per_rank, dtype, routing,
                    quant_mode=quant_mode, x_lo=x_lo, x_hi=x_hi, zero_experts=zero_experts,
                    copy_experts=copy_experts, static_scales=static_scales, const_experts=const_experts)


def static_scales(w: Workload) -> np.ndarray:
    """quantMode 1 coefficients (fp32): 1, h or E*h values, from their own generator."""
    n = {"scalar": 1, "column": w.h, "expert": w.num_experts * w.h}[w.static_scales]
    u = np.random.default_rng(4321 + w.index).uniform(-1.0, 1.0, size=n)
    return (31.75 * np.exp2(u)).astype(np.float32)


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 draws to bf16 (nearest-even) with torch's CPU cast."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def _routing(w: Workload, rng: np.random.Generator):
    N, K = w.num_tokens, w.topk
    E = w.num_experts + w.zero_experts + w.copy_experts + w.const_experts   # every id the router can pick
    if w.routing == "uniform_distinct":
        ids = np.stack([rng.permutation(E)[:K] for _ in range(N)]).astype(np.int32) if N else \
            np.zeros((0, K), np.int32)
        return ids, None
    logits = rng.standard_normal((N, E)).astype(np.float32)
    if w.routing == "zipf_topk":
        p = (np.arange(1, E + 1, dtype=np.float64) ** -w.zipf_s)
        p /= p.sum()
        logits = (logits + np.log(p).astype(np.float32)).astype(np.float32)
    elif w.routing != "gauss_topk":
        raise ValueError(w.routing)
    order = np.argsort(-logits, axis=1, kind="stable")[:, :K]
    ids = order.astype(np.int32)
    chosen = np.take_along_axis(logits, order, axis=1).astype(np.float32)
    z = np.exp(chosen - chosen.max(axis=1, keepdims=True), dtype=np.float32)
    weights = (z / z.sum(axis=1, keepdims=True, dtype=np.float32)).astype(np.float32)
    return ids, weights


def make_inputs(w: Workload, seed: Optional[int] = None) -> dict:
    """Seeded tokens, expert ids and routing weights for a workload.

    Returns a dict with:
      x        [N, h]  int32 | float16 | uint16 (bf16 bits)
      ids      [N, K]  int32
      scales   [N, K]  int32 for int32 tokens (uniform in [1, 4]), else fp32
      quant_scales     fp32 quantMode 1 coefficients (only for quantMode 1)
      mask     uint8 [N] or [N, K] token mask (only when the workload has one;
               drawn after everything else, so the other inputs do not change)
      const_x  [const_experts, h] the const experts' outputs, in the combine's dtype
               (the token dtype, or bf16 bits when dispatch quantises): int32 in the
               token range, else N(0,1); drawn last (only with const experts)
    """
    rng = np.random.default_rng(1234 + w.index if seed is None else seed)
    N, h = w.num_tokens, w.h
    ids, weights = _routing(w, rng)
    if w.dtype == "int32":
        x = rng.integers(w.x_lo, w.x_hi + 1, size=(N, h), dtype=np.int64).astype(np.int32)
        scales = rng.integers(1, 5, size=(N, w.topk), dtype=np.int64).astype(np.int32)
        if weights is not None:
            raise ValueError("int32 workloads use integer weights")
    else:
        g = rng.standard_normal((N, h)).astype(np.float32)
        x = g.astype(np.float16) if w.dtype == "fp16" else f32_to_bf16_bits(g)
        scales = weights if weights is not None else \
            rng.uniform(0.0, 1.0, size=(N, w.topk)).astype(np.float32)
    out = dict(x=x, ids=ids, scales=scales)
    if w.quant_mode == 1:
        out["quant_scales"] = static_scales(w)
    if w.mask == "token_prefix":
        m = np.zeros(N, np.uint8)
        for s in range(w.ep_world):
            m[s * w.bs: s * w.bs + (3 * w.bs) // 4] = 1
        out["mask"] = m
    elif w.mask == "pair":
        out["mask"] = (rng.random((N, w.topk)) < 0.75).astype(np.uint8)
    elif w.mask != "none":
        raise ValueError(w.mask)
    if w.const_experts:
        shape = (w.const_experts, h)
        if w.dtype == "int32":
            out["const_x"] = rng.integers(w.x_lo, w.x_hi + 1, size=shape, dtype=np.int64).astype(np.int32)
        else:
            g = rng.standard_normal(shape).astype(np.float32)
            out["const_x"] = g.astype(np.float16) if (w.dtype == "fp16" and not w.quant_mode) else f32_to_bf16_bits(g)
    return out
