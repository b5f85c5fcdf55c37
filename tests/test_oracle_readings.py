"""Pins of the oracle's arithmetic readings (CPU only).

Three hand-worked fixtures under tests/golden/ fix the readings that decide
single bits of the outputs:
  * quant_int8_quotient.json -- quantMode 2 ("aclnnMoeDistributeDispatchV4",
    参数说明): q = rint(RN32(x / scale)), scale = RN32(max|x| / 127);
  * quant_fp8_quotient.json  -- quantMode 3 (same page): E4M3 of RN32(|x| / scale),
    scale = RN32(group max / 448);
  * combine_fma_order.json   -- the check formula of the combine_doubleplane
    README (功能说明), summed in fp32 with one fused multiply-add per k, k
    ascending, one rounding to the output type.

Each test (a) runs the oracle on the fixture and compares bit for bit, and
(b) re-derives every stored value from exact rational arithmetic, so a stored
value that does not follow from the mathematics fails as well. The planted-
mistake tests then build copies of oracle/moe_oracle.c with one plausible
mistake each (a reciprocal instead of a quotient, a float64 quotient, rounding
ties away from zero, a rounded product before the add, the k loop reversed),
and check that every copy fails at least one fixture, while an unaltered copy
built the same way passes them all.
"""
from __future__ import annotations

import ctypes
import json
import os
import struct
import subprocess
from fractions import Fraction as Fr

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# --------------------------------------------------------------------------
# exact arithmetic: nearest binary floating-point value (ties to even) with
# `frac` fraction bits and smallest normal exponent `emin`
# --------------------------------------------------------------------------

def round_binary(v: Fr, frac: int, emin: int) -> Fr:
    if v == 0:
        return Fr(0)
    a = abs(v)
    e = 0
    while a >= 2:
        a /= 2
        e += 1
    while a < 1:
        a *= 2
        e -= 1
    quantum = Fr(2) ** (max(e, emin) - frac)
    m = abs(v) / quantum
    n = m.numerator // m.denominator
    rest = m - n
    if rest > Fr(1, 2) or (rest == Fr(1, 2) and n % 2 == 1):
        n += 1
    return (1 if v > 0 else -1) * n * quantum


def rn32(v):
    return round_binary(Fr(v), 23, -126)


def rn16(v):
    return round_binary(Fr(v), 10, -14)


def rnbf16(v):
    return round_binary(Fr(v), 7, -126)


def rint_even(v: Fr) -> int:
    n = v.numerator // v.denominator
    rest = v - n
    if rest > Fr(1, 2) or (rest == Fr(1, 2) and n % 2 == 1):
        n += 1
    return n


def f32_hex(v) -> str:
    return struct.pack(">f", float(v)).hex()


def f32_from_hex(s) -> float:
    return struct.unpack(">f", bytes.fromhex(s))[0]


def e4m3_bits(v: Fr) -> int:
    """OCP E4M3 encoding of a value already on the E4M3 grid, |v| <= 448."""
    sign = 0x80 if v < 0 else 0
    a = abs(v)
    if a == 0:
        return sign
    if a < Fr(1, 64):                      # subnormal: f * 2^-9
        f = a * 512
        assert f.denominator == 1 and 0 < f < 8
        return sign | int(f)
    e = 0
    while a >= 2:
        a /= 2
        e += 1
    while a < 1:
        a *= 2
        e -= 1
    f = (a - 1) * 8
    assert f.denominator == 1 and -6 <= e <= 8
    return sign | ((e + 7) << 3) | int(f)


def to_bits(values, dtype):
    a = np.asarray(values, np.float32)
    if dtype == "fp16":
        return a.astype(np.float16)
    import torch

    return torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


# --------------------------------------------------------------------------
# fixture runners: each returns a list of (what, got, want) mismatches
# --------------------------------------------------------------------------

def run_int8_fixture(dtype):
    g = _golden("quant_int8_quotient.json")
    d = g[dtype]
    x = to_bits(d["x"], dtype)
    out = oracle.dispatch(x, np.asarray(g["expert_ids"], np.int32), g["ep_world"], g["experts_per_rank"],
                          quant_mode=2, bf16=dtype == "bf16")
    bad = []
    for row, (s, tok, k) in enumerate(out["assist_info"].tolist()):
        t = s * g["bs"] + tok
        codes = out["expand_x"][row].tolist()
        if codes != d["codes"][t]:
            bad.append(("codes of token %d" % t, codes, d["codes"][t]))
        sc = f32_hex(out["dynamic_scales"][row])
        if sc != d["scales_hex"][t]:
            bad.append(("scale of token %d" % t, sc, d["scales_hex"][t]))
    return bad


def run_fp8_fixture(dtype):
    g = _golden("quant_fp8_quotient.json")
    x = to_bits(g["x"], dtype)
    out = oracle.dispatch(x, np.asarray(g["expert_ids"], np.int32), g["ep_world"], g["experts_per_rank"],
                          quant_mode=3, bf16=dtype == "bf16")
    bad = []
    for row, (s, tok, k) in enumerate(out["assist_info"].tolist()):
        t = s * g["bs"] + tok
        codes = out["expand_x"][row].tolist()
        if codes != g["codes"][t]:
            bad.append(("codes of token %d" % t, codes, g["codes"][t]))
        sc = f32_hex(out["dynamic_scales"][row][0])
        if sc != g["scales_hex"][t]:
            bad.append(("scale of token %d" % t, sc, g["scales_hex"][t]))
    return bad


def combine_fixture_inputs(dtype):
    g = _golden("combine_fma_order.json")
    d = g[dtype]
    ids = np.asarray(g["expert_ids"], np.int32)
    N, K = ids.shape
    W, epr = g["ep_world"], g["experts_per_rank"]
    y = np.asarray(d["y"], np.float32)                         # [N, K]: expert output of pair (t, k)
    w = np.asarray([[f32_from_hex(h) for h in row] for row in d["weights_hex"]], np.float32)
    assist = np.asarray(g["assist_info"], np.int32)
    erc = np.asarray(g["ep_recv_count"], np.int32)
    rows = np.zeros((N * K, g["h"]), np.float32)
    for i, (s, tok, k) in enumerate(assist.tolist()):
        rows[i, :] = y[s * g["bs"] + tok, k]
    return g, d, ids, W, epr, to_bits(rows, dtype), w, assist, erc


def run_combine_fixture(dtype):
    g, d, ids, W, epr, rows, w, assist, erc = combine_fixture_inputs(dtype)
    xo = oracle.combine(rows, assist, erc, ids, w, W, epr, bf16=dtype == "bf16")
    got = np.asarray(xo).view(np.uint16)[:, 0].tolist()
    want = to_bits(np.asarray(d["x_out"], np.float32)[:, None], dtype).view(np.uint16)[:, 0].tolist()
    return [("x_out", got, want)] if got != want else []


FIXTURES = {
    "int8_fp16": lambda: run_int8_fixture("fp16"),
    "int8_bf16": lambda: run_int8_fixture("bf16"),
    "fp8_fp16": lambda: run_fp8_fixture("fp16"),
    "fp8_bf16": lambda: run_fp8_fixture("bf16"),
    "combine_fp16": lambda: run_combine_fixture("fp16"),
    "combine_bf16": lambda: run_combine_fixture("bf16"),
}


# --------------------------------------------------------------------------
# the oracle passes the fixtures, and the fixtures follow from exact arithmetic
# --------------------------------------------------------------------------

@pytest.mark.parametrize("name", sorted(FIXTURES))
def test_oracle_matches_fixture(name):
    assert FIXTURES[name]() == []


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_int8_fixture_follows_from_exact_arithmetic(dtype):
    g = _golden("quant_int8_quotient.json")
    d = g[dtype]
    rn = rn16 if dtype == "fp16" else rnbf16
    for t, xs in enumerate(d["x"]):
        xs = [Fr(v) for v in xs]
        assert all(rn(v) == v for v in xs), "token %d is not exactly representable" % t
        scale = rn32(max(abs(v) for v in xs) / 127)
        assert f32_hex(scale) == d["scales_hex"][t]
        codes = [0 if scale == 0 else max(-127, min(127, rint_even(rn32(v / scale)))) for v in xs]
        assert codes == d["codes"][t], t


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_fp8_fixture_follows_from_exact_arithmetic(dtype):
    g = _golden("quant_fp8_quotient.json")
    rn = rn16 if dtype == "fp16" else rnbf16
    for t, xs in enumerate(g["x"]):
        xs = [Fr(v) for v in xs]
        assert all(rn(v) == v for v in xs)
        scale = rn32(max(abs(v) for v in xs) / 448)
        assert f32_hex(scale) == g["scales_hex"][t]
        codes = []
        for v in xs:
            if scale == 0:
                codes.append(0)
                continue
            q = min(rn32(abs(v) / scale), Fr(448))
            c = round_binary(q, 3, -6)                 # E4M3: 3 fraction bits, normals from 2^-6
            codes.append(e4m3_bits(c) | (0x80 if v < 0 else 0))
        assert codes == g["codes"][t], t


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_combine_fixture_follows_from_exact_arithmetic(dtype):
    g, d, ids, W, epr, rows, w, assist, erc = combine_fixture_inputs(dtype)
    out = rn16 if dtype == "fp16" else rnbf16
    for t in range(ids.shape[0]):
        acc = Fr(0)
        for k in range(ids.shape[1]):
            acc = rn32(Fr(float(d["y"][t][k])) * Fr(float(w[t, k])) + acc)   # one rounding per fused step
        assert float(out(acc)) == d["x_out"][t], t


def test_combine_fixture_layout_is_the_dispatch_layout():
    """The fixture's assist_info and ep_recv_count are what dispatch gives for its routing."""
    g = _golden("combine_fma_order.json")
    ids = np.asarray(g["expert_ids"], np.int32)
    x = np.zeros((ids.shape[0], g["h"]), np.int32)
    out = oracle.dispatch(x, ids, g["ep_world"], g["experts_per_rank"])
    assert out["assist_info"].tolist() == g["assist_info"]
    assert out["ep_recv_count"].tolist() == g["ep_recv_count"]


# --------------------------------------------------------------------------
# planted mistakes: each altered copy of the oracle must fail a fixture
# --------------------------------------------------------------------------

MUTATIONS = {
    # quantMode 2: multiply by the binary32 reciprocal of the scale
    "int8_reciprocal": ("rintf(v / scale)", "rintf(v * (1.0f / scale))"),
    # quantMode 2: round the float64 quotient (close to the exact one) instead of the binary32 quotient
    "int8_f64_quotient": ("rintf(v / scale)", "(float)rint((double)v / (double)scale)"),
    # quantMode 2: ties away from zero
    "int8_ties_away": ("rintf(v / scale)", "roundf(v / scale)"),
    # quantMode 3: multiply by the reciprocal of the group scale
    "fp8_reciprocal": ("float n = v / gs;", "float n = v * (1.0f / gs);"),
    # combine: round each product before adding it
    "combine_mul_then_add": ("acc = fmaf(load_f32(expand_x, (size_t)slot[t * K + k] * h + j, dtype), sc, acc);",
                             "acc = load_f32(expand_x, (size_t)slot[t * K + k] * h + j, dtype) * sc + acc;"),
    # combine: k descending (for token 0 of the fixture this is also the order of its rows)
    "combine_k_descending": ("for (int k = 0; k < K; ++k) {\n                    float sc = ((const float *)scales)",
                             "for (int k = K - 1; k >= 0; --k) {\n                    float sc = ((const float *)scales)"),
}


def _build_variant(tmpdir, name, text):
    src = os.path.join(tmpdir, name + ".c")
    lib = os.path.join(tmpdir, "lib" + name + ".so")
    with open(src, "w") as f:
        f.write(text)
    subprocess.check_call(["gcc", *oracle._CFLAGS, "-o", lib, src, "-lm"])
    return oracle.bind(ctypes.CDLL(lib))


@pytest.fixture(scope="module")
def oracle_source():
    with open(oracle._SRC) as f:
        return f.read()


def _all_fixture_failures(monkeypatch, lib):
    monkeypatch.setattr(oracle, "_lib", lib)
    return {name: run() for name, run in FIXTURES.items()}


def test_unaltered_copy_passes(tmp_path, monkeypatch, oracle_source):
    lib = _build_variant(str(tmp_path), "unaltered", oracle_source)
    fails = _all_fixture_failures(monkeypatch, lib)
    assert all(v == [] for v in fails.values()), fails


@pytest.mark.parametrize("mutation", sorted(MUTATIONS))
def test_planted_mistake_fails_a_fixture(tmp_path, monkeypatch, oracle_source, mutation):
    old, new = MUTATIONS[mutation]
    assert oracle_source.count(old) == 1, "the planted mistake no longer matches the oracle source"
    lib = _build_variant(str(tmp_path), mutation, oracle_source.replace(old, new))
    fails = _all_fixture_failures(monkeypatch, lib)
    assert any(v for v in fails.values()), "%s passed every fixture" % mutation
