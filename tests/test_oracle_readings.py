"""Pins of the oracle's arithmetic readings (CPU only).

Four hand-worked fixtures under tests/golden/ fix the readings that decide
single bits of the outputs:
  * quant_int8_quotient.json -- quantMode 2 ("aclnnMoeDistributeDispatchV4",
    参数说明): q = rint(RN32(x / scale)), scale = RN32(max|x| / 127);
  * quant_fp8_quotient.json  -- quantMode 3 (same page): E4M3 of RN32(|x| / scale),
    scale = RN32(group max / 448);
  * quant_mx_e8m0.json       -- quantMode 4 (same page, "mx"): OCP MXFP8, blocks of 32,
    E8M0 byte = clamp(floor(log2 block max) - 8, -127, 127) + 127, E4M3 codes
    of x * 2^-shared;
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


def mx_fixture_tokens(dtype):
    """Dense [tokens, h] float32 inputs of the MX fixture (elements not listed are 0; "-0" is -0.0)."""
    g = _golden("quant_mx_e8m0.json")
    rows = []
    for tok in g[dtype]["x"]:
        r = np.zeros(g["h"], np.float32)
        for j, v in tok.items():
            r[int(j)] = -0.0 if v == "-0" else v
        rows.append(r)
    return g, np.stack(rows)


def mx_fixture_codes(g, dtype):
    out = np.zeros((len(g[dtype]["codes"]), g["h"]), np.int64)
    for t, tok in enumerate(g[dtype]["codes"]):
        for j, c in tok.items():
            out[t, int(j)] = c
    return out


def run_mx_fixture(dtype):
    g, xf = mx_fixture_tokens(dtype)
    x = to_bits(xf, dtype)
    ids = np.zeros((xf.shape[0], 1), np.int32)
    out = oracle.dispatch(x, ids, g["ep_world"], g["experts_per_rank"], quant_mode=4, bf16=dtype == "bf16")
    want_codes = mx_fixture_codes(g, dtype)
    bad = []
    for row, (s, tok, k) in enumerate(out["assist_info"].tolist()):
        codes = out["expand_x"][row].tolist()
        if codes != want_codes[tok].tolist():
            bad.append(("codes of token %d" % tok, codes, want_codes[tok].tolist()))
        sc = out["dynamic_scales"][row].tolist()
        if sc != g[dtype]["scales"][tok]:
            bad.append(("scale bytes of token %d" % tok, sc, g[dtype]["scales"][tok]))
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
    "mx_fp16": lambda: run_mx_fixture("fp16"),
    "mx_bf16": lambda: run_mx_fixture("bf16"),
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


def floor_log2(a: Fr) -> int:
    e = 0
    while a >= 2:
        a /= 2
        e += 1
    while a < 1:
        a *= 2
        e -= 1
    return e


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_mx_fixture_follows_from_exact_arithmetic(dtype):
    """Every stored byte and code from the OCP MX definition in exact rationals: per block of 32, the shared
    exponent floor(log2 max|x|) - 8 clamped to [-127, 127], byte = shared + 127, and the E4M3 rounding of
    x * 2^-shared clamped to 448, the sign taken from x's sign bit."""
    g, xf = mx_fixture_tokens(dtype)
    rn = rn16 if dtype == "fp16" else rnbf16
    want_codes = mx_fixture_codes(g, dtype)
    h = g["h"]
    for t in range(xf.shape[0]):
        xs = [Fr(float(v)) for v in xf[t]]
        assert all(rn(v) == v for v in xs), "token %d is not exactly representable" % t
        bytes_, codes = [], []
        for b0 in range(0, h, 32):
            blk = xs[b0:b0 + 32]
            amax = max(abs(v) for v in blk)
            shared = -127 if amax == 0 else max(-127, min(127, floor_log2(amax) - 8))
            bytes_.append(shared + 127)
            for j, v in enumerate(blk):
                q = min(abs(v) * Fr(2) ** -shared, Fr(448))
                c = e4m3_bits(round_binary(q, 3, -6))
                codes.append(c | (0x80 if np.signbit(xf[t, b0 + j]) else 0))
        assert bytes_ == g[dtype]["scales"][t], t
        assert codes == want_codes[t].tolist(), t


def test_mx_fixture_covers_its_cases():
    """The fixture holds what it claims: a clamp at 448, the shared-exponent clamp at -127 (a bf16
    subnormal block max among them), a byte near the top of the range, an all-zero block and -0 codes."""
    g, xf = mx_fixture_tokens("bf16")
    sc = np.asarray(g["bf16"]["scales"])
    assert (np.abs(xf[0, :32]) * 64 > 448).any()
    assert sc[2].tolist() == [0, 0] and np.abs(xf[2]).max() > 0
    assert 0 < np.abs(xf[2, 32:]).max() < 2.0 ** -126
    assert sc[3, 0] == 246 and (xf[1] == 0).all()
    assert (mx_fixture_codes(g, "bf16") == 0x80).sum() >= 3


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
    # quantMode 4: the frexp exponent taken as floor(log2) (one too high: a ceiling for non-powers of two)
    "mx_ceil_exponent": ("shared = (e2 - 1) - 8;", "shared = e2 - 8;"),
    # quantMode 4: no clamp of the scaled value to 448
    "mx_no_448_clamp": ("        if (n > 448.0) n = 448.0;\n                        if (n < -448.0) n = -448.0;\n",
                        ""),
    # quantMode 4: no lower clamp of the shared exponent
    "mx_no_low_clamp": ("if (shared < -127) shared = -127;", ""),
    # quantMode 4: E8M0 bias off by one
    "mx_bias_128": ("sb[b] = (uint8_t)(shared + 127);", "sb[b] = (uint8_t)(shared + 128);"),
    # quantMode 4: blocks of 64 instead of 32
    "mx_block_64": ("enum { MX_BLOCK = 32 };", "enum { MX_BLOCK = 64 };"),
    # quantMode 4: E4M3's largest exponent taken as 7 (the exponent of 240, not of 448)
    "mx_emax_7": ("shared = (e2 - 1) - 8;", "shared = (e2 - 1) - 7;"),
    # quantMode 4: the block scale applied the wrong way round
    "mx_scale_inverted": ("ldexp((double)load_f32(x, (size_t)(t * h + j), dtype), -shared)",
                          "ldexp((double)load_f32(x, (size_t)(t * h + j), dtype), shared)"),
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
