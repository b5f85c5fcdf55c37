"""Pins for the CPU oracle: it is checked against things other than itself.

* hand-worked fixtures under tests/golden/ (each cites the page it follows);
* brute-force definitions (segment counts by direct counting, every routing
  of a tiny problem);
* a library routine the result must reduce to (numpy's stable argsort gives
  the expand_x row order; numpy / torch give IEEE binary16 / bfloat16 casts);
* closed forms (identity expert: x_out = x * sum_k s for int32, x_out == x for
  softmax weights), invariants (assist_info is a bijection, counts sum to N*K),
  error bounds (quantisation and the fp32 accumulation), and exact rational
  arithmetic for the large-segment predicate.
"""
import itertools
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _run(w, inp=None):
    inp = inp or wl.make_inputs(w)
    d = oracle.dispatch(inp["x"], inp["ids"], w.ep_world, w.experts_per_rank, w.quant_mode,
                        expert_scales=inp["scales"], bf16=(w.dtype == "bf16"))
    return inp, d


SMALL = [w for w in wl.WORKLOADS if w.h <= 16] + [
    wl.custom(3, 5, 7, 3, 2, "int32", name="w3_ragged"),
    wl.custom(4, 9, 24, 4, 3, "fp16", "gauss_topk", name="w4_fp16"),
    wl.custom(2, 17, 40, 2, 4, "bf16", "zipf_topk", quant_mode=2, name="w2_bf16_q"),
]
ALL = SMALL + [w for w in wl.WORKLOADS if w.h > 16]


# --------------------------------------------------------------------------
# hand-worked fixtures
# --------------------------------------------------------------------------

def test_golden_dispatch_combine_int32():
    g = _golden("dispatch_combine_int32_w2.json")
    x = np.array(g["x"], np.int32)
    ids = np.array(g["expert_ids"], np.int32)
    sc = np.array(g["expert_scales"], np.int32)
    d = oracle.dispatch(x, ids, g["ep_world"], g["experts_per_rank"])
    assert d["expand_x"].tolist() == g["expand_x"]
    assert d["assist_info"].tolist() == g["assist_info"]
    assert d["ep_recv_count"].tolist() == g["ep_recv_count"]
    y = np.array(g["expert_out"], np.int32)
    out = oracle.combine(y, d["assist_info"], d["ep_recv_count"], ids, sc, g["ep_world"],
                         g["experts_per_rank"])
    assert out.tolist() == g["x_out_expert_out"]
    out = oracle.combine(d["expand_x"], d["assist_info"], d["ep_recv_count"], ids, sc,
                         g["ep_world"], g["experts_per_rank"])
    assert out.tolist() == g["x_out_identity"]


def test_golden_quant_ties_to_even():
    g = _golden("quant_fp16_ties.json")
    x = np.array(g["x"], np.float32).astype(np.float16)
    ids = np.array(g["expert_ids"], np.int32)
    d = oracle.dispatch(x, ids, g["ep_world"], g["experts_per_rank"], quant_mode=2)
    assert d["expand_x"].tolist() == g["expand_x"]
    assert d["dynamic_scales"].tolist() == g["dynamic_scales"]
    assert d["assist_info"].tolist() == g["assist_info"]
    assert d["ep_recv_count"].tolist() == g["ep_recv_count"]


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_golden_combine_final_rounding(dtype):
    g = _golden("combine_rounding.json")
    sub = g[dtype]
    y32 = np.array(sub["expert_out"], np.float32)
    y = y32.astype(np.float16) if dtype == "fp16" else wl.f32_to_bf16_bits(y32)
    ids = np.array(g["expert_ids"], np.int32)
    sc = np.array(g["expert_scales"], np.float32)
    out = oracle.combine(y, np.array(g["assist_info"], np.int32), np.array(g["ep_recv_count"], np.int32),
                         ids, sc, g["ep_world"], g["experts_per_rank"], bf16=(dtype == "bf16"))
    want32 = np.array(sub["x_out"], np.float32)
    want = want32.astype(np.float16) if dtype == "fp16" else wl.f32_to_bf16_bits(want32)
    assert out.view(np.uint16).tolist() == want.view(np.uint16).tolist()


# --------------------------------------------------------------------------
# counts, layout, assist_info
# --------------------------------------------------------------------------

def _brute_counts(ids, W, bs, epr):
    """cnt[r][el*W+s] = number of tokens of source rank s routed to expert r*epr+el."""
    E = W * epr
    cnt = np.zeros((W, epr * W), np.int64)
    for s in range(W):
        for e in range(E):
            n = sum(1 for tok in range(bs) if e in set(ids[s * bs + tok].tolist()))
            cnt[e // epr, (e % epr) * W + s] = n
    return cnt


@pytest.mark.parametrize("w", ALL, ids=lambda w: w.name)
def test_counts_match_direct_count(w):
    inp, d = _run(w)
    erc = d["ep_recv_count"].astype(np.int64)
    cnt = _brute_counts(inp["ids"], w.ep_world, w.bs, w.experts_per_rank)
    assert (erc == np.cumsum(cnt, axis=1)).all()
    assert erc[:, -1].sum() == w.num_tokens * w.topk
    assert (np.diff(erc, axis=1) >= 0).all() and (erc[:, :1] >= 0).all()
    assert cnt.max() <= w.bs


@pytest.mark.parametrize("w", ALL, ids=lambda w: w.name)
def test_row_order_is_stable_argsort_by_expert(w):
    inp, d = _run(w)
    a = d["assist_info"].astype(np.int64)
    pair = (a[:, 0] * w.bs + a[:, 1]) * w.topk + a[:, 2]
    assert (pair == np.argsort(inp["ids"].ravel(), kind="stable")).all()


@pytest.mark.parametrize("w", ALL, ids=lambda w: w.name)
def test_assist_info_is_a_bijection_onto_pairs(w):
    inp, d = _run(w)
    a = d["assist_info"]
    W, bs, K, epr = w.ep_world, w.bs, w.topk, w.experts_per_rank
    assert ((a[:, 0] >= 0) & (a[:, 0] < W) & (a[:, 1] >= 0) & (a[:, 1] < bs) & (a[:, 2] >= 0) & (a[:, 2] < K)).all()
    pair = (a[:, 0].astype(np.int64) * bs + a[:, 1]) * K + a[:, 2]
    assert len(set(pair.tolist())) == w.rows == len(pair)
    # every row sits in the segment of its pair's expert and source; src_token ascends inside a segment
    erc = d["ep_recv_count"]
    row = 0
    for r in range(W):
        prev = 0
        for i in range(epr * W):
            e, s = r * epr + i // W, i % W
            seg = a[row:row + erc[r, i] - prev]
            assert (seg[:, 0] == s).all()
            assert (inp["ids"][s * bs + seg[:, 1], seg[:, 2]] == e).all()
            assert (np.diff(seg[:, 1]) > 0).all()
            row += erc[r, i] - prev
            prev = erc[r, i]
    assert row == w.rows


@pytest.mark.parametrize("w", [w for w in ALL if w.quant_mode == 0], ids=lambda w: w.name)
def test_expand_x_rows_are_source_tokens_bitwise(w):
    inp, d = _run(w)
    a = d["assist_info"].astype(np.int64)
    t = a[:, 0] * w.bs + a[:, 1]
    assert d["expand_x"].view(np.uint8).tobytes() == inp["x"][t].view(np.uint8).tobytes()
    assert (d["expand_scales"] == inp["scales"][t, a[:, 2]]).all()


# --------------------------------------------------------------------------
# quantisation
# --------------------------------------------------------------------------

def _token_f32(w, x):
    if w.dtype == "bf16":
        return (x.astype(np.uint32) << 16).view(np.float32)
    return x.astype(np.float32)


@pytest.mark.parametrize("w", [w for w in ALL if w.quant_mode == 2], ids=lambda w: w.name)
def test_quant_bounds_and_ties(w):
    inp, d = _run(w)
    a = d["assist_info"].astype(np.int64)
    t = a[:, 0] * w.bs + a[:, 1]
    xf = _token_f32(w, inp["x"])[t].astype(np.float64)
    q = d["expand_x"].astype(np.float64)
    sc = d["dynamic_scales"].astype(np.float64)
    amax = np.abs(xf).max(axis=1)
    # the scale is the fp32 quotient amax/127 (relative error at most 2^-24)
    assert (np.abs(sc * 127 - amax) <= amax * 2.0 ** -23).all()
    nz = amax > 0
    assert (np.abs(q[nz]).max(axis=1) == 127).all()
    assert (q[~nz] == 0).all() and (sc[~nz] == 0).all()
    # q is a nearest integer of x/scale: |x/scale - q| <= 1/2 up to the fp32 quotient's rounding
    ratio = xf[nz] / sc[nz, None]
    assert (np.abs(ratio - q[nz]) <= 0.5 + 1e-5 * np.maximum(1.0, np.abs(ratio))).all()
    assert (np.abs(q) <= 127).all()


def test_quant_is_odd_and_ties_go_to_even():
    # A token and its negation quantise to negated codes with the same scale; a
    # value whose quotient is an exact half goes to the even neighbour.
    w = wl.custom(2, 4, 64, 1, 1, "fp16", name="odd")
    rng = np.random.default_rng(7)
    x = rng.standard_normal((8, 64)).astype(np.float16)
    # token 0: amax 127 (scale 1.0) and halves in between
    x[0, :8] = np.array([127, 0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 3.5], np.float16)
    x[4:] = -x[:4]
    ids = np.zeros((8, 1), np.int32)
    ids[4:] = 1
    d = oracle.dispatch(x, ids, 2, 1, quant_mode=2)
    a = d["assist_info"].astype(np.int64)
    t = a[:, 0] * 4 + a[:, 1]
    q = np.empty_like(d["expand_x"])
    q[t] = d["expand_x"]
    scl = np.empty_like(d["dynamic_scales"])
    scl[t] = d["dynamic_scales"]
    assert (q[4:] == -q[:4]).all() and (scl[4:] == scl[:4]).all()
    assert q[0, :8].tolist() == [127, 0, 2, 2, 0, -2, -2, 4]
    assert scl[0] == 1.0
    del w


# --------------------------------------------------------------------------
# combine
# --------------------------------------------------------------------------

@pytest.mark.parametrize("w", [w for w in ALL if w.dtype == "int32"], ids=lambda w: w.name)
def test_combine_int32_identity_closed_form(w):
    inp, d = _run(w)
    out = oracle.combine(d["expand_x"], d["assist_info"], d["ep_recv_count"], inp["ids"], inp["scales"],
                         w.ep_world, w.experts_per_rank)
    want = inp["x"].astype(np.int64) * inp["scales"].astype(np.int64).sum(axis=1, keepdims=True)
    assert (out.astype(np.int64) == want).all()


@pytest.mark.parametrize("w", [w for w in ALL if w.dtype != "int32" and w.routing != "uniform_distinct"],
                         ids=lambda w: w.name)
def test_combine_identity_softmax_closed_form(w):
    """Identity expert + softmax weights: sum_k x * s_k rounds back to x exactly."""
    inp, d = _run(w)
    bf = w.dtype == "bf16"
    y = oracle.identity_expert(d["expand_x"], d["dynamic_scales"])
    out = oracle.combine(y, d["assist_info"], d["ep_recv_count"], inp["ids"], inp["scales"],
                         w.ep_world, w.experts_per_rank, bf16=bf)
    if w.quant_mode == 0:
        assert out.view(np.uint16).tobytes() == inp["x"].view(np.uint16).tobytes()
    else:
        # every row of token t carries the same dequantised vector, so x_out[t] is that vector
        a = d["assist_info"].astype(np.int64)
        t = a[:, 0] * w.bs + a[:, 1]
        per_token = np.zeros_like(out.view(np.uint16))
        per_token[t] = y
        assert (out.view(np.uint16) == per_token).all()


def _exact_sum(yf, sc):
    return sum(Fraction(float(a)) * Fraction(float(b)) for a, b in zip(yf, sc))


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_combine_random_rows_within_error_bound(dtype):
    """Random expert outputs and weights: x_out is within half an output ulp
    plus the fp32 accumulation bound of the exact weighted sum."""
    w = wl.custom(2, 6, 33, 5, 4, dtype, "gauss_topk", name="rand")
    inp, d = _run(w)
    rng = np.random.default_rng(99)
    g = (rng.standard_normal(d["expand_x"].shape) * 3).astype(np.float32)
    y = g.astype(np.float16) if dtype == "fp16" else wl.f32_to_bf16_bits(g)
    sc = rng.uniform(-1.0, 1.0, size=inp["scales"].shape).astype(np.float32)
    out = oracle.combine(y, d["assist_info"], d["ep_recv_count"], inp["ids"], sc, w.ep_world,
                         w.experts_per_rank, bf16=(dtype == "bf16"))
    yf = _token_f32(wl.custom(1, 1, 1, 1, 1, dtype), y)
    of = _token_f32(wl.custom(1, 1, 1, 1, 1, dtype), out)
    # pull each pair's row through the library argsort (independent of the oracle's slot table)
    order = np.argsort(inp["ids"].ravel(), kind="stable")
    row_of = np.empty_like(order)
    row_of[order] = np.arange(order.size)
    K = w.topk
    mant = 10 if dtype == "fp16" else 7
    for t in range(w.num_tokens):
        rows = row_of[t * K:(t + 1) * K]
        for j in range(w.h):
            terms = yf[rows, j]
            ex = _exact_sum(terms, sc[t])
            mag = float(sum(abs(Fraction(float(a)) * Fraction(float(b))) for a, b in zip(terms, sc[t])))
            got = float(of[t, j])
            ulp = 2.0 ** (np.floor(np.log2(max(abs(got), 2.0 ** -14))) - mant)
            assert abs(got - float(ex)) <= ulp / 2 + K * 2.0 ** -24 * mag + 1e-30, (t, j)


def test_combine_rejects_tampered_assist():
    w = wl.WORKLOADS[0]
    inp, d = _run(w)
    a = d["assist_info"].copy()
    a[0, 2] = (a[0, 2] + 1) % w.topk    # row 0 now claims a pair routed to another expert
    with pytest.raises(oracle.OracleError):
        oracle.combine(d["expand_x"], a, d["ep_recv_count"], inp["ids"], inp["scales"], w.ep_world,
                       w.experts_per_rank)


def test_dispatch_rejects_bad_ids():
    x = np.zeros((4, 2), np.int32)
    ids = np.array([[0, 0], [1, 2], [3, 1], [2, 0]], np.int32)   # duplicate in token 0
    with pytest.raises(oracle.OracleError):
        oracle.dispatch(x, ids, 2, 2)
    ids[0] = [0, 4]                                                # out of range
    with pytest.raises(oracle.OracleError):
        oracle.dispatch(x, ids, 2, 2)


def test_empty_batch():
    x = np.zeros((0, 8), np.float16)
    ids = np.zeros((0, 2), np.int32)
    d = oracle.dispatch(x, ids, 4, 2)
    assert d["expand_x"].shape == (0, 8) and (d["ep_recv_count"] == 0).all()
    out = oracle.combine(d["expand_x"], d["assist_info"], d["ep_recv_count"], ids,
                         np.zeros((0, 2), np.float32), 4, 2)
    assert out.shape == (0, 8)


# --------------------------------------------------------------------------
# every routing of a tiny problem
# --------------------------------------------------------------------------

def test_all_1296_routings_end_to_end():
    W, bs, epr, K, h = 2, 2, 2, 2, 4
    E, N = W * epr, W * bs
    rng = np.random.default_rng(5)
    x = rng.integers(-50, 51, size=(N, h)).astype(np.int32)
    sc = rng.integers(1, 5, size=(N, K)).astype(np.int32)
    choices = list(itertools.permutations(range(E), K))   # ordered, distinct
    pick = [c for c in choices if c[0] < c[1]]             # 6 per token -> 6^4 = 1296 routings
    assert len(pick) ** N == 1296
    for combo in itertools.product(pick, repeat=N):
        ids = np.array(combo, np.int32)
        d = oracle.dispatch(x, ids, W, epr)
        cnt = _brute_counts(ids, W, bs, epr)
        assert (d["ep_recv_count"] == np.cumsum(cnt, axis=1)).all()
        order = np.argsort(ids.ravel(), kind="stable")
        a = d["assist_info"].astype(np.int64)
        assert ((a[:, 0] * bs + a[:, 1]) * K + a[:, 2] == order).all()
        assert (d["expand_x"] == x[order // K]).all()
        y = (np.arange(N * K * h, dtype=np.int32).reshape(N * K, h) * 7 - 11)
        out = oracle.combine(y, d["assist_info"], d["ep_recv_count"], ids, sc, W, epr)
        row_of = np.empty_like(order)
        row_of[order] = np.arange(order.size)
        want = sum(y[row_of[np.arange(N) * K + k]].astype(np.int64) * sc[:, k:k + 1] for k in range(K))
        assert (out == want).all()


# --------------------------------------------------------------------------
# IEEE conversions used by the oracle
# --------------------------------------------------------------------------

def test_f16_decode_all_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    want = bits.view(np.float16).astype(np.float32)
    got = np.array([oracle.f16_to_f32(int(b)) for b in bits], np.float32)
    fin = np.isfinite(want)
    assert (got[fin].view(np.uint32) == want[fin].view(np.uint32)).all()
    assert np.isnan(got[np.isnan(want)]).all()


def test_f16_encode_matches_numpy():
    rng = np.random.default_rng(3)
    vals = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * 10.0 ** rng.integers(-9, 6, 20000),
        np.arange(65536, dtype=np.uint32).astype(np.uint16).view(np.float16).astype(np.float32),
        # exact midpoints between neighbouring halves (ties), incl. subnormal and overflow edges
        ((np.arange(65535, dtype=np.uint32).astype(np.uint16).view(np.float16).astype(np.float64)
          + np.arange(1, 65536, dtype=np.uint32).astype(np.uint16).view(np.float16).astype(np.float64)) / 2
         ).astype(np.float32),
        np.array([65504, 65519.99, 65520, 70000, 2.0 ** -25, 2.0 ** -24, 3 * 2.0 ** -26, 1e-30], np.float32),
    ]).astype(np.float32)
    vals = vals[np.isfinite(vals)]
    vals = np.concatenate([vals, -vals])
    want = vals.astype(np.float16).view(np.uint16)
    got = np.array([oracle.f32_to_f16(float(v)) for v in vals], np.uint16)
    assert (got == want).all()


def test_bf16_roundtrip_matches_torch():
    import torch

    rng = np.random.default_rng(4)
    u = rng.integers(0, 2 ** 32, size=40000, dtype=np.uint64).astype(np.uint32)
    u = np.concatenate([u, (rng.integers(0, 2 ** 16, 2000).astype(np.uint32) << 16) | 0x8000])  # ties
    f = u.view(np.float32)
    f = f[np.isfinite(f)]
    want = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([oracle.f32_to_bf16(float(v)) for v in f], np.uint16)
    assert (got == want).all()
    back = np.array([oracle.bf16_to_f32(int(b)) for b in want[:5000]], np.float32)
    tb = torch.from_numpy(want[:5000].view(np.int16).copy()).view(torch.bfloat16).float().numpy()
    fin = np.isfinite(tb)
    assert (back[fin].view(np.uint32) == tb[fin].view(np.uint32)).all()


# --------------------------------------------------------------------------
# the large-segment predicate
# --------------------------------------------------------------------------

def _rule_exact(erc, W, epr, h, sz, T):
    S = epr * W
    out = np.zeros((W, S), np.uint8)
    for r in range(W):
        c = np.diff(np.concatenate([[0], erc[r].astype(np.int64)]))
        remote = sum(int(c[i]) for i in range(S) if i % W != r)
        mean = Fraction(remote * h * sz, max(W - 1, 1) * epr)
        for i in range(S):
            b = int(c[i]) * h * sz
            out[r, i] = (i % W != r) and c[i] > 0 and b >= T and Fraction(b) > mean
    return out


def test_large_segment_predicate_matches_exact_rationals():
    rng = np.random.default_rng(11)
    n = 0
    for W in (2, 3, 4, 5):
        for epr in (1, 2, 3):
            for h, sz in ((1, 1), (3, 2), (7, 4), (7168, 2)):
                for _ in range(12):
                    cnt = rng.integers(0, 9, size=(W, epr * W)) * rng.integers(0, 2, size=(W, epr * W))
                    erc = np.cumsum(cnt, axis=1).astype(np.int32)
                    for T in (0, 1, 5 * h * sz, 2 * 1024 * 1024):
                        got = oracle.large_segments(erc, W, epr, h, sz, T)
                        assert (got == _rule_exact(erc, W, epr, h, sz, T)).all()
                        n += 1
    assert n > 500


def test_literal_2mib_rule_selects_nothing_on_the_page_workloads():
    """A segment holds at most bs tokens: at most 32*7168*2 B = 448 KiB on the
    8-rank h=7168 workloads, so the literal 2 MiB threshold never fires there."""
    for w in wl.WORKLOADS:
        inp, d = _run(w)
        sz = 1 if w.quant_mode == 2 else (4 if w.dtype == "int32" else 2)
        flags = oracle.large_segments(d["ep_recv_count"], w.ep_world, w.experts_per_rank, w.h, sz,
                                      2 * 1024 * 1024)
        assert flags.sum() == 0, w.name
    # and a skewed shape with bs >= 147 at h=7168 fp16 does fire
    w = wl.custom(4, 192, 7168, 4, 2, "fp16", "zipf_topk", name="big_zipf")
    inp = wl.make_inputs(w)
    d = oracle.dispatch(inp["x"], inp["ids"], w.ep_world, w.experts_per_rank)
    flags = oracle.large_segments(d["ep_recv_count"], w.ep_world, w.experts_per_rank, w.h, 2,
                                  2 * 1024 * 1024)
    assert flags.sum() > 0
    assert (flags == _rule_exact(d["ep_recv_count"], w.ep_world, w.experts_per_rank, w.h, 2,
                                 2 * 1024 * 1024)).all()


# --------------------------------------------------------------------------
# token masks (aclnnMoeDistributeDispatchV4 参数说明, xActiveMaskOptional):
# an inactive pair is not exchanged, so it has no row and no count
# --------------------------------------------------------------------------

def _mask_cases(rng, N, K, bs):
    """(name, mask) pairs: per-token masks (each rank's active tokens first, as
    the pages ask, and an arbitrary pattern) and per-pair masks (random, with
    whole tokens switched off, and all off)."""
    W = N // bs
    prefix = np.zeros(N, bool)
    for s in range(W):
        prefix[s * bs: s * bs + rng.integers(0, bs + 1)] = True
    pair = rng.random((N, K)) < 0.6
    pair[rng.random(N) < 0.3] = False
    return [("token_prefix", prefix), ("token_any", rng.random(N) < 0.5), ("pair", pair),
            ("pair_all_off", np.zeros((N, K), bool)), ("token_all_on", np.ones(N, bool))]


def _active(mask, N, K):
    return np.repeat(mask[:, None], K, axis=1) if mask.ndim == 1 else mask


def _brute_force_layout(ids, act, W, bs, epr):
    """Rows by sorting the active pairs on (rank, local expert, source rank,
    token): the definition of the row order, without the counting sort."""
    N, K = ids.shape
    keys = sorted((int(ids[t, k]) // epr, int(ids[t, k]) % epr, t // bs, t % bs, k)
                  for t in range(N) for k in range(K) if act[t, k])
    assist = np.array([[s, tok, k] for (_, _, s, tok, k) in keys], np.int32).reshape(-1, 3)
    cnt = np.zeros((W, epr * W), np.int64)
    for (r, el, s, _, _) in keys:
        cnt[r, el * W + s] += 1
    return assist, np.cumsum(cnt, axis=1).astype(np.int32)


@pytest.mark.parametrize("w", [wl.custom(3, 7, 5, 3, 2, "int32", name="int32_small"),
                               wl.custom(4, 9, 16, 4, 3, "bf16", "zipf_topk", quant_mode=2, name="bf16_q")],
                         ids=lambda w: w.name)
def test_masked_dispatch_matches_a_sort_of_the_active_pairs(w):
    inp = wl.make_inputs(w)
    N, K, bs = w.num_tokens, w.topk, w.bs
    full = oracle.dispatch(inp["x"], inp["ids"], w.ep_world, w.experts_per_rank, w.quant_mode,
                           bf16=w.dtype == "bf16")
    full_row = {tuple(a): i for i, a in enumerate(full["assist_info"].tolist())}
    for name, mask in _mask_cases(np.random.default_rng(7), N, K, bs):
        act = _active(mask, N, K)
        d = oracle.dispatch(inp["x"], inp["ids"], w.ep_world, w.experts_per_rank, w.quant_mode,
                            bf16=w.dtype == "bf16", mask=mask)
        assist, erc = _brute_force_layout(inp["ids"], act, w.ep_world, bs, w.experts_per_rank)
        A = len(assist)
        assert d["rows"] == A == int(act.sum()), name
        assert (d["assist_info"][:A] == assist).all(), name
        assert (d["ep_recv_count"] == erc).all(), name
        # each row holds its token's payload exactly as the unmasked dispatch does
        for i, a in enumerate(assist.tolist()):
            j = full_row[tuple(a)]
            assert d["expand_x"][i].tobytes() == full["expand_x"][j].tobytes(), name
            if w.quant_mode == 2:
                assert d["dynamic_scales"][i] == full["dynamic_scales"][j], name


def test_masked_int32_combine_closed_form():
    """Identity expert, int32: x_out[t] = x[t] * sum over active k of s[t,k]
    (wrapping), and 0 for a token with no active pair."""
    w = wl.custom(4, 11, 6, 3, 2, "int32", name="int32_mask")
    inp = wl.make_inputs(w)
    N, K = w.num_tokens, w.topk
    for name, mask in _mask_cases(np.random.default_rng(3), N, K, w.bs):
        act = _active(mask, N, K)
        d = oracle.dispatch(inp["x"], inp["ids"], w.ep_world, w.experts_per_rank, mask=mask)
        out = oracle.combine(d["expand_x"], d["assist_info"], d["ep_recv_count"], inp["ids"], inp["scales"],
                             w.ep_world, w.experts_per_rank, mask=mask)
        ssum = (inp["scales"].astype(np.int64) * act).sum(axis=1)
        want = ((inp["x"].astype(np.int64) * ssum[:, None]) & 0xFFFFFFFF).astype(np.uint32).view(np.int32)
        assert (out == want).all(), name


@pytest.mark.parametrize("dt", ["fp16", "bf16"])
def test_masked_combine_equals_zero_weights(dt):
    """fp16/bf16: skipping an inactive pair gives the same bits as keeping it
    with weight 0 (fma(y, 0, acc) == acc for finite y, and acc never becomes
    -0 from +0), so the masked combine must equal the unmasked one on weights
    zeroed where the mask is off. Tokens with no active pair come out +0."""
    w = wl.custom(3, 13, 24, 4, 3, dt, "gauss_topk", name="half_mask")
    inp = wl.make_inputs(w)
    N, K = w.num_tokens, w.topk
    bf = dt == "bf16"
    full = oracle.dispatch(inp["x"], inp["ids"], w.ep_world, w.experts_per_rank, bf16=bf)
    for name, mask in _mask_cases(np.random.default_rng(5), N, K, w.bs):
        act = _active(mask, N, K)
        d = oracle.dispatch(inp["x"], inp["ids"], w.ep_world, w.experts_per_rank, bf16=bf, mask=mask)
        got = oracle.combine(d["expand_x"], d["assist_info"], d["ep_recv_count"], inp["ids"], inp["scales"],
                             w.ep_world, w.experts_per_rank, bf16=bf, mask=mask)
        zeroed = (inp["scales"] * act).astype(np.float32)
        want = oracle.combine(full["expand_x"], full["assist_info"], full["ep_recv_count"], inp["ids"], zeroed,
                              w.ep_world, w.experts_per_rank, bf16=bf)
        assert got.view(np.uint16).tobytes() == want.view(np.uint16).tobytes(), name
        assert (got.view(np.uint16)[~act.any(axis=1)] == 0).all(), name


def test_masks_that_keep_everything_change_nothing_and_mismatches_are_rejected():
    w = wl.custom(2, 8, 16, 3, 3, "fp16", "gauss_topk", quant_mode=2, name="all_on")
    inp = wl.make_inputs(w)
    N, K = w.num_tokens, w.topk
    ref = oracle.dispatch(inp["x"], inp["ids"], w.ep_world, w.experts_per_rank, 2)
    for mask in (np.ones(N, np.uint8), np.full((N, K), 3, np.uint8)):
        d = oracle.dispatch(inp["x"], inp["ids"], w.ep_world, w.experts_per_rank, 2, mask=mask)
        for key in ("expand_x", "dynamic_scales", "assist_info", "ep_recv_count"):
            assert d[key].tobytes() == ref[key].tobytes(), key
    # outputs of an unmasked dispatch do not describe a masked exchange
    y = oracle.identity_expert(ref["expand_x"], ref["dynamic_scales"])
    mask = np.ones((N, K), bool)
    mask[0, 0] = False
    with pytest.raises(oracle.OracleError):
        oracle.combine(y, ref["assist_info"], ref["ep_recv_count"], inp["ids"], inp["scales"], w.ep_world,
                       w.experts_per_rank, bf16=True, mask=mask)
    # an inactive pair's id is never read: garbage there is accepted
    ids = inp["ids"].copy()
    ids[0, 0] = 10 ** 6
    d = oracle.dispatch(inp["x"], ids, w.ep_world, w.experts_per_rank, 2, mask=mask)
    assert d["rows"] == N * K - 1
    with pytest.raises(oracle.OracleError):
        oracle.dispatch(inp["x"], ids, w.ep_world, w.experts_per_rank, 2)


# --------------------------------------------------------------------------
# quantMode 3 (per-group dynamic, reading: groups of 128, OCP E4M3 codes,
# scale = max|x| / 448): the E4M3 conversions and the quantiser
# --------------------------------------------------------------------------

def _e4m3_table():
    """Every finite E4M3 value, from the format's definition (bias 7, 3
    fraction bits, subnormals f * 2^-9, exponent 15 / fraction 7 is NaN)."""
    vals = {}
    for c in range(256):
        s, e, f = c >> 7, (c >> 3) & 15, c & 7
        if e == 15 and f == 7:
            continue
        v = f * 2.0 ** -9 if e == 0 else (1 + f / 8) * 2.0 ** (e - 7)
        vals[c] = -v if s else v
    return vals


def test_e4m3_decode_matches_the_definition_and_torch():
    import torch
    tab = _e4m3_table()
    ref = torch.from_numpy(np.arange(256, dtype=np.uint8)).view(torch.float8_e4m3fn).float().numpy()
    for c in range(256):
        got = oracle.e4m3_to_f32(c)
        if c in tab:
            assert got == tab[c] == ref[c], c
        else:
            assert np.isnan(got) and np.isnan(ref[c]), c
    assert max(tab.values()) == 448.0 and min(v for v in tab.values() if v > 0) == 2.0 ** -9


def test_e4m3_encode_is_nearest_ties_to_even():
    """Brute-force nearest search over every finite code (ties to the even
    code, the sign kept), and torch's float8_e4m3fn cast, on every
    representable value, every midpoint, one float32 ulp either side of each
    midpoint, and random values in [-448, 448]."""
    import torch
    tab = _e4m3_table()
    pos = sorted((v, c) for c, v in tab.items() if v >= 0 and not (v == 0 and c == 0x80))
    vals = [v for v, _ in pos]
    pts = set(vals)
    for a, b in zip(vals, vals[1:]):
        m = np.float32((a + b) / 2)
        pts.update([float(m), float(np.nextafter(m, np.float32(0))), float(np.nextafter(m, np.float32(1e9)))])
    rng = np.random.default_rng(11)
    pts.update(rng.uniform(0, 448, 3000).astype(np.float32).tolist())
    pts.update((2.0 ** rng.uniform(-12, 8.8, 3000)).astype(np.float32).clip(0, 448).tolist())
    xs = np.array(sorted(pts), np.float32)
    xs = np.concatenate([xs, -xs])
    want_torch = torch.from_numpy(xs).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    pos_codes = [(v, c) for v, c in pos]
    n = 0
    for x, wt in zip(xs.tolist(), want_torch.tolist()):
        a = abs(x)
        best = min(pos_codes, key=lambda vc: (abs(vc[0] - a), vc[1] & 1))
        code = best[1] | (0x80 if np.signbit(np.float32(x)) else 0)
        got = oracle.f32_to_e4m3(x)
        assert got == code == wt, (x, got, code, wt)
        n += 1
    assert n > 10000


def test_group_quantiser_properties():
    """Per group of 128: scale = amax / 448 in fp32; the largest element maps to
    +-448; every code decodes to within half an E4M3 quantum of x / scale; an
    all-zero group has scale 0 and codes 0; a ragged last group is its own
    group; -0 keeps its sign bit in a group with a nonzero scale."""
    h = 128 * 3 + 40
    rng = np.random.default_rng(4)
    x = (rng.standard_normal((6, h)) * 2.0 ** rng.integers(-20, 10, size=(6, 1))).astype(np.float16)
    x[2, 128:256] = 0.0                      # an all-zero group
    x[3, 5] = -0.0
    ids = np.array([[0], [1], [2], [3], [0], [1]], np.int32)
    d = oracle.dispatch(x, ids, 2, 2, quant_mode=3)
    assert d["expand_x"].dtype == np.uint8 and d["dynamic_scales"].shape == (6, 4)
    row_of = {tuple(a): i for i, a in enumerate(d["assist_info"].tolist())}
    dec = np.array([oracle.e4m3_to_f32(c) for c in range(256)], np.float32)
    xf = x.astype(np.float32)
    for t in range(6):
        i = row_of[(t // 3, t % 3, 0)]
        q, sc = d["expand_x"][i], d["dynamic_scales"][i]
        for g in range(4):
            seg = slice(g * 128, min(h, g * 128 + 128))
            amax = np.abs(xf[t, seg]).max()
            assert sc[g] == np.float32(amax) / np.float32(448.0)
            if amax == 0:
                assert sc[g] == 0 and (q[seg] == 0).all()
                continue
            quot = xf[t, seg] / sc[g]
            deq = dec[q[seg]]
            assert np.abs(deq).max() == 448.0
            quantum = np.where(np.abs(quot) < 2.0 ** -6, 2.0 ** -9, 2.0 ** (np.floor(np.log2(np.maximum(np.abs(quot), 1e-30))) - 3))
            assert (np.abs(deq - np.clip(quot, -448, 448)) <= quantum / 2 + 1e-12).all(), (t, g)
    i = row_of[(1, 0, 0)]
    assert d["expand_x"][i, 5] == 0x80


# --------------------------------------------------------------------------
# quantMode 4 ("mx" dynamic quantisation, reading: OCP MXFP8, E4M3 elements,
# blocks of 32, one E8M0 scale byte per block)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_mx_quantiser_against_frexp_and_torch_e4m3(dtype):
    """Per block of 32 (the last one ragged): byte = clip(e - 1 - 8, -127, 127) + 127 with e from numpy's
    frexp of the block max (0 for an all-zero block); codes equal torch's float8_e4m3fn cast of
    clip(x * 2^-shared, -448, 448); the block max lands in [256, 448] after scaling; -0 keeps its sign."""
    import torch

    h = 32 * 5 + 8
    rng = np.random.default_rng(8)
    g = rng.standard_normal((8, h)) * 2.0 ** rng.integers(-30, 30, size=(8, 1))
    g[2, 32:64] = 0.0                                    # an all-zero block
    g[3, 7] = -0.0
    g[5, 160:] *= 2.0 ** -12                             # a ragged block far below the others
    if dtype == "fp16":
        g = np.clip(g, -60000, 60000)
        x = g.astype(np.float16)
        xf = x.astype(np.float32)
    else:
        x = wl.f32_to_bf16_bits(g.astype(np.float32))
        xf = (x.astype(np.uint32) << 16).view(np.float32)
    ids = np.arange(8, dtype=np.int32)[:, None] % 2
    d = oracle.dispatch(x, ids, 2, 1, quant_mode=4, bf16=dtype == "bf16")
    B = (h + 31) // 32
    assert d["expand_x"].dtype == np.uint8 and d["dynamic_scales"].dtype == np.uint8
    assert d["dynamic_scales"].shape == (8, B)
    row_of = {tuple(a): i for i, a in enumerate(d["assist_info"].tolist())}
    dec = torch.from_numpy(np.arange(256, dtype=np.uint8)).view(torch.float8_e4m3fn).float().numpy()
    for t in range(8):
        i = row_of[(t // 4, t % 4, 0)]
        q, sb = d["expand_x"][i], d["dynamic_scales"][i]
        for b in range(B):
            seg = slice(32 * b, min(h, 32 * b + 32))
            amax = np.abs(xf[t, seg]).max()
            shared = -127 if amax == 0 else int(np.clip(np.frexp(np.float64(amax))[1] - 1 - 8, -127, 127))
            assert sb[b] == shared + 127, (t, b)
            n = np.clip(xf[t, seg].astype(np.float64) * 2.0 ** -shared, -448, 448).astype(np.float32)
            want = torch.from_numpy(n).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
            assert (q[seg] == want).all(), (t, b)
            if amax > 0:
                assert 256 <= np.abs(dec[q[seg]]).max() <= 448
    assert d["expand_x"][row_of[(0, 3, 0)], 7] == 0x80
    assert (d["dynamic_scales"][row_of[(0, 2, 0)], 1] == 0)


def test_mx_identity_expert_matches_torch():
    """bf16(e4m3(q) * 2^(byte - 127)) per 32-element block, against torch's float8_e4m3fn decoding, fp32
    multiply by a power of two and round-to-nearest-even bfloat16 cast."""
    import torch

    rng = np.random.default_rng(43)
    rows, h = 29, 200
    codes = rng.integers(0, 256, size=(rows, h)).astype(np.uint8)
    codes[(codes & 0x7f) == 0x7f] = 0                  # the NaN codes are not produced by the quantiser
    sb = rng.integers(0, 247, size=(rows, (h + 31) // 32)).astype(np.uint8)
    got = oracle.identity_expert(codes, sb)
    dec = torch.from_numpy(codes).view(torch.float8_e4m3fn).float()
    full = torch.exp2(torch.from_numpy(sb.astype(np.float32) - 127.0)).repeat_interleave(32, dim=1)[:, :h]
    want = (dec * full).bfloat16().view(torch.int16).numpy()
    assert got.view(np.int16).tobytes() == want.tobytes()


# --------------------------------------------------------------------------
# special experts (aclnnMoeDistributeDispatchV4 参数说明, zeroExpertNum /
# copyExpertNum: id ranges after the E real experts). Reading: not exchanged;
# a zero expert adds nothing, a copy expert adds the token itself
# --------------------------------------------------------------------------

def test_special_experts_match_a_dispatch_without_those_pairs():
    """Pairs routed to a zero or copy expert behave exactly like pairs switched
    off by a per-pair mask (a different code path in the oracle)."""
    for w in (wl.custom(3, 7, 5, 3, 2, "int32", zero_experts=2, copy_experts=2, const_experts=2,
                        name="int32_special"),
              wl.custom(4, 9, 16, 4, 3, "bf16", "zipf_topk", quant_mode=2, zero_experts=3, copy_experts=1,
                        const_experts=2, name="bf16_special")):
        inp = wl.make_inputs(w)
        E = w.num_experts
        special = inp["ids"] >= E
        assert special.any() and (~special).any()
        assert (inp["ids"] >= E + w.zero_experts + w.copy_experts).any()      # some const pairs
        d = oracle.dispatch(inp["x"], inp["ids"], w.ep_world, w.experts_per_rank, w.quant_mode,
                            bf16=w.dtype == "bf16", zero_experts=w.zero_experts, copy_experts=w.copy_experts,
                            const_experts=w.const_experts)
        ids_masked = np.where(special, 0, inp["ids"]).astype(np.int32)
        m = oracle.dispatch(inp["x"], ids_masked, w.ep_world, w.experts_per_rank, w.quant_mode,
                            bf16=w.dtype == "bf16", mask=~special)
        for key in ("expand_x", "assist_info", "ep_recv_count"):
            assert d[key].tobytes() == m[key].tobytes(), (w.name, key)
        # ids beyond the special ranges are still an error
        bad = inp["ids"].copy()
        bad[0, 0] = E + w.zero_experts + w.copy_experts + w.const_experts
        with pytest.raises(oracle.OracleError):
            oracle.dispatch(inp["x"], bad, w.ep_world, w.experts_per_rank, w.quant_mode, bf16=w.dtype == "bf16",
                            zero_experts=w.zero_experts, copy_experts=w.copy_experts, const_experts=w.const_experts)


def test_special_experts_int32_combine_closed_form():
    """Identity expert, int32: x_out[t] = x[t] * (sum of the weights of its real
    and copy experts), wrapping; zero experts add nothing."""
    w = wl.custom(4, 11, 6, 4, 2, "int32", zero_experts=3, copy_experts=3, name="int32_special_combine")
    inp = wl.make_inputs(w)
    E, Z, C = w.num_experts, w.zero_experts, w.copy_experts
    ids = inp["ids"]
    d = oracle.dispatch(inp["x"], ids, w.ep_world, w.experts_per_rank, zero_experts=Z, copy_experts=C)
    out = oracle.combine(d["expand_x"], d["assist_info"], d["ep_recv_count"], ids, inp["scales"], w.ep_world,
                         w.experts_per_rank, zero_experts=Z, copy_experts=C, ori_x=inp["x"])
    counted = (ids < E) | ((ids >= E + Z) & (ids < E + Z + C))
    assert ((ids >= E) & (ids < E + Z)).any() and ((ids >= E + Z) & (ids < E + Z + C)).any()
    ssum = (inp["scales"].astype(np.int64) * counted).sum(axis=1)
    want = ((inp["x"].astype(np.int64) * ssum[:, None]) & 0xFFFFFFFF).astype(np.uint32).view(np.int32)
    assert (out == want).all()


def test_const_experts_int32_combine_closed_form():
    """Identity expert, int32, with const experts ("aclnnMoeDistributeDispatchV4" 参数说明,
    constExpertNum; reading: const expert j outputs the fixed row const_x[j]):
    x_out[t] = x[t] * (sum of real and copy weights) + sum over const pairs of
    const_x[j] * weight, in wrapping 32-bit arithmetic; zero experts add nothing."""
    w = wl.custom(4, 11, 6, 4, 2, "int32", zero_experts=2, copy_experts=2, const_experts=3,
                  name="int32_const_combine")
    inp = wl.make_inputs(w)
    E, Z, C, Q = w.num_experts, w.zero_experts, w.copy_experts, w.const_experts
    ids, sc, cx = inp["ids"], inp["scales"].astype(np.int64), inp["const_x"].astype(np.int64)
    assert cx.shape == (Q, w.h)
    d = oracle.dispatch(inp["x"], ids, w.ep_world, w.experts_per_rank, zero_experts=Z, copy_experts=C,
                        const_experts=Q)
    out = oracle.combine(d["expand_x"], d["assist_info"], d["ep_recv_count"], ids, inp["scales"], w.ep_world,
                         w.experts_per_rank, zero_experts=Z, copy_experts=C, ori_x=inp["x"], const_experts=Q,
                         const_x=inp["const_x"])
    is_const = (ids >= E + Z + C) & (ids < E + Z + C + Q)
    assert is_const.any() and ((ids >= E) & (ids < E + Z)).any()
    token_w = (sc * ((ids < E) | ((ids >= E + Z) & (ids < E + Z + C)))).sum(axis=1)
    want = inp["x"].astype(np.int64) * token_w[:, None]
    for t, k in zip(*np.nonzero(is_const)):
        want[t] += cx[ids[t, k] - (E + Z + C)] * sc[t, k]
    want = (want & 0xFFFFFFFF).astype(np.uint32).view(np.int32)
    assert (out == want).all()
    # a zero table makes const experts zero experts
    zero = oracle.combine(d["expand_x"], d["assist_info"], d["ep_recv_count"], ids, inp["scales"], w.ep_world,
                          w.experts_per_rank, zero_experts=Z, copy_experts=C, ori_x=inp["x"], const_experts=Q,
                          const_x=np.zeros_like(inp["const_x"]))
    as_zero = np.where(is_const, E, ids).astype(np.int32)        # E is the first zero expert
    ref = oracle.combine(d["expand_x"], d["assist_info"], d["ep_recv_count"], as_zero, inp["scales"], w.ep_world,
                         w.experts_per_rank, zero_experts=Z, copy_experts=C, ori_x=inp["x"])
    assert (zero == ref).all()


def test_const_expert_adds_its_row_in_k_order():
    """fp16/bf16: a const pair's term is fma(const_x[j], w, acc) at its own k; the same sum
    is obtained when the pair goes to an unused real expert whose output row is const_x[j]."""
    for dt in ("fp16", "bf16"):
        w = wl.custom(3, 13, 24, 4, 3, dt, "gauss_topk", const_experts=3, name="const_" + dt)
        inp = wl.make_inputs(w)
        E, bf = w.num_experts, dt == "bf16"
        ids, cx = inp["ids"], inp["const_x"]
        assert (ids >= E).any()
        d = oracle.dispatch(inp["x"], ids, w.ep_world, w.experts_per_rank, bf16=bf, const_experts=3)
        got = oracle.combine(d["expand_x"], d["assist_info"], d["ep_recv_count"], ids, inp["scales"], w.ep_world,
                             w.experts_per_rank, bf16=bf, const_experts=3, const_x=cx)
        real = ids.copy()
        for t in range(w.num_tokens):
            free = [e for e in range(E) if e not in set(ids[t].tolist())]
            for k in range(w.topk):
                if real[t, k] >= E:
                    real[t, k] = free.pop()
        r = oracle.dispatch(inp["x"], real, w.ep_world, w.experts_per_rank, bf16=bf)
        rows = r["expand_x"].copy()
        for i, (s, tok, k) in enumerate(r["assist_info"].tolist()):   # the expert's output for those pairs
            t = s * w.bs + tok
            if ids[t, k] >= E:
                rows[i] = cx[ids[t, k] - E]
        want = oracle.combine(rows, r["assist_info"], r["ep_recv_count"], real, inp["scales"], w.ep_world,
                              w.experts_per_rank, bf16=bf)
        assert got.view(np.uint16).tobytes() == want.view(np.uint16).tobytes(), dt


def test_copy_expert_adds_the_token_in_k_order():
    """fp16/bf16: a copy expert's term is fma(x[t], w, acc) at its own k; the
    same sum is obtained when that pair is instead sent to a real expert whose
    output is the token itself (identity expert)."""
    for dt in ("fp16", "bf16"):
        w = wl.custom(3, 13, 24, 4, 3, dt, "gauss_topk", copy_experts=4, name="copy_" + dt)
        inp = wl.make_inputs(w)
        E, bf = w.num_experts, dt == "bf16"
        ids = inp["ids"]
        assert (ids >= E).any()
        d = oracle.dispatch(inp["x"], ids, w.ep_world, w.experts_per_rank, bf16=bf, copy_experts=4)
        got = oracle.combine(d["expand_x"], d["assist_info"], d["ep_recv_count"], ids, inp["scales"], w.ep_world,
                             w.experts_per_rank, bf16=bf, copy_experts=4, ori_x=inp["x"])
        # route every copy pair to a real expert the token does not use: the identity expert then returns
        # x[t] for it, so the sum must be bitwise the same
        real = ids.copy()
        for t in range(w.num_tokens):
            free = [e for e in range(E) if e not in set(ids[t].tolist())]
            for k in range(w.topk):
                if real[t, k] >= E:
                    real[t, k] = free.pop()
        r = oracle.dispatch(inp["x"], real, w.ep_world, w.experts_per_rank, bf16=bf)
        want = oracle.combine(r["expand_x"], r["assist_info"], r["ep_recv_count"], real, inp["scales"], w.ep_world,
                              w.experts_per_rank, bf16=bf)
        assert got.view(np.uint16).tobytes() == want.view(np.uint16).tobytes(), dt


# --------------------------------------------------------------------------
# static quantisation (aclnnMoeDistributeDispatchV4 参数说明, quantMode 1: the
# coefficient input is one value, a per-column smoothing vector or per-expert
# fused coefficients). Reading: q = sat_int8(rint(x * c)), the exact product
# rounded once to the nearest integer (ties to even)
# --------------------------------------------------------------------------

def _codes_by_pair(d, bs):
    """expand_x rows keyed by (token, k), from assist_info."""
    a = d["assist_info"].astype(np.int64)
    return {(int(s) * bs + int(tok), int(k)): d["expand_x"][i] for i, (s, tok, k) in enumerate(a)}


def test_static_unit_coefficient_is_a_saturating_round():
    """c = 1 on fp16 tokens: integers pass through, saturating at -128 and 127;
    halves go to the even neighbour; NaN gives -128 and infinities saturate."""
    x = np.zeros((4, 16), np.float16)
    x[0] = np.arange(-8, 8) * 20                       # -160 .. 140: both ends saturate
    x[1, :8] = [0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 126.5, -127.5]
    x[1, 8:12] = [np.nan, np.inf, -np.inf, -0.0]
    x[2] = -x[0]
    ids = np.array([[0], [1], [2], [3]], np.int32)
    d = oracle.dispatch(x, ids, 2, 2, quant_mode=1, quant_scales=np.ones(1, np.float32))
    assert d["dynamic_scales"] is None and d["expand_x"].dtype == np.int8
    q = _codes_by_pair(d, 2)
    assert q[(0, 0)].tolist() == [-128, -128, -120, -100, -80, -60, -40, -20, 0, 20, 40, 60, 80, 100, 120, 127]
    assert q[(1, 0)][:12].tolist() == [0, 2, 2, 0, -2, -2, 126, -128, -128, 127, -128, 0]
    assert q[(2, 0)].tolist() == [127, 127, 120, 100, 80, 60, 40, 20, 0, -20, -40, -60, -80, -100, -120, -128]
    assert (q[(3, 0)] == 0).all()


def test_static_coefficient_tables_name_their_expert_and_column():
    """With x = 1 the code is the coefficient itself, so a table whose entries
    encode (expert, column) shows which entry each code came from: the per-expert
    table must be indexed by the row's own expert, the per-column one by the
    column; all three shapes agree when they hold the same value."""
    W, epr, h, K, bs = 3, 2, 24, 3, 5
    E = W * epr
    rng = np.random.default_rng(11)
    ids = np.stack([rng.permutation(E)[:K] for _ in range(W * bs)]).astype(np.int32)
    for bf in (False, True):
        x = np.ones((W * bs, h), np.float32)
        x = wl.f32_to_bf16_bits(x) if bf else x.astype(np.float16)
        ce = np.array([[(5 * e + j) % 120 - 60 for j in range(h)] for e in range(E)], np.float32)
        d = oracle.dispatch(x, ids, W, epr, quant_mode=1, quant_scales=ce, bf16=bf)
        for (t, k), code in _codes_by_pair(d, bs).items():
            assert code.tolist() == ce[ids[t, k]].astype(int).tolist(), (t, k)
        cc = np.arange(h, dtype=np.float32) * 7 - 80
        d = oracle.dispatch(x, ids, W, epr, quant_mode=1, quant_scales=cc, bf16=bf)
        assert all(code.tolist() == np.clip(cc, -128, 127).astype(int).tolist()
                   for code in _codes_by_pair(d, bs).values())
        outs = [oracle.dispatch(x, ids, W, epr, quant_mode=1, quant_scales=np.full(n, 0.75, np.float32),
                                bf16=bf)["expand_x"] for n in (1, h, E * h)]
        assert (outs[0] == outs[1]).all() and (outs[0] == outs[2]).all() and (outs[0] == 1).all()


def test_static_codes_are_nearest_integers_of_the_product():
    """On the static workload's own inputs (per-expert coefficients, N(0,1) bf16
    tokens at a reduced batch): each code is within 1/2 of x * c[e] (exact in
    float64), or saturated beyond the range."""
    w = wl.custom(4, 16, 256, 8, 4, "bf16", "gauss_topk", quant_mode=1, name="static_small", index=4)
    inp = wl.make_inputs(w)
    c = inp["quant_scales"].reshape(w.num_experts, w.h).astype(np.float64)
    d = oracle.dispatch(inp["x"], inp["ids"], w.ep_world, w.experts_per_rank, 1, quant_scales=inp["quant_scales"],
                        bf16=True)
    xf = (inp["x"].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    nsat = 0
    for (t, k), code in _codes_by_pair(d, w.bs).items():
        p = xf[t] * c[inp["ids"][t, k]]
        q = code.astype(np.float64)
        inside = (p > -128.5) & (p < 127.5)
        assert (np.abs(p[inside] - q[inside]) <= 0.5).all()
        assert (q[p >= 127.5] == 127).all() and (q[p <= -128.5] == -128).all()
        nsat += int((~inside).sum())
    assert nsat > 0          # the coefficient range makes a few codes saturate


def test_static_quant_rejects_bad_coefficient_counts():
    x = np.ones((4, 8), np.float16)
    ids = np.array([[0], [1], [2], [3]], np.int32)
    for n in (0, 2, 7, 9, 4 * 8 + 1):
        with pytest.raises(oracle.OracleError):
            oracle.dispatch(x, ids, 2, 2, quant_mode=1, quant_scales=np.ones(n, np.float32))


def test_static_codes_round_the_exact_product_once():
    """Products whose binary32 rounding lands on a half-integer while the exact
    value does not: the code follows the exact product (a plain rint of x * c),
    not a rounding of the rounded product. The products are exact in float64
    (8-bit by 24-bit significands), and numpy's rint is the reference."""
    xs = (1.0 + np.arange(128) / 128.0).astype(np.float32)          # every bf16 in [1, 2)
    k = np.arange(120, dtype=np.float64)
    cs = ((2 * k[:, None] + 1) / (2 * xs[None, :].astype(np.float64))).astype(np.float32)   # x * c near k + 1/2
    p64 = xs[None, :].astype(np.float64) * cs.astype(np.float64)
    p32 = (xs[None, :] * cs).astype(np.float64)
    ki, xi = np.nonzero(np.rint(p64) != np.rint(p32))
    assert ki.size >= 16                                              # such products exist
    sel = list(zip(ki[:64], xi[:64]))
    n = len(sel)
    x = wl.f32_to_bf16_bits(np.array([[xs[j]] * 16 for _, j in sel], np.float32))
    ids = np.arange(n, dtype=np.int32)[:, None]                       # W = n, token r -> expert r
    ce = np.repeat(np.array([cs[i, j] for i, j in sel], np.float32)[:, None], 16, axis=1)
    d = oracle.dispatch(x, ids, n, 1, quant_mode=1, quant_scales=ce, bf16=True)
    for r, (i, j) in enumerate(sel):                                  # row r belongs to expert r
        assert (d["expand_x"][r] == np.rint(p64[i, j])).all(), (cs[i, j], xs[j])


def test_identity_expert_dequantisation_matches_torch():
    """The harness's identity expert, bf16(f32(q) * scale) with one scale per row (int8) or per 128-element
    group (E4M3), against torch's int8 / float8_e4m3fn decoding, fp32 multiply and round-to-nearest-even
    bfloat16 cast."""
    import torch

    rng = np.random.default_rng(41)
    rows, h = 37, 300
    q = rng.integers(-128, 128, size=(rows, h)).astype(np.int8)
    sc = (rng.uniform(0.0, 1.0, rows) * 2.0 ** rng.integers(-30, 30, rows)).astype(np.float32)
    sc[3] = 0.0
    got = oracle.identity_expert(q, sc)
    want = (torch.from_numpy(q).float() * torch.from_numpy(sc)[:, None]).bfloat16().view(torch.int16).numpy()
    assert got.view(np.int16).tobytes() == want.tobytes()
    codes = rng.integers(0, 256, size=(rows, h)).astype(np.uint8)
    codes[(codes & 0x7f) == 0x7f] = 0                  # the two NaN codes are not produced by the quantiser
    gs = (rng.uniform(0.0, 1.0, (rows, (h + 127) // 128)) * 2.0 ** rng.integers(-20, 20, (rows, 1))).astype(np.float32)
    got = oracle.identity_expert(codes, gs)
    dec = torch.from_numpy(codes).view(torch.float8_e4m3fn).float()
    full = torch.from_numpy(gs).repeat_interleave(128, dim=1)[:, :h]
    want = (dec * full).bfloat16().view(torch.int16).numpy()
    assert got.view(np.int16).tobytes() == want.tobytes()
