"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Index/count outputs, int32 data, int8 codes and fp32 scales must be bitwise
equal. fp16/bf16 x_out must meet max relative error 1e-3 under the metric
|g - r| / max(sum_k |y_k * s_k|, FLT_MIN); since both sides use one fp32 FMA
per k in the same order and round once, they are also checked for bitwise
equality. Combine runs on the GPU's own dispatch outputs passed through the
identity expert (for int8 rows: bf16(f32(q) * scale)), the oracle's on the
oracle's; the two never exchange data.
"""
import dataclasses

import numpy as np
import pytest
import torch

import combine_ep_recv_amd as moe
import oracle
import workloads as wl

pytestmark = pytest.mark.gpu
DEV = "cuda"
TWO_MIB = 2 * 1024 * 1024


# --------------------------------------------------------------------------
# helpers
# --------------------------------------------------------------------------

def to_dev(a: np.ndarray, bf16=False) -> torch.Tensor:
    if bf16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(DEV)
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def to_np(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).numpy()
    return t.numpy()


def mx_scale_f32(sb):
    """2^(byte - 127) as float32, built from its bits (byte 0 is the subnormal 2^-127)."""
    b = sb.to(torch.int32)
    normal = (b << 23).view(torch.float32)
    return torch.where(b > 0, normal, torch.full_like(normal, 2.0 ** -127))


def gpu_identity_expert(expand_x, dyn):
    """bf16(f32(q) * scale): one scale per row (int8), per 128-element group (E4M3), or 2^(byte - 127) per
    32-element block (MX: uint8 scale bytes)."""
    if dyn is None:
        return expand_x
    if dyn.dtype == torch.uint8:
        sc = mx_scale_f32(dyn).repeat_interleave(32, dim=1)[:, :expand_x.shape[1]]
        return (expand_x.float() * sc).to(torch.bfloat16)
    if dyn.dim() == 2:
        sc = dyn.repeat_interleave(128, dim=1)[:, :expand_x.shape[1]]
        return (expand_x.float() * sc).to(torch.bfloat16)
    return (expand_x.float() * dyn[:, None]).to(torch.bfloat16)


def gpu_quant_scales(w, inp):
    return to_dev(inp["quant_scales"]) if w.quant_mode == 1 else None


def special_args(w):
    """The workload's special-expert counts (dispatch and combine take the same)."""
    return dict(zero_experts=w.zero_experts, copy_experts=w.copy_experts, const_experts=w.const_experts)


def gpu_combine_special(w, inp, x):
    """Combine's special-expert inputs on the GPU: the tokens for copy experts (the combine's dtype:
    bf16 tokens for quantised runs) and the const experts' outputs."""
    cbf = w.dtype == "bf16" or w.quant_mode != 0
    return dict(special_args(w), ori_x=x if w.copy_experts else None,
                const_x=to_dev(inp["const_x"], cbf) if w.const_experts else None)


def oracle_combine_special(w, inp):
    return dict(special_args(w), ori_x=inp["x"] if w.copy_experts else None,
                const_x=inp["const_x"] if w.const_experts else None)


def run_gpu(w, inp, schedule=None):
    bf = w.dtype == "bf16"
    x, ids, sc = to_dev(inp["x"], bf), to_dev(inp["ids"]), to_dev(inp["scales"])
    ex, dyn, assist, erc, esc = moe.dispatch(x, ids, w.ep_world, w.experts_per_rank, w.quant_mode,
                                             expert_scales=sc, schedule=schedule,
                                             quant_scales=gpu_quant_scales(w, inp), **special_args(w))
    y = gpu_identity_expert(ex, dyn if w.quant_mode != 1 else torch.ones(ex.shape[0], device=DEV))
    xo = moe.combine(y, assist, erc, ids, sc, w.ep_world, w.experts_per_rank, **gpu_combine_special(w, inp, x))
    torch.cuda.synchronize()
    return dict(expand_x=to_np(ex), dynamic_scales=None if dyn is None else to_np(dyn),
                assist_info=to_np(assist), ep_recv_count=to_np(erc), expand_scales=to_np(esc),
                x_out=to_np(xo))


def run_oracle(w, inp):
    bf = w.dtype == "bf16"
    d = oracle.dispatch(inp["x"], inp["ids"], w.ep_world, w.experts_per_rank, w.quant_mode,
                        expert_scales=inp["scales"], bf16=bf, quant_scales=inp.get("quant_scales"),
                        **special_args(w))
    y = oracle.identity_expert(d["expand_x"], d["dynamic_scales"] if w.quant_mode != 1
                               else np.ones(w.rows, np.float32))
    out_bf = bf or w.quant_mode != 0
    d["x_out"] = oracle.combine(y, d["assist_info"], d["ep_recv_count"], inp["ids"], inp["scales"],
                                w.ep_world, w.experts_per_rank, bf16=out_bf, **oracle_combine_special(w, inp))
    d["y"] = y
    return d


def as_f32(a, bf16):
    if bf16:
        return (a.astype(np.uint32) << 16).view(np.float32)
    return a.astype(np.float32)


def rel_err_metric(g, r, y, assist, scales, W, bs, K, bf16):
    """max_j |g - r| / max(sum_k |y_k s_k|, FLT_MIN) over all outputs."""
    a = assist.astype(np.int64)
    pair = (a[:, 0] * bs + a[:, 1]) * K + a[:, 2]
    row_of = np.empty_like(pair)
    row_of[pair] = np.arange(pair.size)
    N = scales.shape[0]
    yf = as_f32(y, bf16)
    den = np.zeros((N, y.shape[1]), np.float64)
    for k in range(K):
        den += np.abs(yf[row_of[np.arange(N) * K + k]].astype(np.float64)) * np.abs(scales[:, k:k + 1].astype(np.float64))
    diff = np.abs(as_f32(g, bf16).astype(np.float64) - as_f32(r, bf16).astype(np.float64))
    return float((diff / np.maximum(den, np.finfo(np.float32).tiny)).max()) if diff.size else 0.0


def assert_parity(w, g, o):
    A = o["rows"]          # rows written: N*K, fewer when pairs go to special experts
    assert (g["ep_recv_count"] == o["ep_recv_count"]).all(), "ep_recv_count"
    assert (g["assist_info"][:A] == o["assist_info"][:A]).all(), "assist_info"
    assert g["expand_x"][:A].tobytes() == o["expand_x"][:A].tobytes(), "expand_x"
    assert g["expand_scales"][:A].view(np.uint32).tobytes() == o["expand_scales"][:A].view(np.uint32).tobytes()
    if w.quant_mode in (2, 3):
        assert (g["dynamic_scales"][:A].view(np.uint32).tobytes()
                == o["dynamic_scales"][:A].view(np.uint32).tobytes()), "dynamic_scales"
    if w.quant_mode == 4:
        assert g["dynamic_scales"].dtype == np.uint8
        assert g["dynamic_scales"][:A].tobytes() == o["dynamic_scales"][:A].tobytes(), "scale bytes"
    if w.dtype == "int32":
        assert (g["x_out"] == o["x_out"]).all(), "x_out"
    else:
        bf = w.dtype == "bf16" or w.quant_mode != 0
        if A == w.rows:    # the tolerance metric's denominator sums the K exchanged rows
            err = rel_err_metric(g["x_out"], o["x_out"], o["y"], o["assist_info"], o["scales_in"], w.ep_world,
                                 w.bs, w.topk, bf)
            assert err <= 1e-3, err
        # stricter: same operation order on both sides, so the bits agree
        assert g["x_out"].view(np.uint16).tobytes() == o["x_out"].view(np.uint16).tobytes(), "x_out bits"


def check(w, inp=None, schedule=None):
    inp = inp or wl.make_inputs(w)
    print("parity case %s W=%d bs=%d h=%d K=%d epr=%d %s q%d sched=%s" % (
        w.name, w.ep_world, w.bs, w.h, w.topk, w.experts_per_rank, w.dtype, w.quant_mode,
        None if schedule is None else (schedule.mode, schedule.large_segment_bytes)), flush=True)
    g = run_gpu(w, inp, schedule)
    o = run_oracle(w, inp)
    o["scales_in"] = inp["scales"]
    assert_parity(w, g, o)
    return g, o


# --------------------------------------------------------------------------
# the page workloads, full size
# --------------------------------------------------------------------------

@pytest.mark.parametrize("w", wl.WORKLOADS, ids=lambda w: w.name)
def test_page_workloads_full_size(w):
    check(w)


@pytest.mark.parametrize("name", ["w16_h7168_bf16_q8_pair_mask", "w16_h7168_bf16_q8_special"])
def test_benchmarked_mask_and_special_expert_workloads_full_size(name):
    """The bench's masked and special-expert lines, at their full size and with their own inputs."""
    w = wl.BY_NAME[name]
    if w.mask == "none":
        check(w)
    else:
        check_masked(w, "workload")


# --------------------------------------------------------------------------
# edge cases
# --------------------------------------------------------------------------

EDGE = [
    wl.custom(3, 5, 7, 3, 2, "int32", name="int32_h7_scalar_path"),
    wl.custom(4, 9, 13, 3, 3, "fp16", "gauss_topk", name="fp16_h13_scalar_path"),
    wl.custom(2, 17, 40, 2, 4, "bf16", "zipf_topk", quant_mode=2, name="bf16_q_h40"),
    wl.custom(2, 6, 12, 2, 2, "fp16", "gauss_topk", quant_mode=2, name="fp16_q_h12_scalar_quant"),
    wl.custom(2, 3, 8200, 2, 2, "bf16", "gauss_topk", quant_mode=2, name="bf16_q_h8200_two_pass"),
    wl.custom(2, 600, 64, 3, 4, "fp16", "zipf_topk", name="bs600_three_route_blocks"),
    wl.custom(768, 1, 16, 1, 1, "int32", name="w768_max_world"),
    wl.custom(8, 16, 32, 8, 128, "bf16", "gauss_topk", name="e1024_max_experts"),
    wl.custom(2, 5, 16, 4, 2, "int32", name="topk_equals_experts"),
    wl.custom(4, 1, 24, 1, 1, "fp16", "gauss_topk", name="topk1_bs1"),
    wl.custom(3, 70, 7176, 5, 3, "bf16", "zipf_topk", name="bf16_h7176_ragged_tiles"),
    # h = 1, the smallest hidden size: scalar copy, scalar gather and the block quantiser on one element
    wl.custom(2, 4, 1, 2, 2, "int32", name="int32_h1"),
    wl.custom(3, 5, 1, 2, 2, "fp16", "gauss_topk", name="fp16_h1"),
    wl.custom(2, 7, 1, 3, 2, "bf16", "gauss_topk", quant_mode=2, name="bf16_q_h1_block_quant"),
    wl.custom(2, 3, 16, 70, 40, "int32", name="topk70_copy_lds_path"),
    wl.custom(2, 2, 32, 66, 40, "bf16", "gauss_topk", quant_mode=2, name="topk66_quant_block_path"),
    # the copy with one wavefront per token (from 1024 tokens): rows of 1, 14 and 16 pieces per lane, a row
    # length between template sizes, and the fallbacks beyond 16 pieces or 64 copies
    wl.custom(8, 128, 7168, 8, 8, "bf16", "gauss_topk", name="copy_wave_h7168_j14"),
    wl.custom(4, 300, 8192, 4, 4, "fp16", "zipf_topk", name="copy_wave_h8192_j16"),
    wl.custom(16, 128, 32, 4, 8, "int32", name="copy_wave_int32_j1"),
    wl.custom(2, 700, 1040, 3, 4, "bf16", "gauss_topk", name="copy_wave_h1040_j3_ragged_chunks"),
    wl.custom(2, 512, 8200, 2, 2, "fp16", "gauss_topk", name="copy_slices_h8200_past_16_pieces"),
    wl.custom(4, 256, 16, 65, 20, "int32", name="copy_slices_topk65"),
    # 66 route chunks (the scan kernel), loaded 16 at a time with a partial last batch; ragged chunks of 44
    wl.custom(33, 300, 64, 4, 2, "bf16", "zipf_topk", name="scan_66_chunks"),
    wl.custom(33, 300, 64, 4, 2, "bf16", "gauss_topk", quant_mode=2, name="scan_66_chunks_q8"),
]


@pytest.mark.parametrize("w", EDGE, ids=lambda w: w.name)
def test_edge_shapes(w):
    check(w)


# outputs past the store-policy thresholds: quantised rows above 320 MiB keep a quarter of their stores plain,
# above 512 MiB none, and a copy above 640 MiB of rows goes back to the (token, slice) blocks
LARGE_OUTPUTS = [
    wl.custom(16, 448, 7168, 8, 16, "bf16", "gauss_topk", quant_mode=2, index=4, name="int8_411MB_quarter_plain"),
    wl.custom(16, 448, 7168, 8, 16, "bf16", "gauss_topk", quant_mode=3, index=4, name="fp8_411MB_quarter_plain"),
    wl.custom(16, 448, 7168, 8, 16, "bf16", "gauss_topk", quant_mode=1, index=4, name="static_411MB_nt_stores"),
    wl.custom(16, 448, 7168, 8, 16, "fp16", "zipf_topk", quant_mode=1, static_scales="column", index=4,
              name="static_column_411MB_quarter_plain"),
    wl.custom(16, 600, 7168, 8, 16, "bf16", "gauss_topk", quant_mode=2, index=4, name="int8_551MB_nt_stores"),
    wl.custom(16, 384, 7168, 8, 16, "bf16", "gauss_topk", index=4, name="copy_705MB_slices"),
]


@pytest.mark.parametrize("w", LARGE_OUTPUTS, ids=lambda w: w.name)
def test_large_outputs(w):
    check(w)


def test_hot_experts_max_segments():
    """Every token goes to experts 0..3: four segments per source hold all rows."""
    w = wl.custom(4, 64, 256, 4, 2, "fp16", "gauss_topk", name="hot")
    inp = wl.make_inputs(w)
    inp["ids"] = np.tile(np.array([[3, 0, 2, 1]], np.int32), (w.num_tokens, 1))
    check(w, inp)


def test_zero_tokens_quantise_to_zero():
    w = wl.custom(2, 8, 64, 2, 2, "bf16", "gauss_topk", quant_mode=2, name="zero_rows")
    inp = wl.make_inputs(w)
    inp["x"][[0, 5, 9]] = 0
    g, o = check(w, inp)
    a = g["assist_info"].astype(np.int64)
    t = a[:, 0] * w.bs + a[:, 1]
    assert (g["dynamic_scales"][np.isin(t, [0, 5, 9])] == 0).all()


@pytest.mark.parametrize("exp", [-90, -120], ids=["tiny_fast_path", "subnormal_division_path"])
def test_tiny_tokens_quantise_exactly(exp):
    """Scales below 2^-100 take the IEEE division; just above it the FMA step."""
    w = wl.custom(2, 8, 64, 2, 2, "bf16", "gauss_topk", quant_mode=2, name="tiny")
    inp = wl.make_inputs(w)
    g = np.random.default_rng(17).standard_normal((w.num_tokens, w.h)).astype(np.float32) * np.float32(2.0 ** exp)
    inp["x"] = wl.f32_to_bf16_bits(g)
    check(w, inp)


# --------------------------------------------------------------------------
# quantMode 3: per-group (128) dynamic FP8 E4M3 (readings: group size, E4M3,
# scale = max|x| / 448)
# --------------------------------------------------------------------------

GROUP_QUANT = [
    wl.custom(16, 256, 7168, 8, 16, "bf16", "gauss_topk", quant_mode=3, name="w16_h7168_bf16_fp8"),
    wl.custom(3, 300, 1040, 4, 3, "fp16", "zipf_topk", quant_mode=3, name="fp16_h1040_ragged_group"),
    wl.custom(2, 5, 16, 3, 2, "bf16", "gauss_topk", quant_mode=3, name="h16_one_partial_group"),
    wl.custom(4, 257, 8192, 2, 4, "bf16", "gauss_topk", quant_mode=3, name="h8192_j8"),
    wl.custom(65, 2, 256, 2, 4, "fp16", "gauss_topk", quant_mode=3, name="65_chunks_scanned_offsets"),
    wl.custom(2, 2, 128, 64, 40, "bf16", "gauss_topk", quant_mode=3, name="topk64"),
    wl.custom(2, 40, 12288, 4, 4, "bf16", "gauss_topk", quant_mode=3, name="h12288_j12"),
    wl.custom(2, 40, 16384, 4, 4, "fp16", "zipf_topk", quant_mode=3, name="h16384_j16"),
    wl.custom(2, 40, 16384, 4, 4, "bf16", "gauss_topk", quant_mode=2, name="h16384_int8_j16"),
    wl.custom(2, 40, 16400, 4, 4, "bf16", "gauss_topk", quant_mode=2, name="h16400_int8_block_kernel"),
]


@pytest.mark.parametrize("w", GROUP_QUANT, ids=lambda w: w.name)
def test_group_quant_shapes(w):
    check(w)


@pytest.mark.parametrize("exp", [-90, -125], ids=["tiny_fast_path", "subnormal_division_path"])
def test_group_quant_tiny_and_zero_groups(exp):
    """Group scales below 2^-100 take the IEEE division; zero groups give scale
    0 and codes 0; -0 keeps its sign bit."""
    w = wl.custom(2, 8, 512, 2, 2, "bf16", "gauss_topk", quant_mode=3, name="fp8_tiny")
    inp = wl.make_inputs(w)
    rng = np.random.default_rng(23)
    g = rng.standard_normal((w.num_tokens, w.h)).astype(np.float32)
    g[:, 128:256] *= np.float32(2.0 ** exp)
    g[:, 256:384] = 0.0
    g[3, 300] = -0.0
    g[4] = -0.0
    inp["x"] = wl.f32_to_bf16_bits(g)
    gg, o = check(w, inp)
    assert (gg["dynamic_scales"][:, 2] == 0).all()


def test_group_quant_with_a_mask():
    check_masked(wl.custom(4, 96, 2048, 6, 4, "bf16", "zipf_topk", quant_mode=3, name="fp8_masked"), "pair")


# --------------------------------------------------------------------------
# quantMode 4: MX (OCP MXFP8: E4M3 codes, one E8M0 byte per 32-element block)
# --------------------------------------------------------------------------

MX_QUANT = [
    wl.BY_NAME["w16_h7168_bf16_mxfp8"],                                                   # 224 bytes a row
    wl.custom(3, 300, 1040, 4, 3, "fp16", "zipf_topk", quant_mode=4, name="fp16_h1040_ragged_block"),   # 33
    wl.custom(2, 5, 16, 3, 2, "bf16", "gauss_topk", quant_mode=4, name="h16_one_partial_block"),
    wl.custom(2, 7, 48, 2, 2, "fp16", "gauss_topk", quant_mode=4, name="h48_two_bytes"),
    wl.custom(4, 257, 8192, 2, 4, "bf16", "gauss_topk", quant_mode=4, name="h8192_j8_64_words"),
    wl.custom(65, 2, 256, 2, 4, "fp16", "gauss_topk", quant_mode=4, name="65_chunks_scanned_offsets"),
    wl.custom(2, 2, 128, 64, 40, "bf16", "gauss_topk", quant_mode=4, name="topk64"),
    wl.custom(2, 40, 12288, 4, 4, "bf16", "gauss_topk", quant_mode=4, name="h12288_j12_two_word_passes"),
    wl.custom(2, 40, 16384, 4, 4, "fp16", "zipf_topk", quant_mode=4, name="h16384_j16"),
    wl.custom(2, 33, 16336, 3, 4, "bf16", "zipf_topk", quant_mode=4, name="h16336_j16_511_bytes"),
    wl.custom(16, 448, 7168, 8, 16, "bf16", "gauss_topk", quant_mode=4, index=4, name="mx_411MB"),
]


@pytest.mark.parametrize("w", MX_QUANT, ids=lambda w: w.name)
def test_mx_quant_shapes(w):
    check(w)


def test_mx_quant_tiny_huge_subnormal_and_zero_blocks():
    """Block maxima that clamp the shared exponent at -127 (2^-125, and bf16 subnormals around 2^-130), a
    block near the top of bf16's range (byte 246), all-zero blocks (byte 0) and -0 codes; the dispatch outputs
    bit for bit (the identity expert's products would be subnormal here, so the combine is left out)."""
    w = wl.custom(2, 8, 512, 2, 2, "bf16", "gauss_topk", quant_mode=4, name="mx_edges")
    inp = wl.make_inputs(w)
    rng = np.random.default_rng(29)
    g = rng.standard_normal((w.num_tokens, w.h)).astype(np.float32)
    g[:, 32:64] *= np.float32(2.0 ** -125)
    g[:, 64:96] *= np.float32(2.0 ** -131)               # bf16 subnormals
    g[:, 96:128] = 0.0
    g[:, 128:160] = (g[:, 128:160] * np.float32(2.0 ** 124)).astype(np.float32)
    g[3, 300] = -0.0
    g[4] = -0.0
    g[5, 200:232] = -0.0
    inp["x"] = wl.f32_to_bf16_bits(g)
    x, ids = to_dev(inp["x"], True), to_dev(inp["ids"])
    ex, dyn, assist, erc = moe.dispatch(x, ids, w.ep_world, w.experts_per_rank, 4)
    torch.cuda.synchronize()
    d = oracle.dispatch(inp["x"], inp["ids"], w.ep_world, w.experts_per_rank, 4, bf16=True)
    assert (to_np(erc) == d["ep_recv_count"]).all()
    assert (to_np(assist) == d["assist_info"]).all()
    assert to_np(ex).tobytes() == d["expand_x"].tobytes()
    sb = to_np(dyn)
    assert sb.tobytes() == d["dynamic_scales"].tobytes()
    assert (sb[:, 1] == 0).all() and (sb[:, 2] == 0).all() and (sb[:, 3] == 0).all()
    assert sb[:, 4].max() >= 240 and (to_np(ex) == 0x80).any()


def test_mx_quant_with_a_mask_and_special_experts():
    check_masked(wl.custom(4, 96, 2048, 6, 4, "bf16", "zipf_topk", quant_mode=4, name="mx_masked"), "pair")
    check(wl.custom(4, 33, 2048, 8, 4, "bf16", "zipf_topk", quant_mode=4, zero_experts=4, copy_experts=8,
                    const_experts=2, name="mx_special"))


def test_mx_scale_bytes_at_any_alignment():
    """Scale rows of 224 bytes (words) and 33 bytes (bytes), written at an odd address: the bytes are the
    ones written at an aligned address."""
    for w in (wl.custom(2, 64, 7168, 4, 4, "bf16", "gauss_topk", quant_mode=4, name="mx_words"),
              wl.custom(2, 64, 1040, 4, 4, "fp16", "gauss_topk", quant_mode=4, name="mx_bytes")):
        inp = wl.make_inputs(w)
        bf = w.dtype == "bf16"
        x, ids = to_dev(inp["x"], bf), to_dev(inp["ids"])
        B = (w.h + 31) // 32
        buf = moe.DispatchBuffers(w.ep_world, w.bs, w.experts_per_rank, w.h, w.topk, x.dtype, 4, DEV)
        store = torch.zeros(w.rows * B + 1, dtype=torch.uint8, device=DEV)
        buf.dynamic_scales = store[1:].view(w.rows, B)
        moe.dispatch_into(buf, x, ids)
        torch.cuda.synchronize()
        d = oracle.dispatch(inp["x"], inp["ids"], w.ep_world, w.experts_per_rank, 4, bf16=bf)
        assert to_np(buf.dynamic_scales).tobytes() == d["dynamic_scales"].tobytes(), w.name
        assert to_np(buf.expand_x).tobytes() == d["expand_x"].tobytes(), w.name
        assert int(store[0]) == 0


def random_mx_case(i):
    rng = np.random.default_rng(2900 + i)
    W = int(rng.choice([2, 3, 4, 8, 16, 65]))
    bs = int(rng.integers(1, max(2, 2048 // W)))
    epr = int(rng.integers(1, max(2, min(9, 1024 // W))))
    K = int(rng.integers(1, min(W * epr, 12) + 1))
    dtype = str(rng.choice(["fp16", "bf16"]))
    h = 16 * int(rng.integers(1, 400))
    routing = str(rng.choice(["gauss_topk", "zipf_topk"]))
    zero = int(rng.integers(0, 3))
    copy = 0 if dtype != "bf16" else int(rng.integers(0, 3))
    kind = str(rng.choice(["none", "token_any", "pair"]))
    w = wl.custom(W, bs, h, K, epr, dtype, routing, quant_mode=4, zero_experts=zero, copy_experts=copy,
                  index=2300 + i, name="random_mx%d" % i)
    return w, kind


RANDOM_MX_CASES = [random_mx_case(i) for i in range(12)]


@pytest.mark.parametrize("w,kind", RANDOM_MX_CASES, ids=lambda v: v if isinstance(v, str) else v.name)
def test_random_configurations_mx(w, kind):
    if kind == "none":
        check(w)
    else:
        check_masked(w, kind)


# --------------------------------------------------------------------------
# quantMode 1: static int8, q = sat8(rint(x * c)) with one coefficient, one per
# column or one per expert and column (the page's three coefficient shapes)
# --------------------------------------------------------------------------

STATIC_QUANT = [
    wl.BY_NAME["w16_h7168_bf16_static_q8"],
    wl.custom(16, 256, 7168, 8, 16, "bf16", "gauss_topk", quant_mode=1, static_scales="scalar", index=4,
              name="w16_h7168_bf16_static_one"),
    wl.custom(8, 32, 7168, 8, 8, "fp16", "zipf_topk", quant_mode=1, static_scales="column", name="fp16_h7168_column"),
    wl.custom(2, 5, 16, 3, 2, "bf16", "gauss_topk", quant_mode=1, name="h16_j1_expert"),
    wl.custom(3, 300, 1040, 4, 3, "fp16", "zipf_topk", quant_mode=1, static_scales="column", name="h1040_j2_ragged"),
    wl.custom(4, 100, 4096, 6, 4, "bf16", "gauss_topk", quant_mode=1, name="h4096_j4_expert"),
    wl.custom(4, 257, 8192, 2, 4, "fp16", "gauss_topk", quant_mode=1, static_scales="scalar", name="h8192_j8_one"),
    wl.custom(4, 257, 8192, 2, 4, "bf16", "gauss_topk", quant_mode=1, name="h8192_j8_expert"),
    wl.custom(65, 2, 256, 2, 4, "fp16", "gauss_topk", quant_mode=1, name="65_chunks_scanned_offsets"),
    wl.custom(2, 2, 128, 64, 40, "bf16", "gauss_topk", quant_mode=1, name="topk64_expert"),
    # per-expert coefficients run in groups of source ranks (about 1170 tokens at h = 7168): a ragged last group,
    # several workgroups per (expert, group), and skewed expert loads
    wl.custom(7, 300, 7168, 8, 4, "bf16", "gauss_topk", quant_mode=1, name="expert_ragged_groups"),
    wl.custom(2, 2048, 7168, 2, 2, "fp16", "gauss_topk", quant_mode=1, name="expert_32_parts_per_group"),
    wl.custom(8, 400, 4096, 8, 8, "bf16", "zipf_topk", quant_mode=1, name="expert_zipf_groups"),
    # over 64 rows per wavefront (64 parts of 4 wavefronts per expert): the rows' assist_info entries are loaded
    # 64 at a time, one per lane, so the wavefronts of the busier expert take a second batch
    wl.custom(2, 20000, 16, 1, 1, "bf16", "zipf_topk", quant_mode=1, name="expert_over_64_rows_per_wave"),
    # rows past 8192 elements: 12 and 16 pieces per lane, two pieces per lane in the source-group kernel
    wl.custom(2, 40, 12288, 4, 4, "bf16", "gauss_topk", quant_mode=1, name="h12288_expert"),
    wl.custom(2, 40, 16384, 4, 4, "fp16", "gauss_topk", quant_mode=1, name="h16384_expert"),
    wl.custom(2, 40, 16384, 4, 4, "bf16", "gauss_topk", quant_mode=1, static_scales="column", name="h16384_column"),
    wl.custom(2, 40, 8208, 4, 4, "bf16", "gauss_topk", quant_mode=1, name="h8208_expert_ragged_slices"),
]


@pytest.mark.parametrize("w", STATIC_QUANT, ids=lambda w: w.name)
def test_static_quant_shapes(w):
    check(w)


@pytest.mark.parametrize("kind", ["scalar", "column", "expert"])
def test_static_quant_saturation_nan_and_infinities(kind):
    """Products beyond the int8 range saturate, NaN gives -128, ties go to even."""
    w = wl.custom(2, 8, 64, 2, 2, "bf16", "gauss_topk", quant_mode=1, static_scales=kind, name="static_edges")
    inp = wl.make_inputs(w)
    g = np.random.default_rng(29).standard_normal((w.num_tokens, w.h)).astype(np.float32) * 8
    g[0, :6] = [np.nan, np.inf, -np.inf, -0.0, 1e30, -1e30]
    g[1] = np.arange(w.h) - 32.5                  # halves: ties with a unit coefficient
    inp["x"] = wl.f32_to_bf16_bits(g)
    inp["quant_scales"][: min(4, inp["quant_scales"].size)] = 1.0
    gg, o = check(w, inp)
    assert (gg["expand_x"][:w.rows] == 127).any() and (gg["expand_x"][:w.rows] == -128).any()


def test_static_quant_subnormal_tokens_and_large_coefficients():
    """bf16 subnormal tokens times 2^127: the product is rounded exactly (no flush to zero)."""
    w = wl.custom(2, 8, 64, 2, 2, "bf16", "gauss_topk", quant_mode=1, static_scales="scalar", name="static_subnormal")
    inp = wl.make_inputs(w)
    g = np.random.default_rng(31).standard_normal((w.num_tokens, w.h)).astype(np.float32)
    g *= np.float32(2.0 ** -128)                 # mostly bf16 subnormals
    g[0, :4] = [2.0 ** -127, -(2.0 ** -127), 2.0 ** -130, 3 * 2.0 ** -128]
    inp["x"] = wl.f32_to_bf16_bits(g)
    inp["quant_scales"][:] = 2.0 ** 127
    gg, o = check(w, inp)
    assert (np.abs(gg["expand_x"][:w.rows].astype(int)) > 0).any()


def test_static_quant_with_a_mask_and_special_experts():
    check_masked(wl.custom(4, 96, 2048, 6, 4, "bf16", "zipf_topk", quant_mode=1, name="static_masked"), "pair")
    check(wl.custom(4, 33, 7168, 8, 4, "bf16", "gauss_topk", quant_mode=1, zero_experts=6, copy_experts=6,
                    name="static_special"))


# --------------------------------------------------------------------------
# special experts (zeroExpertNum / copyExpertNum): no row, no count; a zero
# expert adds nothing, a copy expert adds the token itself
# --------------------------------------------------------------------------

SPECIAL = [
    wl.custom(4, 9, 16, 3, 2, "int32", zero_experts=2, copy_experts=3, name="int32_vec"),
    wl.custom(3, 7, 13, 3, 2, "int32", zero_experts=1, copy_experts=1, name="int32_scalar_path"),
    wl.custom(4, 33, 7168, 8, 4, "bf16", "gauss_topk", quant_mode=2, zero_experts=6, copy_experts=6,
              name="bf16_q8_h7168"),
    wl.custom(4, 33, 2048, 8, 4, "bf16", "zipf_topk", quant_mode=3, zero_experts=4, copy_experts=8,
              name="bf16_fp8"),
    wl.custom(3, 70, 7176, 5, 3, "bf16", "zipf_topk", zero_experts=3, copy_experts=3, name="bf16_h7176_scalar"),
    wl.custom(8, 16, 64, 4, 2, "fp16", "gauss_topk", copy_experts=40, name="fp16_mostly_copy"),
    wl.custom(8, 128, 1024, 8, 4, "bf16", "zipf_topk", zero_experts=8, copy_experts=8, name="bf16_copy_wave"),
    wl.custom(2, 6, 32, 2, 1, "fp16", "gauss_topk", zero_experts=30, name="fp16_mostly_zero"),
    # const experts (constExpertNum): const expert j adds row j of the const table
    wl.custom(4, 9, 16, 3, 2, "int32", zero_experts=1, copy_experts=1, const_experts=3, name="int32_const"),
    wl.custom(3, 7, 13, 3, 2, "int32", const_experts=2, name="int32_const_scalar_path"),
    wl.custom(4, 33, 7168, 8, 4, "bf16", "gauss_topk", quant_mode=2, zero_experts=4, copy_experts=4,
              const_experts=4, name="bf16_q8_zero_copy_const"),
    wl.custom(8, 32, 7168, 8, 8, "fp16", "gauss_topk", const_experts=8, name="fp16_w8_const"),
    wl.custom(2, 1100, 64, 8, 4, "bf16", "zipf_topk", zero_experts=2, copy_experts=2, const_experts=2,
              name="bf16_slot_path_special"),
]


@pytest.mark.parametrize("w", SPECIAL, ids=lambda w: w.name)
def test_special_experts(w):
    g, o = check(w)
    assert o["rows"] < w.rows


@pytest.mark.parametrize("kind", ["token_any", "pair"])
def test_special_experts_with_a_mask_and_the_segment_schedule(kind):
    w = wl.custom(4, 40, 512, 4, 3, "bf16", "zipf_topk", zero_experts=3, copy_experts=3, name="special_masked")
    check_masked(w, kind, schedule=moe.MoeSchedule(mode=moe.MOE_SCHED_SEGMENT, large_segment_bytes=1024))


# --------------------------------------------------------------------------
# one launch per call (rows by counting) against the route / slot-pass paths:
# shapes on both sides of each threshold (dispatch: N*K <= 4096, K <= 16,
# W*E <= 4096; combine: bs*K <= 1024, K <= 16, N*K < 2^16, ep_recv_count in
# LDS for W*E <= 2048)
# --------------------------------------------------------------------------

FUSED = [
    wl.custom(8, 64, 2048, 8, 8, "fp16", "gauss_topk", name="fused_nk4096_k8"),
    wl.custom(4, 16, 1024, 16, 8, "bf16", "zipf_topk", name="fused_k16_nk1024"),
    wl.custom(4, 48, 1024, 16, 8, "bf16", "gauss_topk", name="fused_k16_nk3072"),
    wl.custom(2, 257, 512, 8, 4, "fp16", "zipf_topk", name="route_nk4112_fused_combine"),
    wl.custom(4, 8, 256, 17, 8, "bf16", "gauss_topk", name="k17_no_fused_path"),
    wl.custom(64, 2, 64, 4, 2, "bf16", "zipf_topk", name="w64_e128_counts_past_lds"),
    wl.custom(16, 16, 512, 8, 16, "fp16", "gauss_topk", name="w16_e256_combine_erc_global"),
    # 1024 ep_recv_count values: the combine's deeper LDS staging (more than 512, at most 2048)
    wl.custom(8, 16, 512, 8, 16, "fp16", "gauss_topk", name="w8_e128_combine_erc_lds16"),
    wl.custom(16, 8, 256, 16, 4, "bf16", "zipf_topk", name="w16_e64_k16_combine_erc_lds16"),
    wl.custom(2, 1025, 128, 8, 4, "bf16", "gauss_topk", name="bsk8200_slot_pass"),
    wl.custom(4, 128, 256, 8, 4, "fp16", "zipf_topk", name="bsk1024_last_fused_combine"),
    wl.custom(4, 129, 256, 8, 4, "fp16", "zipf_topk", name="bsk1032_slot_pass"),
    wl.custom(5, 3, 8, 7, 3, "int32", name="int32_h8_two_chunks"),
    wl.custom(2, 1, 16, 1, 1, "int32", name="one_token_per_rank_top1"),
]


@pytest.mark.parametrize("w", FUSED, ids=lambda w: w.name)
def test_one_launch_paths_and_their_thresholds(w):
    check(w)


MASKED_FUSED = ("fused_nk4096_k8", "fused_k16_nk3072", "bsk8200_slot_pass", "w8_e128_combine_erc_lds16",
                "w16_e64_k16_combine_erc_lds16")


@pytest.mark.parametrize("kind", ["token_any", "pair"])
@pytest.mark.parametrize("w", [f for f in FUSED if f.name in MASKED_FUSED], ids=lambda w: w.name)
def test_one_launch_paths_with_a_mask(w, kind):
    check_masked(w, kind)


def test_int32_combine_wraps_like_the_oracle():
    w = wl.custom(2, 4, 16, 2, 2, "int32", x_lo=-(2 ** 31), x_hi=2 ** 31 - 1, name="int32_wrap")
    check(w)


def test_empty_batch_writes_zero_counts():
    W, epr, h, K = 4, 2, 16, 2
    x = torch.empty((0, h), dtype=torch.float16, device=DEV)
    ids = torch.empty((0, K), dtype=torch.int32, device=DEV)
    ex, dyn, assist, erc = moe.dispatch(x, ids, W, epr)
    torch.cuda.synchronize()
    assert ex.shape == (0, h) and assist.shape == (0, 3) and dyn is None
    assert (to_np(erc) == 0).all() and erc.shape == (W, epr * W)
    buf = moe.DispatchBuffers(W, 0, epr, h, K, torch.float16)
    buf.ep_recv_count.fill_(7)                   # the counts are written, not left as they were
    moe.dispatch_into(buf, x, ids)
    torch.cuda.synchronize()
    assert (to_np(buf.ep_recv_count) == 0).all()
    xo = moe.combine(ex, assist, erc, ids, torch.empty((0, K), dtype=torch.float32, device=DEV), W, epr)
    assert xo.shape == (0, h)
    # and with each quantiser: zero counts, empty codes and scales
    xb = torch.empty((0, h), dtype=torch.bfloat16, device=DEV)
    for q in (moe.MOE_QUANT_DYN_TOKEN, moe.MOE_QUANT_DYN_GROUP, moe.MOE_QUANT_MX):
        ex, dyn, assist, erc = moe.dispatch(xb, ids, W, epr, q)
        torch.cuda.synchronize()
        assert ex.shape == (0, h) and dyn.shape[0] == 0 and (to_np(erc) == 0).all(), q


# --------------------------------------------------------------------------
# schedules: result-neutral, and the large-segment predicate matches
# --------------------------------------------------------------------------

SCHED_CASES = [wl.WORKLOADS[1], wl.WORKLOADS[2], wl.WORKLOADS[3], wl.WORKLOADS[4],
               wl.custom(4, 192, 7168, 4, 2, "fp16", "zipf_topk", name="zipf_bs192_literal_rule_fires"),
               wl.custom(3, 70, 7176, 5, 3, "bf16", "zipf_topk", quant_mode=2, name="bf16_q_ragged"),
               # the segment payload's wavefront kernels at 16 pieces per lane and a ragged 2-piece row, the
               # block kernel for rows that are not 16-byte pieces, and 104 ranks (10,816 segments: the most,
               # 11, per thread of the plan's scans)
               wl.custom(4, 100, 8192, 4, 4, "fp16", "zipf_topk", name="copy_h8192_j16"),
               wl.custom(2, 40, 16384, 4, 4, "bf16", "gauss_topk", quant_mode=2, name="q8_h16384_j16"),
               wl.custom(3, 300, 1040, 4, 3, "fp16", "zipf_topk", quant_mode=2, name="q8_h1040_j2"),
               wl.custom(3, 20, 13, 3, 2, "int32", name="int32_h13_block_path"),
               wl.custom(104, 3, 16, 2, 1, "bf16", "zipf_topk", name="w104_11_segments_per_thread"),
               # topk > 64 (the token-major kernels' LDS row path), and 66 route chunks (offsets from the
               # scan block instead of per-pair chunk sums)
               wl.custom(2, 24, 64, 70, 40, "fp16", "zipf_topk", name="copy_k70_lds_rows"),
               wl.custom(2, 24, 64, 70, 40, "bf16", "gauss_topk", quant_mode=2, name="q8_k70_block_kernel"),
               wl.custom(2, 8300, 32, 2, 2, "bf16", "zipf_topk", quant_mode=2, name="q8_66_chunks_scan_offsets")]


@pytest.mark.parametrize("w", SCHED_CASES, ids=lambda w: w.name)
@pytest.mark.parametrize("mode", [moe.MOE_SCHED_TOKEN, moe.MOE_SCHED_SEGMENT, moe.MOE_SCHED_ADAPTIVE],
                         ids=["token", "segment", "adaptive"])
@pytest.mark.parametrize("T", [-1, 0, 64 * 1024, 1 << 40], ids=["T2MiB", "T0", "T64KiB", "Tinf"])
def test_schedules_are_result_neutral_and_flag_the_right_segments(w, mode, T):
    inp = wl.make_inputs(w)
    flags = torch.full((w.ep_world, w.experts_per_rank * w.ep_world), -1, dtype=torch.int32, device=DEV)
    sched = moe.MoeSchedule(mode=mode, large_segment_bytes=T, segment_is_large=flags.data_ptr())
    g, o = check(w, inp, sched)
    elem = 1 if w.quant_mode != 0 else (4 if w.dtype == "int32" else 2)
    want = oracle.large_segments(o["ep_recv_count"], w.ep_world, w.experts_per_rank, w.h, elem,
                                 TWO_MIB if T < 0 else T)
    assert (to_np(flags) == want.astype(np.int32)).all()
    if T < 0 and w.name != "zipf_bs192_literal_rule_fires":
        assert want.sum() == 0     # the README's 2 MiB never fires on the page workloads


@pytest.mark.parametrize("q", [1, 3, 4], ids=["static", "fp8_group", "mx"])
@pytest.mark.parametrize("mode", [moe.MOE_SCHED_TOKEN, moe.MOE_SCHED_ADAPTIVE], ids=["token", "adaptive"])
def test_token_major_quantisers_report_segment_flags(q, mode):
    """The quantisers that run token-major only, with segment flags requested: the scan block then forms the
    offsets (and the flags) in place of the per-pair chunk sums; outputs and flags match the oracle."""
    w = wl.custom(4, 192, 2048, 4, 2, "bf16", "zipf_topk", quant_mode=q, name="flags_q%d" % q)
    inp = wl.make_inputs(w)
    flags = torch.full((w.ep_world, w.experts_per_rank * w.ep_world), -1, dtype=torch.int32, device=DEV)
    sched = moe.MoeSchedule(mode=mode, large_segment_bytes=4096, segment_is_large=flags.data_ptr())
    g, o = check(w, inp, sched)
    want = oracle.large_segments(o["ep_recv_count"], w.ep_world, w.experts_per_rank, w.h, 1, 4096)
    assert want.sum() > 0 and (to_np(flags) == want.astype(np.int32)).all()


ADAPTIVE_FLAG_CASES = [SCHED_CASES[i] for i in (2, 3, 4, 5, 6, 9, 12, 13)]


def adaptive_row_flags(w, workspace):
    """The adaptive schedule's per-row flags, read from the dispatch workspace (white box): one byte per row in
    the segment plan's region, which follows pc, pci and boff ([NB, E] int32 each) and lr ([N*K] int32), each
    region 256-byte aligned."""
    nb = w.ep_world * ((w.bs + 255) // 256)
    r256 = lambda n: (n + 255) // 256 * 256
    off = 3 * r256(nb * w.num_experts * 4) + r256(w.rows * 4)
    return to_np(workspace[off:off + w.rows])


@pytest.mark.parametrize("w", ADAPTIVE_FLAG_CASES, ids=lambda w: w.name)
@pytest.mark.parametrize("T", [0, 64 * 1024, -1], ids=["T0", "T64KiB", "T2MiB"])
def test_adaptive_schedule_leaves_out_exactly_the_rows_of_large_segments(w, T):
    """The token-major kernels evaluate the predicate per pair and flag the rows they leave to the second pass;
    the flagged rows are exactly the rows of the segments the oracle's predicate selects (outputs alone cannot
    show this: either pass writes the same bytes)."""
    elem = 1 if w.quant_mode != 0 else (4 if w.dtype == "int32" else 2)
    thr = TWO_MIB if T < 0 else T
    if w.bs * w.h * elem < thr:
        pytest.skip("no segment can reach the threshold: the adaptive pass is not engaged")
    inp = wl.make_inputs(w)
    bf = w.dtype == "bf16"
    x, ids, sc = to_dev(inp["x"], bf), to_dev(inp["ids"]), to_dev(inp["scales"])
    tdt = {"int32": torch.int32, "fp16": torch.float16, "bf16": torch.bfloat16}[w.dtype]
    print("adaptive flags case %s T=%d" % (w.name, thr), flush=True)
    buf = moe.DispatchBuffers(w.ep_world, w.bs, w.experts_per_rank, w.h, w.topk, tdt, w.quant_mode, DEV)
    moe.dispatch_into(buf, x, ids, expert_scales=sc,
                      schedule=moe.MoeSchedule(mode=moe.MOE_SCHED_ADAPTIVE, large_segment_bytes=T))
    torch.cuda.synchronize()
    o = oracle.dispatch(inp["x"], inp["ids"], w.ep_world, w.experts_per_rank, w.quant_mode, bf16=bf)
    erc = o["ep_recv_count"]
    large = oracle.large_segments(erc, w.ep_world, w.experts_per_rank, w.h, elem, thr)
    want = np.zeros(w.rows, np.uint8)
    base = 0
    for r in range(w.ep_world):
        for g in range(erc.shape[1]):
            lo = base + (erc[r, g - 1] if g else 0)
            if large[r, g]:
                want[lo:base + erc[r, g]] = 1
        base += erc[r, -1]
    got = adaptive_row_flags(w, buf.workspace)
    assert (got[:base] == want[:base]).all(), (int(got[:base].sum()), int(want[:base].sum()))
    if T == 0:
        assert want.sum() > 0      # the case exercises the second pass


def test_default_schedule_splits_off_the_segments_the_literal_rule_selects():
    """With no schedule the dispatch is adaptive at the README's 2 MiB: on this shape (192 tokens per rank of 7168
    fp16, Zipf routing) a segment can reach 2 MiB, so the large-segment pass runs, and some segments are large."""
    w = SCHED_CASES[4]
    assert w.name == "zipf_bs192_literal_rule_fires"
    inp = wl.make_inputs(w)
    _, o = check(w, inp, None)
    assert oracle.large_segments(o["ep_recv_count"], w.ep_world, w.experts_per_rank, w.h, 2, TWO_MIB).sum() > 0


# --------------------------------------------------------------------------
# the wavefront-per-token quantiser across its row-length templates and the
# two offset paths (chunk prefixes summed per pair up to 64 chunks, scan beyond)
# --------------------------------------------------------------------------

QUANT_WAVE = [
    wl.custom(2, 5, 16, 3, 2, "bf16", "gauss_topk", quant_mode=2, name="h16_one_chunk_per_lane"),
    wl.custom(3, 300, 1040, 4, 3, "fp16", "zipf_topk", quant_mode=2, name="h1040_two_chunks_per_rank"),
    wl.custom(4, 257, 8192, 2, 4, "bf16", "gauss_topk", quant_mode=2, name="h8192_ragged_chunks"),
    wl.custom(64, 3, 64, 2, 4, "fp16", "gauss_topk", quant_mode=2, name="64_chunks_direct_offsets"),
    wl.custom(8, 16, 32, 8, 128, "bf16", "gauss_topk", quant_mode=2, name="e1024_quantised"),
    wl.custom(65, 2, 64, 2, 4, "bf16", "gauss_topk", quant_mode=2, name="65_chunks_scanned_offsets"),
    wl.custom(4, 601, 7168, 8, 4, "fp16", "zipf_topk", quant_mode=2, name="138MB_mixed_store_kinds"),
]


@pytest.mark.parametrize("w", QUANT_WAVE, ids=lambda w: w.name)
def test_quantiser_shapes(w):
    check(w)


def test_workspace_contents_on_entry_do_not_matter():
    """Dispatch into a workspace holding other bytes, or an earlier call's
    counts for other ids, gives the same outputs."""
    w = wl.custom(4, 300, 256, 4, 3, "bf16", "zipf_topk", quant_mode=2, name="stale_workspace")
    print("parity case %s" % w.name, flush=True)
    inp_a, inp_b = wl.make_inputs(w, seed=11), wl.make_inputs(w, seed=12)
    o = run_oracle(w, inp_b)
    buf = moe.DispatchBuffers(w.ep_world, w.bs, w.experts_per_rank, w.h, w.topk, torch.bfloat16, 2, DEV)
    xa, ida = to_dev(inp_a["x"], True), to_dev(inp_a["ids"])
    xb, idb = to_dev(inp_b["x"], True), to_dev(inp_b["ids"])
    for fill in (None, 0x00, 0xFF, 0x80):
        if fill is None:
            moe.dispatch_into(buf, xa, ida)          # leaves this call's counts behind
        else:
            buf.workspace.fill_(fill)
        moe.dispatch_into(buf, xb, idb)
        torch.cuda.synchronize()
        assert to_np(buf.expand_x).tobytes() == o["expand_x"].tobytes(), fill
        assert to_np(buf.dynamic_scales).view(np.uint32).tobytes() == o["dynamic_scales"].view(np.uint32).tobytes()
        assert (to_np(buf.assist_info) == o["assist_info"]).all(), fill
        assert (to_np(buf.ep_recv_count) == o["ep_recv_count"]).all(), fill


# --------------------------------------------------------------------------
# token masks (aclnnMoeDistributeDispatchV4 参数说明, xActiveMaskOptional):
# inactive pairs get no row and no count; the A active pairs fill rows 0..A-1;
# a token with no active pair combines to 0
# --------------------------------------------------------------------------

def _make_mask(kind, w, seed):
    rng = np.random.default_rng(seed)
    N, K, bs = w.num_tokens, w.topk, w.bs
    if kind == "token_prefix":          # each rank's active tokens first, as the pages ask
        m = np.zeros(N, bool)
        for s in range(w.ep_world):
            m[s * bs: s * bs + rng.integers(0, bs + 1)] = True
        return m
    if kind == "token_any":
        return rng.random(N) < 0.6
    if kind == "pair":
        m = rng.random((N, K)) < 0.7
        m[rng.random(N) < 0.2] = False  # some tokens switched off entirely
        return m
    if kind == "pair_all_off":
        return np.zeros((N, K), bool)
    raise ValueError(kind)


def check_masked(w, kind, seed=1, schedule=None):
    inp = wl.make_inputs(w)
    mask = inp["mask"].astype(bool) if kind == "workload" else _make_mask(kind, w, seed)
    print("parity case %s mask=%s seed=%d W=%d bs=%d h=%d K=%d %s q%d sched=%s" % (
        w.name, kind, seed, w.ep_world, w.bs, w.h, w.topk, w.dtype, w.quant_mode,
        None if schedule is None else schedule.mode), flush=True)
    bf = w.dtype == "bf16"
    x, ids, sc = to_dev(inp["x"], bf), to_dev(inp["ids"]), to_dev(inp["scales"])
    m = torch.from_numpy(mask).to(DEV)
    ex, dyn, assist, erc, esc = moe.dispatch(x, ids, w.ep_world, w.experts_per_rank, w.quant_mode,
                                             expert_scales=sc, schedule=schedule, x_active_mask=m,
                                             quant_scales=gpu_quant_scales(w, inp), **special_args(w))
    y = gpu_identity_expert(ex, dyn if w.quant_mode != 1 else torch.ones(ex.shape[0], device=DEV))
    xo = moe.combine(y, assist, erc, ids, sc, w.ep_world, w.experts_per_rank, x_active_mask=m,
                     **gpu_combine_special(w, inp, x))
    torch.cuda.synchronize()
    d = oracle.dispatch(inp["x"], inp["ids"], w.ep_world, w.experts_per_rank, w.quant_mode,
                        expert_scales=inp["scales"], bf16=bf, mask=mask, quant_scales=inp.get("quant_scales"),
                        **special_args(w))
    yo = oracle.identity_expert(d["expand_x"], d["dynamic_scales"] if w.quant_mode != 1
                                else np.ones(w.rows, np.float32))
    xo_o = oracle.combine(yo, d["assist_info"], d["ep_recv_count"], inp["ids"], inp["scales"], w.ep_world,
                          w.experts_per_rank, bf16=bf or w.quant_mode != 0, mask=mask,
                          **oracle_combine_special(w, inp))
    A = d["rows"]
    assert (to_np(erc) == d["ep_recv_count"]).all(), "ep_recv_count"
    assert (to_np(assist)[:A] == d["assist_info"][:A]).all(), "assist_info"
    assert to_np(ex)[:A].tobytes() == d["expand_x"][:A].tobytes(), "expand_x"
    assert to_np(esc)[:A].view(np.uint32).tobytes() == d["expand_scales"][:A].view(np.uint32).tobytes()
    if w.quant_mode in (2, 3):
        assert to_np(dyn)[:A].view(np.uint32).tobytes() == d["dynamic_scales"][:A].view(np.uint32).tobytes()
    if w.quant_mode == 4:
        assert to_np(dyn)[:A].tobytes() == d["dynamic_scales"][:A].tobytes(), "scale bytes"
    g = to_np(xo)
    if w.dtype == "int32":
        assert (g == xo_o).all(), "x_out"
    else:
        assert g.view(np.uint16).tobytes() == xo_o.view(np.uint16).tobytes(), "x_out bits"
    if w.dtype != "int32" and not (w.zero_experts or w.copy_experts or w.const_experts):
        # and the tolerance metric over the active pairs
        act = np.repeat(mask[:, None], w.topk, axis=1) if mask.ndim == 1 else mask
        yf = as_f32(yo, True if (bf or w.quant_mode != 0) else False)
        den = np.zeros(g.shape, np.float64)
        a3 = d["assist_info"][:A].astype(np.int64)
        row_of = np.full(w.num_tokens * w.topk, -1, np.int64)
        row_of[(a3[:, 0] * w.bs + a3[:, 1]) * w.topk + a3[:, 2]] = np.arange(A)
        for k in range(w.topk):
            t_on = np.nonzero(act[:, k])[0]
            r = row_of[t_on * w.topk + k]
            assert (r >= 0).all()
            den[t_on] += np.abs(yf[r].astype(np.float64)) * np.abs(inp["scales"][t_on, k].astype(np.float64))[:, None]
        bfo = bf or w.quant_mode != 0
        diff = np.abs(as_f32(g, bfo).astype(np.float64) - as_f32(xo_o, bfo).astype(np.float64))
        assert (diff / np.maximum(den, np.finfo(np.float32).tiny)).max() <= 1e-3
    return A


MASK_CASES = [
    (wl.WORKLOADS[1], "token_prefix"),
    (wl.WORKLOADS[1], "pair"),
    (wl.WORKLOADS[2], "token_prefix"),
    (wl.WORKLOADS[3], "token_any"),
    (wl.WORKLOADS[4], "pair"),
    (wl.custom(3, 70, 7176, 5, 3, "bf16", "zipf_topk", name="bf16_h7176_scalar_copy"), "pair"),
    (wl.custom(4, 9, 13, 3, 3, "fp16", "gauss_topk", quant_mode=2, name="fp16_q_h13_block_quant"), "token_any"),
    (wl.custom(2, 2, 32, 66, 40, "bf16", "gauss_topk", quant_mode=2, name="topk66_quant_block"), "pair"),
    (wl.custom(65, 2, 64, 2, 4, "bf16", "gauss_topk", quant_mode=2, name="65_chunks_scan"), "pair"),
    (wl.custom(2, 600, 64, 3, 4, "fp16", "zipf_topk", name="bs600"), "token_prefix"),
    (wl.custom(2, 5, 16, 4, 2, "int32", name="topk_equals_experts"), "pair_all_off"),
]


@pytest.mark.parametrize("w,kind", MASK_CASES, ids=lambda v: v if isinstance(v, str) else v.name)
def test_token_masks(w, kind):
    A = check_masked(w, kind)
    if kind == "pair_all_off":
        assert A == 0


@pytest.mark.parametrize("kind", ["token_prefix", "pair"])
def test_token_masks_with_the_segment_schedule(kind):
    w = wl.custom(4, 192, 7168, 4, 2, "fp16", "zipf_topk", name="zipf_bs192")
    check_masked(w, kind, schedule=moe.MoeSchedule(mode=moe.MOE_SCHED_SEGMENT, large_segment_bytes=64 * 1024))


# --------------------------------------------------------------------------
# seeded random configurations: features combined in ways the lists above do
# not (quant mode x mask kind x special experts x ragged shapes x chunk counts)
# --------------------------------------------------------------------------

def random_case(i):
    rng = np.random.default_rng(900 + i)
    W = int(rng.choice([2, 3, 4, 8, 16, 65]))
    bs = int(rng.integers(1, max(2, 2048 // W)))
    epr = int(rng.integers(1, max(2, min(9, 1024 // W))))
    K = int(rng.integers(1, min(W * epr, 12) + 1))
    dtype = str(rng.choice(["int32", "fp16", "bf16"]))
    quant = 0 if dtype == "int32" else int(rng.choice([0, 1, 2, 3]))
    h = 16 * int(rng.integers(1, 257)) if quant in (1, 3) else int(rng.integers(1, 3000))
    routing = "uniform_distinct" if dtype == "int32" else str(rng.choice(["gauss_topk", "zipf_topk"]))
    zero = int(rng.integers(0, 3))
    copy = 0 if (quant and dtype != "bf16") else int(rng.integers(0, 3))     # copy tokens in the combine's dtype
    kind = str(rng.choice(["none", "token_any", "pair"]))
    sk = str(rng.choice(["scalar", "column", "expert"]))
    w = wl.custom(W, bs, h, K, epr, dtype, routing, quant_mode=quant, zero_experts=zero, copy_experts=copy,
                  static_scales=sk, index=300 + i, name="random%d" % i)
    return w, kind


RANDOM_CASES = [random_case(i) for i in range(28)]


@pytest.mark.parametrize("w,kind", RANDOM_CASES, ids=lambda v: v if isinstance(v, str) else v.name)
def test_random_configurations(w, kind):
    if kind == "none":
        check(w)
    else:
        check_masked(w, kind)


def random_small_case(i):
    """Small batches, mostly on the one-launch paths (dispatch: copies with N*K <= 4096, K <= 16;
    combine: bs*K <= 1024), with const experts beside zero and copy ones."""
    rng = np.random.default_rng(1900 + i)
    W = int(rng.choice([2, 3, 4, 5, 8, 12]))
    K = int(rng.integers(1, 17))
    epr = int(rng.integers(max(1, -(-K // W)), 9))
    bs = int(rng.integers(1, max(2, min(1024 // K, 4096 // (W * K)) + 1)))
    dtype = str(rng.choice(["int32", "fp16", "bf16"]))
    quant = 0 if dtype == "int32" else int(rng.choice([0, 0, 0, 2]))
    step = 4 if dtype == "int32" else 8                # 16-byte rows, except now and then
    h = step * int(rng.integers(1, 400)) if rng.random() < 0.85 else int(rng.integers(1, 300))
    routing = "uniform_distinct" if dtype == "int32" else str(rng.choice(["gauss_topk", "zipf_topk"]))
    zero, const = int(rng.integers(0, 3)), int(rng.integers(0, 3))
    copy = 0 if (quant and dtype != "bf16") else int(rng.integers(0, 3))
    kind = str(rng.choice(["none", "token_any", "pair"]))
    w = wl.custom(W, bs, h, K, epr, dtype, routing, quant_mode=quant, zero_experts=zero, copy_experts=copy,
                  const_experts=const, index=1300 + i, name="small%d" % i)
    return w, kind


RANDOM_SMALL_CASES = [random_small_case(i) for i in range(24)]


@pytest.mark.parametrize("w,kind", RANDOM_SMALL_CASES, ids=lambda v: v if isinstance(v, str) else v.name)
def test_random_small_batches(w, kind):
    if kind == "none":
        check(w)
    else:
        check_masked(w, kind)


def random_segment_case(i):
    """A random configuration through the segment schedule at a random large-segment threshold (the schedule
    takes copies and per-token int8; its segment counts stay within the scan's LDS)."""
    w, kind = random_case(i)
    if w.quant_mode in (1, 3):
        w = dataclasses.replace(w, quant_mode=2, copy_experts=w.copy_experts if w.dtype == "bf16" else 0)
    while w.ep_world * w.ep_world * w.experts_per_rank > 11264:
        w = dataclasses.replace(w, experts_per_rank=max(1, w.experts_per_rank // 2),
                                topk=min(w.topk, w.ep_world * max(1, w.experts_per_rank // 2)))
    T = int(np.random.default_rng(i).choice([0, 4096, 65536, -1]))
    return w, kind, T


RANDOM_SEGMENT_CASES = [random_segment_case(i) for i in range(100, 112)]
RANDOM_ADAPTIVE_CASES = [random_segment_case(i) for i in range(112, 124)]


@pytest.mark.parametrize("w,kind,T", RANDOM_SEGMENT_CASES,
                         ids=lambda v: v if isinstance(v, (str, int)) else v.name)
def test_random_configurations_segment_schedule(w, kind, T):
    sched = moe.MoeSchedule(mode=moe.MOE_SCHED_SEGMENT, large_segment_bytes=T)
    if kind == "none":
        check(w, schedule=sched)
    else:
        check_masked(w, kind, schedule=sched)


@pytest.mark.parametrize("w,kind,T", RANDOM_ADAPTIVE_CASES,
                         ids=lambda v: v if isinstance(v, (str, int)) else v.name)
def test_random_configurations_adaptive_schedule(w, kind, T):
    sched = moe.MoeSchedule(mode=moe.MOE_SCHED_ADAPTIVE, large_segment_bytes=T)
    if kind == "none":
        check(w, schedule=sched)
    else:
        check_masked(w, kind, schedule=sched)


def random_large_case(i):
    """Batches of 300 to 600 MB of rows, around the store-policy and copy-kernel thresholds (FP8 has its own
    large case: its oracle is the slowest)."""
    rng = np.random.default_rng(700 + i)
    W = int(rng.choice([8, 16, 32]))
    h = 16 * int(rng.integers(256, 513))                     # 4096 .. 8192
    K = int(rng.choice([4, 6, 8]))
    quant = int(rng.choice([0, 1, 2]))
    dtype = "bf16" if quant else str(rng.choice(["fp16", "bf16"]))
    target = float(rng.uniform(3e8, 6e8))                     # bytes of expand_x rows
    bs = max(1, int(target / (W * K * h * (1 if quant else 2))))
    epr = int(rng.choice([4, 8, 16]))
    kind = str(rng.choice(["none", "pair"]))
    w = wl.custom(W, bs, h, K, epr, dtype, str(rng.choice(["gauss_topk", "zipf_topk"])), quant_mode=quant,
                  zero_experts=int(rng.integers(0, 2)), copy_experts=int(rng.integers(0, 2)) if dtype == "bf16" else 0,
                  static_scales=str(rng.choice(["scalar", "column", "expert"])), index=500 + i,
                  name="random_large%d" % i)
    return w, kind


RANDOM_LARGE_CASES = [random_large_case(i) for i in range(4)]


@pytest.mark.parametrize("w,kind", RANDOM_LARGE_CASES, ids=lambda v: v if isinstance(v, str) else v.name)
def test_random_large_configurations(w, kind):
    if kind == "none":
        check(w)
    else:
        check_masked(w, kind)


def random_sweep_case(i):
    """A wider random draw than the lists above: up to 768 ranks with tiny batches, the one-launch region, topk
    up to 64, ragged h, every quantiser, mask kind and special-expert kind, and now and then the segment schedule
    (copies and per-token int8) at a random threshold. Sized so the oracle stays fast."""
    rng = np.random.default_rng(50000 + i)
    region = rng.random()
    if region < 0.15:
        W, bs, epr = int(rng.choice([96, 128, 200, 384, 768])), int(rng.integers(1, 4)), 1
    elif region < 0.5:
        W = int(rng.choice([2, 3, 4, 6, 8, 16, 32, 64, 65]))
        bs = int(rng.integers(1, max(2, 4096 // (W * 4))))
        epr = int(rng.integers(1, max(2, min(9, 1024 // W))))
    else:
        W = int(rng.choice([2, 3, 4, 5, 8, 16, 24]))
        bs = int(rng.integers(1, 700 // max(1, W // 4)))
        epr = int(rng.integers(1, max(2, min(17, 1024 // W))))
    K = int(rng.integers(1, min(W * epr, 64 if rng.random() < 0.1 else 16) + 1))
    dtype = str(rng.choice(["int32", "fp16", "bf16"]))
    quant = 0 if dtype == "int32" else int(rng.choice([0, 0, 1, 2, 2, 3]))
    if quant in (1, 3):
        h = 16 * int(rng.integers(1, 200))
    else:
        h = int(rng.choice([8, 16, 24, 64, 1024, 7168])) if rng.random() < 0.6 else int(rng.integers(1, 2000))
    routing = "uniform_distinct" if dtype == "int32" else str(rng.choice(["gauss_topk", "zipf_topk"]))
    zero, const = int(rng.integers(0, 3)), int(rng.integers(0, 3))
    copy = 0 if (quant and dtype != "bf16") else int(rng.integers(0, 3))
    sk = str(rng.choice(["scalar", "column", "expert"]))
    kind = str(rng.choice(["none", "none", "token_any", "token_prefix", "pair"]))
    w = wl.custom(W, bs, h, K, epr, dtype, routing, quant_mode=quant, zero_experts=zero, copy_experts=copy,
                  const_experts=const, static_scales=sk, index=20000 + i, name="sweep%d" % i)
    T = None
    if quant in (0, 2) and rng.random() < 0.2 and W * W * epr <= 11264:
        T = int(rng.choice([0, 4096, 65536, -1]))
    return w, kind, T


RANDOM_SWEEP_CASES = [c for c in (random_sweep_case(i) for i in range(170))
                      if c[0].num_tokens * c[0].topk * c[0].h <= 6e7][:150]


@pytest.mark.parametrize("w,kind,T", RANDOM_SWEEP_CASES,
                         ids=lambda v: v if isinstance(v, (str, int)) or v is None else v.name)
def test_random_sweep(w, kind, T):
    sched = None if T is None else moe.MoeSchedule(mode=moe.MOE_SCHED_SEGMENT, large_segment_bytes=T)
    if kind == "none":
        check(w, schedule=sched)
    else:
        check_masked(w, kind, seed=int(w.name[5:]), schedule=sched)


# --------------------------------------------------------------------------
# determinism (aclnnMoeDistributeDispatchV4 约束说明: deterministic by default)
# --------------------------------------------------------------------------

def test_repeat_runs_are_bitwise_identical():
    w = wl.WORKLOADS[3]
    inp = wl.make_inputs(w)
    a = run_gpu(w, inp)
    b = run_gpu(w, inp)
    for k in a:
        if a[k] is not None:
            assert a[k].tobytes() == b[k].tobytes(), k


# --------------------------------------------------------------------------
# HIP graphs: every launch goes on the caller's stream, with no allocation and
# no memset, so a step can be captured and replayed; each replay must equal
# the eager result (checked after eager work between replays)
# --------------------------------------------------------------------------

GRAPH_CASES = [
    (wl.WORKLOADS[2], None),
    (wl.custom(4, 64, 1024, 8, 4, "bf16", "gauss_topk", quant_mode=2, name="bf16_q8_graph"), None),
    # the adaptive schedule's second pass and the segment-major schedule's scan and plan, both engaged at T = 0
    (wl.custom(4, 64, 1024, 8, 4, "bf16", "zipf_topk", quant_mode=2, name="bf16_q8_graph_adaptive_T0"),
     (moe.MOE_SCHED_ADAPTIVE, 0)),
    (wl.custom(4, 64, 1024, 8, 4, "fp16", "zipf_topk", name="fp16_copy_graph_segment_T0"), (moe.MOE_SCHED_SEGMENT, 0)),
    # MXFP8 codes and scale bytes (h = 1040: 33 bytes a row, byte stores)
    (wl.custom(4, 64, 1040, 8, 4, "bf16", "gauss_topk", quant_mode=4, name="bf16_mx_graph"), None),
]


@pytest.mark.parametrize("w,sched", GRAPH_CASES, ids=lambda v: v.name if hasattr(v, "name") else str(v))
def test_graph_replay_matches_eager(w, sched):
    print("parity case %s graph replay" % w.name, flush=True)
    schedule = None if sched is None else moe.MoeSchedule(mode=sched[0], large_segment_bytes=sched[1])
    inp = wl.make_inputs(w)
    bf = w.dtype == "bf16"
    x, ids, sc = to_dev(inp["x"], bf), to_dev(inp["ids"]), to_dev(inp["scales"])
    tdt = torch.bfloat16 if bf else torch.float16
    buf = moe.DispatchBuffers(w.ep_world, w.bs, w.experts_per_rank, w.h, w.topk, tdt, w.quant_mode, DEV)
    moe.dispatch_into(buf, x, ids, schedule=schedule)
    y = gpu_identity_expert(buf.expand_x, buf.dynamic_scales)   # for copies: expand_x itself, rewritten each step
    out = torch.empty((w.num_tokens, w.h), dtype=y.dtype, device=DEV)
    cws = moe.combine_workspace(w.ep_world, w.bs, w.experts_per_rank, w.h, w.topk, y.dtype, DEV)

    def step():
        moe.dispatch_into(buf, x, ids, schedule=schedule)
        moe.combine_into(out, y, buf.assist_info, buf.ep_recv_count, ids, sc, w.ep_world, w.experts_per_rank, cws)

    def snapshot():
        torch.cuda.synchronize()
        return [t.clone() for t in (buf.expand_x, buf.assist_info, buf.ep_recv_count, out)] + \
               ([buf.dynamic_scales.clone()] if buf.dynamic_scales is not None else [])

    step()
    want = snapshot()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()                                   # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(3):
        for t in (buf.expand_x, buf.assist_info, buf.ep_recv_count, out):
            t.zero_()                            # eager work between replays
        step() if rep == 1 else None             # and an eager step
        g.replay()
        got = snapshot()
        for a, b in zip(got, want):
            assert torch.equal(a.view(torch.uint8) if a.dtype == torch.float8_e4m3fn else a,
                               b.view(torch.uint8) if b.dtype == torch.float8_e4m3fn else b), rep
