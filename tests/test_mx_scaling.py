"""The MX quantiser (quantMode 4) takes its E8M0 byte from the block max's
binary32 exponent field (minus 8, at least 0) and scales each element by a
binary32 multiply with 2^(127 - byte) before the E4M3 conversion. Here that
arithmetic, emulated in numpy's IEEE binary32 (subnormals kept, as the kernels
run), is compared with the oracle's definition (frexp exponent, clamp at -127,
exact scaling) for every finite 16-bit block max of fp16 and bf16, with 31
further elements per block drawn at or below the max (subnormals included). The
E4M3 conversion of the emulation is torch's float8_e4m3fn cast, which the
oracle pins match the brute-force nearest-value search for |v| <= 448."""
import numpy as np
import pytest

import oracle
import workloads as wl


def _blocks(fmt, rng):
    """[M, 32] float32 blocks whose element 0 is each finite non-negative 16-bit value in turn and whose other
    elements lie at or below it in magnitude, with random signs; and their 16-bit encodings."""
    if fmt == "fp16":
        m = np.arange(0, 0x7C00, dtype=np.uint16).view(np.float16).astype(np.float32)
    else:
        m = (np.arange(0, 0x7F80, dtype=np.uint32) << 16).view(np.float32)
    u = rng.random((m.size, 31)).astype(np.float32)
    u[:, :4] = rng.random((m.size, 4)).astype(np.float32) * np.float32(2.0 ** -20)   # far below the max
    u[:, 4] = 1.0                                                                   # the max again
    x = np.concatenate([m[:, None], m[:, None] * u], axis=1)
    x *= np.where(rng.random(x.shape) < 0.5, -1.0, 1.0).astype(np.float32)
    x[:, 0] = np.abs(x[:, 0])
    if fmt == "fp16":
        bits = x.astype(np.float16)
        xf = bits.astype(np.float32)
    else:
        bits = wl.f32_to_bf16_bits(x)
        xf = (bits.astype(np.uint32) << 16).view(np.float32)
    assert (np.abs(xf) <= xf[:, :1]).all()
    return bits, xf


def _kernel_arithmetic(xf):
    import torch

    amax = np.abs(xf).max(axis=1)
    byte = np.maximum((amax.view(np.uint32) >> 23).astype(np.int64) - 8, 0)
    mult = ((254 - byte).astype(np.uint32) << 23).view(np.float32)
    q = np.minimum(np.abs(xf) * mult[:, None], np.float32(448.0))                  # binary32 multiply
    q = np.where(np.signbit(xf), -q, q).astype(np.float32)
    codes = torch.from_numpy(q).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return byte.astype(np.uint8), codes


@pytest.mark.parametrize("fmt", ["fp16", "bf16"])
def test_kernel_scaling_matches_the_definition_for_every_16bit_block_max(fmt):
    bits, xf = _blocks(fmt, np.random.default_rng(77 if fmt == "fp16" else 78))
    n = bits.shape[0]
    d = oracle.dispatch(bits, np.zeros((n, 1), np.int32), 1, 1, quant_mode=4, bf16=fmt == "bf16")
    assert (d["assist_info"][:, 1] == np.arange(n)).all()          # one expert: row t is token t
    byte, codes = _kernel_arithmetic(xf)
    assert (d["dynamic_scales"][:, 0] == byte).all()
    assert (d["expand_x"] == codes).all()
    # the range the blocks cover: bytes from 0 (subnormal and tiny maxima) to the format's top
    assert byte.min() == 0 and byte.max() == (134 if fmt == "fp16" else 246)
