"""Quantizer parity: the GPU kernel is bit-exact against the oracle."""

import os

import numpy as np
import pytest

import oracle
from fp8_block_scaled_03_amd import workloads as W

from gpu_util import gpu_quantize, say

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _check(x_bits, label):
    say(f"quantize {label} shape={x_bits.shape}")
    q, s = gpu_quantize(x_bits)
    qo, so = oracle.quantize_blocks(x_bits)
    assert np.array_equal(s.view(np.uint32), so.view(np.uint32)), f"{label}: scales differ"
    bad = np.argwhere(q != qo)
    assert len(bad) == 0, f"{label}: {len(bad)} codes differ, first at {bad[:5].tolist()}"


@pytest.mark.parametrize("rows,cols", [(256, 256), (1, 32), (33, 64), (100, 96), (64, 8192)])
def test_random_normal(rows, cols):
    _check(W.normal_bf16(1000, 0, rows, cols), "normal")


def test_square_256_operands():
    wl = W.square_256()
    _check(wl.a_bits(), "square-256 A")
    _check(wl.b_bits(), "square-256 B")


def test_scale_one_exhaustive():
    bits = np.arange(0, 1 << 16, dtype=np.uint32)
    x = (bits << 16).view(np.float32)
    xb = bits[np.isfinite(x) & (np.abs(x) <= 448)].astype(np.uint16)
    per = 1023
    nblk = -(-len(xb) // per)
    pad = np.zeros(nblk * per, np.uint16)
    pad[:len(xb)] = xb
    blocks = np.concatenate([np.full((nblk, 1), 0x43E0, np.uint16), pad.reshape(nblk, per)], axis=1)
    _check(blocks.reshape(nblk, 32, 32).transpose(1, 0, 2).reshape(32, nblk * 32), "scale-1 sweep")


def test_many_scales_all_bf16():
    """Every finite bf16 value quantized under 64 different non-power-of-two
    block maxima: exercises the fp32 division and the E4M3 rounding at every
    midpoint neighbourhood."""
    g = np.random.default_rng(5)
    bits = np.arange(0, 1 << 16, dtype=np.uint32)
    x = (bits << 16).view(np.float32)
    allb = bits[np.isfinite(x)].astype(np.uint16)
    amax_list = (g.uniform(1, 2, 64) * np.exp2(g.integers(-100, 100, 64))).astype(np.float32)
    for amax in amax_list[:64]:
        ab = np.uint16(np.float32(amax).view(np.uint32) >> 16)
        af = np.array([np.uint32(ab) << np.uint32(16)], dtype=np.uint32).view(np.float32)[0]
        xf = (allb.astype(np.uint32) << 16).view(np.float32)
        keep = allb[np.abs(xf) <= af]
        per = 1023
        nblk = -(-len(keep) // per)
        pad = np.zeros(nblk * per, np.uint16)
        pad[:len(keep)] = keep
        blocks = np.concatenate([np.full((nblk, 1), ab, np.uint16), pad.reshape(nblk, per)], axis=1)
        _check(blocks.reshape(nblk, 32, 32).transpose(1, 0, 2).reshape(32, nblk * 32), f"amax={float(af):.3e}")


def _all_bf16_under(ab):
    """Blocks holding every finite bf16 value |x| <= amax (bits ab), each block
    led by the amax element itself."""
    bits = np.arange(0, 1 << 16, dtype=np.uint32)
    xf = (bits << 16).view(np.float32)
    allb = bits[np.isfinite(xf)].astype(np.uint16)
    af = np.array([np.uint32(ab) << np.uint32(16)], dtype=np.uint32).view(np.float32)[0]
    keep = allb[np.abs((allb.astype(np.uint32) << 16).view(np.float32)) <= af]
    per = 1023
    nblk = -(-len(keep) // per)
    pad = np.zeros(nblk * per, np.uint16)
    pad[:len(keep)] = keep
    blocks = np.concatenate([np.full((nblk, 1), ab, np.uint16), pad.reshape(nblk, per)], axis=1)
    return blocks.reshape(nblk, 32, 32).transpose(1, 0, 2).reshape(32, nblk * 32)


@pytest.mark.parametrize("amax_bits", [
    0x2200, 0x21FF, 0x2180, 0x2100, 0x20FF,     # around 2^-60, where the quotient method switches
    0x0001, 0x0040, 0x0080, 0x00FF, 0x1000,     # subnormal and tiny block maxima
    0x43E0, 0x3F80, 0x4060, 0x7F60, 0x7F7F,     # 448, 1, 3.5, 448 * 2^120, the largest bf16
    0x3DE0, 0x48E0, 0x3F81, 0x3FFF, 0x4001,     # 448 * 2^-k, 448 * 2^k, near-power-of-two maxima
])
def test_targeted_scales_all_bf16(amax_bits):
    """Every finite bf16 value under block maxima chosen at the edges of the
    quotient computation: exact powers of two times 448 (s a power of two),
    maxima around the switch to direct division, subnormal and huge maxima."""
    _check(_all_bf16_under(np.uint16(amax_bits)), f"amax bits {amax_bits:#06x}")


def test_golden_examples_on_gpu():
    x = np.full((32, 32), 0x3F80, dtype=np.uint16)
    x[0, 0] = 0x3FA3
    x[7, 9] = 0x37A3
    say("quantize golden divide example")
    q, s = gpu_quantize(x)
    assert s.view(np.uint32)[0, 0] == 0x3B3A4925 and q[7, 9] == 0x03


def test_edge_values():
    x = W.normal_bf16(1000, 5, 64, 128)
    x[:, 0:32] = 0                      # zero block
    x[3, 5] = 0x8000                    # -0 in the zero block
    x[40, 40] = 0x8000                  # -0 in a live block
    x[32:64, 96:128] = W.f32_to_bf16_bits(np.float32(1e-39) * np.ones((32, 32), np.float32))  # tiny block
    x[0:32, 64:96] = W.f32_to_bf16_bits(np.float32(3e38) * np.ones((32, 32), np.float32))     # huge block
    x[5, 70] = W.f32_to_bf16_bits(np.float32([-1.0]))[0]
    _check(x, "edge values")
