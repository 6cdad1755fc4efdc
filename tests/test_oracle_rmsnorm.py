"""Pins for the oracle's residual add and RMSNorm (CPU only).

The norm follows the Determinism article, part 三 section 1
(y = x / sqrt(mean(x**2) + eps) * gamma per token); the residual add is one
bf16 rounding of the exact sum (its section 2 lists the fused add form)."""

import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import residual_add, rmsnorm_ref, rmsnorm_tolerance_ok
from fp8_block_scaled_03_amd.workloads import normal_bf16

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _f32_bits_to_bf16(v):
    """fp32 values that are bf16 values -> their bf16 bits (truncation is exact here)."""
    return (np.asarray(v, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def test_residual_add_golden():
    rows = [ln.split("#")[0].split() for ln in open(os.path.join(GOLDEN, "residual_add_examples.txt"))]
    rows = [[int(t, 16) for t in r] for r in rows if r]
    assert len(rows) == 12
    x = np.array([r[0] for r in rows], np.uint16)
    r = np.array([r[1] for r in rows], np.uint16)
    want = np.array([r[2] for r in rows], np.uint16)
    assert np.array_equal(residual_add(x, r), want)


def _exact_bf16_round(v: Fraction) -> int:
    """Round an exact rational to bf16 (nearest, ties to even) with integers
    only; returns the bit pattern (finite results only)."""
    if v == 0:
        return 0
    sign = 0x8000 if v < 0 else 0
    a = abs(v)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    e = max(e, -126)                       # subnormal range shares the spacing of 2**-126
    scaled = a / Fraction(2) ** (e - 7)    # 8 significant bits
    n = scaled.numerator // scaled.denominator
    rem = scaled - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    if n == 256:                           # carried into the next binade
        n, e = 128, e + 1
    if n < 128:                            # subnormal
        return sign | n
    return sign | ((e + 127) << 7) | (n - 128)


def _bits_to_fraction(b: int) -> Fraction:
    return Fraction(float(np.array([b << 16], np.uint32).view(np.float32)[0]))


def test_residual_add_matches_exact_rational_rounding():
    g = np.random.default_rng(5)
    # wide exponent spread: sums that are exact, that round, and where one
    # operand vanishes below half an ulp of the other
    exps = g.integers(-40, 40, size=(2, 3000))
    mant = g.integers(0, 128, size=(2, 3000))
    signs = g.integers(0, 2, size=(2, 3000))
    bits = ((signs << 15) | ((exps + 127) << 7) | mant).astype(np.uint16)
    h = residual_add(bits[0], bits[1])
    for i in range(bits.shape[1]):
        want = _exact_bf16_round(_bits_to_fraction(int(bits[0, i])) + _bits_to_fraction(int(bits[1, i])))
        if want == 0 and (bits[0, i] & 0x8000) and (bits[1, i] & 0x8000):
            want = 0x8000
        assert int(h[i]) == want, (hex(bits[0, i]), hex(bits[1, i]), hex(h[i]), hex(want))


def test_rmsnorm_closed_forms():
    d = 64
    one = np.full(d, 0x3F80, np.uint16)
    # a constant row: the RMS is |c|, so y = sign(c) exactly (eps = 0)
    h = np.full((2, d), 0x4040, np.uint16)      # 3.0
    h[1] = 0xC0A0                               # -5.0
    y = rmsnorm_ref(h, one, 0.0)
    assert np.all(y[0] == 1.0) and np.all(y[1] == -1.0)
    # one non-zero entry v: RMS = |v| / sqrt(d), so y = sign(v) * sqrt(d) = 8
    h = np.zeros((1, d), np.uint16)
    h[0, 17] = 0xC0A0
    y = rmsnorm_ref(h, one, 0.0)
    assert y[0, 17] == -8.0 and np.count_nonzero(y) == 1
    # gamma scales element-wise
    gam = one.copy()
    gam[17] = 0x3E80                            # 0.25
    assert rmsnorm_ref(h, gam, 0.0)[0, 17] == -2.0
    # eps sits inside the square root: c = 1, eps = 3 -> 1 / sqrt(1 + 3) = 0.5
    h = np.full((1, d), 0x3F80, np.uint16)
    assert np.all(rmsnorm_ref(h, one, 3.0) == 0.5)
    # half threes and half fours: RMS = sqrt(12.5)
    h = np.array([[0x4040] * 32 + [0x4080] * 32], np.uint16)
    y = rmsnorm_ref(h, one, 0.0)
    assert abs(y[0, 0] - 3 / math.sqrt(12.5)) <= 2e-16 and abs(y[0, 40] - 4 / math.sqrt(12.5)) <= 2e-16
    # an all-zero row with eps > 0 gives zeros
    assert np.all(rmsnorm_ref(np.zeros((1, d), np.uint16), one, 1e-6) == 0.0)


@pytest.mark.parametrize("p", [-20, -3, 5, 30])
def test_rmsnorm_power_of_two_invariance(p):
    """With eps = 0, scaling a row by 2**p leaves y unchanged bitwise."""
    x = normal_bf16(3, 0, 4, 96)
    xs = _f32_bits_to_bf16((x.astype(np.uint32) << 16).view(np.float32) * np.float32(2.0 ** p))
    gam = normal_bf16(3, 1, 1, 96)[0]
    assert np.array_equal(rmsnorm_ref(x, gam, 0.0), rmsnorm_ref(xs, gam, 0.0))


def test_rmsnorm_matches_torch_rms_norm_fp64():
    """torch.nn.functional.rms_norm computes the same definition; in fp64 on
    the CPU it agrees to rounding level."""
    x = normal_bf16(4, 0, 16, 7168, 1.0, 0.01)
    gam = normal_bf16(4, 1, 1, 7168, 0.5)[0]
    for eps in (1e-6, 1e-2):
        y = rmsnorm_ref(x, gam, eps)
        xt = torch.from_numpy((x.astype(np.uint32) << 16).view(np.float32).astype(np.float64))
        gt = torch.from_numpy((gam.astype(np.uint32) << 16).view(np.float32).astype(np.float64))
        yt = torch.nn.functional.rms_norm(xt, (7168,), gt, float(np.float32(eps))).numpy()
        assert np.all(np.abs(y - yt) <= 1e-13 * np.abs(yt) + 1e-300)


def test_rmsnorm_tolerance_accepts_rounding_and_rejects_one_ulp_more():
    """A correctly rounded bf16 y passes; moving one element by one bf16 ulp
    away from the reference fails."""
    x = normal_bf16(6, 0, 8, 128)
    gam = normal_bf16(6, 1, 1, 128)[0]
    y = rmsnorm_ref(x, gam, 1e-5)
    from oracle import BF16
    yb = BF16.encode(y, overflow="inf").astype(np.uint16)
    assert rmsnorm_tolerance_ok(yb, y).all()
    bad = yb.copy()
    i = np.unravel_index(np.argmax(np.abs(y)), y.shape)
    yv = abs(float(y[i]))
    cur = abs(float(np.array([int(yb[i]) << 16], np.uint32).view(np.float32)[0]))
    # sign-magnitude bits: +1 raises the magnitude, -1 lowers it
    bad[i] = np.uint16(int(yb[i]) + (1 if cur >= yv else -1))   # one ulp further from the reference
    assert not rmsnorm_tolerance_ok(bad, y)[i]
