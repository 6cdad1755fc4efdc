"""Residual add + RMSNorm reference in fp64 (test oracle only).

What is computed (Determinism article, part 三, section 1): every token (row) of
an activation matrix [num_tokens, hidden] is normalised by the root mean square
of its own hidden vector and scaled element-wise by a learned weight gamma,

    y = x / RMS(x) * gamma,      RMS(x) = sqrt( (1/d) * sum_i x_i**2 + eps ).

Section 2 of that part lists the serving variants: with a residual stream the
input is first added to it (the "fused add" form), and for FP8 with block
scales the per-token-group quantizer runs in the same kernel.

Readings taken here where the pages leave a step open:

* residual: h = bf16(x + r), the exact sum of the two bf16 inputs rounded
  once to bf16 (nearest, ties to even).  h is the updated residual stream
  (stored as bf16) and the norm's input.  The fp64 sum of two bf16 values is
  exact unless their exponents differ by more than 45; then the smaller one is
  far below half a bf16 ulp of the larger, and the exact sum and the fp64 sum
  both round to the larger, so fp64 addition followed by one bf16 rounding is
  the definition.
* the normalised value is delivered as bf16 (nearest, ties to even), which is
  what the quantizer reads; the fused quantization is ``quantize_token_groups``
  of those bf16 values.  The oracle gives y in fp64; a computed bf16 y is
  accepted when |y - ref| <= RMS_REL_TOL * |ref| + RMS_ABS_TOL (the bf16
  rounding, 2**-8 relative, plus 2**-15 for fp32 arithmetic before it: a sum
  of at most 256 squares per lane and six pairwise levels, a divide, a square
  root, a reciprocal and two products, each within 2**-24 relative).
"""

from __future__ import annotations

import numpy as np

from .minifloat import BF16

RMS_REL_TOL = 2.0 ** -8 + 2.0 ** -15
RMS_ABS_TOL = 2.0 ** -133  # half the smallest bf16 subnormal


def _bf16_to_f64(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def residual_add(x_bits, r_bits):
    """h = bf16(x + r) for bf16 bit patterns of equal shape; returns bf16 bits."""
    s = _bf16_to_f64(x_bits) + _bf16_to_f64(r_bits)
    return BF16.encode(s, overflow="inf").astype(np.uint16)


def rmsnorm_ref(h_bits, gamma_bits, eps):
    """y[i, :] = h[i, :] * gamma / sqrt(mean(h[i, :]**2) + eps), fp64 [R, d].

    h_bits [R, d] and gamma_bits [d] are bf16 bit patterns; eps is an fp32
    value (taken exactly)."""
    h = _bf16_to_f64(h_bits)
    g = _bf16_to_f64(gamma_bits)
    if h.ndim != 2 or g.shape != (h.shape[1],):
        raise ValueError(f"shapes {h.shape} and {g.shape} do not match")
    ms = np.mean(h * h, axis=1) + float(np.float32(eps))
    return h * g[None, :] / np.sqrt(ms)[:, None]


def rmsnorm_tolerance_ok(y_bits, y_ref):
    """Element-wise acceptance of a computed bf16 y against the fp64 reference."""
    y = _bf16_to_f64(y_bits)
    return np.abs(y - y_ref) <= RMS_REL_TOL * np.abs(y_ref) + RMS_ABS_TOL
