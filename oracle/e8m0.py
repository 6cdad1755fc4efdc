"""Block quantizer with power-of-two (E8M0) scales and its GEMM reference
(test oracle only).

The block layout is the DeepGEMM write-up's (section 2.2: one scale per 32x32
block; section 5.2: from the block's absolute maximum; section 2.1: E4M3
tops out at 448).  Here the scale is restricted to a power of two 2**E, kept
as one E8M0 byte (E + 127), the form a hardware-scaled MFMA can apply.  The
pages describe no such variant; the readings taken:

* E is the smallest integer with 448 * 2**E >= amax, so that no value of the
  block exceeds the E4M3 range (none saturates); E is clamped to
  [-127, 127] (the E8M0 byte range without its NaN code 0xFF);
* each code is E4M3(x * 2**-E): the scaling by a power of two is exact, then
  one round half to even; the sign is kept (-0 gives 0x80);
* an all-zero block gets E = -127 (byte 0x00) and codes of its zeros.

GEMM: C[i, j] = sum_k dec(A[i, k]) 2**Ea[i//32, k//32] * dec(Bt[j, k]) 2**Eb[j//32, k//32],
the plain definition, with the weight K-major (Bt [N, K]).
"""

from __future__ import annotations

import numpy as np

from .minifloat import E4M3FN
from .e4m3 import decode_e4m3

BLOCK = 32
E_MIN, E_MAX = -127, 127


def _bf16_to_f64(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def e8m0_exponent(amax):
    """Smallest integer E with 448 * 2**E >= amax (exact test), clamped to
    [E_MIN, E_MAX]; E_MIN for amax == 0.  amax: fp64 array of bf16 values."""
    amax = np.asarray(amax, dtype=np.float64)
    nz = amax > 0
    E = np.zeros(amax.shape, dtype=np.int64)
    guess = np.ceil(np.log2(np.where(nz, amax, 1.0) / 448.0)).astype(np.int64)
    # the fp64 logarithm can be off by one near a power of two: settle it with
    # the exact comparison (448 * 2**E is exact in fp64)
    for _ in range(2):
        guess = np.where(np.ldexp(448.0, guess - 1) >= amax, guess - 1, guess)
        guess = np.where(np.ldexp(448.0, guess) < amax, guess + 1, guess)
    E[nz] = guess[nz]
    E[~nz] = E_MIN
    return np.clip(E, E_MIN, E_MAX)


def quantize_blocks_e8m0(x_bits):
    """bf16 bits [R, C] (C % 32 == 0) -> (codes uint8 [R, C], E8M0 bytes uint8 [ceil(R/32), C/32])."""
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    if x_bits.ndim != 2 or x_bits.shape[1] % BLOCK:
        raise ValueError("quantize_blocks_e8m0 takes [R, C] with C a multiple of 32")
    R, C = x_bits.shape
    x = _bf16_to_f64(x_bits)
    nrb, ncb = -(-R // BLOCK), C // BLOCK
    q = np.zeros((R, C), np.uint8)
    e = np.zeros((nrb, ncb), np.uint8)
    for rb in range(nrb):
        r0, r1 = rb * BLOCK, min(rb * BLOCK + BLOCK, R)
        xb = x[r0:r1].reshape(r1 - r0, ncb, BLOCK)
        E = e8m0_exponent(np.abs(xb).max(axis=(0, 2)))                  # [ncb]
        t = np.ldexp(xb, -E[None, :, None])                                # exact
        q[r0:r1] = E4M3FN.encode(t, overflow="saturate").astype(np.uint8).reshape(r1 - r0, C)
        e[rb] = (E + 127).astype(np.uint8)
    return q, e


def dequantize_e8m0(q, e):
    """dec(q) * 2**(e - 127) with each 32x32 block's exponent, exact in fp64."""
    q = np.asarray(q, dtype=np.uint8)
    R, C = q.shape
    E = np.asarray(e, dtype=np.int64) - 127
    if E.shape != (-(-R // BLOCK), C // BLOCK):
        raise ValueError(f"exponent grid {E.shape} does not match operand {q.shape}")
    Ef = np.repeat(np.repeat(E, BLOCK, axis=0)[:R], BLOCK, axis=1)
    return np.ldexp(decode_e4m3(q), Ef)


def gemm_ref_e8m0_nt(qa, ea, qbt, ebt):
    """A [M, K] with E8M0 grid [ceil(M/32), K/32]; Bt [N, K] with [N/32, K/32].
    Returns (ref, absref): the fp64 product and sum_k |a' b'|."""
    a = dequantize_e8m0(qa, ea)
    bt = dequantize_e8m0(qbt, ebt)
    return a @ bt.T, np.abs(a) @ np.abs(bt).T
