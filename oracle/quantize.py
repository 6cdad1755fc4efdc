"""bf16 -> E4M3 block quantizer (test oracle only).

DeepGEMM write-up:
* section 2.2 - the matrix is cut into 32x32 blocks and each block gets its own
  scale;
* section 5.2 - the scale comes from the block's absolute maximum;
* section 2.1 - E4M3's largest finite value is 448.

Reading adopted for the steps the pages leave open (all recorded in the design
notes): the scale is the fp32 quotient amax / 448 (IEEE round to nearest
even); each element is divided by that scale in fp32, and the fp32 quotient is
rounded to E4M3 (round half to even, saturating at +-448, sign kept); a block
whose amax is 0 gets scale 0 and all-zero (0x00) codes.  A final row-block
shorter than 32 rows covers only the rows that exist; the column count must be
a multiple of 32.

Input is the bf16 bit pattern (uint16); bf16 -> fp32 is exact (shift left 16).
"""

from __future__ import annotations

import numpy as np

from .e4m3 import encode_e4m3

BLOCK = 32
E4M3_MAX = np.float32(448.0)


def bf16_bits_to_f32(bits) -> np.ndarray:
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32)


def quantize_blocks(x_bits):
    """x_bits: uint16 bf16 patterns [R, C] with C % 32 == 0.

    Returns (q uint8 [R, C], s float32 [ceil(R/32), C/32]).
    """
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    if x_bits.ndim != 2:
        raise ValueError("quantize_blocks takes a 2-D matrix")
    R, C = x_bits.shape
    if C % BLOCK:
        raise ValueError("column count must be a multiple of 32")
    x = bf16_bits_to_f32(x_bits)
    nrb, ncb = -(-R // BLOCK), C // BLOCK
    q = np.zeros((R, C), dtype=np.uint8)
    s = np.zeros((nrb, ncb), dtype=np.float32)
    for rb in range(nrb):
        r0, r1 = rb * BLOCK, min(R, rb * BLOCK + BLOCK)
        # [rows, ncb, 32]: one slice per 32-column block of this row-block
        xb = x[r0:r1].reshape(r1 - r0, ncb, BLOCK)
        amax = np.abs(xb).max(axis=(0, 2)).astype(np.float32)        # [ncb]
        sc = (amax / E4M3_MAX).astype(np.float32)                      # fp32 divide
        s[rb] = sc
        nz = sc != 0
        t = np.zeros_like(xb)
        # fp32 quotient element by element; zero blocks never divide
        t[:, nz, :] = (xb[:, nz, :] / sc[nz][None, :, None]).astype(np.float32)
        qb = encode_e4m3(t)
        qb[:, ~nz, :] = 0x00
        q[r0:r1] = qb.reshape(r1 - r0, C)
    return q, s


def quantize_token_groups(x_bits):
    """Per-token groups of 1 row x 32 columns (test oracle only).

    The activation-side granularity that the determinism article's RMSNorm
    part (三, section 2, the vLLM table) lists for a norm fused with FP8
    quantization: one scale per token (row) and group of columns.  The group
    width is 32 here, matching the 32-deep K-blocks of the weight's 32x32
    scales.  Per group, the element rule of the block quantizer (DeepGEMM
    write-up, sections 2.1 and 5.2): amax = max |x| over the group's 32
    values, s = fp32(amax / 448), each code = E4M3(fp32(x / s)) (round half to
    even, saturating at +-448, sign kept), an all-zero group gets s = 0 and
    0x00 codes.

    x_bits: uint16 bf16 patterns [R, C], C % 32 == 0.
    Returns (q uint8 [R, C], s float32 [R, C/32]).
    """
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    if x_bits.ndim != 2:
        raise ValueError("quantize_token_groups takes a 2-D matrix")
    R, C = x_bits.shape
    if C % BLOCK:
        raise ValueError("column count must be a multiple of 32")
    ncb = C // BLOCK
    xg = bf16_bits_to_f32(x_bits).reshape(R, ncb, BLOCK)
    amax = np.abs(xg).max(axis=2).astype(np.float32)                   # [R, ncb]
    sc = (amax / E4M3_MAX).astype(np.float32)
    nz = sc != 0
    t = np.zeros_like(xg)
    t[nz] = (xg[nz] / sc[nz][:, None]).astype(np.float32)
    q = encode_e4m3(t)
    q[~nz] = 0x00
    return q.reshape(R, C), sc
