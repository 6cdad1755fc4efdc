"""Exact rational GEMM for tiny shapes (test oracle only; checks ``gemm_ref``).

Every E4M3 value is an integer multiple of 2**-9 (DeepGEMM write-up, section
2.1 fixes the 4/3 bit split; the smallest step is the subnormal 2**-9), so
ai = dec(a) * 2**9 and bi = dec(b) * 2**9 are integers and each 32-deep block
sum P_kb = sum_k ai * bi is an exact integer.  With fp32 scales taken as exact
fractions,

    C_ij = sum_kb  sa[i//32, kb] * sb[kb, j//32] * P_kb / 2**18

is the exact value of the block-scaled product (no rounding anywhere).  Pure
Python integers and ``fractions.Fraction``: only for M, N, K of a few dozen.
"""

from __future__ import annotations

from fractions import Fraction

import numpy as np

BLOCK = 32


def _int_units(code: int) -> int:
    """dec(code) * 2**9 from the E4M3 bit fields, as a Python int."""
    code = int(code)
    if (code & 0x7F) == 0x7F:
        raise ValueError("NaN code")
    sign = -1 if code & 0x80 else 1
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0:
        mag = m                      # (m/8) * 2**-6 * 2**9
    else:
        mag = (8 + m) << (e - 1)     # (1 + m/8) * 2**(e-7) * 2**9
    return sign * mag


def gemm_exact(qa, sa, qb, sb):
    """Exact C as an object array of Fractions, shape [M, N]."""
    qa = np.asarray(qa)
    qb = np.asarray(qb)
    M, K = qa.shape
    K2, N = qb.shape
    if K != K2 or K % BLOCK or N % BLOCK:
        raise ValueError("shape mismatch or K, N not multiples of 32")
    ai = [[_int_units(qa[i, k]) for k in range(K)] for i in range(M)]
    bi = [[_int_units(qb[k, j]) for j in range(N)] for k in range(K)]
    sa_f = [[Fraction(float(v)) for v in row] for row in np.asarray(sa, dtype=np.float32)]
    sb_f = [[Fraction(float(v)) for v in row] for row in np.asarray(sb, dtype=np.float32)]
    out = np.empty((M, N), dtype=object)
    for i in range(M):
        for j in range(N):
            total = Fraction(0)
            for kb in range(K // BLOCK):
                p = 0
                for k in range(kb * BLOCK, kb * BLOCK + BLOCK):
                    p += ai[i][k] * bi[k][j]
                total += sa_f[i // BLOCK][kb] * sb_f[kb][j // BLOCK] * p
            out[i, j] = total / (1 << 18)
    return out
