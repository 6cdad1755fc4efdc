"""Block-scaled GEMM reference in fp64 (test oracle only).

What the method computes (DeepGEMM write-up, sections 2.2-2.3): with one scale
per 32x32 block of each operand, the product is the plain matrix product of the
dequantized operands,

    C[i, j] = sum_k  dec(A[i, k]) * sa[i // 32, k // 32] * dec(B[k, j]) * sb[k // 32, j // 32]

(section 2.2 has the scales enter during accumulation rather than in a
separate dequantize pass over C; that says where a kernel applies them, not
that the result differs).  The Determinism article (part 一, section 1) states the
plain definition C_ij = sum_k A_ik B_kj.  This module is that definition
written out: dequantize both operands in fp64 (exact: a 4-bit significand times
a 24-bit one) and call one fp64 matmul.  It also returns the magnitude sum
sum_k |a' * b'| used by the acceptance bound.

Grouped variant (DeepGEMM write-up, sections 4.1-4.2): consecutive row ranges
[off[g], off[g+1]) of A are multiplied by their own B_g / sb_g; empty ranges
produce nothing.

K-major weights (section 6 passes the weight as [N, K] with scales
[N/32, K/32]): ``gemm_ref_nt`` / ``grouped_gemm_ref_nt`` take B transposed;
the product is the same definition with B[k, j] = Bt[j, k].

Per-token-group activation scales (``gemm_ref_tg``, ``gemm_ref_tg_nt``): A's
scale grid is [M, K/32], one scale per row and 32 columns; the product is the
same definition with sa[i // 32, k // 32] replaced by sa_rows[i, k // 32].

Acceptance bound per element (the tolerance the GPU result is held to):
    |C - ref| <= 2**-8 * |ref| + 1e-6 * sum_k |a' b'|
"""

from __future__ import annotations

import numpy as np

from .e4m3 import decode_e4m3

BLOCK = 32
REL_TOL = 2.0 ** -8
ABS_SUM_TOL = 1e-6


def _expand_rows(s, n_rows):
    """scale grid [ceil(R/32), X] -> per-row [R, X] (row r uses scale row r // 32)."""
    return np.repeat(np.asarray(s, dtype=np.float64), BLOCK, axis=0)[:n_rows]


def dequantize(q, s):
    """A' = dec(q) * expand32(s) in fp64.

    For A [M, K] with sa [ceil(M/32), K/32] and for B [K, N] with sb [K/32, N/32]
    the expansion is the same: entry (r, c) uses s[r // 32, c // 32].
    """
    q = np.asarray(q, dtype=np.uint8)
    v = decode_e4m3(q)
    R, C = q.shape
    s = np.asarray(s, dtype=np.float64)
    if s.shape != (-(-R // BLOCK), C // BLOCK):
        raise ValueError(f"scale grid {s.shape} does not match operand {q.shape}")
    full = np.repeat(_expand_rows(s, R), BLOCK, axis=1)[:, :C]
    return v * full


def gemm_ref(qa, sa, qb, sb):
    """Full reference: returns (ref, absref), both fp64 [M, N]."""
    a = dequantize(qa, sa)
    b = dequantize(qb, sb)
    return a @ b, np.abs(a) @ np.abs(b)


def gemm_ref_at(qa, sa, qb, sb, rows, cols):
    """Reference for the sub-matrix rows x cols only (for full-size checks)."""
    rows = np.asarray(rows)
    cols = np.asarray(cols)
    qa = np.asarray(qa)
    qb = np.asarray(qb)
    a = decode_e4m3(qa[rows]) * np.repeat(np.asarray(sa, np.float64)[rows // BLOCK], BLOCK, axis=1)
    b = decode_e4m3(qb[:, cols]) * np.repeat(np.asarray(sb, np.float64)[:, cols // BLOCK], BLOCK, axis=0)
    return a @ b, np.abs(a) @ np.abs(b)


def gemm_ref_nt(qa, sa, qbt, sbt):
    """K-major weights: qbt [N, K] with scales sbt [N/32, K/32] (the weight
    layout of the DeepGEMM write-up's call interface, section 6).

        C[i, j] = sum_k dec(A[i, k]) sa[i//32, k//32] * dec(Bt[j, k]) sbt[j//32, k//32]

    Both operands are dequantized with their own grids (entry (r, c) uses
    [r // 32, c // 32]) and contracted over K.  Returns (ref, absref)."""
    a = dequantize(qa, sa)
    bt = dequantize(qbt, sbt)
    return a @ bt.T, np.abs(a) @ np.abs(bt).T


def dequantize_token_groups(q, s):
    """A' = dec(q) * s expanded along columns: entry (r, c) uses s[r, c // 32]
    (per-token groups of 1 x 32; s is [R, C/32])."""
    q = np.asarray(q, dtype=np.uint8)
    R, C = q.shape
    s = np.asarray(s, dtype=np.float64)
    if s.shape != (R, C // BLOCK):
        raise ValueError(f"token-group scales {s.shape} do not match operand {q.shape}")
    return decode_e4m3(q) * np.repeat(s, BLOCK, axis=1)


def gemm_ref_tg(qa, sa_rows, qb, sb):
    """Activations with per-token-group scales sa_rows [M, K/32], weight
    B [K, N] with 32x32 block scales sb [K/32, N/32]:

        C[i, j] = sum_k dec(A[i, k]) sa_rows[i, k//32] * dec(B[k, j]) sb[k//32, j//32]

    Returns (ref, absref)."""
    a = dequantize_token_groups(qa, sa_rows)
    b = dequantize(qb, sb)
    return a @ b, np.abs(a) @ np.abs(b)


def gemm_ref_tg_nt(qa, sa_rows, qbt, sbt):
    """As ``gemm_ref_tg`` with the weight K-major: qbt [N, K], sbt [N/32, K/32]."""
    a = dequantize_token_groups(qa, sa_rows)
    bt = dequantize(qbt, sbt)
    return a @ bt.T, np.abs(a) @ np.abs(bt).T


def _check_offsets(offsets, M_total):
    off = np.asarray(offsets, dtype=np.int64)
    if off[0] != 0 or off[-1] != M_total or np.any(np.diff(off) < 0) or np.any(off % BLOCK):
        raise ValueError("offsets must start at 0, end at M_total, be non-decreasing multiples of 32")
    return off


def grouped_gemm_ref(qa, sa, qb, sb, offsets):
    """qb [G, K, N], sb [G, K/32, N/32]; rows off[g]..off[g+1] use group g."""
    qa = np.asarray(qa)
    off = _check_offsets(offsets, qa.shape[0])
    M, N = qa.shape[0], qb.shape[2]
    ref = np.zeros((M, N))
    absref = np.zeros((M, N))
    for g in range(len(off) - 1):
        r0, r1 = off[g], off[g + 1]
        if r1 == r0:
            continue
        r, ar = gemm_ref(qa[r0:r1], np.asarray(sa)[r0 // BLOCK:r1 // BLOCK], qb[g], sb[g])
        ref[r0:r1] = r
        absref[r0:r1] = ar
    return ref, absref


def grouped_gemm_ref_nt(qa, sa, qbt, sbt, offsets):
    """qbt [G, N, K], sbt [G, N/32, K/32]; rows off[g]..off[g+1] use group g."""
    qa = np.asarray(qa)
    off = _check_offsets(offsets, qa.shape[0])
    M, N = qa.shape[0], qbt.shape[1]
    ref = np.zeros((M, N))
    absref = np.zeros((M, N))
    for g in range(len(off) - 1):
        r0, r1 = off[g], off[g + 1]
        if r1 == r0:
            continue
        r, ar = gemm_ref_nt(qa[r0:r1], np.asarray(sa)[r0 // BLOCK:r1 // BLOCK], qbt[g], sbt[g])
        ref[r0:r1] = r
        absref[r0:r1] = ar
    return ref, absref


def grouped_gemm_ref_at(qa, sa, qb, sb, offsets, rows, cols):
    """Grouped reference for selected rows (any order) x cols."""
    qa = np.asarray(qa)
    off = _check_offsets(offsets, qa.shape[0])
    rows = np.asarray(rows)
    grp = np.searchsorted(off, rows, side="right") - 1
    ref = np.zeros((len(rows), len(cols)))
    absref = np.zeros((len(rows), len(cols)))
    for g in np.unique(grp):
        sel = np.nonzero(grp == g)[0]
        r, ar = gemm_ref_at(qa, sa, qb[g], sb[g], rows[sel], cols)
        ref[sel] = r
        absref[sel] = ar
    return ref, absref


def tolerance_bound(ref, absref):
    return REL_TOL * np.abs(ref) + ABS_SUM_TOL * absref


def tolerance_ok(c, ref, absref):
    """Element-wise acceptance of a computed C (any float array) against ref."""
    c = np.asarray(c, dtype=np.float64)
    return np.abs(c - ref) <= tolerance_bound(ref, absref)


def bf16_bits_to_f64(bits):
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
