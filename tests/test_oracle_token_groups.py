"""Pins for the oracle's per-token-group quantizer and GEMM references (CPU only)."""

import os

import numpy as np
import pytest

from oracle import (FINITE_E4M3_CODES, gemm_exact, gemm_ref_tg, gemm_ref_tg_nt, quantize_blocks,
                    quantize_token_groups)
from fp8_block_scaled_03_amd.workloads import normal_bf16

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_hand_derived_group_ignores_other_rows():
    """Golden codes for a group with amax 7 (scale 2**-6), taken from the
    hand-derived block file: a row holding the pairs and its maximum 7.0 gets
    exactly those codes although another row of the same 32-column block holds
    a much larger value (which would change a 32x32 block's scale)."""
    lines = [ln.split("#")[0].split() for ln in open(os.path.join(GOLDEN, "quantize_hand_examples.txt"))]
    lines = [ln for ln in lines if ln]
    scale_bits = int(lines[0][1], 16)
    pairs = [(int(a, 16), int(b, 16)) for a, b in lines[1:]]
    assert len(pairs) <= 31
    x = np.full((3, 64), 0x3F80, dtype=np.uint16)
    x[1, 0] = 0x40E0                          # row 1, group 0: maximum 7.0
    for i, (xb, _) in enumerate(pairs):
        x[1, 1 + i] = xb
    x[2, 5] = 0x4380                          # 256.0 in another row of the same block
    q, s = quantize_token_groups(x)
    assert s.shape == (3, 2)
    assert s.view(np.uint32)[1, 0] == scale_bits
    for i, (_, code) in enumerate(pairs):
        assert q[1, 1 + i] == code, (hex(pairs[i][0]), hex(q[1, 1 + i]))
    assert s[2, 0] == np.float32(256.0) / np.float32(448.0)
    qb, sb = quantize_blocks(x)
    assert sb[0, 0] != s[1, 0]                # the block scale does see row 2


def test_token_groups_are_one_row_blocks():
    """A one-row matrix is quantized by quantize_blocks with 1 x 32 blocks, so
    per-token groups are quantize_blocks applied row by row."""
    x = normal_bf16(77, 0, 40, 96, 1.0, 0.01)
    x[3, 0:32] = 0                            # a zero group
    x[7, 40] = 0x8000                         # -0
    q, s = quantize_token_groups(x)
    for r in range(x.shape[0]):
        qr, sr = quantize_blocks(x[r:r + 1])
        assert np.array_equal(q[r], qr[0]) and np.array_equal(s[r].view(np.uint32), sr[0].view(np.uint32)), r


def _rand_codes(g, shape):
    return FINITE_E4M3_CODES[g.integers(0, len(FINITE_E4M3_CODES), shape)]


def _rand_scales(g, shape):
    return (g.uniform(1.0, 2.0, shape) * np.exp2(g.integers(-12, 6, shape))).astype(np.float32)


@pytest.mark.parametrize("M,N,K", [(3, 32, 64), (5, 64, 32)])
def test_token_group_gemm_matches_exact_rational_per_row(M, N, K):
    """Each row of gemm_ref_tg against the exact rational product of that row
    alone (a one-row A has one scale row: its token-group scales)."""
    g = np.random.default_rng(M + N + K)
    qa, qb = _rand_codes(g, (M, K)), _rand_codes(g, (K, N))
    sa, sb = _rand_scales(g, (M, K // 32)), _rand_scales(g, (K // 32, N // 32))
    ref, absref = gemm_ref_tg(qa, sa, qb, sb)
    ref_nt, _ = gemm_ref_tg_nt(qa, sa, np.ascontiguousarray(qb.T), np.ascontiguousarray(sb.T))
    u = 2.0 ** -53
    gam = (K + 2) * u / (1 - (K + 2) * u)
    for i in range(M):
        ex = np.vectorize(float)(gemm_exact(qa[i:i + 1], sa[i:i + 1], qb, sb))[0]
        assert np.all(np.abs(ref[i] - ex) <= gam * absref[i] + 1e-300), i
        assert np.all(np.abs(ref_nt[i] - ex) <= gam * absref[i] + 1e-300), i


def test_token_group_gemm_with_block_scales_repeated_is_block_gemm():
    """Token-group scales that repeat a 32x32 grid's scale on each of its rows
    describe the same dequantized A, so the two references agree exactly."""
    from oracle import gemm_ref
    g = np.random.default_rng(9)
    M, N, K = 70, 64, 96
    qa, qb = _rand_codes(g, (M, K)), _rand_codes(g, (K, N))
    sa, sb = _rand_scales(g, (3, K // 32)), _rand_scales(g, (K // 32, N // 32))
    sa_rows = np.repeat(sa, 32, axis=0)[:M]
    ref_tg, abs_tg = gemm_ref_tg(qa, sa_rows, qb, sb)
    ref, absref = gemm_ref(qa, sa, qb, sb)
    assert np.array_equal(ref_tg, ref) and np.array_equal(abs_tg, absref)
