"""Pins for the oracle's GEMM reference (CPU only)."""

import numpy as np
import pytest

from oracle import (FINITE_E4M3_CODES, decode_e4m3, gemm_exact, gemm_ref, gemm_ref_at, gemm_ref_nt,
                    grouped_gemm_ref, grouped_gemm_ref_at, grouped_gemm_ref_nt, quantize_blocks, tolerance_ok,
                    tolerance_bound)
from oracle.exact import _int_units


def _rand_codes(g, shape):
    return FINITE_E4M3_CODES[g.integers(0, len(FINITE_E4M3_CODES), shape)]


def _rand_scales(g, shape):
    # positive fp32 scales that are not powers of two, spread over many binades
    return (g.uniform(1.0, 2.0, shape) * np.exp2(g.integers(-12, 6, shape))).astype(np.float32)


@pytest.mark.parametrize("M,N,K", [(1, 32, 32), (8, 32, 64), (33, 64, 32), (40, 32, 96)])
def test_fp64_reference_matches_exact_rational(M, N, K):
    g = np.random.default_rng(M * 1000 + N + K)
    qa, qb = _rand_codes(g, (M, K)), _rand_codes(g, (K, N))
    sa, sb = _rand_scales(g, (-(-M // 32), K // 32)), _rand_scales(g, (K // 32, N // 32))
    ref, absref = gemm_ref(qa, sa, qb, sb)
    exact = gemm_exact(qa, sa, qb, sb)
    ex = np.vectorize(float)(exact)
    # fp64 matmul error bound: gamma_{K+2} * sum |a' b'|
    u = 2.0 ** -53
    gam = (K + 2) * u / (1 - (K + 2) * u)
    assert np.all(np.abs(ref - ex) <= gam * absref + 1e-300)


def test_exact_units_closed_form():
    assert _int_units(0x38) == 512          # 1.0 * 2**9
    assert _int_units(0x7E) == 448 * 512
    assert _int_units(0x01) == 1            # 2**-9
    assert _int_units(0x81) == -1
    assert _int_units(0x08) == 8            # 2**-6 * 2**9
    for c in FINITE_E4M3_CODES:
        assert _int_units(c) == decode_e4m3(np.array([c]))[0] * 512


def test_unit_scales_reduce_to_integer_matmul():
    """With unit scales the block-scaled product is the plain product (the
    Triton-cutlass article's tiled listing: fp32 accumulation, no scales);
    in units of 2**-18 it is an exact int64 matmul."""
    g = np.random.default_rng(3)
    M, N, K = 48, 64, 128
    qa, qb = _rand_codes(g, (M, K)), _rand_codes(g, (K, N))
    ia = np.vectorize(_int_units)(qa).astype(np.int64)
    ib = np.vectorize(_int_units)(qb).astype(np.int64)
    exact_units = ia @ ib                       # |entries| < 2**53: exact in fp64 too
    ref, _ = gemm_ref(qa, np.ones((2, 4), np.float32), qb, np.ones((4, 2), np.float32))
    assert np.array_equal(ref * 2.0 ** 18, exact_units.astype(np.float64))


def test_identity_and_one_hot():
    g = np.random.default_rng(4)
    K, N = 64, 96
    qb = _rand_codes(g, (K, N))
    sb = _rand_scales(g, (K // 32, N // 32))
    qa = np.zeros((K, K), np.uint8)
    qa[np.arange(K), np.arange(K)] = 0x38       # identity in E4M3
    ref, _ = gemm_ref(qa, np.ones((2, 2), np.float32), qb, sb)
    expect = decode_e4m3(qb) * np.repeat(np.repeat(sb.astype(np.float64), 32, 0), 32, 1)
    assert np.array_equal(ref, expect)
    # one-hot row: a single code at (i, k) picks row k of B
    qa = np.zeros((5, K), np.uint8)
    qa[2, 37] = 0xC4                            # -3.0
    sa = _rand_scales(g, (1, K // 32))
    ref, _ = gemm_ref(qa, sa, qb, sb)
    assert np.all(ref[[0, 1, 3, 4]] == 0)
    assert np.array_equal(ref[2], -3.0 * np.float64(sa[0, 1]) * expect[37])


def test_power_of_two_scales_commute():
    g = np.random.default_rng(5)
    qa, qb = _rand_codes(g, (64, 64)), _rand_codes(g, (64, 32))
    sa, sb = _rand_scales(g, (2, 2)), _rand_scales(g, (2, 1))
    r0, a0 = gemm_ref(qa, sa, qb, sb)
    r1, a1 = gemm_ref(qa, sa * np.float32(2.0 ** 7), qb, sb * np.float32(2.0 ** -3))
    assert np.array_equal(r1, r0 * 2.0 ** 4) and np.array_equal(a1, a0 * 2.0 ** 4)


def test_zero_blocks_give_zero():
    g = np.random.default_rng(6)
    qa, qb = _rand_codes(g, (32, 64)), _rand_codes(g, (64, 64))
    sa = _rand_scales(g, (1, 2))
    sa[0, 0] = 0.0
    sb = _rand_scales(g, (2, 2))
    qb[32:, :] = 0
    ref, absref = gemm_ref(qa, sa, qb, sb)
    assert np.all(ref == 0) and np.all(absref == 0)


def test_submatrix_reference_matches_full():
    g = np.random.default_rng(7)
    qa, qb = _rand_codes(g, (70, 96)), _rand_codes(g, (96, 128))
    sa, sb = _rand_scales(g, (3, 3)), _rand_scales(g, (3, 4))
    ref, absref = gemm_ref(qa, sa, qb, sb)
    rows, cols = np.array([69, 0, 33, 5]), np.array([127, 3, 64])
    r, a = gemm_ref_at(qa, sa, qb, sb, rows, cols)
    # the two fp64 matmuls may sum in different orders: compare within gamma_K * absref
    sub = np.ix_(rows, cols)
    assert np.all(np.abs(r - ref[sub]) <= 1e-14 * absref[sub])
    assert np.all(np.abs(a - absref[sub]) <= 1e-14 * absref[sub])


def test_grouped_is_per_group_gemm():
    g = np.random.default_rng(8)
    G, K, N = 5, 64, 64
    rows = np.array([64, 0, 32, 96, 0])
    off = np.concatenate([[0], np.cumsum(rows)]).astype(np.int32)
    M = int(off[-1])
    qa, sa = _rand_codes(g, (M, K)), _rand_scales(g, (M // 32, K // 32))
    qb, sb = _rand_codes(g, (G, K, N)), _rand_scales(g, (G, K // 32, N // 32))
    ref, absref = grouped_gemm_ref(qa, sa, qb, sb, off)
    for gi in range(G):
        r0, r1 = off[gi], off[gi + 1]
        if r1 > r0:
            r, a = gemm_ref(qa[r0:r1], sa[r0 // 32:r1 // 32], qb[gi], sb[gi])
            assert np.array_equal(ref[r0:r1], r)
    sel = np.array([M - 1, 0, 70, 100])
    r, a = grouped_gemm_ref_at(qa, sa, qb, sb, off, sel, np.arange(N))
    assert np.all(np.abs(r - ref[sel]) <= 1e-14 * absref[sel])
    with pytest.raises(ValueError):
        grouped_gemm_ref(qa, sa, qb, sb, np.array([0, 16, M]))


@pytest.mark.parametrize("M,N,K", [(8, 32, 64), (33, 64, 32), (32, 32, 32)])
def test_k_major_reference_matches_exact_rational(M, N, K):
    """gemm_ref_nt on Bt [N, K] against the exact rational product of the same
    values laid out [K, N]; a square case so that a missing transpose or a
    scale grid read the wrong way round cannot pass by shape."""
    g = np.random.default_rng(M * 7 + N + K)
    qa, qbt = _rand_codes(g, (M, K)), _rand_codes(g, (N, K))
    sa, sbt = _rand_scales(g, (-(-M // 32), K // 32)), _rand_scales(g, (N // 32, K // 32))
    ref, absref = gemm_ref_nt(qa, sa, qbt, sbt)
    ex = np.vectorize(float)(gemm_exact(qa, sa, np.ascontiguousarray(qbt.T), np.ascontiguousarray(sbt.T)))
    u = 2.0 ** -53
    gam = (K + 2) * u / (1 - (K + 2) * u)
    assert np.all(np.abs(ref - ex) <= gam * absref + 1e-300)


def test_k_major_grouped_is_per_group():
    g = np.random.default_rng(9)
    G, K, N = 4, 64, 32
    off = np.array([0, 32, 32, 96, 128], np.int32)
    qa, sa = _rand_codes(g, (128, K)), _rand_scales(g, (4, K // 32))
    qbt, sbt = _rand_codes(g, (G, N, K)), _rand_scales(g, (G, N // 32, K // 32))
    ref, _ = grouped_gemm_ref_nt(qa, sa, qbt, sbt, off)
    for gi in range(G):
        r0, r1 = off[gi], off[gi + 1]
        if r1 > r0:
            ex = np.vectorize(float)(gemm_exact(qa[r0:r1], sa[r0 // 32:r1 // 32], qbt[gi].T, sbt[gi].T))
            assert np.all(np.abs(ref[r0:r1] - ex) <= 1e-12 * np.abs(ex) + 1e-300)


def test_quantizer_is_orientation_symmetric():
    """A 32x32 block holds the same elements read row- or column-major, so
    quantizing B^T gives the transposed codes and the transposed scale grid:
    the K-major weight path needs no quantizer of its own."""
    g = np.random.default_rng(10)
    x = (g.standard_normal((96, 64)).astype(np.float32) * np.float32(0.02)).view(np.uint32)
    bits = ((x + 0x7FFF + ((x >> 16) & 1)) >> 16).astype(np.uint16)
    q, s = quantize_blocks(bits)
    qt, st = quantize_blocks(np.ascontiguousarray(bits.T))
    assert np.array_equal(qt, q.T) and np.array_equal(st, s.T)


def test_tolerance_accepts_exact_and_rejects_outside():
    ref = np.array([1.0, -3.0, 0.0, 1e-3])
    absref = np.array([2.0, 5.0, 10.0, 100.0])
    b = tolerance_bound(ref, absref)
    assert np.array_equal(b, 2.0 ** -8 * np.abs(ref) + 1e-6 * absref)
    assert tolerance_ok(ref, ref, absref).all()
    assert tolerance_ok(ref + 0.99 * b, ref, absref).all()
    assert not tolerance_ok(ref + 1.01 * b, ref, absref).any()
    assert not tolerance_ok(ref - 1.01 * b, ref, absref).any()
