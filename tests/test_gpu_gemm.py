"""GEMM parity against the oracle, exact special cases, and batch invariance."""

import numpy as np
import pytest
import torch

import oracle
import fp8_block_scaled_03_amd as fp8bs
from fp8_block_scaled_03_amd import workloads as W

from gpu_util import bits_np, bits_to_f64, f32_dev, gpu_gemm, gpu_grouped, gpu_grouped_nt, say, u8_dev

pytestmark = pytest.mark.gpu


def _rand_codes(g, shape):
    return oracle.FINITE_E4M3_CODES[g.integers(0, len(oracle.FINITE_E4M3_CODES), shape)]


def _rand_scales(g, shape):
    return (g.uniform(1.0, 2.0, shape) * np.exp2(g.integers(-10, 4, shape))).astype(np.float32)


def _quantized(seed, rows, cols, std=1.0, outlier=0.0):
    return oracle.quantize_blocks(W.normal_bf16(seed, 0, rows, cols, std, outlier))


def _assert_tol(c_bits, ref, absref, label):
    c = bits_to_f64(c_bits)
    ok = oracle.tolerance_ok(c, ref, absref)
    bad = np.argwhere(~ok)
    assert len(bad) == 0, (f"{label}: {len(bad)} of {ok.size} outside the bound; first {bad[:4].tolist()}, "
                           f"worst ratio {np.max(np.abs(c - ref) / oracle.tolerance_bound(ref, absref)):.3g}")


@pytest.mark.parametrize("M,N,K", [
    (256, 256, 256),      # square-256 shape, tile kernel
    (300, 96, 96),        # ragged M and N (N < tile), several K-blocks
    (520, 288, 160),      # three M-tiles, two N-tiles, ragged tails
    (1, 64, 256), (8, 96, 128), (33, 32, 64), (64, 160, 96),   # small-M kernel
    (65, 64, 64),         # just above the small-M limit
    (1, 24576, 96), (40, 24576, 64),      # small-M kernel, 128-column slices
    (64, 12288, 96), (17, 12288, 320),    # small-M kernel, 64-column slices; ragged last round
    # tile kernel, odd numbers of K-blocks (the last one paired with an empty,
    # zero-scale block): one, seven, and 65 (past a 64-block scale window)
    (100, 64, 32), (130, 96, 32 * 7), (257, 64, 32 * 65),
    # small-M kernel, 128-column slices, 17-32 rows: A decoded once per
    # workgroup into a shared bf16 area (several rounds, a ragged last round)
    (17, 24576, 32 * 9), (32, 24576, 32 * 17), (24, 24576, 64),
])
def test_gemm_matches_oracle(M, N, K):
    qa, sa = _quantized(2000 + M, M, K)
    qb, sb = _quantized(3000 + N, K, N, std=0.02)
    say(f"gemm M={M} N={N} K={K}")
    c = gpu_gemm(qa, sa, qb, sb)
    ref, absref = oracle.gemm_ref(qa, sa, qb, sb)
    _assert_tol(c, ref, absref, f"M={M} N={N} K={K}")


def test_square_256_workload():
    wl = W.square_256()
    qa, sa = oracle.quantize_blocks(wl.a_bits())
    qb, sb = oracle.quantize_blocks(wl.b_bits())
    say("gemm square-256 workload")
    c = gpu_gemm(qa, sa, qb, sb)
    ref, absref = oracle.gemm_ref(qa, sa, qb, sb)
    _assert_tol(c, ref, absref, "square-256")


@pytest.mark.parametrize("M", [1, 40, 300])
def test_random_codes_and_scales(M):
    """Arbitrary finite codes (subnormals included) and non-power-of-two scales."""
    g = np.random.default_rng(M)
    K, N = 128, 64
    qa, qb = _rand_codes(g, (M, K)), _rand_codes(g, (K, N))
    sa, sb = _rand_scales(g, (-(-M // 32), K // 32)), _rand_scales(g, (K // 32, N // 32))
    say(f"gemm random codes M={M}")
    c = gpu_gemm(qa, sa, qb, sb)
    ref, absref = oracle.gemm_ref(qa, sa, qb, sb)
    _assert_tol(c, ref, absref, f"random codes M={M}")


@pytest.mark.parametrize("M", [64, 256])
def test_identity_is_exact(M):
    """A = I (code 0x38) with unit scales: C = bf16(dec(B)) bit for bit (E4M3 is a
    subset of bf16).  Pins operand decode, the B layout and OCP E4M3."""
    g = np.random.default_rng(11)
    K = M
    N = 96
    qa = np.zeros((M, K), np.uint8)
    qa[np.arange(M), np.arange(M)] = 0x38
    qb = _rand_codes(g, (K, N))
    say(f"gemm identity M={M}")
    c = gpu_gemm(qa, np.ones((M // 32, K // 32), np.float32), qb, np.ones((K // 32, N // 32), np.float32))
    expect = W.f32_to_bf16_bits(oracle.decode_e4m3(qb).astype(np.float32))
    expect[expect == 0x8000] = 0          # -0 * 1 + (+0 products) sums to +0
    assert np.array_equal(c, expect)


def test_power_of_two_scales_commute_bitwise():
    qa, sa = _quantized(21, 96, 128)
    qb, sb = _quantized(22, 128, 64, std=0.02)
    say("gemm power-of-two scaling")
    c0 = gpu_gemm(qa, sa, qb, sb)
    c1 = gpu_gemm(qa, sa * np.float32(2.0 ** 5), qb, sb * np.float32(2.0 ** -2))
    assert np.array_equal(bits_to_f64(c1), bits_to_f64(c0) * 8.0)


def test_zero_blocks_and_empty_k():
    qa, sa = _quantized(23, 80, 64)
    qb, sb = _quantized(24, 64, 64, std=0.02)
    sa[:, 0] = 0.0
    qb[32:, :] = 0
    say("gemm zero blocks")
    c = gpu_gemm(qa, sa, qb, sb)
    assert np.all(c == 0)
    for m in (70, 5):  # tile kernel, small-M kernel
        say(f"gemm K=0 M={m}")
        c = gpu_gemm(np.zeros((m, 0), np.uint8), np.zeros((-(-m // 32), 0), np.float32),
                     np.zeros((0, 64), np.uint8), np.zeros((0, 2), np.float32))
        assert c.shape == (m, 64) and np.all(c == 0)
    say("grouped K=0")
    off = np.array([0, 32, 32, 96], np.int32)
    c = gpu_grouped(np.zeros((96, 0), np.uint8), np.zeros((3, 0), np.float32), np.zeros((3, 0, 64), np.uint8),
                    np.zeros((3, 0, 2), np.float32), off)
    assert c.shape == (96, 64) and np.all(c == 0)


def test_zero_results_are_plus_zero_in_every_kernel():
    """Outputs whose promotions all underflow to a signed zero: an odd number
    of K-blocks (the tile kernel pairs the last one with a zero-scale block,
    the small-M kernels do not), scale products far below the fp32 normal
    range, negative or zero partials.  Every kernel stores such a result as +0,
    so rows agree bitwise between M = 1, M = 40 and M = 65, and between the
    [K, N] and K-major entry points."""
    M, N, K = 65, 64, 96
    qa = np.zeros((M, K), np.uint8)
    qb = np.zeros((K, N), np.uint8)
    qa[:, [0, 32, 64]] = 0x81        # -2^-9 in every K-block
    qa[1::2, [0, 32, 64]] = 0x80     # -0 codes on odd rows
    qb[[0, 32, 64], :] = 0x01        # +2^-9
    qb[[0, 32, 64], 1::3] = 0x81     # -2^-9 in some columns
    sa = np.full((3, 3), 2.0 ** -70, np.float32)
    sb = np.full((3, 2), 2.0 ** -70, np.float32)   # s = 2^-140: every product 2^-158 rounds to a zero
    say("gemm signed-zero results, tile kernel")
    full = gpu_gemm(qa, sa, qb, sb)
    assert np.all(full == 0x0000), "zero results stored as +0"
    for m in (1, 40):
        say(f"gemm signed-zero results, M={m}")
        assert np.array_equal(gpu_gemm(qa[:m], sa[:-(-m // 32)], qb, sb), full[:m]), m
    say("gemm_nt signed-zero results")
    c_nt = fp8bs.gemm_nt(u8_dev(qa), f32_dev(sa), u8_dev(np.ascontiguousarray(qb.T)),
                         f32_dev(np.ascontiguousarray(sb.T)))
    torch.cuda.synchronize()
    assert np.array_equal(bits_np(c_nt), full)


def test_rows_independent_of_batch():
    """Row i of C is bitwise the same computed alone (M=1, small-M kernel),
    inside M=64 (small-M kernel), inside M=100 (one light tile), M=200 and
    M=320 (tile kernel; the last 64 rows of M=320 form a light tile)."""
    qa, sa = _quantized(25, 320, 256)
    qb, sb = _quantized(26, 256, 96, std=0.02)
    say("invariance full M=320")
    full = gpu_gemm(qa, sa, qb, sb)
    say("invariance M=64")
    part = gpu_gemm(qa[:64], sa[:2], qb, sb)
    assert np.array_equal(part, full[:64])
    say("invariance M=100 (a light tile) and M=200 (a full one)")
    assert np.array_equal(gpu_gemm(qa[:100], sa[:4], qb, sb), full[:100])
    assert np.array_equal(gpu_gemm(qa[:200], sa[:7], qb, sb), full[:200])
    for i in (0, 5, 31, 32, 63, 64, 100, 255, 319):
        say(f"invariance row {i}")
        one = gpu_gemm(qa[i:i + 1], sa[i // 32:i // 32 + 1], qb, sb)
        assert np.array_equal(one[0], full[i]), f"row {i}"
    for m in (1, 8, 32):
        say(f"invariance prefix M={m}")
        pre = gpu_gemm(qa[:m], sa[:-(-m // 32)], qb, sb)
        assert np.array_equal(pre, full[:m])


@pytest.mark.parametrize("N", [12288, 24576])
def test_rows_independent_of_batch_wide_slices(N):
    """The small-M kernel's 64- and 128-column slice variants give the tile
    kernel's bits, row by row."""
    qa, sa = _quantized(29, 320, 160)
    qb, sb = _quantized(30, 160, N, std=0.02)
    say(f"wide invariance full M=320 N={N}")
    full = gpu_gemm(qa, sa, qb, sb)
    ref, absref = oracle.gemm_ref(qa, sa, qb, sb)
    _assert_tol(full, ref, absref, f"wide M=320 N={N}")
    for m in (64, 33, 32, 20, 8, 1):
        say(f"wide invariance prefix M={m} N={N}")
        pre = gpu_gemm(qa[:m], sa[:-(-m // 32)], qb, sb)
        assert np.array_equal(pre, full[:m]), f"M={m}"
    for i in (7, 200):
        say(f"wide invariance row {i} N={N}")
        one = gpu_gemm(qa[i:i + 1], sa[i // 32:i // 32 + 1], qb, sb)
        assert np.array_equal(one[0], full[i]), f"row {i}"


def test_row_blocks_permute_and_repeat():
    qa, sa = _quantized(27, 512, 128)
    qb, sb = _quantized(28, 128, 64, std=0.02)
    say("permutation base")
    c = gpu_gemm(qa, sa, qb, sb)
    perm = np.random.default_rng(0).permutation(16)
    rows = (perm[:, None] * 32 + np.arange(32)[None, :]).reshape(-1)
    say("permutation permuted")
    cp = gpu_gemm(qa[rows], sa[perm], qb, sb)
    assert np.array_equal(cp, c[rows])
    for _ in range(2):
        assert np.array_equal(gpu_gemm(qa, sa, qb, sb), c)


@pytest.mark.parametrize("K", [128, 96, 32])   # even, odd and single K-block counts
def test_grouped_matches_oracle_and_single_gemm(K):
    g = np.random.default_rng(31)
    G, N = 6, 96
    rows = np.array([64, 0, 288, 32, 0, 96])
    off = W.offsets_from_rows(rows)
    M = int(off[-1])
    qa, sa = _quantized(32, M, K)
    qb = np.stack([_quantized(40 + i, K, N, std=0.02)[0] for i in range(G)])
    sb = np.stack([_quantized(40 + i, K, N, std=0.02)[1] for i in range(G)])
    say(f"grouped small K={K}")
    c = gpu_grouped(qa, sa, qb, sb, off)
    ref, absref = oracle.grouped_gemm_ref(qa, sa, qb, sb, off)
    _assert_tol(c, ref, absref, "grouped")
    for gi in range(G):
        r0, r1 = off[gi], off[gi + 1]
        if r1 > r0:
            say(f"grouped vs single group {gi}")
            single = gpu_gemm(qa[r0:r1], sa[r0 // 32:r1 // 32], qb[gi], sb[gi])
            assert np.array_equal(single, c[r0:r1])
    del g


def test_grouped_all_empty_but_one_and_untouched_rows():
    K, N = 64, 64
    off = np.array([0, 0, 64, 64], np.int32)
    qa, sa = _quantized(50, 64, K)
    qb = np.stack([_quantized(51 + i, K, N)[0] for i in range(3)])
    sb = np.stack([_quantized(51 + i, K, N)[1] for i in range(3)])
    say("grouped one live group")
    c = gpu_grouped(qa, sa, qb, sb, off)
    ref, absref = oracle.grouped_gemm_ref(qa, sa, qb, sb, off)
    _assert_tol(c, ref, absref, "grouped one live group")


def test_grouped_many_groups_heavy_and_light_tiles():
    """130 groups (the tile lookup walks the offsets 64 groups at a time) with
    sizes from 0 to 544 rows in 32-row steps: full 256-row tiles, tails above
    and at most 128 rows, empty groups.  Every group's rows equal a single
    GEMM on them, bitwise, and the whole output is within the bound."""
    G, K, N = 130, 96, 64
    g = np.random.default_rng(77)
    rows = 32 * g.integers(0, 18, G)
    rows[[3, 64, 65, 129]] = 0
    off = np.concatenate([[0], np.cumsum(rows)]).astype(np.int32)
    M = int(off[-1])
    qa, sa = _quantized(70, M, K)
    qb = np.stack([_quantized(1000 + i, K, N, std=0.02)[0] for i in range(G)])
    sb = np.stack([_quantized(1000 + i, K, N, std=0.02)[1] for i in range(G)])
    say(f"grouped G={G} M={M}")
    c = gpu_grouped(qa, sa, qb, sb, off)
    ref, absref = oracle.grouped_gemm_ref(qa, sa, qb, sb, off)
    _assert_tol(c, ref, absref, "grouped many groups")
    for gi in (0, 1, 63, 66, 100, 128):
        r0, r1 = int(off[gi]), int(off[gi + 1])
        if r1 > r0:
            say(f"grouped many groups: group {gi} as a single GEMM")
            assert np.array_equal(c[r0:r1], gpu_gemm(qa[r0:r1], sa[r0 // 32:r1 // 32], qb[gi], sb[gi])), gi


@pytest.mark.parametrize("K", [352, 64])   # eleven K-blocks (odd), two
def test_grouped_light_tiles_every_column_band(K):
    """Group tails of at most 128 rows run as light tiles (eight 64 x 64 wave
    tiles over 128 rows x 256 columns): tails of 32, 64, 96 and 128 rows, and
    groups with full tiles before them, at N = 544 (two full column tiles and
    a 32-column rest).  Each group equals a single GEMM of its rows bitwise,
    in both weight layouts, and the whole output is within the bound."""
    G, N = 7, 544
    rows = np.array([32, 64, 96, 128, 288, 416, 0])
    off = W.offsets_from_rows(rows)
    M = int(off[-1])
    qa, sa = _quantized(90, M, K)
    qb = np.stack([_quantized(91 + i, K, N, std=0.02)[0] for i in range(G)])
    sb = np.stack([_quantized(91 + i, K, N, std=0.02)[1] for i in range(G)])
    say(f"grouped light tiles K={K}")
    c = gpu_grouped(qa, sa, qb, sb, off)
    ref, absref = oracle.grouped_gemm_ref(qa, sa, qb, sb, off)
    _assert_tol(c, ref, absref, "grouped light tiles")
    qbt = np.ascontiguousarray(qb.transpose(0, 2, 1))
    sbt = np.ascontiguousarray(sb.transpose(0, 2, 1))
    say("grouped light tiles, K-major weight")
    assert np.array_equal(c, gpu_grouped_nt(qa, sa, qbt, sbt, off))
    for gi in range(G):
        r0, r1 = int(off[gi]), int(off[gi + 1])
        if r1 > r0:
            say(f"grouped light tiles: group {gi} ({r1 - r0} rows) as a single GEMM")
            assert np.array_equal(c[r0:r1], gpu_gemm(qa[r0:r1], sa[r0 // 32:r1 // 32], qb[gi], sb[gi])), gi


def _effective_ranges(off, M_total):
    """The documented treatment of a bad offsets table: each range clipped to
    [0, M_total], started no earlier than the previous range's end, and empty
    when it would run backwards."""
    out, prev_end = [], 0
    for g in range(len(off) - 1):
        s0 = min(max(int(off[g]), 0), M_total)
        s1 = min(max(int(off[g + 1]), 0), M_total)
        s0 = max(s0, prev_end)
        s1 = max(s1, s0)
        prev_end = s1
        out.append((s0, s1))
    return out


def test_grouped_bad_offsets_are_clipped_not_faulted():
    """Negative, decreasing, overlapping and out-of-range entries (multiples of
    32): every clipped range holds exactly the plain GEMM's rows for its group,
    rows outside every range are untouched.  An unaligned table runs too (its
    rows may use the wrong scale rows; the call must only stay in bounds)."""
    G, K, N, M = 4, 64, 64, 192
    qa, sa = _quantized(60, M, K)
    qb = np.stack([_quantized(61 + i, K, N, std=0.02)[0] for i in range(G)])
    sb = np.stack([_quantized(61 + i, K, N, std=0.02)[1] for i in range(G)])
    singles = []
    for gi in range(G):
        say(f"bad offsets: single GEMM group {gi}")
        singles.append(gpu_gemm(qa, sa, qb[gi], sb[gi]))
    sentinel = np.full((M, N), 0x7FC1, np.uint16)
    for off in ([-64, 64, 32, 320, 128], [32, 32, 96, 64, 160], [0, 192, 0, 192, 0]):
        off = np.array(off, np.int32)
        say(f"bad offsets {off.tolist()}")
        c = gpu_grouped(qa, sa, qb, sb, off, c_init=sentinel)
        covered = np.zeros(M, bool)
        for gi, (s0, s1) in enumerate(_effective_ranges(off, M)):
            if s1 > s0:
                assert np.array_equal(c[s0:s1], singles[gi][s0:s1]), (off.tolist(), gi)
                covered[s0:s1] = True
        assert np.all(c[~covered] == 0x7FC1), off.tolist()
    say("unaligned offsets")
    gpu_grouped(qa, sa, qb, sb, np.array([0, 40, 100, 150, 192], np.int32))
    assert np.array_equal(gpu_gemm(qa, sa, qb[1], sb[1]), singles[1])
