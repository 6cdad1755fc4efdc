"""Whole-output oracle checks at the workload sizes (test infrastructure).

The oracle's quantizers and dequantizers are plain numpy and single threaded;
at the workload sizes (up to 8192 x 28672) they are run here on a thread pool
over slabs of rows.  That changes nothing they compute:

* the block quantizer and dequantizer look only inside 32 x 32 blocks, so
  slabs that start on a multiple of 32 rows give exactly the codes, scales and
  values of one call on the whole matrix;
* the token-group quantizer looks only inside one row.

``tests/test_fullsize_util.py`` pins both statements on the CPU.

The GEMM reference (the plain fp64 product of the dequantized operands and
the magnitude sum sum_k |a' b'|) is formed in column chunks, and every element
of C is held to the oracle's acceptance bound.
"""

from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

import oracle

THREADS = max(1, min(16, len(os.sched_getaffinity(0))))
ROWS_PER_JOB = 256            # a multiple of 32


def _row_slabs(R, rows_per_job=ROWS_PER_JOB):
    return [(r0, min(R, r0 + rows_per_job)) for r0 in range(0, R, rows_per_job)]


def _pool_map(fn, items):
    with ThreadPoolExecutor(THREADS) as ex:
        return list(ex.map(fn, items))


def quantize_full(bits, token_groups=False, rows_per_job=ROWS_PER_JOB):
    """oracle.quantize_blocks (or quantize_token_groups) of the whole matrix,
    computed slab by slab.  Returns (codes uint8, scales float32)."""
    assert rows_per_job % 32 == 0
    fn = oracle.quantize_token_groups if token_groups else oracle.quantize_blocks
    bits = np.asarray(bits)
    parts = _pool_map(lambda s: fn(bits[s[0]:s[1]]), _row_slabs(bits.shape[0], rows_per_job))
    return np.concatenate([p[0] for p in parts]), np.concatenate([p[1] for p in parts])


def dequantize_full(q, s, token_groups=False, rows_per_job=ROWS_PER_JOB):
    """oracle.dequantize (or dequantize_token_groups) in fp64, slab by slab."""
    assert rows_per_job % 32 == 0
    q = np.asarray(q)
    s = np.asarray(s)
    out = np.empty(q.shape, dtype=np.float64)

    def job(sl):
        r0, r1 = sl
        if token_groups:
            out[r0:r1] = oracle.dequantize_token_groups(q[r0:r1], s[r0:r1])
        else:
            out[r0:r1] = oracle.dequantize(q[r0:r1], s[r0 // 32:-(-r1 // 32)])

    _pool_map(job, _row_slabs(q.shape[0], rows_per_job))
    return out


def assert_same_codes(q_got, s_got, q_ref, s_ref, label):
    """Quantizer output bit for bit: every code and every scale."""
    q_got, q_ref = np.asarray(q_got), np.asarray(q_ref)
    s_got, s_ref = np.asarray(s_got, np.float32), np.asarray(s_ref, np.float32)
    assert q_got.shape == q_ref.shape and s_got.shape == s_ref.shape, (label, q_got.shape, q_ref.shape)
    bad_s = np.argwhere(s_got.view(np.uint32) != s_ref.view(np.uint32))
    assert len(bad_s) == 0, f"{label}: {len(bad_s)} of {s_ref.size} scales differ, first {bad_s[:4].tolist()}"
    bad_q = np.argwhere(q_got != q_ref)
    assert len(bad_q) == 0, f"{label}: {len(bad_q)} of {q_ref.size} codes differ, first {bad_q[:4].tolist()}"


def check_c_full(c_bits, a_deq, b_deq=None, bt_deq=None, label="", col_chunk=2048):
    """Every element of C (bf16 bit patterns [M, N]) against the fp64 reference
    A' @ B' (B' [K, N], or B'^T given as bt_deq [N, K]), held to
    oracle.tolerance_ok.  Returns the number of elements checked."""
    c_bits = np.asarray(c_bits, dtype=np.uint16)
    M, N = c_bits.shape
    assert (b_deq is None) != (bt_deq is None)
    abs_a = np.abs(a_deq)
    bad_total, worst, first_bad = 0, 0.0, None
    for c0 in range(0, N, col_chunk):
        c1 = min(N, c0 + col_chunk)
        bc = b_deq[:, c0:c1] if b_deq is not None else bt_deq[c0:c1].T
        ref = a_deq @ bc
        absref = abs_a @ np.abs(bc)
        got = oracle.bf16_bits_to_f64(c_bits[:, c0:c1])
        ok = oracle.tolerance_ok(got, ref, absref)
        if not ok.all():
            bad = np.argwhere(~ok)
            bad_total += len(bad)
            ratio = np.abs(got - ref)[~ok] / oracle.tolerance_bound(ref, absref)[~ok]
            worst = max(worst, float(np.max(ratio)))
            if first_bad is None:
                i, j = bad[0]
                first_bad = (int(i), int(j) + c0, float(got[i, j]), float(ref[i, j]))
    assert bad_total == 0, (f"{label}: {bad_total} of {M * N} outputs outside the bound, worst |C-ref|/bound "
                            f"{worst:.3g}, first (row, col, C, ref) {first_bad}")
    return M * N


def spread_rows(M, count=64, seed=0):
    """`count` distinct rows of [0, M): evenly spread plus random ones, always
    with the first two and the last."""
    rng = np.random.default_rng(seed)
    pick = {0, 1, M - 1}
    pick.update(int(r) for r in np.linspace(0, M - 1, count // 2).round())
    while len(pick) < min(count, M):
        pick.add(int(rng.integers(0, M)))
    return sorted(pick)
