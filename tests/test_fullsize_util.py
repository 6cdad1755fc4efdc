"""The slab-parallel oracle calls used by the whole-output GPU checks give
exactly what one oracle call on the whole matrix gives, and the whole-output
comparison rejects what oracle.tolerance_ok rejects (CPU only)."""

import numpy as np
import pytest

import oracle
from fp8_block_scaled_03_amd import workloads as W

import fullsize_util as FU


@pytest.mark.parametrize("rows,cols,per_job", [(1000, 96, 64), (33, 64, 32), (256, 32, 256), (1, 160, 32)])
def test_slab_quantize_and_dequantize_equal_whole_calls(rows, cols, per_job):
    x = W.normal_bf16(9100 + rows, 0, rows, cols, 1.0, 0.01)
    x[5 % rows, :32] = 0
    q, s = FU.quantize_full(x, rows_per_job=per_job)
    qo, so = oracle.quantize_blocks(x)
    assert np.array_equal(q, qo) and np.array_equal(s.view(np.uint32), so.view(np.uint32))
    assert np.array_equal(FU.dequantize_full(q, s, rows_per_job=per_job), oracle.dequantize(qo, so))
    qt, st = FU.quantize_full(x, token_groups=True, rows_per_job=per_job)
    qto, sto = oracle.quantize_token_groups(x)
    assert np.array_equal(qt, qto) and np.array_equal(st.view(np.uint32), sto.view(np.uint32))
    assert np.array_equal(FU.dequantize_full(qt, st, token_groups=True, rows_per_job=per_job),
                          oracle.dequantize_token_groups(qto, sto))


def _bf16_rne_bits(x):
    return W.f32_to_bf16_bits(np.asarray(x, np.float32))


def test_whole_output_check_agrees_with_tolerance_ok():
    qa, sa = oracle.quantize_blocks(W.normal_bf16(9201, 0, 70, 96, 1.0))
    qb, sb = oracle.quantize_blocks(W.normal_bf16(9202, 0, 96, 160, 0.02))
    ref, absref = oracle.gemm_ref(qa, sa, qb, sb)
    a_deq, b_deq = oracle.dequantize(qa, sa), oracle.dequantize(qb, sb)
    good = _bf16_rne_bits(ref)
    assert FU.check_c_full(good, a_deq, b_deq, label="rounded ref", col_chunk=64) == 70 * 160
    # the same through the K-major form
    FU.check_c_full(good, a_deq, bt_deq=np.ascontiguousarray(b_deq.T), label="rounded ref nt", col_chunk=48)
    # plant one element just outside the bound, in the last column chunk
    bad = good.copy()
    i, j = 69, 150
    bound = oracle.tolerance_bound(ref, absref)[i, j]
    v = np.float32(ref[i, j] + 1.01 * bound + abs(ref[i, j]) * 2.0 ** -8)
    bad[i, j] = _bf16_rne_bits(np.array([v]))[0]
    assert not oracle.tolerance_ok(oracle.bf16_bits_to_f64(bad), ref, absref)[i, j]
    with pytest.raises(AssertionError, match="1 of 11200 outputs"):
        FU.check_c_full(bad, a_deq, b_deq, label="planted", col_chunk=64)


def test_spread_rows():
    r = FU.spread_rows(4096, 64, seed=1)
    assert len(r) == 64 and r[0] == 0 and r[1] == 1 and r[-1] == 4095 and len(set(r)) == 64
    assert FU.spread_rows(10, 64) == list(range(10))
