"""Seeded random shapes through every entry point, against the oracle, and
concurrent calls from two host threads on two streams."""

import threading

import numpy as np
import pytest
import torch

import oracle
import fp8_block_scaled_03_amd as fp8bs
from fp8_block_scaled_03_amd import workloads as W

from gpu_util import DEV, bf16_dev, bits_np, bits_to_f64, f32_dev, say, u8_dev

pytestmark = pytest.mark.gpu


def _shapes(seed, n):
    g = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        M = int(g.choice([int(g.integers(1, 65)), int(g.integers(65, 700))]))
        N = 32 * int(g.integers(1, 40))
        K = 32 * int(g.integers(1, 20))
        out.append((M, N, K))
    return out


@pytest.mark.parametrize("seed", [7001, 7002])
def test_random_quantizer_shapes_bit_exact(seed):
    g = np.random.default_rng(seed)
    for i in range(12):
        rows, cols = int(g.integers(1, 400)), 32 * int(g.integers(1, 70))
        x = W.normal_bf16(seed + i, 0, rows, cols, float(2.0 ** g.integers(-20, 20)), 0.01)
        say(f"random quantizers {rows}x{cols}")
        q, s = fp8bs.quantize(bf16_dev(x))
        qt, st = fp8bs.quantize_tg(bf16_dev(x))
        torch.cuda.synchronize()
        qo, so = oracle.quantize_blocks(x)
        qto, sto = oracle.quantize_token_groups(x)
        assert np.array_equal(q.cpu().numpy(), qo) and np.array_equal(s.cpu().numpy(), so), (rows, cols)
        assert np.array_equal(qt.cpu().numpy(), qto) and np.array_equal(st.cpu().numpy(), sto), (rows, cols)


@pytest.mark.parametrize("seed", [7101, 7102, 7103])
def test_random_gemm_shapes_all_entry_points(seed):
    for (M, N, K) in _shapes(seed, 8):
        x = W.normal_bf16(seed + M, 0, M, K, 1.0, 0.01)
        qa, sa = oracle.quantize_blocks(x)
        qat, sat = oracle.quantize_token_groups(x)
        qb, sb = oracle.quantize_blocks(W.normal_bf16(seed + N, 1, K, N, 0.02))
        qbt, sbt = np.ascontiguousarray(qb.T), np.ascontiguousarray(sb.T)
        say(f"random gemm M={M} N={N} K={K}")
        da, dsa, dat, dsat = u8_dev(qa), f32_dev(sa), u8_dev(qat), f32_dev(sat)
        db, dsb, dbt, dsbt = u8_dev(qb), f32_dev(sb), u8_dev(qbt), f32_dev(sbt)
        c = bits_np(fp8bs.gemm(da, dsa, db, dsb))
        c_nt = bits_np(fp8bs.gemm_nt(da, dsa, dbt, dsbt))
        c_tg = bits_np(fp8bs.gemm_tg(dat, dsat, db, dsb))
        c_tg_nt = bits_np(fp8bs.gemm_tg_nt(dat, dsat, dbt, dsbt))
        torch.cuda.synchronize()
        ref, absref = oracle.gemm_ref(qa, sa, qb, sb)
        assert oracle.tolerance_ok(bits_to_f64(c), ref, absref).all(), (M, N, K)
        assert np.array_equal(c, c_nt), (M, N, K)
        ref, absref = oracle.gemm_ref_tg(qat, sat, qb, sb)
        assert oracle.tolerance_ok(bits_to_f64(c_tg), ref, absref).all(), (M, N, K)
        assert np.array_equal(c_tg, c_tg_nt), (M, N, K)


def test_concurrent_calls_from_two_threads_on_two_streams():
    """Two host threads, each on its own stream, issue GEMMs and quantizations
    at the same time; every result equals the serial one bit for bit."""
    M, N, K = 320, 1024, 512
    xs = [W.normal_bf16(7200 + i, 0, M, K) for i in range(2)]
    qb, sb = oracle.quantize_blocks(W.normal_bf16(7210, 1, K, N, 0.02))
    db, dsb = u8_dev(qb), f32_dev(sb)
    dxs = [bf16_dev(x) for x in xs]

    def work(i):
        qa, sa = fp8bs.quantize(dxs[i])
        c = fp8bs.gemm(qa, sa, db, dsb)
        c1 = fp8bs.gemm(qa[:7].contiguous(), sa[:1].contiguous(), db, dsb)
        return c, c1

    say("concurrency: serial reference")
    serial = [work(i) for i in range(2)]
    torch.cuda.synchronize()
    serial = [(bits_np(c), bits_np(c1)) for c, c1 in serial]
    results = [None, None]
    errors = []

    def run(i):
        try:
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                outs = []
                for _ in range(5):
                    outs.append(work(i))
                s.synchronize()
                results[i] = [(bits_np(c), bits_np(c1)) for c, c1 in outs]
        except Exception as e:  # reported below
            errors.append(e)

    say("concurrency: two threads")
    threads = [threading.Thread(target=run, args=(i,)) for i in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=60)
    assert not errors, errors
    for i in range(2):
        assert results[i] is not None
        for c, c1 in results[i]:
            assert np.array_equal(c, serial[i][0]) and np.array_equal(c1, serial[i][1])
            assert np.array_equal(c1, c[:7])
