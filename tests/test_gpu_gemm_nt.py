"""K-major weights (B^T [N, K], scales [N/32, K/32]): parity against the
oracle, and bitwise equality with the [K, N] entry points on the transposed
weight (the per-element recipe is the same, so the bits must be too)."""

import numpy as np
import pytest
import torch

import oracle
import fp8_block_scaled_03_amd as fp8bs
from fp8_block_scaled_03_amd import workloads as W

import fullsize_util as FU
from gpu_util import (DEV, bf16_dev, bits_np, bits_to_f64, f32_dev, gpu_gemm, gpu_grouped, gpu_grouped_nt, i32_dev, say,
                      u8_dev)

pytestmark = pytest.mark.gpu


def _quantized(seed, rows, cols, std=1.0):
    return oracle.quantize_blocks(W.normal_bf16(seed, 0, rows, cols, std))


def gpu_gemm_nt(qa, sa, qbt, sbt):
    c = fp8bs.gemm_nt(u8_dev(qa), f32_dev(sa), u8_dev(qbt), f32_dev(sbt))
    torch.cuda.synchronize()
    return bits_np(c)


def _assert_tol(c_bits, ref, absref, label):
    ok = oracle.tolerance_ok(bits_to_f64(c_bits), ref, absref)
    assert ok.all(), f"{label}: {int((~ok).sum())} of {ok.size} outside the bound"


@pytest.mark.parametrize("M,N,K", [
    (256, 256, 256), (300, 96, 96), (520, 288, 160),     # tile kernel, ragged M and N
    (1, 64, 256), (8, 96, 320), (33, 32, 64), (64, 160, 96),   # small-M, 32-column slices, ragged rounds
    (17, 12288, 96),                                     # small-M, 64-column slices
    (40, 28672, 64), (1, 28672, 320),                    # small-M, 128-column slices
    (65, 64, 64),
    (9, 12288, 96), (16, 12288, 320),                   # K-blocks split over waves, 64-column slices
    (24, 96, 160), (32, 64, 288),                        # K-blocks split over waves, 17-32 rows
    # deeper K: several rounds of the small-M rings plus ragged tails, for
    # 1-4 row tiles, and a grid wider than 16384 columns
    (1, 32, 32 * 31), (5, 64, 32 * 32), (16, 32, 32 * 33), (3, 96, 32 * 70),
    (17, 32, 32 * 15), (32, 64, 32 * 16), (20, 32, 32 * 37),
    (33, 32, 32 * 7), (48, 64, 32 * 8), (64, 32, 32 * 9), (57, 96, 32 * 25),
    (2, 16416, 32 * 17), (30, 16416, 32 * 9), (64, 16416, 32 * 5),
    (100, 64, 32), (130, 96, 32 * 7),                     # tile kernel, odd K-block counts
    # 128-column slices, 17-32 rows: A decoded once per workgroup into a
    # shared bf16 area (several rounds, ragged last rounds)
    (17, 32768, 32 * 9), (32, 28672, 32 * 17), (24, 28672, 64),
])
def test_gemm_nt_matches_oracle_and_kn_path(M, N, K):
    qa, sa = _quantized(4000 + M, M, K)
    qb, sb = _quantized(5000 + N, K, N, std=0.02)
    qbt, sbt = np.ascontiguousarray(qb.T), np.ascontiguousarray(sb.T)
    say(f"gemm_nt M={M} N={N} K={K}")
    c_nt = gpu_gemm_nt(qa, sa, qbt, sbt)
    ref, absref = oracle.gemm_ref_nt(qa, sa, qbt, sbt)
    _assert_tol(c_nt, ref, absref, f"nt M={M} N={N} K={K}")
    say(f"gemm (K, N layout) M={M} N={N} K={K}")
    assert np.array_equal(c_nt, gpu_gemm(qa, sa, qb, sb)), "K-major and [K, N] results differ"


def test_gemm_nt_rows_independent_of_batch():
    qa, sa = _quantized(61, 320, 256)
    qbt, sbt = _quantized(62, 28672 // 4, 256, std=0.02)   # N = 7168
    say("nt invariance full M=320")
    full = gpu_gemm_nt(qa, sa, qbt, sbt)
    for m in (64, 8, 1):
        say(f"nt invariance prefix M={m}")
        assert np.array_equal(gpu_gemm_nt(qa[:m], sa[:-(-m // 32)], qbt, sbt), full[:m]), f"M={m}"
    for i in (3, 200):
        say(f"nt invariance row {i}")
        assert np.array_equal(gpu_gemm_nt(qa[i:i + 1], sa[i // 32:i // 32 + 1], qbt, sbt)[0], full[i])


def test_gemm_nt_rows_independent_of_batch_wide_slices():
    """128-column K-major slices (N = 28672): prefixes of 17-32 rows (A decoded
    once per workgroup) and of 1-16 and 33-64 rows give the tile kernel's bits."""
    qa, sa = _quantized(63, 320, 32 * 11)
    qbt, sbt = _quantized(64, 28672, 32 * 11, std=0.02)
    say("nt wide invariance full M=320")
    full = gpu_gemm_nt(qa, sa, qbt, sbt)
    for m in (64, 40, 32, 20, 17, 16, 1):
        say(f"nt wide invariance prefix M={m}")
        assert np.array_equal(gpu_gemm_nt(qa[:m], sa[:-(-m // 32)], qbt, sbt), full[:m]), f"M={m}"


def test_gemm_nt_empty_k():
    for m in (70, 5):
        say(f"gemm_nt K=0 M={m}")
        c = gpu_gemm_nt(np.zeros((m, 0), np.uint8), np.zeros((-(-m // 32), 0), np.float32),
                        np.zeros((64, 0), np.uint8), np.zeros((2, 0), np.float32))
        assert c.shape == (m, 64) and np.all(c == 0)


@pytest.mark.parametrize("K", [128, 96, 32])   # even, odd and single K-block counts
def test_grouped_nt_matches_oracle_and_kn_path(K):
    G, N = 5, 96
    rows = np.array([64, 0, 288, 32, 96])
    off = W.offsets_from_rows(rows)
    M = int(off[-1])
    qa, sa = _quantized(70, M, K)
    qb = np.stack([_quantized(71 + i, K, N, std=0.02)[0] for i in range(G)])
    sb = np.stack([_quantized(71 + i, K, N, std=0.02)[1] for i in range(G)])
    qbt = np.ascontiguousarray(qb.transpose(0, 2, 1))
    sbt = np.ascontiguousarray(sb.transpose(0, 2, 1))
    say(f"grouped_nt small K={K}")
    c = gpu_grouped_nt(qa, sa, qbt, sbt, off)
    ref, absref = oracle.grouped_gemm_ref_nt(qa, sa, qbt, sbt, off)
    _assert_tol(c, ref, absref, "grouped nt")
    say("grouped (K, N layout)")
    assert np.array_equal(c, gpu_grouped(qa, sa, qb, sb, off))


def test_decode_nt_full_size():
    """Decode shapes, K = 8192, M = 64 and prefixes: the K-major kernel at full
    size, every element against the oracle and bitwise equal to the [K, N]
    kernel's, prefixes bitwise equal to the M = 64 rows."""
    for N in (8192, 28672):
        wl = W.decode(64, N)
        a_bits, b_bits = wl.a_bits(), wl.b_bits()
        bt_bits = np.ascontiguousarray(b_bits.T)
        say(f"decode nt N={N}: quantize")
        qa, sa = fp8bs.quantize(bf16_dev(a_bits))
        qbt, sbt = fp8bs.quantize(bf16_dev(bt_bits))
        qb, sb = fp8bs.quantize(bf16_dev(b_bits))
        say(f"decode nt N={N}: gemm_nt and gemm")
        c_nt = fp8bs.gemm_nt(qa, sa, qbt, sbt)
        c_kn = fp8bs.gemm(qa, sa, qb, sb)
        torch.cuda.synchronize()
        assert torch.equal(c_nt.view(torch.int16), c_kn.view(torch.int16))
        for m in (1, 8, 32):
            cm = fp8bs.gemm_nt(qa[:m].contiguous(), sa[:(m + 31) // 32].contiguous(), qbt, sbt)
            torch.cuda.synchronize()
            assert torch.equal(cm.view(torch.int16), c_nt[:m].view(torch.int16)), f"N={N} M={m}"
        say(f"decode nt N={N}: oracle")
        qa_o, sa_o = FU.quantize_full(a_bits)
        qbt_o, sbt_o = FU.quantize_full(bt_bits)
        FU.assert_same_codes(qbt.cpu().numpy(), sbt.cpu().numpy(), qbt_o, sbt_o, f"decode nt N={N} weight")
        FU.check_c_full(bits_np(c_nt), FU.dequantize_full(qa_o, sa_o), bt_deq=FU.dequantize_full(qbt_o, sbt_o),
                        label=f"decode nt N={N}")
        del qa, sa, qbt, sbt, qb, sb, c_nt, c_kn
        torch.cuda.empty_cache()


def test_prefill_nt_full_size():
    """Prefill M = K = 8192, N = 28672 with the weight K-major: every element
    against the oracle (which quantizes both operands itself)."""
    wl = W.prefill(28672)
    a_bits = wl.a_bits()
    bt_bits = np.ascontiguousarray(wl.b_bits().T)
    say("prefill nt N=28672: quantize + gemm_nt")
    qa, sa = fp8bs.quantize(bf16_dev(a_bits))
    qbt, sbt = fp8bs.quantize(bf16_dev(bt_bits))
    c = fp8bs.gemm_nt(qa, sa, qbt, sbt)
    torch.cuda.synchronize()
    c_host = bits_np(c)
    del c
    say("prefill nt N=28672: oracle")
    qa_o, sa_o = FU.quantize_full(a_bits)
    FU.assert_same_codes(qa.cpu().numpy(), sa.cpu().numpy(), qa_o, sa_o, "prefill nt A")
    qbt_o, sbt_o = FU.quantize_full(bt_bits)
    FU.assert_same_codes(qbt.cpu().numpy(), sbt.cpu().numpy(), qbt_o, sbt_o, "prefill nt weight")
    del qa, sa, qbt, sbt
    torch.cuda.empty_cache()
    FU.check_c_full(c_host, FU.dequantize_full(qa_o, sa_o), bt_deq=FU.dequantize_full(qbt_o, sbt_o),
                    label="prefill nt N=28672")
