"""Per-token-group activation scales (1 row x 32 columns): the quantizer is
bit-exact against the oracle, the GEMMs (both weight layouts, every kernel)
are within the tolerance, and the whole bf16 -> quantize -> GEMM chain is
batch invariant: a row's codes, scales and outputs do not depend on the other
rows."""

import numpy as np
import pytest
import torch

import oracle
import fp8_block_scaled_03_amd as fp8bs
from fp8_block_scaled_03_amd import workloads as W

import fullsize_util as FU
from gpu_util import bf16_dev, bits_np, bits_to_f64, f32_dev, say, u8_dev

pytestmark = pytest.mark.gpu


def gpu_quantize_tg(x_bits):
    q, s = fp8bs.quantize_tg(bf16_dev(x_bits))
    torch.cuda.synchronize()
    return q.cpu().numpy(), s.cpu().numpy()


def gpu_gemm_tg(qa, sa_rows, qb, sb, k_major=False):
    fn = fp8bs.gemm_tg_nt if k_major else fp8bs.gemm_tg
    c = fn(u8_dev(qa), f32_dev(sa_rows), u8_dev(qb), f32_dev(sb))
    torch.cuda.synchronize()
    return bits_np(c)


def _check_quant(x_bits, label):
    say(f"quantize_tg {label} shape={x_bits.shape}")
    q, s = gpu_quantize_tg(x_bits)
    qo, so = oracle.quantize_token_groups(x_bits)
    assert np.array_equal(s.view(np.uint32), so.view(np.uint32)), f"{label}: scales differ"
    bad = np.argwhere(q != qo)
    assert len(bad) == 0, f"{label}: {len(bad)} codes differ, first {bad[:5].tolist()}"


@pytest.mark.parametrize("rows,cols", [(1, 32), (33, 64), (100, 96), (64, 8192), (300, 160)])
def test_quantize_tg_random(rows, cols):
    _check_quant(W.normal_bf16(1100, 0, rows, cols, 1.0, 0.01), "normal with outliers")


@pytest.mark.parametrize("amax_bits", [0x43E0, 0x3F80, 0x0001, 0x2100, 0x2180, 0x7F7F, 0x3FFF])
def test_quantize_tg_all_bf16_under_group_maxima(amax_bits):
    """Every finite bf16 |x| <= amax in groups of 31 led by the maximum itself."""
    bits = np.arange(0, 1 << 16, dtype=np.uint32)
    xf = (bits << 16).view(np.float32)
    allb = bits[np.isfinite(xf)].astype(np.uint16)
    af = np.array([np.uint32(amax_bits) << np.uint32(16)], dtype=np.uint32).view(np.float32)[0]
    keep = allb[np.abs((allb.astype(np.uint32) << 16).view(np.float32)) <= af]
    n = -(-len(keep) // 31)
    pad = np.zeros(n * 31, np.uint16)
    pad[:len(keep)] = keep
    x = np.concatenate([np.full((n, 1), amax_bits, np.uint16), pad.reshape(n, 31)], axis=1)
    _check_quant(x, f"amax bits {amax_bits:#06x}")


def test_quantize_tg_ignores_other_rows():
    x = W.normal_bf16(1101, 0, 64, 64)
    q, s = gpu_quantize_tg(x)
    x2 = x.copy()
    x2[5, 3] = 0x4700      # 32768 in another row of the same 32x32 block
    q2, s2 = gpu_quantize_tg(x2)
    keep = np.ones(64, bool)
    keep[5] = False
    assert np.array_equal(q[keep], q2[keep]) and np.array_equal(s[keep], s2[keep])


@pytest.mark.parametrize("k_major", [False, True])
@pytest.mark.parametrize("M,N,K", [
    (256, 256, 256), (300, 96, 96), (520, 288, 160),          # tile kernel, ragged
    (1, 64, 256), (8, 96, 320), (33, 32, 64), (64, 160, 96),    # small-M, narrow slices, ragged rounds
    (17, 12288, 96), (40, 28672, 64), (64, 24576, 64),          # small-M, wide slices
    (9, 12288, 96), (24, 96, 160), (32, 64, 288),                # K-blocks split over waves (K-major)
    # deeper K with ragged tails, and a grid wider than 16384 columns
    (1, 32, 32 * 33), (16, 64, 32 * 32), (31, 32, 32 * 17), (50, 96, 32 * 9),
    (4, 16416, 32 * 17), (64, 16416, 32 * 5),
    # tile kernel, odd K-block counts: one, and 17 (past a 16-block scale window)
    (100, 64, 32), (130, 96, 32 * 17),
    # small-M, 128-column slices, 17-32 rows: packed scale record and A decoded
    # once per workgroup
    (20, 28672, 32 * 9), (32, 28672, 32 * 5),
])
def test_gemm_tg_matches_oracle(M, N, K, k_major):
    qa, sa_rows = oracle.quantize_token_groups(W.normal_bf16(1200 + M, 0, M, K, 1.0, 0.01))
    qb, sb = oracle.quantize_blocks(W.normal_bf16(1300 + N, 1, K, N, 0.02))
    say(f"gemm_tg M={M} N={N} K={K} k_major={k_major}")
    if k_major:
        c = gpu_gemm_tg(qa, sa_rows, np.ascontiguousarray(qb.T), np.ascontiguousarray(sb.T), k_major=True)
    else:
        c = gpu_gemm_tg(qa, sa_rows, qb, sb)
    ref, absref = oracle.gemm_ref_tg(qa, sa_rows, qb, sb)
    ok = oracle.tolerance_ok(bits_to_f64(c), ref, absref)
    assert ok.all(), f"{int((~ok).sum())} of {ok.size} outside the bound"


def test_gemm_tg_layouts_agree_bitwise_and_k0():
    qa, sa_rows = oracle.quantize_token_groups(W.normal_bf16(1400, 0, 72, 192))
    qb, sb = oracle.quantize_blocks(W.normal_bf16(1401, 1, 192, 288, 0.02))
    say("gemm_tg both layouts")
    c_kn = gpu_gemm_tg(qa, sa_rows, qb, sb)
    c_nt = gpu_gemm_tg(qa, sa_rows, np.ascontiguousarray(qb.T), np.ascontiguousarray(sb.T), k_major=True)
    assert np.array_equal(c_kn, c_nt)
    for m in (70, 5):
        say(f"gemm_tg K=0 M={m}")
        c = gpu_gemm_tg(np.zeros((m, 0), np.uint8), np.zeros((m, 0), np.float32), np.zeros((0, 64), np.uint8),
                        np.zeros((0, 2), np.float32))
        assert c.shape == (m, 64) and np.all(c == 0)


@pytest.mark.parametrize("k_major", [False, True])
def test_chain_is_batch_invariant_end_to_end(k_major):
    """bf16 rows -> quantize_tg -> gemm_tg: a row computed alone (small-M
    kernel) or inside M = 320 (tile kernel) or M = 40 gives the same codes,
    scales and output bits."""
    a_bits = W.normal_bf16(1500, 0, 320, 256, 1.0, 0.01)
    qb, sb = oracle.quantize_blocks(W.normal_bf16(1501, 1, 256, 7168, 0.02))
    w, sw = (np.ascontiguousarray(qb.T), np.ascontiguousarray(sb.T)) if k_major else (qb, sb)
    say(f"chain full M=320 k_major={k_major}")
    qa, sa_rows = gpu_quantize_tg(a_bits)
    full = gpu_gemm_tg(qa, sa_rows, w, sw, k_major)
    for lo, hi in ((0, 40), (100, 101), (7, 8), (319, 320)):
        say(f"chain rows {lo}:{hi}")
        q1, s1 = gpu_quantize_tg(a_bits[lo:hi])
        assert np.array_equal(q1, qa[lo:hi]) and np.array_equal(s1, sa_rows[lo:hi])
        assert np.array_equal(gpu_gemm_tg(q1, s1, w, sw, k_major), full[lo:hi]), (lo, hi)


def test_decode_and_prefill_tg_full_size():
    """Decode K = 8192 (M = 64 and prefixes, both N, K-major weight) and
    prefill M = K = 8192, N = 10240 ([K, N] weight): every code and scale of A
    bit-exact, every element of C against the oracle, which quantizes both
    operands itself."""
    for N in (8192, 28672):
        wl = W.decode(64, N)
        a_bits, b_bits = wl.a_bits(), wl.b_bits()
        bt_bits = np.ascontiguousarray(b_bits.T)
        say(f"decode tg N={N}")
        qa, sa = fp8bs.quantize_tg(bf16_dev(a_bits))
        qbt, sbt = fp8bs.quantize(bf16_dev(bt_bits))
        c = fp8bs.gemm_tg_nt(qa, sa, qbt, sbt)
        torch.cuda.synchronize()
        for m in (1, 8, 32):
            cm = fp8bs.gemm_tg_nt(qa[:m].contiguous(), sa[:m].contiguous(), qbt, sbt)
            torch.cuda.synchronize()
            assert torch.equal(cm.view(torch.int16), c[:m].view(torch.int16)), f"N={N} M={m}"
        qa_o, sa_o = FU.quantize_full(a_bits, token_groups=True)
        FU.assert_same_codes(qa.cpu().numpy(), sa.cpu().numpy(), qa_o, sa_o, f"decode tg N={N} A")
        qbt_o, sbt_o = FU.quantize_full(bt_bits)
        FU.check_c_full(bits_np(c), FU.dequantize_full(qa_o, sa_o, token_groups=True),
                        bt_deq=FU.dequantize_full(qbt_o, sbt_o), label=f"decode tg N={N}")
        del qa, sa, qbt, sbt, c
        torch.cuda.empty_cache()
    wl = W.prefill(10240)
    a_bits, b_bits = wl.a_bits(), wl.b_bits()
    say("prefill tg N=10240")
    qa, sa = fp8bs.quantize_tg(bf16_dev(a_bits))
    qb, sb = fp8bs.quantize(bf16_dev(b_bits))
    c = fp8bs.gemm_tg(qa, sa, qb, sb)
    torch.cuda.synchronize()
    c_host = bits_np(c)
    qa_o, sa_o = FU.quantize_full(a_bits, token_groups=True)
    FU.assert_same_codes(qa.cpu().numpy(), sa.cpu().numpy(), qa_o, sa_o, "prefill tg A")
    qb_o, sb_o = FU.quantize_full(b_bits)
    del qa, sa, qb, sb, c
    torch.cuda.empty_cache()
    FU.check_c_full(c_host, FU.dequantize_full(qa_o, sa_o, token_groups=True), FU.dequantize_full(qb_o, sb_o),
                    label="prefill tg N=10240")
