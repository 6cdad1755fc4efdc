"""Which MFMA forms a 32-deep K-block partial P = sum_{k in block} dec(a) dec(b)
(DeepGEMM write-up on hncyxsy.com, section 2.2) accurately enough for the
acceptance bound: v_mfma_f32_16x16x32_bf16 on exactly decoded codes (what
every kernel of the library uses) against v_mfma_f32_16x16x32_fp8_fp8 on the
raw codes (the instruction the FP8 data type suggests).  Both run through the
plain probe GEMM (libfp8bs_probe.so), on the square-4096 workload's quantized
operands; the exact partials are integers in units of 2^-18.

What is asserted:
* the bf16 form's partials are within 7.5e-8 of the block's magnitude sum
  sum |a b| of the exact value, and its GEMM output is bitwise the library's;
* the FP8 form's partials miss by far more (over 100 times the bf16 form's
  worst), and its whole-output GEMM breaks the acceptance bound somewhere at
  4096^3 - the reason the library decodes to bf16 instead.
The FP8 form's violation rate is printed."""

import numpy as np
import pytest
import torch

import oracle
import fp8_block_scaled_03_amd as fp8bs
from fp8_block_scaled_03_amd import probe
from fp8_block_scaled_03_amd import workloads as W

import fullsize_util as FU
from gpu_util import bf16_dev, bits_np, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def square4096():
    wl = W.square_4096()
    a_bits, b_bits = wl.a_bits(), wl.b_bits()
    qa, sa = fp8bs.quantize(bf16_dev(a_bits))
    qb, sb = fp8bs.quantize(bf16_dev(b_bits))
    torch.cuda.synchronize()
    yield qa, sa, qb, sb
    del qa, sa, qb, sb
    torch.cuda.empty_cache()


def _exact_partials(qa, qb):
    """P[kb, i, j] and sum |a b| per K-block, exactly (fp64 holds integers < 2^53)."""
    ai = np.rint(oracle.decode_e4m3(qa) * 512).astype(np.int64)
    bi = np.rint(oracle.decode_e4m3(qb) * 512).astype(np.int64)
    KB = qa.shape[1] // 32
    P = np.empty((KB, qa.shape[0], qb.shape[1]))
    S = np.empty_like(P)
    for kb in range(KB):
        a, b = ai[:, 32 * kb:32 * kb + 32], bi[32 * kb:32 * kb + 32]
        P[kb] = (a @ b) / 2.0 ** 18
        S[kb] = (np.abs(a) @ np.abs(b)) / 2.0 ** 18
    return P, S


def test_partials_bf16_form_near_exact_fp8_form_not(square4096):
    qa, sa, qb, sb = square4096
    a, s_a = qa[:128].contiguous(), sa[:4].contiguous()
    b, s_b = qb[:, :128].contiguous(), sb[:, :4].contiguous()
    say("probe gemm with partials, bf16 and FP8 forms, 128 x 128 x 4096")
    c16, p16 = probe.gemm(a, s_a, b, s_b, fp8_form=False, with_partials=True)
    c8, p8 = probe.gemm(a, s_a, b, s_b, fp8_form=True, with_partials=True)
    c_lib = fp8bs.gemm(a, s_a, b, s_b)
    torch.cuda.synchronize()
    assert torch.equal(c16.view(torch.int16), c_lib.view(torch.int16)), "probe bf16 form != library GEMM"
    P, S = _exact_partials(a.cpu().numpy(), b.cpu().numpy())
    e16 = np.abs(p16.cpu().numpy() - P) / S
    e8 = np.abs(p8.cpu().numpy() - P) / S
    exact32 = P.astype(np.float32).astype(np.float64)
    say(f"  bf16 form: max |P - exact| / sum|ab| {e16.max():.3g}, correctly rounded "
        f"{np.mean(p16.cpu().numpy() == exact32):.5f}")
    say(f"  FP8 form:  max {e8.max():.3g}, mean {e8.mean():.3g}, correctly rounded "
        f"{np.mean(p8.cpu().numpy() == exact32):.5f}")
    assert e16.max() <= 7.5e-8
    assert e8.max() > 100 * e16.max()


def test_fp8_form_breaks_the_bound_at_4096(square4096):
    qa, sa, qb, sb = square4096
    say("probe gemm FP8 form, 4096^3")
    c8, _ = probe.gemm(qa, sa, qb, sb, fp8_form=True)
    torch.cuda.synchronize()
    c8_host = bits_np(c8)
    del c8
    a_deq = FU.dequantize_full(qa.cpu().numpy(), sa.cpu().numpy())
    b_deq = FU.dequantize_full(qb.cpu().numpy(), sb.cpu().numpy())
    bad = 0
    for c0 in range(0, 4096, 1024):
        ref = a_deq @ b_deq[:, c0:c0 + 1024]
        absref = np.abs(a_deq) @ np.abs(b_deq[:, c0:c0 + 1024])
        bad += int((~oracle.tolerance_ok(oracle.bf16_bits_to_f64(c8_host[:, c0:c0 + 1024]), ref, absref)).sum())
    say(f"  FP8 form: {bad} of {4096 * 4096} outputs outside the acceptance bound "
        f"({bad / 4096 ** 2:.2e}); the library's bf16 form: none (test_gpu_fullsize)")
    assert bad > 0
