"""Parity at the full workload sizes, every element, through the entry points
the bench times (GPU quantize of A and B, then the GEMM).

For each of the five workloads:
* every code and every scale that the GPU quantizer writes for A and B is
  compared bit for bit with the oracle's quantization of the same bf16 input;
* every element of C is held to the oracle's acceptance bound against the fp64
  reference formed from the oracle's own codes and scales (the oracle never
  takes a GPU result as input);
* batch invariance: decode rows at M = 1, 8, 32 (prefixes) and every row
  alone equal the M = 64 rows; 64 spread rows of the square and prefill
  workloads equal their M = 1 recomputation; every live group of the grouped
  workload equals a single GEMM on its rows.

Sizes: square 256^3 and 4096^3; prefill M = K = 8192 with N = 10240, 8192,
28672; decode K = 8192, M in {1, 8, 32, 64}, N in {8192, 28672}; grouped
G = 16, K = 7168, N = 4096, 8192 rows.
"""

import numpy as np
import pytest
import torch

import fp8_block_scaled_03_amd as fp8bs
from fp8_block_scaled_03_amd import workloads as W

import fullsize_util as FU
from gpu_util import DEV, bf16_dev, bits_np, say

pytestmark = pytest.mark.gpu


def _gpu_quantize(bits):
    q, s = fp8bs.quantize(bf16_dev(bits))
    torch.cuda.synchronize()
    return q, s


def _oracle_operand(bits, q_dev, s_dev, label):
    """Oracle codes and scales of `bits`, compared bitwise with the GPU's;
    returns the oracle's dequantized operand (fp64)."""
    say(f"{label}: oracle quantize {bits.shape}")
    q_o, s_o = FU.quantize_full(bits)
    FU.assert_same_codes(q_dev.cpu().numpy(), s_dev.cpu().numpy(), q_o, s_o, label)
    return FU.dequantize_full(q_o, s_o)


def _rows_alone(qa, sa, qb, sb, c, rows, label):
    for i in rows:
        one = fp8bs.gemm(qa[i:i + 1].contiguous(), sa[i // 32:i // 32 + 1].contiguous(), qb, sb)
        torch.cuda.synchronize()
        assert torch.equal(one[0].view(torch.int16), c[i].view(torch.int16)), f"{label}: row {i} alone"


def _plain_full(wl_a_bits, wl_b_bits, label, a_deq=None, spread=64):
    qa, sa = _gpu_quantize(wl_a_bits)
    qb, sb = _gpu_quantize(wl_b_bits)
    say(f"{label}: gemm {qa.shape[0]}x{qb.shape[1]}x{qa.shape[1]}")
    c = fp8bs.gemm(qa, sa, qb, sb)
    torch.cuda.synchronize()
    c_host = bits_np(c)
    if a_deq is None:
        a_deq = _oracle_operand(wl_a_bits, qa, sa, f"{label} A")
    b_deq = _oracle_operand(wl_b_bits, qb, sb, f"{label} B")
    say(f"{label}: whole-output check")
    FU.check_c_full(c_host, a_deq, b_deq, label=label)
    del b_deq
    if spread:
        say(f"{label}: {spread} rows alone")
        _rows_alone(qa, sa, qb, sb, c, FU.spread_rows(qa.shape[0], spread, seed=qa.shape[0] + qb.shape[1]), label)
    return qa, sa, qb, sb, c


def test_square_256_full():
    wl = W.square_256()
    _plain_full(wl.a_bits(), wl.b_bits(), "square-256", spread=256)


def test_square_4096_full_and_row_invariance():
    wl = W.square_4096()
    _plain_full(wl.a_bits(), wl.b_bits(), "square-4096")
    torch.cuda.empty_cache()


@pytest.fixture(scope="module")
def prefill_a():
    """The prefill activations do not depend on N: draw, quantize (GPU and
    oracle) and dequantize them once for the three N."""
    bits = W.prefill(8192).a_bits()
    qa, sa = _gpu_quantize(bits)
    a_deq = _oracle_operand(bits, qa, sa, "prefill A")
    del qa, sa
    torch.cuda.empty_cache()
    yield bits, a_deq


@pytest.mark.parametrize("N", [10240, 8192, 28672])
def test_prefill_full_and_row_invariance(N, prefill_a):
    a_bits, a_deq = prefill_a
    _plain_full(a_bits, W.prefill(N).b_bits(), f"prefill N={N}", a_deq=a_deq)
    torch.cuda.empty_cache()


@pytest.mark.parametrize("N", [8192, 28672])
def test_decode_full_and_prefix_invariance(N):
    wl = W.decode(64, N)
    qa, sa, qb, sb, c = _plain_full(wl.a_bits(), wl.b_bits(), f"decode N={N}", spread=0)
    for m in (1, 8, 32):
        say(f"decode N={N}: prefix M={m}")
        cm = fp8bs.gemm(qa[:m].contiguous(), sa[:(m + 31) // 32].contiguous(), qb, sb)
        torch.cuda.synchronize()
        assert torch.equal(cm.view(torch.int16), c[:m].view(torch.int16)), f"M={m}"
    say(f"decode N={N}: every row alone")
    _rows_alone(qa, sa, qb, sb, c, range(64), f"decode N={N}")
    torch.cuda.empty_cache()


def test_grouped_full_and_single_gemm():
    wl = W.grouped()
    a_bits, b_bits, off = wl.a_bits(), wl.b_bits(), wl.offsets()
    G, K, N = wl.groups, wl.K, wl.N
    say(f"grouped G={G} K={K} N={N} offsets={off.tolist()}")
    qa, sa = _gpu_quantize(a_bits)
    qb2, sb2 = _gpu_quantize(b_bits.reshape(G * K, N))
    qb, sb = qb2.view(G, K, N), sb2.view(G, K // 32, N // 32)
    off_dev = torch.from_numpy(off).to(DEV)
    c = fp8bs.grouped_gemm(qa, sa, qb, sb, off_dev)
    torch.cuda.synchronize()
    c_host = bits_np(c)
    a_deq = _oracle_operand(a_bits, qa, sa, "grouped A")
    b_deq = _oracle_operand(b_bits.reshape(G * K, N), qb2, sb2, "grouped B").reshape(G, K, N)
    live = [g for g in range(G) if off[g + 1] > off[g]]
    assert len(live) == G - 2
    for g in live:
        r0, r1 = int(off[g]), int(off[g + 1])
        say(f"grouped g={g}: rows {r0}:{r1} whole-output check")
        FU.check_c_full(c_host[r0:r1], a_deq[r0:r1], b_deq[g], label=f"grouped g={g}")
        single = fp8bs.gemm(qa[r0:r1], sa[r0 // 32:r1 // 32], qb[g].contiguous(), sb[g].contiguous())
        torch.cuda.synchronize()
        assert torch.equal(single.view(torch.int16), c[r0:r1].view(torch.int16)), f"group {g}"
