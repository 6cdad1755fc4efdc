"""Parity at the full workload sizes, through the same entry points the bench
times (GPU quantize of A and B, then the GEMM), on sampled outputs.

The oracle never sees a GPU result as input: for every sampled 32x32 output
block it quantizes the bf16 row slab of A and column slab of B itself
(quantization is local to 32x32 blocks, so a slab quantizes exactly as it does
inside the whole matrix) and forms the fp64 reference of that block.  The GPU's
quantized slabs are also compared bit for bit with the oracle's.

Sizes: square 4096^3; prefill M = K = 8192 with N = 10240, 8192, 28672;
decode K = 8192, M in {1, 8, 32, 64}, N in {8192, 28672}; grouped G = 16,
K = 7168, N = 4096, 8192 rows.  Batch invariance at these sizes: decode rows
against the M = 64 rows, square-4096 rows against their M = 1 recomputation.
"""

import functools

import numpy as np
import pytest
import torch

import oracle
import fp8_block_scaled_03_amd as fp8bs
from fp8_block_scaled_03_amd import workloads as W

from gpu_util import DEV, bf16_dev, bits_np, bits_to_f64, say

pytestmark = pytest.mark.gpu


@functools.lru_cache(maxsize=2)
def _bits(name, which, *args):
    wl = getattr(W, name)(*args)
    return wl.a_bits() if which == "a" else wl.b_bits()


def _blocks(rng, n_blocks, count):
    """`count` distinct block indices out of n_blocks, always with the first and last."""
    pick = {0, n_blocks - 1}
    while len(pick) < min(count, n_blocks):
        pick.add(int(rng.integers(0, n_blocks)))
    return sorted(pick)


def _check_block(c_dev, a_bits, b_bits, qa_dev, sa_dev, qb_dev, sb_dev, rb, cb, label, row_limit=None):
    """Oracle-quantize the slabs of output block (rb, cb), compare the GPU's
    quantized slabs bitwise and the GPU's C block within the tolerance."""
    r0 = rb * 32
    r1 = min(r0 + 32, a_bits.shape[0] if row_limit is None else row_limit)
    cols = slice(cb * 32, cb * 32 + 32)
    qa_o, sa_o = oracle.quantize_blocks(a_bits[r0:r1])
    qb_o, sb_o = oracle.quantize_blocks(np.ascontiguousarray(b_bits[:, cols]))
    assert np.array_equal(qa_dev[r0:r1].cpu().numpy(), qa_o), f"{label}: A slab codes, row block {rb}"
    assert np.array_equal(sa_dev[rb:rb + 1].cpu().numpy(), sa_o), f"{label}: A slab scales, row block {rb}"
    assert np.array_equal(qb_dev[:, cols].cpu().numpy(), qb_o), f"{label}: B slab codes, column block {cb}"
    assert np.array_equal(sb_dev[:, cb:cb + 1].cpu().numpy(), sb_o), f"{label}: B slab scales, column block {cb}"
    ref, absref = oracle.gemm_ref(qa_o, sa_o, qb_o, sb_o)
    got = bits_to_f64(bits_np(c_dev[r0:r1, cols].contiguous()))
    ok = oracle.tolerance_ok(got, ref, absref)
    assert ok.all(), (f"{label}: block ({rb},{cb}) {int((~ok).sum())} outputs outside the bound, worst ratio "
                      f"{np.max(np.abs(got - ref) / oracle.tolerance_bound(ref, absref)):.3g}")


def _run_plain(a_bits, b_bits):
    a = bf16_dev(a_bits)
    b = bf16_dev(b_bits)
    qa, sa = fp8bs.quantize(a)
    qb, sb = fp8bs.quantize(b)
    c = fp8bs.gemm(qa, sa, qb, sb)
    torch.cuda.synchronize()
    del a, b
    return qa, sa, qb, sb, c


def test_square_4096_sampled_and_row_invariance():
    a_bits, b_bits = _bits("square_4096", "a"), _bits("square_4096", "b")
    say("fullsize square-4096 quantize + gemm")
    qa, sa, qb, sb, c = _run_plain(a_bits, b_bits)
    rng = np.random.default_rng(7)
    rbs, cbs = _blocks(rng, 128, 5), _blocks(rng, 128, 5)
    for rb in rbs:
        for cb in cbs:
            _check_block(c, a_bits, b_bits, qa, sa, qb, sb, rb, cb, "square-4096")
    for i in (0, 1, 2047, 4095):
        say(f"fullsize square-4096 row {i} alone (small-M kernel)")
        one = fp8bs.gemm(qa[i:i + 1].contiguous(), sa[i // 32:i // 32 + 1].contiguous(), qb, sb)
        torch.cuda.synchronize()
        assert torch.equal(one[0].view(torch.int16), c[i].view(torch.int16)), f"row {i}"


@pytest.mark.parametrize("N", [10240, 8192, 28672])
def test_prefill_sampled(N):
    a_bits, b_bits = _bits("prefill", "a", N), _bits("prefill", "b", N)
    say(f"fullsize prefill M=8192 K=8192 N={N} quantize + gemm")
    qa, sa, qb, sb, c = _run_plain(a_bits, b_bits)
    rng = np.random.default_rng(N)
    for rb in _blocks(rng, 256, 4):
        for cb in _blocks(rng, N // 32, 4):
            _check_block(c, a_bits, b_bits, qa, sa, qb, sb, rb, cb, f"prefill N={N}")
    del qa, sa, qb, sb, c
    torch.cuda.empty_cache()


@pytest.mark.parametrize("N", [8192, 28672])
def test_decode_sampled_and_prefix_invariance(N):
    wl = W.decode(64, N)
    a_bits, b_bits = wl.a_bits(), wl.b_bits()
    say(f"fullsize decode M=64 K=8192 N={N}")
    qa, sa, qb, sb, c = _run_plain(a_bits, b_bits)
    rng = np.random.default_rng(N + 1)
    for rb in (0, 1):
        for cb in _blocks(rng, N // 32, 6):
            _check_block(c, a_bits, b_bits, qa, sa, qb, sb, rb, cb, f"decode N={N}")
    for m in (1, 8, 32):
        say(f"fullsize decode prefix M={m} N={N}")
        cm = fp8bs.gemm(qa[:m].contiguous(), sa[:(m + 31) // 32].contiguous(), qb, sb)
        torch.cuda.synchronize()
        assert torch.equal(cm.view(torch.int16), c[:m].view(torch.int16)), f"M={m}"
    for i in (0, 13, 63):
        say(f"fullsize decode single row {i} N={N}")
        one = fp8bs.gemm(qa[i:i + 1].contiguous(), sa[i // 32:i // 32 + 1].contiguous(), qb, sb)
        torch.cuda.synchronize()
        assert torch.equal(one[0].view(torch.int16), c[i].view(torch.int16)), f"row {i}"


def test_grouped_sampled_and_single_gemm():
    wl = W.grouped()
    a_bits, b_bits, off = wl.a_bits(), wl.b_bits(), wl.offsets()
    G, K, N = wl.groups, wl.K, wl.N
    say(f"fullsize grouped G={G} K={K} N={N} offsets={off.tolist()}")
    a = bf16_dev(a_bits)
    b = bf16_dev(b_bits.reshape(G * K, N))
    qa, sa = fp8bs.quantize(a)
    qb2, sb2 = fp8bs.quantize(b)
    qb, sb = qb2.view(G, K, N), sb2.view(G, K // 32, N // 32)
    off_dev = torch.from_numpy(off).to(DEV)
    c = fp8bs.grouped_gemm(qa, sa, qb, sb, off_dev)
    torch.cuda.synchronize()
    del a, b
    rng = np.random.default_rng(44)
    live = [g for g in range(G) if off[g + 1] > off[g]]
    assert len(live) == G - 2
    for g in live:
        r0, r1 = int(off[g]), int(off[g + 1])
        rb = int(rng.integers(r0 // 32, r1 // 32))
        cb = int(rng.integers(0, N // 32))
        _check_block(c, a_bits, b_bits[g], qa, sa, qb[g], sb[g], rb, cb, f"grouped g={g}")
    for g in (live[0], live[-1]):
        r0, r1 = int(off[g]), int(off[g + 1])
        say(f"fullsize grouped group {g} as a single gemm")
        single = fp8bs.gemm(qa[r0:r1], sa[r0 // 32:r1 // 32], qb[g].contiguous(), sb[g].contiguous())
        torch.cuda.synchronize()
        assert torch.equal(single.view(torch.int16), c[r0:r1].view(torch.int16)), f"group {g}"
