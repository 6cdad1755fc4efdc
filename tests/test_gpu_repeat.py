"""Run-to-run determinism: the same inputs give the same output bits on every
call ("AI Infra 进阶：如何让大模型输出确定的结果", part 一: a fixed reduction
order makes a result reproducible, not only batch invariant).  Every kernel
family runs six times back to back on one set of inputs, with a fresh output
buffer filled with a sentinel each time, and every run must equal the first
bit for bit (and no sentinel may survive).  The shapes put each kernel under
full load: all CUs busy, several waves per SIMD, so that scheduling differs
between runs."""

import numpy as np
import pytest
import torch

import fp8_block_scaled_03_amd as fp8bs
from fp8_block_scaled_03_amd import workloads as W

from gpu_util import bf16_dev, i32_dev, say

pytestmark = pytest.mark.gpu

RUNS = 6
SENTINEL = 0x7FC1   # a bf16 NaN no kernel writes


def _repeat(label, fn, shape):
    first = None
    for r in range(RUNS):
        out = torch.full(shape, SENTINEL, dtype=torch.int16, device="cuda").view(torch.bfloat16)
        fn(out)
        torch.cuda.synchronize()
        bits = out.view(torch.int16)
        assert not torch.any(bits == SENTINEL), f"{label}: run {r} left outputs unwritten"
        if first is None:
            first = bits.clone()
        else:
            diff = int((bits != first).sum())
            assert diff == 0, f"{label}: run {r} differs from run 0 in {diff} outputs"
    say(f"  {label}: {RUNS} runs bitwise identical")


@pytest.fixture(scope="module")
def square():
    wl = W.square_4096()
    a, b = bf16_dev(wl.a_bits()), bf16_dev(wl.b_bits())
    qa, sa = fp8bs.quantize(a)
    qb, sb = fp8bs.quantize(b)
    qbt, sbt = fp8bs.quantize(bf16_dev(np.ascontiguousarray(wl.b_bits().T)))
    qa_tg, sa_tg = fp8bs.quantize_tg(a)
    torch.cuda.synchronize()
    yield dict(qa=qa, sa=sa, qb=qb, sb=sb, qbt=qbt, sbt=sbt, qa_tg=qa_tg, sa_tg=sa_tg)
    torch.cuda.empty_cache()


def test_tile_kernels_repeat(square):
    s = square
    say("repeat: 4096^3 tile kernel, both weight layouts, token groups")
    _repeat("gemm", lambda o: fp8bs.gemm(s["qa"], s["sa"], s["qb"], s["sb"], out=o), (4096, 4096))
    _repeat("gemm_nt", lambda o: fp8bs.gemm_nt(s["qa"], s["sa"], s["qbt"], s["sbt"], out=o), (4096, 4096))
    _repeat("gemm_tg", lambda o: fp8bs.gemm_tg(s["qa_tg"], s["sa_tg"], s["qb"], s["sb"], out=o), (4096, 4096))
    # M = 3904: the last M-tile holds 64 rows and runs the light body
    _repeat("gemm M=3904", lambda o: fp8bs.gemm(s["qa"][:3904], s["sa"][:122], s["qb"], s["sb"], out=o), (3904, 4096))


def test_small_m_kernels_repeat(square):
    s = square
    say("repeat: decode shapes, both weight layouts")
    for m in (1, 8, 64):
        _repeat(f"gemm M={m}", lambda o, m=m: fp8bs.gemm(s["qa"][:m], s["sa"][:-(-m // 32)], s["qb"], s["sb"], out=o),
                (m, 4096))
        _repeat(f"gemm_nt M={m}",
                lambda o, m=m: fp8bs.gemm_nt(s["qa"][:m], s["sa"][:-(-m // 32)], s["qbt"], s["sbt"], out=o),
                (m, 4096))


def test_grouped_repeat():
    wl = W.grouped()
    off = wl.offsets()
    qa, sa = fp8bs.quantize(bf16_dev(wl.a_bits()))
    b_bits = wl.b_bits()
    qb2, sb2 = fp8bs.quantize(bf16_dev(b_bits.reshape(wl.groups * wl.K, wl.N)))
    qb = qb2.view(wl.groups, wl.K, wl.N)
    sb = sb2.view(wl.groups, wl.K // 32, wl.N // 32)
    qbt2, sbt2 = fp8bs.quantize(bf16_dev(np.ascontiguousarray(b_bits.transpose(0, 2, 1)).reshape(wl.groups * wl.N, wl.K)))
    qbt = qbt2.view(wl.groups, wl.N, wl.K)
    sbt = sbt2.view(wl.groups, wl.N // 32, wl.K // 32)
    doff = i32_dev(off)
    say("repeat: grouped workload, both weight layouts")
    _repeat("grouped", lambda o: fp8bs.grouped_gemm(qa, sa, qb, sb, doff, out=o), (wl.M, wl.N))
    _repeat("grouped_nt", lambda o: fp8bs.grouped_gemm_nt(qa, sa, qbt, sbt, doff, out=o), (wl.M, wl.N))


def test_e8m0_kernels_repeat():
    wl = W.square_4096()
    qa, ea = fp8bs.quantize_e8m0(bf16_dev(wl.a_bits()))
    qbt, ebt = fp8bs.quantize_e8m0(bf16_dev(np.ascontiguousarray(wl.b_bits().T)))
    say("repeat: E8M0 GEMM, 256x256 / 128x128 / small-M kernels")
    _repeat("gemm_e8m0 4096^3", lambda o: fp8bs.gemm_e8m0_nt(qa, ea, qbt, ebt, out=o), (4096, 4096))
    _repeat("gemm_e8m0 M=1024", lambda o: fp8bs.gemm_e8m0_nt(qa[:1024], ea[:32], qbt, ebt, out=o), (1024, 4096))
    _repeat("gemm_e8m0 M=8", lambda o: fp8bs.gemm_e8m0_nt(qa[:8], ea[:1], qbt, ebt, out=o), (8, 4096))
