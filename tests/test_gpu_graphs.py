"""The entry points under HIP graph capture.

The grouped GEMM reads its row offsets from device memory, so one captured
graph serves every grouping: the DeepGEMM write-up (section 4.3) makes the
shape table device-resident for exactly this.  Each replay is checked against
an eager call on the same inputs, with eager work and synchronizations between
the replays; nothing captured records a memset."""

import numpy as np
import pytest
import torch

import oracle
import fp8_block_scaled_03_amd as fp8bs
from fp8_block_scaled_03_amd import workloads as W

from gpu_util import DEV, bf16_dev, bits_np, f32_dev, i32_dev, say, u8_dev

pytestmark = pytest.mark.gpu


def _capture(fn):
    """Warm up on a side stream, then capture fn() into a graph."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("k_major", [False, True])
def test_grouped_graph_follows_device_offsets(k_major):
    G, K, N = 4, 128, 96
    groupings = [np.array([64, 0, 96, 32]), np.array([32, 128, 0, 32]), np.array([0, 0, 0, 192])]
    M = 192
    qa, sa = oracle.quantize_blocks(W.normal_bf16(3000, 0, M, K))
    qbs = [oracle.quantize_blocks(W.normal_bf16(3001 + i, 1, K, N, 0.02)) for i in range(G)]
    qb = np.stack([q for q, _ in qbs])
    sb = np.stack([s for _, s in qbs])
    if k_major:
        qb, sb = np.ascontiguousarray(qb.transpose(0, 2, 1)), np.ascontiguousarray(sb.transpose(0, 2, 1))
    fn_raw = fp8bs.grouped_gemm_nt if k_major else fp8bs.grouped_gemm
    da, dsa, db, dsb = u8_dev(qa), f32_dev(sa), u8_dev(qb), f32_dev(sb)
    off_dev = i32_dev(W.offsets_from_rows(groupings[0]))
    c = torch.zeros((M, N), dtype=torch.bfloat16, device=DEV)

    eager = []
    for rows in groupings:
        say(f"grouped eager rows={rows.tolist()} k_major={k_major}")
        e = fn_raw(da, dsa, db, dsb, i32_dev(W.offsets_from_rows(rows)))
        torch.cuda.synchronize()
        eager.append(bits_np(e))

    say("grouped capture")
    graph = _capture(lambda: fn_raw(da, dsa, db, dsb, off_dev, out=c))
    for rep in range(2):
        for i, rows in enumerate(groupings):
            say(f"grouped replay {rep} rows={rows.tolist()}")
            off_dev.copy_(torch.from_numpy(W.offsets_from_rows(rows)).to(DEV))
            c.zero_()
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            assert np.array_equal(bits_np(c), eager[i]), (rep, rows.tolist())


def test_norm_quantize_gemm_chain_graph_replays():
    """Residual add + RMSNorm + token-group quantizer, then the token-group GEMM
    on a K-major weight, captured once: every replay equals the eager chain
    bit for bit (the residual is reset before each run)."""
    rows, d, N = 40, 1024, 2048
    x = bf16_dev(W.normal_bf16(3100, 0, rows, d, 1.0, 0.01))
    r0 = bf16_dev(W.normal_bf16(3100, 5, rows, d))
    gam = bf16_dev(W.f32_to_bf16_bits(1.0 + 0.1 * W.rng_for(3100, 6).standard_normal(d).astype(np.float32)))
    qw, sw = oracle.quantize_blocks(W.normal_bf16(3101, 1, N, d, 0.02))
    wt, swt = u8_dev(qw), f32_dev(sw)
    res = r0.clone()
    q = torch.empty((rows, d), dtype=torch.uint8, device=DEV)
    s = torch.empty((rows, d // 32), dtype=torch.float32, device=DEV)
    c = torch.empty((rows, N), dtype=torch.bfloat16, device=DEV)

    def chain():
        fp8bs.rmsnorm_quantize_tg(x, gam, 1e-6, residual=res, q=q, scales=s)
        fp8bs.gemm_tg_nt(q, s, wt, swt, out=c)

    say("chain eager")
    res.copy_(r0)
    chain()
    torch.cuda.synchronize()
    want_c, want_res = bits_np(c), bits_np(res)
    say("chain capture")
    res.copy_(r0)
    graph = _capture(chain)
    for rep in range(3):
        say(f"chain replay {rep}")
        res.copy_(r0)
        c.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bits_np(c), want_c), rep
        assert np.array_equal(bits_np(res), want_res), rep
