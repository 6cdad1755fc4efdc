"""Host-side input generators (CPU only)."""

import numpy as np
import torch

from fp8_block_scaled_03_amd import workloads as W


def test_bf16_packing_matches_torch():
    g = np.random.default_rng(0)
    x = (g.standard_normal(100000) * np.exp2(g.integers(-60, 60, 100000))).astype(np.float32)
    ours = W.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_draws_are_reproducible_and_row_prefix_stable():
    a = W.normal_bf16(1003, W.T_A, 64, 256)
    b = W.normal_bf16(1003, W.T_A, 64, 256)
    assert np.array_equal(a, b)
    # decode workloads rely on this: the first M rows of the 64-row draw equal the M-row draw
    assert np.array_equal(W.normal_bf16(1003, W.T_A, 8, 256), a[:8])


def test_outliers_present_at_about_one_percent():
    x = W.normal_bf16(1002, W.T_A, 256, 1024, outlier_frac=0.01)
    xf = (x.astype(np.uint32) << 16).view(np.float32)
    frac = np.mean(np.abs(xf) > 6.0)            # N(0,1) alone essentially never exceeds 6
    assert 0.006 < frac < 0.012


def test_group_sizes():
    wl = W.grouped()
    off = wl.offsets()
    rows = np.diff(off)
    assert len(off) == 17 and off[0] == 0 and off[-1] == 8192
    assert np.all(rows % 32 == 0) and np.sum(rows == 0) >= 2
    assert np.array_equal(off, wl.offsets())


def test_workload_shapes():
    assert (W.square_256().M, W.square_256().N, W.square_256().K) == (256, 256, 256)
    assert W.square_4096().flops() == 2.0 * 4096 ** 3
    assert W.prefill(28672).N == 28672 and W.prefill(28672).a_outlier_frac == 0.01
    assert W.decode(8, 8192).M == 8 and W.decode(8, 8192).b_std == 0.02
