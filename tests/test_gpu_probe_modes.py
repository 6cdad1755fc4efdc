"""The instruction-rate probes behind the bench's ceiling figures run on the
GPU in every mode (the exact recipe's mix of one bf16 MFMA and four fp32
FMAs per step, its parts, the burst orders, and the hardware-scaled f8f6f4
MFMA alone): every wave writes its sum, and two runs give the same bits.
The sums only keep the work alive; modes that feed raw bf16 bits to an FP8
instruction may legitimately produce NaN."""

import pytest
import torch

from fp8_block_scaled_03_amd import probe

from gpu_util import say

pytestmark = pytest.mark.gpu

SENTINEL = 0x7FC12345   # an fp32 NaN payload the probes never write


@pytest.mark.parametrize("mode", range(9))
def test_probe_mode_runs_and_repeats(mode):
    wg, iters = 4, 16
    outs = []
    for _ in range(2):
        out = torch.full((wg * 8,), SENTINEL, dtype=torch.int32, device="cuda").view(torch.float32)
        probe.promote_ceiling(out, wg, iters, mode)
        torch.cuda.synchronize()
        outs.append(out.view(torch.int32).cpu())
    say(f"  probe mode {mode}: first wave sums {outs[0][:2].view(torch.float32).tolist()}")
    assert not (outs[0] == SENTINEL).any(), f"mode {mode}: a wave wrote no sum"
    assert torch.equal(outs[0], outs[1]), f"mode {mode}: two runs differ"
    if mode not in (3, 8):   # bf16 and fp32 arithmetic on finite operands
        assert torch.isfinite(outs[0].view(torch.float32)).all(), f"mode {mode}: non-finite sum"
