"""Benchmark of the E4M3 block-scaled GEMM hot path on one MI355X.

One step = one pass of the whole path over one batch: quantize the bf16
activations A and weights B to E4M3 with 32x32 block scales, then the
block-scaled GEMM to bf16 C, on the square 4096 x 4096 x 4096 workload (inputs
N(0,1), seeded, already resident in HBM).  `value` is 2*M*N*K per step over the
measured step time (TFLOP/s of the whole path).

"roofline" is the GEMM kernel of the timed steps: HIP events on the launch
stream around the GEMM launch of every timed step, their mean against
MI355X's dense FP8 MFMA peak.  `--roofline-only` runs just the warm-up and the
timed steps, so that a rocprofv3 kernel trace of it averages exactly those
launches.

Also measured (same run, reported under "detail"; median and min per entry):
  * the GEMM kernel alone, per launch with the caches flushed before each
    launch (a 1 GiB read), and the streaming-read rate of that flush read,
    which the decode rows are also reported against;
  * the square 256^3 workload in microseconds (GEMM alone and the whole step);
  * the prefill GEMM, M = K = 8192, N in {10240, 8192, 28672}, and the grouped
    GEMM (G = 16, K = 7168, N = 4096, 8192 rows);
  * the small-M (decode) GEMM at K=8192, M in {1, 8, 32, 64}, N in
    {8192, 28672}: algorithmic HBM bytes per launch over the kernel time;
  * the quantizer alone (HBM bytes per launch over its time);
  * the same for per-token-group (1 x 32) activation scales: quantizer, square
    GEMM and the decode sweep in both weight layouts;
  * the fused residual add + RMSNorm + token-group quantizer at d = 8192
    (8192 rows, and 1 / 8 / 64 rows);
  * power-of-two (E8M0) block scales, weight K-major: quantizer, the square
    and prefill GEMMs, decode M = 8 / 64;
  * the CPU oracle on a bounded sample of the same workload ("cpu_baseline").

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--quick]
       python bench.py --roofline-only      (the timed steps only, for the kernel trace)
       python bench.py --profile-kernels    (a short run for rocprofv3 counter passes)
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0           # MI355X HBM3E, GB/s
FP8_DENSE_PEAK_TFLOPS = 5000.0  # MI355X dense FP8 MFMA, TFLOP/s
BF16_DENSE_PEAK_TFLOPS = 2500.0
METRIC = "FP8 block-scaled GEMM TFLOPS & % MFMA peak @4096³; small-M HBM GB/s"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_gemm_tile_square4096.txt")
# An idle MI355X runs its first few hundred steps at a lower shader clock
# (measured with 20 timed steps: 676 TFLOP/s after 5 warm-up steps, 766 after
# 50, 804 after 100, 849 after 300).  Before the requested warm-up steps the
# step therefore runs, untimed, for at least this long, so that the timed
# steps measure the sustained rate whatever --warmup is.
PREWARM_SECONDS = 0.5


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)
    # untimed: about 20 ms of steps, enough for the clocks to settle (a 10-step
    # warm-up measured ~10% slower steps than the same steps a hundred later)
    p.add_argument("--warmup", type=int, default=100)
    p.add_argument("--reps", type=int, default=50, help="per-kernel timed launches (flushed)")
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--quick", action="store_true", help="fewer reps, no decode sweep (for profiling)")
    p.add_argument("--no-sclk", action="store_true",
                   help="skip the one-second shader-clock sample (for profiler runs: its back-to-back GEMMs "
                        "would dominate the kernel statistics)")
    p.add_argument("--profile-kernels", action="store_true",
                   help="run each kernel a few times without timing (for rocprofv3 counter passes)")
    p.add_argument("--roofline-only", action="store_true",
                   help="only the warm-up and timed steps and the JSON line (for the rocprofv3 kernel-trace "
                        "summary of the roofline kernel: every GEMM launch of the run is then a step launch)")
    return p.parse_args()


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the path has no multi-GPU mode (it shards along M or N "
              "with no exchange, so one GPU's share is the measured unit); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import fp8_block_scaled_03_amd as fp8bs
    from fp8_block_scaled_03_amd import probe
    from fp8_block_scaled_03_amd import workloads as W

    fp8bs.load_library()  # fail loudly before any work if the library is missing
    probe.load_probe_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)

    def to_dev_bf16(bits):
        return torch.from_numpy(bits.view(np.int16)).to(dev).view(torch.bfloat16)

    # Decode weights (K = 8192, N = 8192 and 28672; [K, N], K-major, and K-major
    # with E8M0 exponents) are allocated before anything else, as a model's
    # weights are at load time, and quantized once on first use.  A K-major
    # decode launch reads one K window of every weight row at once, so its
    # whole weight is in use concurrently: the same launch on a 235 MB weight
    # allocated after other large allocations had come and gone measured
    # about 30% slower (57 against 43.6 us at M = 8); the [K, N] layout and the
    # 67 MB weight showed no such difference.
    DEC_K = 8192
    dec_w = {}
    if not args.quick and not args.profile_kernels:
        for n_dec in (8192, 28672):
            for kind in ("kn", "nt", "e8m0"):
                shape = (DEC_K, n_dec) if kind == "kn" else (n_dec, DEC_K)
                sdt = torch.uint8 if kind == "e8m0" else torch.float32
                dec_w[(n_dec, kind)] = [torch.zeros(shape, dtype=torch.uint8, device=dev),
                                        torch.zeros((shape[0] // 32, shape[1] // 32), dtype=sdt, device=dev), False]

    def dec_weight(n_dec, kind):
        """The decode workload's weight, quantized into its start-up buffers once."""
        q, sc, done = dec_w[(n_dec, kind)]
        if not done:
            w_bits = W.decode(64, n_dec).b_bits()
            if kind != "kn":
                w_bits = np.ascontiguousarray(w_bits.T)
            x = to_dev_bf16(w_bits)
            (fp8bs.quantize_e8m0 if kind == "e8m0" else fp8bs.quantize)(x, q, sc)
            del x, w_bits
            dec_w[(n_dec, kind)][2] = True
        return q, sc

    # Cache flush between timed launches: READ 1 GiB (written once, here) with
    # the probe library's streaming read.  A read evicts L2 and the 256 MB
    # Infinity Cache and leaves only clean lines; a write flush would leave
    # dirty lines whose write-back then runs inside the next timed launch and
    # halves the bandwidth it sees.
    flush_buf = torch.ones(1 << 28, dtype=torch.int32, device=dev)
    FLUSH_WG = 256                      # one workgroup per CU read 1 GiB fastest
    flush_out = torch.empty(8 * 2048, dtype=torch.int32, device=dev)
    torch.cuda.synchronize()

    def flush():
        probe.stream_read(flush_buf, flush_out[:8 * FLUSH_WG], FLUSH_WG)

    def time_launch(fn, reps, do_flush=True):
        """Median and min per-launch time in ms, HIP events on the launch stream."""
        times = []
        for _ in range(reps):
            if do_flush:
                flush()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            e1.synchronize()
            times.append(e0.elapsed_time(e1))
        times.sort()
        return times[len(times) // 2], times[0], sum(times) / len(times)

    # ---- headline workload: square 4096^3
    wl = W.square_4096()
    M, N, K = wl.M, wl.N, wl.K
    a = to_dev_bf16(wl.a_bits())
    b = to_dev_bf16(wl.b_bits())
    qa = torch.empty((M, K), dtype=torch.uint8, device=dev)
    qb = torch.empty((K, N), dtype=torch.uint8, device=dev)
    sa = torch.empty((M // 32, K // 32), dtype=torch.float32, device=dev)
    sb = torch.empty((K // 32, N // 32), dtype=torch.float32, device=dev)
    c = torch.empty((M, N), dtype=torch.bfloat16, device=dev)

    def step():
        fp8bs.quantize(a, qa, sa)
        fp8bs.quantize(b, qb, sb)
        fp8bs.gemm(qa, sa, qb, sb, out=c)

    def gemm_only():
        fp8bs.gemm(qa, sa, qb, sb, out=c)

    if args.profile_kernels:
        for _ in range(3):
            step()
        torch.cuda.synchronize()
        # decode M=8 at both widths so both small-M kernel variants show up
        for n_dec in (8192, 28672):
            dwl = W.decode(8, n_dec)
            da = to_dev_bf16(dwl.a_bits())
            db = to_dev_bf16(dwl.b_bits())
            dqa, dsa = fp8bs.quantize(da)
            dqb, dsb = fp8bs.quantize(db)
            for _ in range(3):
                flush()
                fp8bs.gemm(dqa, dsa, dqb, dsb)
            del da, db, dqa, dsa, dqb, dsb
        # the same decode shapes with the weight K-major
        for n_dec in (8192, 28672):
            dwl = W.decode(8, n_dec)
            dqa, dsa = fp8bs.quantize(to_dev_bf16(dwl.a_bits()))
            dqbt, dsbt = fp8bs.quantize(to_dev_bf16(np.ascontiguousarray(dwl.b_bits().T)))
            for _ in range(3):
                flush()
                fp8bs.gemm_nt(dqa, dsa, dqbt, dsbt)
            del dqa, dsa, dqbt, dsbt
        # token-group activation scales on the square workload
        sa_tg = torch.empty((M, K // 32), dtype=torch.float32, device=dev)
        for _ in range(3):
            flush()
            fp8bs.quantize_tg(a, qa, sa_tg)
            flush()
            fp8bs.gemm_tg(qa, sa_tg, qb, sb, out=c)
        del sa_tg
        # fused residual add + RMSNorm + token-group quantizer, 8192 x 8192
        nwl = W.norm_prefill()
        nx, nr = to_dev_bf16(nwl.x_bits()), to_dev_bf16(nwl.residual_bits())
        ng = to_dev_bf16(nwl.gamma_bits())
        for _ in range(3):
            flush()
            fp8bs.rmsnorm_quantize_tg(nx, ng, nwl.eps, residual=nr)
        del nx, nr, ng
        # power-of-two (E8M0) scales: quantizer and GEMM on the square workload
        # (weight K-major), and decode M = 8 at N = 8192
        eqa, eea = fp8bs.quantize_e8m0(a)
        eqb, eeb = fp8bs.quantize_e8m0(to_dev_bf16(np.ascontiguousarray(wl.b_bits().T)))
        dwl = W.decode(8, 8192)
        dqa, dea = fp8bs.quantize_e8m0(to_dev_bf16(dwl.a_bits()))
        dqw, dew = fp8bs.quantize_e8m0(to_dev_bf16(np.ascontiguousarray(dwl.b_bits().T)))
        for _ in range(3):
            flush()
            fp8bs.quantize_e8m0(a, eqa, eea)
            flush()
            fp8bs.gemm_e8m0_nt(eqa, eea, eqb, eeb, out=c)
            flush()
            fp8bs.gemm_e8m0_nt(dqa, dea, dqw, dew)
        del eqa, eea, eqb, eeb, dqa, dea, dqw, dew
        # plain copy of known size, for scaling the HBM byte counters
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev).fill_(3)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"profile_kernels": "done", "copy_bytes": 256 << 20}))
        return

    # The GEMM launch of every timed step is bracketed by HIP events on the
    # launch stream; the roofline figure is their mean.  (Recording an event
    # costs the GPU nothing measurable; the step time is the wall clock.)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]

    def timed_step(i):
        fp8bs.quantize(a, qa, sa)
        fp8bs.quantize(b, qb, sb)
        ev[i][0].record(stream)
        fp8bs.gemm(qa, sa, qb, sb, out=c)
        ev[i][1].record(stream)

    prewarm_steps = 0
    t_pw = time.perf_counter()
    while time.perf_counter() - t_pw < PREWARM_SECONDS:
        for _ in range(20):
            step()
        prewarm_steps += 20
        torch.cuda.synchronize()
    prewarm_s = time.perf_counter() - t_pw
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        timed_step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    value = 2.0 * M * N * K / (ms_per_step * 1e-3) / 1e12
    step_gemm_ms = sorted(e0.elapsed_time(e1) for e0, e1 in ev)
    g_avg = sum(step_gemm_ms) / len(step_gemm_ms)

    gemm_flops = 2.0 * M * N * K
    # algorithmic bytes of one GEMM launch: A + B (E4M3) + both scale grids + C (bf16)
    gemm_bytes = M * K + K * N + 4 * (M // 32) * (K // 32) + 4 * (K // 32) * (N // 32) + 2 * M * N
    achieved = gemm_flops / (g_avg * 1e-3) / 1e12

    # HBM bytes per launch from the committed rocprofv3 counter summary, only
    # while the GEMM sources are the ones that were profiled
    from fp8_block_scaled_03_amd import profiling
    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        tr = profiling.read_traffic(TRAFFIC_FILE)
        if tr.get("source_sha") == profiling.source_sha():
            traffic = int(float(tr["hbm_bytes_per_launch"]))

    roofline = {"bound": "mfma", "achieved": round(achieved, 1), "peak": FP8_DENSE_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / FP8_DENSE_PEAK_TFLOPS, 4), "traffic": traffic,
                "kernel": "gemm_tile_kernel", "per_launch_flops": gemm_flops, "per_launch_alg_bytes": gemm_bytes,
                "avg_ms": round(g_avg, 5), "launches": len(step_gemm_ms),
                "timing": "HIP events around the GEMM launch of every timed step, on its stream"}
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "e4m3 (exact bf16 MFMA products, fp32 accumulation)",
        "data": "synthetic",
        "config": {"workload": "square-4096: quantize A, B (bf16 -> E4M3, 32x32 scales) + block-scaled GEMM",
                   "M": M, "N": N, "K": K, "block": 32, "seed": wl.seed},
        "roofline": roofline,
        "prewarm": {"steps": prewarm_steps, "seconds": round(prewarm_s, 3),
                    "what": "untimed steps run before the warm-up steps until the GPU holds its sustained clock"},
    }
    if args.roofline_only:
        print(json.dumps(out), flush=True)
        return

    reps = 10 if args.quick else args.reps

    def ms_entry(med, mn):
        return {"median": round(med, 5), "min": round(mn, 5)}

    # streaming-read ceilings of this GPU in this run: the 1 GiB flush read
    # itself, and a plain read of a decode weight's byte count after a flush
    flush()
    fl_med, fl_min, _ = time_launch(flush, 10, do_flush=False)
    stream_gbs = flush_buf.numel() * 4 / (fl_med * 1e-3) / 1e9

    def stream_ceiling(nbytes):
        """GB/s of a plain read of nbytes (a view of the flush buffer) with cold caches."""
        view = flush_buf[: nbytes // 4]
        best = None
        for wg in (512, 1024, 2048):
            med, _, _ = time_launch(lambda: probe.stream_read(view, flush_out[:8 * wg], wg), 10)
            best = med if best is None else min(best, med)
        return nbytes / (best * 1e-3) / 1e9

    # the exact recipe's instruction-mix ceiling (one 16x16x32 bf16 MFMA and
    # four fp32 FMAs per step, registers only), and the same steps' MFMAs alone
    # and FMAs alone: on gfx950 the mix takes about the sum of the two
    pc_wg, pc_iters = 512, 4000
    pc_out = torch.empty(pc_wg * 8, dtype=torch.float32, device=dev)
    pc_us = {}
    for mode in (0, 1, 2, 3):
        probe.promote_ceiling(pc_out, pc_wg, 200, mode)
        med, _, _ = time_launch(lambda mode=mode: probe.promote_ceiling(pc_out, pc_wg, pc_iters, mode), 5,
                                do_flush=False)
        pc_us[mode] = med * 1e3
    promote_ceiling_tflops = (pc_wg * 8 * pc_iters * 8 * probe.PROMOTE_CEILING_FLOPS_PER_STEP
                              / (pc_us[0] * 1e-6) / 1e12)
    # the same mix at two waves per SIMD (the tile kernel's occupancy): the
    # interleaved loop, then bursts of 2, 3, 4 and 6 MFMAs each followed by the
    # previous burst's FMAs; reported in nanoseconds per step and SIMD
    pc2_wg, pc2_steps = 256, 48000
    pc2_ns = {}
    for mode in (0, 4, 5, 6, 7):
        it = pc2_steps // probe.PROMOTE_STEPS_PER_ITER[mode]
        pc2_out = pc_out[:pc2_wg * 8]
        probe.promote_ceiling(pc2_out, pc2_wg, 200, mode)
        med, _, _ = time_launch(lambda mode=mode, it=it: probe.promote_ceiling(pc2_out, pc2_wg, it, mode), 5,
                                do_flush=False)
        pc2_ns[mode] = med * 1e6 / (pc2_wg * 8 * pc2_steps / 1024)
    # the burst orders at four waves per SIMD as well; the best rate over every
    # order and occupancy measured is the ceiling the GEMM is compared with
    pc4_ns = {}
    for mode in (4, 5, 6, 7):
        it = pc2_steps // probe.PROMOTE_STEPS_PER_ITER[mode]
        probe.promote_ceiling(pc_out, pc_wg, 200, mode)
        med, _, _ = time_launch(lambda mode=mode, it=it: probe.promote_ceiling(pc_out, pc_wg, it, mode), 5,
                                do_flush=False)
        pc4_ns[mode] = med * 1e6 / (pc_wg * 8 * pc2_steps / 1024)
    ns_to_tflops = lambda ns: probe.PROMOTE_CEILING_FLOPS_PER_STEP * 1024 / (ns * 1e-9) / 1e12
    mix_best_tflops = max([promote_ceiling_tflops] + [ns_to_tflops(v) for v in pc2_ns.values()]
                          + [ns_to_tflops(v) for v in pc4_ns.values()])
    # the hardware-scaled f8f6f4 MFMA alone (the power-of-two-scale contract's
    # instruction), 512 workgroups of eight waves
    probe.promote_ceiling(pc_out, pc_wg, 200, 8)
    sm_med, _, _ = time_launch(lambda: probe.promote_ceiling(pc_out, pc_wg, pc_iters, 8), 5, do_flush=False)
    scaled_mfma_tflops = pc_wg * 8 * pc_iters * 8 * probe.SCALED_MFMA_FLOPS / (sm_med * 1e-3) / 1e12

    for _ in range(5):
        gemm_only()
    g_med, g_min, g_favg = time_launch(gemm_only, reps)
    q_med, q_min, q_avg = time_launch(lambda: fp8bs.quantize(a, qa, sa), reps)

    detail = {
        "sclk_mhz_during_gemm": None if args.no_sclk else sample_sclk(gemm_only, torch),
        "gemm_in_step_ms": {"median": round(step_gemm_ms[len(step_gemm_ms) // 2], 5),
                            "min": round(step_gemm_ms[0], 5), "mean": round(g_avg, 5)},
        "gemm_flushed_ms": {"median": round(g_med, 5), "min": round(g_min, 5), "mean": round(g_favg, 5)},
        "gemm_flushed_tflops_median": round(gemm_flops / (g_med * 1e-3) / 1e12, 1),
        "gemm_frac_of_bf16_mfma_peak": round(achieved / BF16_DENSE_PEAK_TFLOPS, 4),
        "quantize_4096x4096_ms": ms_entry(q_med, q_min),
        "quantize_4096x4096_gbs": round(3.0 * M * K / (q_med * 1e-3) / 1e9, 1),
        "stream_read_ceiling": {"gbs": round(stream_gbs, 1), "frac_hbm_peak": round(stream_gbs / HBM_PEAK_GBS, 4),
                                "what": "the 1 GiB cache-flush read (probe streaming read), median of 10"},
        "promote_ceiling": {"tflops": round(promote_ceiling_tflops, 1),
                            "frac_fp8_peak": round(promote_ceiling_tflops / FP8_DENSE_PEAK_TFLOPS, 4),
                            "gemm_in_step_frac_of_it": round(achieved / promote_ceiling_tflops, 4),
                            "us_mix_mfma_only_fma_only_fp8mfma_only": [round(pc_us[m], 1) for m in (0, 1, 2, 3)],
                            "what": "registers-only loop of one 16x16x32 bf16 MFMA + four fp32 FMAs per step, "
                                    "512 workgroups of eight waves (4 waves per SIMD); also the same "
                                    "steps with the MFMAs alone, with the FMAs alone, and with the FP8 form of "
                                    "the MFMA alone",
                            "two_waves_per_simd_ns_per_step": {
                                "interleaved": round(pc2_ns[0], 3),
                                **{f"bursts_of_{probe.PROMOTE_BURSTS[m]}": round(pc2_ns[m], 3) for m in (4, 5, 6, 7)}},
                            "four_waves_per_simd_ns_per_step": {
                                f"bursts_of_{probe.PROMOTE_BURSTS[m]}": round(pc4_ns[m], 3) for m in (4, 5, 6, 7)},
                            "two_waves_what": "256 workgroups of eight waves; nanoseconds per step and SIMD "
                                              "(times the shader clock: cycles per step)",
                            "best_tflops": round(mix_best_tflops, 1),
                            "gemm_in_step_frac_of_best": round(achieved / mix_best_tflops, 4),
                            "best_what": "the fastest of every order and occupancy above: the exact recipe's "
                                         "instruction-mix ceiling",
                            "scaled_fp8_mfma_only_tflops": round(scaled_mfma_tflops, 1)},
    }

    # square 256^3 (quantize both operands + GEMM, and the GEMM alone): a
    # launch-latency-bound size, reported in microseconds
    s_wl = W.square_256()
    s_a, s_b = to_dev_bf16(s_wl.a_bits()), to_dev_bf16(s_wl.b_bits())
    s_qa, s_sa = fp8bs.quantize(s_a)
    s_qb, s_sb = fp8bs.quantize(s_b)
    s_c = torch.empty((256, 256), dtype=torch.bfloat16, device=dev)
    s_gemm = lambda: fp8bs.gemm(s_qa, s_sa, s_qb, s_sb, out=s_c)
    s_step = lambda: (fp8bs.quantize(s_a, s_qa, s_sa), fp8bs.quantize(s_b, s_qb, s_sb), s_gemm())
    for _ in range(5):
        s_step()
    sg_med, sg_min, _ = time_launch(s_gemm, reps)
    ss_med, ss_min, _ = time_launch(s_step, reps)
    detail["square_256"] = {"gemm_us": {"median": round(sg_med * 1e3, 2), "min": round(sg_min * 1e3, 2)},
                            "step_us": {"median": round(ss_med * 1e3, 2), "min": round(ss_min * 1e3, 2)}}
    del s_a, s_b, s_qa, s_sa, s_qb, s_sb, s_c

    weight_ceiling = {}

    def decode_entry(m, n_dec, k, nbytes, d_med, d_min):
        gbs = nbytes / (d_med * 1e-3) / 1e9
        if n_dec not in weight_ceiling:
            weight_ceiling[n_dec] = stream_ceiling(k * n_dec)
        return {"M": m, "N": n_dec, "K": k, "median_us": round(d_med * 1e3, 2), "min_us": round(d_min * 1e3, 2),
                "gbs": round(gbs, 1), "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
                "frac_stream_read": round(gbs / weight_ceiling[n_dec], 4)}

    if not args.quick:
        def decode_sweep(k_major, token_groups):
            """K = 8192, M in {1, 8, 32, 64} (prefixes of one 64-row A), both N:
            algorithmic bytes (codes, both scale grids, C) over the kernel time."""
            gemm = {(False, False): fp8bs.gemm, (True, False): fp8bs.gemm_nt,
                    (False, True): fp8bs.gemm_tg, (True, True): fp8bs.gemm_tg_nt}[(k_major, token_groups)]
            quant_a = fp8bs.quantize_tg if token_groups else fp8bs.quantize
            rows_out = []
            for n_dec in (8192, 28672):
                dwl = W.decode(64, n_dec)
                KB = dwl.K // 32
                q64, s64 = quant_a(to_dev_bf16(dwl.a_bits()))
                dqw, dsw = dec_weight(n_dec, "nt" if k_major else "kn")
                for m in (1, 8, 32, 64):
                    sa_rows = m if token_groups else (m + 31) // 32
                    dqa, dsa = q64[:m].contiguous(), s64[:sa_rows].contiguous()
                    dc = torch.empty((m, n_dec), dtype=torch.bfloat16, device=dev)
                    fn = (lambda dqa=dqa, dsa=dsa, dc=dc: gemm(dqa, dsa, dqw, dsw, out=dc))
                    for _ in range(3):
                        fn()
                    d_med, d_min, d_avg = time_launch(fn, reps)
                    nbytes = m * dwl.K + dwl.K * n_dec + 4 * sa_rows * KB + 4 * KB * (n_dec // 32) + 2 * m * n_dec
                    rows_out.append(decode_entry(m, n_dec, dwl.K, nbytes, d_med, d_min))
                del q64, s64, dqw, dsw
            return rows_out

        detail["decode_small_m"] = decode_sweep(False, False)
        detail["stream_read_ceiling"]["weight_gbs"] = {
            str(n): round(v, 1) for n, v in weight_ceiling.items()}
        detail["stream_read_ceiling"]["weight_what"] = ("a plain read of the decode weight's byte count (K x N) "
                                                        "after a flush, best of 512 / 1024 / 2048 workgroups; "
                                                        "the rows' frac_stream_read is against it")
        # the weight K-major (B^T [N, K], the layout of the pages' call
        # interface): each workgroup streams whole weight rows
        detail["decode_small_m_k_major_weight"] = decode_sweep(True, False)

        # per-token-group activation scales (1 x 32): quantizer, square GEMM, decode
        sa_tg = torch.empty((M, K // 32), dtype=torch.float32, device=dev)
        fp8bs.quantize_tg(a, qa, sa_tg)
        tq_med, tq_min, _ = time_launch(lambda: fp8bs.quantize_tg(a, qa, sa_tg), reps)
        tg_fn = lambda: fp8bs.gemm_tg(qa, sa_tg, qb, sb, out=c)
        for _ in range(3):
            tg_fn()
        tg_med, tg_min, tg_avg = time_launch(tg_fn, reps)
        detail["token_groups"] = {
            "quantize_tg_4096x4096_ms": ms_entry(tq_med, tq_min),
            "quantize_tg_4096x4096_gbs": round((2 * M * K + M * K + 4 * M * (K // 32)) / (tq_med * 1e-3) / 1e9, 1),
            "gemm_tg_4096_ms": ms_entry(tg_med, tg_min),
            "gemm_tg_4096_tflops_median": round(gemm_flops / (tg_med * 1e-3) / 1e12, 1),
            "decode_k_major_weight": decode_sweep(True, True),
            "decode": decode_sweep(False, True),
        }
        del sa_tg

        # fused residual add + RMSNorm + token-group quantizer, d = 8192: bytes =
        # x, residual in and out (bf16), codes, scales per row, gamma once
        norm = []
        for nwl in (W.norm_prefill(), W.norm_decode(64)):
            nx, nr = to_dev_bf16(nwl.x_bits()), to_dev_bf16(nwl.residual_bits())
            ng = to_dev_bf16(nwl.gamma_bits())
            nq = torch.empty((nwl.rows, nwl.d), dtype=torch.uint8, device=dev)
            ns = torch.empty((nwl.rows, nwl.d // 32), dtype=torch.float32, device=dev)
            for m in ((nwl.rows,) if nwl.rows > 64 else (1, 8, 64)):
                fn = (lambda m=m: fp8bs.rmsnorm_quantize_tg(nx[:m], ng, nwl.eps, residual=nr[:m], q=nq[:m],
                                                            scales=ns[:m]))
                for _ in range(3):
                    fn()
                n_med, n_min, _ = time_launch(fn, reps)
                nbytes = m * (7 * nwl.d + 4 * (nwl.d // 32)) + 2 * nwl.d
                norm.append({"rows": m, "d": nwl.d, "median_us": round(n_med * 1e3, 2),
                             "min_us": round(n_min * 1e3, 2),
                             "gbs": round(nbytes / (n_med * 1e-3) / 1e9, 1),
                             "frac_hbm_peak": round(nbytes / (n_med * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)})
            del nx, nr, ng, nq, ns
        detail["rmsnorm_residual_quantize_tg"] = norm

        # prefill M = K = 8192, N in {10240, 8192, 28672}, and the grouped
        # workload (GEMM only)
        pqa, psa = fp8bs.quantize(to_dev_bf16(W.prefill(8192).a_bits()))
        prefill = []
        for n_pre in (10240, 8192, 28672):
            pwl = W.prefill(n_pre)
            pqb, psb = fp8bs.quantize(to_dev_bf16(pwl.b_bits()))
            pc = torch.empty((pwl.M, pwl.N), dtype=torch.bfloat16, device=dev)
            pfn = lambda: fp8bs.gemm(pqa, psa, pqb, psb, out=pc)
            pfn()
            p_med, p_min, _ = time_launch(pfn, 20)
            prefill.append({"M": pwl.M, "N": n_pre, "K": pwl.K, "median_ms": round(p_med, 4),
                            "min_ms": round(p_min, 4), "tflops": round(pwl.flops() / (p_med * 1e-3) / 1e12, 1)})
            del pqb, psb, pc
        detail["prefill_K8192_M8192"] = prefill
        del pqa, psa
        gwl = W.grouped()
        off = gwl.offsets()
        gqa, gsa = fp8bs.quantize(to_dev_bf16(gwl.a_bits()))
        gqb2, gsb2 = fp8bs.quantize(to_dev_bf16(gwl.b_bits().reshape(gwl.groups * gwl.K, gwl.N)))
        gqb = gqb2.view(gwl.groups, gwl.K, gwl.N)
        gsb = gsb2.view(gwl.groups, gwl.K // 32, gwl.N // 32)
        goff = torch.from_numpy(off).to(dev)
        gc = torch.empty((gwl.M, gwl.N), dtype=torch.bfloat16, device=dev)
        gfn = lambda: fp8bs.grouped_gemm(gqa, gsa, gqb, gsb, goff, out=gc)
        gfn()
        g_med2, g_min2, _ = time_launch(gfn, 20)
        live = int(np.count_nonzero(np.diff(off)))
        detail["grouped_G16_M8192_K7168_N4096"] = {"median_ms": round(g_med2, 4), "min_ms": round(g_min2, 4),
                                                   "tflops": round(gwl.flops() / (g_med2 * 1e-3) / 1e12, 1),
                                                   "live_groups": live}
        del gqa, gsa, gqb2, gsb2, gc

        # power-of-two (E8M0) block scales on the hardware-scaled MFMA, weight
        # K-major: quantizer, the square and prefill GEMMs, decode M = 8 / 64
        e8 = {}
        bt_sq = np.ascontiguousarray(wl.b_bits().T)
        eqa, eea = fp8bs.quantize_e8m0(a)
        eqb, eeb = fp8bs.quantize_e8m0(to_dev_bf16(bt_sq))
        del bt_sq
        eq_med, eq_min, _ = time_launch(lambda: fp8bs.quantize_e8m0(a, eqa, eea), reps)
        e8["quantize_e8m0_4096x4096_ms"] = ms_entry(eq_med, eq_min)
        e8["quantize_e8m0_4096x4096_gbs"] = round((3 * M * K + (M // 32) * (K // 32)) / (eq_med * 1e-3) / 1e9, 1)
        efn = lambda: fp8bs.gemm_e8m0_nt(eqa, eea, eqb, eeb, out=c)
        for _ in range(3):
            efn()
        e_med, e_min, _ = time_launch(efn, reps)
        e8["gemm_e8m0_4096_ms"] = ms_entry(e_med, e_min)
        e8["gemm_e8m0_4096_tflops_median"] = round(gemm_flops / (e_med * 1e-3) / 1e12, 1)
        e8["gemm_e8m0_4096_frac_of_scaled_mfma_loop"] = round(gemm_flops / (e_med * 1e-3) / 1e12 / scaled_mfma_tflops, 4)
        del eqa, eea, eqb, eeb
        pwl = W.prefill(28672)
        pqa, pea = fp8bs.quantize_e8m0(to_dev_bf16(pwl.a_bits()))
        pqb, peb = fp8bs.quantize_e8m0(to_dev_bf16(np.ascontiguousarray(pwl.b_bits().T)))
        pc = torch.empty((pwl.M, pwl.N), dtype=torch.bfloat16, device=dev)
        pfn = lambda: fp8bs.gemm_e8m0_nt(pqa, pea, pqb, peb, out=pc)
        pfn()
        pe_med, pe_min, _ = time_launch(pfn, 20)
        e8["prefill_M8192_K8192_N28672"] = {"median_ms": round(pe_med, 4), "min_ms": round(pe_min, 4),
                                            "tflops": round(pwl.flops() / (pe_med * 1e-3) / 1e12, 1)}
        del pqa, pea, pqb, peb, pc
        e8_dec = []
        for n_dec in (8192, 28672):
            dwl = W.decode(64, n_dec)
            KB = dwl.K // 32
            q64, e64 = fp8bs.quantize_e8m0(to_dev_bf16(dwl.a_bits()))
            dqw, dew = dec_weight(n_dec, "e8m0")
            for m in (8, 64):
                ea_rows = (m + 31) // 32
                dqa, dea = q64[:m].contiguous(), e64[:ea_rows].contiguous()
                dc = torch.empty((m, n_dec), dtype=torch.bfloat16, device=dev)
                fn = (lambda dqa=dqa, dea=dea, dc=dc: fp8bs.gemm_e8m0_nt(dqa, dea, dqw, dew, out=dc))
                for _ in range(3):
                    fn()
                d_med, d_min, _ = time_launch(fn, reps)
                nbytes = m * dwl.K + dwl.K * n_dec + ea_rows * KB + KB * (n_dec // 32) + 2 * m * n_dec
                e8_dec.append(decode_entry(m, n_dec, dwl.K, nbytes, d_med, d_min))
            del q64, e64, dqw, dew
        e8["decode_k_major_weight"] = e8_dec
        detail["e8m0"] = e8

        # The same K-major decode launch (M = 8, N = 28672) on a copy of its
        # weight allocated now, after the run's other large allocations: the
        # placement sensitivity noted where the decode weights are allocated.
        lwl = W.decode(64, 28672)
        lq64, ls64 = fp8bs.quantize(to_dev_bf16(lwl.a_bits()))
        lqw, lsw = fp8bs.quantize(to_dev_bf16(np.ascontiguousarray(lwl.b_bits().T)))
        lqa, lsa = lq64[:8].contiguous(), ls64[:1].contiguous()
        lc = torch.empty((8, 28672), dtype=torch.bfloat16, device=dev)
        lfn = lambda: fp8bs.gemm_nt(lqa, lsa, lqw, lsw, out=lc)
        for _ in range(3):
            lfn()
        l_med, l_min, _ = time_launch(lfn, reps)
        lbytes = 8 * lwl.K + lwl.K * 28672 + 4 * (lwl.K // 32) + 4 * (lwl.K // 32) * (28672 // 32) + 2 * 8 * 28672
        detail["decode_k_major_weight_allocated_late"] = {
            "M": 8, "N": 28672, "K": lwl.K, "median_us": round(l_med * 1e3, 2), "min_us": round(l_min * 1e3, 2),
            "gbs": round(lbytes / (l_med * 1e-3) / 1e9, 1)}
        del lq64, ls64, lqw, lsw, lqa, lsa, lc

    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(wl)

    out["cpu_baseline"] = cpu
    out["detail"] = detail
    print(json.dumps(out), flush=True)


def current_sclk_mhz(table: str):
    """The level marked current ('*') in the driver's shader-clock table, in
    MHz (lines like '1: 2309Mhz *'; 'S: 95Mhz *' is the deep-sleep level), or
    None when no line is marked."""
    for line in table.splitlines():
        line = line.strip()
        if line.endswith("*") and ":" in line:
            value = line.split(":", 1)[1].rstrip("*").strip().lower()
            if value.endswith("mhz") and value[:-3].strip().isdigit():
                return int(value[:-3])
    return None


def sample_sclk(fn, torch, seconds=1.0):
    """Shader clock while `fn` runs back to back for about `seconds`: median of
    the current level read from the driver's sysfs clock table every 20 ms
    (after the first 0.3 s), or None where that file does not exist."""
    import glob
    import threading
    files = sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
    if not files:
        return None
    samples, stop = [], threading.Event()

    def read_current():
        with open(files[0]) as f:
            return current_sclk_mhz(f.read())

    def sampler():
        t_start = time.perf_counter()
        while not stop.is_set():
            v = read_current()
            if v is not None and time.perf_counter() - t_start > 0.3:
                samples.append(v)
            time.sleep(0.02)

    th = threading.Thread(target=sampler)
    th.start()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(20):
            fn()
        torch.cuda.synchronize()
    stop.set()
    th.join()
    if not samples:
        return None
    samples.sort()
    return {"median": samples[len(samples) // 2], "min": samples[0], "max": samples[-1], "samples": len(samples),
            "source": files[0]}


def cpu_baseline(wl):
    """The oracle, as it stands, on a bounded sample of the square-4096 step:
    quantize all of B and the first `rows` rows of A, then the fp64 reference for
    those rows x all columns.  Throughput is that sample's 2*rows*N*K over its
    wall time."""
    import oracle
    from threadpoolctl import threadpool_info

    rows = 4096
    a_bits = wl.a_bits()[:rows]
    b_bits = wl.b_bits()
    t0 = time.perf_counter()
    qa, sa = oracle.quantize_blocks(a_bits)
    qb, sb = oracle.quantize_blocks(b_bits)
    oracle.gemm_ref(qa, sa, qb, sb)
    dt = time.perf_counter() - t0
    info = threadpool_info()
    threads = max([i.get("num_threads", 1) for i in info] or [1])
    blas = [f"{i.get('internal_api')} {i.get('version')} ({i.get('threading_layer')}, {i.get('num_threads')} threads)"
            for i in info if i.get("user_api") == "blas"]
    return {"value": round(2.0 * rows * wl.N * wl.K / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle", "seconds": round(dt, 2), "blas": "; ".join(blas) or None,
            "sample": f"square-4096 step restricted to A rows 0..{rows - 1}: oracle quantize (A rows, all of B) "
                      f"+ fp64 reference GEMM {rows}x{wl.N}x{wl.K}",
            "host_cpus": len(os.sched_getaffinity(0))}


if __name__ == "__main__":
    main()
