/*
 * fp8bs_probe.h - measurement and test support for libfp8bs (gfx950).
 *
 * These calls live in their own library, libfp8bs_probe.so.  No entry point
 * of fp8bs.h uses them; they expose single gfx950 instructions so that the
 * tests can check the instruction choices the library makes and the bench
 * can measure the ceiling of its arithmetic.
 *
 * Source pages cited below:
 *   [DG]  the featured DeepGEMM FP8 write-up on hncyxsy.com (news item 241433)
 *
 * Conventions: device pointers owned by the caller, row-major, E4M3 = OCP
 * E4M3FN bytes; work is enqueued on `stream` (hipStream_t, NULL = the null
 * stream) and nothing synchronizes.  Return value: 0 = enqueued, 1 = a null
 * pointer, 2 = a size out of range, 4 = the launch failed.  Nothing is
 * checked on the device (buffers must be as large as stated).
 */
#ifndef FP8BS_PROBE_H
#define FP8BS_PROBE_H

#ifdef __cplusplus
extern "C" {
#endif

/*
 * fp8bs_probe_gemm - the block-scaled GEMM of fp8bs_gemm, written plainly
 * (one wave per 16x16 tile of C, operands read from global memory), with a
 * choice of the instruction that forms each 32-deep K-block partial
 * P = sum_{k in block} dec(a_ik) dec(b_kj) [DG 2.2]:
 *   fp8_form == 0: v_mfma_f32_16x16x32_bf16 on the exactly decoded codes
 *                  (the instruction every fp8bs kernel uses);
 *   fp8_form != 0: v_mfma_f32_16x16x32_fp8_fp8 on the raw codes.
 * Promotion is fp8bs_gemm's: s = RN32(sa * sb), acc = fma(P, s, acc), K-blocks
 * ascending; C = bf16(acc), round to nearest even, zero stored as +0.
 *   a [M, K] E4M3, sa [M/32, K/32] fp32, b [K, N] E4M3, sb [K/32, N/32] fp32,
 *   c [M, N] bf16 out; partials (may be NULL) [K/32, M, N] fp32 out: P of
 *   every element and K-block.  M, N, K > 0 and multiples of 32 (else 2).
 */
int fp8bs_probe_gemm(const void* a, const float* sa, const void* b, const float* sb, void* c, float* partials,
                     int M, int N, int K, int fp8_form, void* stream);

/*
 * fp8bs_probe_mfma_scale - `count` independent single
 * v_mfma_scale_f32_16x16x128_f8f6f4 instructions (E4M3 operands, E8M0 scale
 * bytes per row and 32-deep K-block).  For problem q and m, n in [0, 16):
 *   d[q][m][n] = cin[q][m][n] + sum_{k<128} dec(a[q][m][k]) 2^(ea[q][m][k/32] - 127)
 *                                          * dec(bt[q][n][k]) 2^(eb[q][n][k/32] - 127)
 * as the instruction computes it (its own summation and rounding).
 *   a, bt [count][16][128] E4M3; ea, eb [count][16][4] E8M0 bytes;
 *   cin, d [count][16][16] fp32.  a, bt 16-byte aligned.  count > 0.
 */
int fp8bs_probe_mfma_scale(const void* a, const void* bt, const void* ea, const void* eb, const float* cin,
                           float* d, int count, void* stream);

/*
 * fp8bs_probe_promote_ceiling - `workgroups` workgroups of eight waves run
 * `iters` x 8 steps each of the exact recipe's instruction mix, registers
 * only: one v_mfma_f32_16x16x32_bf16 (16384 flops) and four fp32 FMAs that
 * promote a partial formed four steps earlier [DG 2.2-2.3].  Its rate bounds
 * any kernel that forms every 32-deep partial with that MFMA and promotes it
 * with non-packed fp32 FMAs.  mode 0: that mix; mode 1: the MFMAs alone;
 * mode 2: the FMAs alone (the same counts), so that the three rates show how
 * far the two kinds of work overlap; mode 3: v_mfma_f32_16x16x32_fp8_fp8
 * alone, the FP8 form of the same partial.  Modes 4-7 run the mix in bursts
 * of 2, 3, 4 and 6 MFMAs, each followed by the FMAs that promote the previous
 * burst's partials, `iters` x 12 steps (iters even).  Mode 8 runs
 * v_mfma_scale_f32_16x16x128_f8f6f4 alone on E4M3 operands with unit
 * scales (65536 flops each), `iters` x 8 instructions per wave: the rate of
 * the power-of-two-scale contract.  out [workgroups * 8] fp32 (one value per
 * wave, written so that nothing is dead code).  workgroups, iters > 0, mode
 * in 0..8; 2 for any other value.
 */
int fp8bs_probe_promote_ceiling(float* out, int workgroups, int iters, int mode, void* stream);

/*
 * fp8bs_probe_stream_read - read `bytes` of `buf` once (16-byte loads,
 * grid-strided, eight per thread in flight) with `workgroups` workgroups of
 * 512 threads; the rate of a plain streaming read, the ceiling of the
 * memory-bound kernels.  out [workgroups * 8] (one xor fold per wave).
 * bytes > 0 and a multiple of 16; buf 16-byte aligned.
 */
int fp8bs_probe_stream_read(const void* buf, long long bytes, unsigned* out, int workgroups, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FP8BS_PROBE_H */
