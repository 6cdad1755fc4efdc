/*
 * fp8bs.h - C ABI of the FP8 (E4M3) GEMM with 32x32 block scales, for AMD
 * MI355X (gfx950).
 *
 * Source pages cited below:
 *   [DG]  the featured DeepGEMM FP8 write-up on hncyxsy.com (news item 241433)
 *   [DET] "AI Infra 进阶：如何让大模型输出确定的结果" (aif.amtbbs.org, post 29992)
 *
 * Conventions shared by every entry point
 *   - All pointers are DEVICE pointers owned by the caller (the library
 *     allocates nothing and keeps no state besides its code object).
 *   - Matrices are dense row-major.  E4M3 means OCP E4M3FN bytes (bias 7, no
 *     infinity, 0x7F/0xFF NaN, largest finite 448) [DG 2.1].  bf16 means the
 *     upper 16 bits of an IEEE fp32.  Scale grids are row-major fp32.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream)
 *     and runs asynchronously; nothing synchronizes.  Calls are reentrant.
 *   - Argument checks happen on the host before any launch; a non-OK status
 *     means nothing was enqueued (except FP8BS_EHIP, returned when the launch
 *     itself failed).  No exception or abort crosses the ABI.
 *   - Device-side preconditions that are NOT checked: inputs finite, scales
 *     finite, outputs not aliasing inputs, buffers as large as stated.
 *   - Results are batch invariant [DET part 一, sections 6-7]: an element of C
 *     depends only on its row of A, its column of B and the scales, never on
 *     M, on the row's position in the batch or on which kernel ran.  K is
 *     never split; the 32-deep K-blocks are accumulated in ascending order.
 */
#ifndef FP8BS_H
#define FP8BS_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FP8BS_OK = 0,
  FP8BS_EINVAL = 1, /* null pointer with a non-zero size, negative size, bad G  */
  FP8BS_ESHAPE = 2, /* a dimension that must be a multiple of 32 is not, or a
                       dimension is too large                                  */
  FP8BS_EALIGN = 3, /* a matrix pointer not 16-byte aligned, or a scale/offset
                       pointer not 4-byte aligned                              */
  FP8BS_EHIP = 4,   /* the HIP runtime reported an error at launch              */
  FP8BS_ENOSYS = 5  /* not built for this device                               */
} fp8bs_status;

/* Largest accepted group count for fp8bs_grouped_gemm. */
#define FP8BS_MAX_GROUPS 1024

/*
 * fp8bs_quantize - bf16 -> E4M3 with one fp32 scale per 32x32 block.
 *   [DG 2.2]: one scale per 32x32 block; [DG 5.2]: scale from the block's
 *   absolute maximum; [DG 2.1]: E4M3 tops out at 448.
 *   For block (rb, cb) covering rows [32rb, min(32rb+32, rows)) and columns
 *   [32cb, 32cb+32):
 *     amax = max |x| over the block;   s = amax / 448   (fp32, round to nearest)
 *     s == 0:  every code of the block is 0x00
 *     else:    q = E4M3(x / s), the quotient taken in fp32 (round to nearest)
 *              and then rounded to E4M3 with ties to even, clamped to +-448,
 *              sign kept (so -0 and negative underflow give 0x80).
 *   x      [rows, cols]              bf16, 16-byte aligned
 *   q      [rows, cols]              E4M3 out, 16-byte aligned
 *   scales [ceil(rows/32), cols/32]  fp32 out, 4-byte aligned
 *   cols % 32 == 0 (else FP8BS_ESHAPE); rows == 0 or cols == 0 is a no-op.
 */
fp8bs_status fp8bs_quantize(const void* x_bf16, int64_t rows, int64_t cols, void* q_e4m3, float* scales,
                            void* stream);

/*
 * fp8bs_gemm - C = dequant(A) . dequant(B) with the scales folded in per
 *   32-deep K-block [DG 2.2-2.3]:
 *     C[i,j] = sum_kb  sa[i/32, kb] * sb[kb, j/32] * sum_{k in kb} A[i,k] B[k,j]
 *   Each 32-deep partial is formed exactly from the decoded E4M3 values (fp32
 *   result), multiplied by the fp32 product sa*sb and added into one fp32
 *   accumulator, K-blocks in ascending order; C is rounded once to bf16
 *   (nearest, ties to even).
 *   a  [M, K] E4M3, 16-byte aligned      sa [ceil(M/32), K/32] fp32
 *   b  [K, N] E4M3, 16-byte aligned      sb [K/32, N/32] fp32
 *   c  [M, N] bf16 out, 16-byte aligned
 *   K % 32 == 0 and N % 32 == 0 (else FP8BS_ESHAPE); M, N, K <= 2^30.
 *   M == 0 or N == 0: no-op.  K == 0: C is filled with +0.
 */
fp8bs_status fp8bs_gemm(const void* a, const float* sa, const void* b, const float* sb, void* c_bf16, int64_t M,
                        int64_t N, int64_t K, void* stream);

/*
 * fp8bs_grouped_gemm - G independent GEMMs over consecutive row ranges of one
 *   A, each with its own B_g [DG 4.1-4.2].  Row range g is
 *   [offsets[g], offsets[g+1]); its rows are multiplied by b[g] with sb[g]
 *   exactly as fp8bs_gemm would; empty ranges produce no work.  The offsets
 *   live in DEVICE memory, so a captured graph stays valid when the group
 *   sizes change [DG 4.3].
 *   a       [M_total, K] E4M3          sa [M_total/32, K/32] fp32
 *   b       [G, K, N] E4M3             sb [G, K/32, N/32] fp32
 *   offsets [G+1] int32 on the device: 0 = off[0] <= off[1] <= ... <= off[G] = M_total,
 *           every entry a multiple of 32.  Not checked on the host.  The kernel
 *           clamps each range into [0, M_total], starts it no earlier than the
 *           previous range's end and treats a range that would run backwards as
 *           empty, so a bad table gives wrong rows (with unaligned entries also
 *           wrong scale rows), never an out-of-bounds access.
 *   c       [M_total, N] bf16 out (rows outside every range are left untouched)
 *   1 <= G <= FP8BS_MAX_GROUPS (else FP8BS_EINVAL); M_total, K, N multiples of 32.
 */
fp8bs_status fp8bs_grouped_gemm(const void* a, const float* sa, const void* b, const float* sb,
                                const int32_t* offsets_dev, int32_t G, void* c_bf16, int64_t M_total, int64_t N,
                                int64_t K, void* stream);

/*
 * fp8bs_gemm_nt - fp8bs_gemm with the weight K-major, the layout of the
 *   call interface in [DG 6] (weight [N, K], its scales [N/32, K/32]):
 *     C[i,j] = sum_kb  sa[i/32, kb] * sbt[j/32, kb] * sum_{k in kb} A[i,k] Bt[j,k]
 *   with the same per-element recipe as fp8bs_gemm, so every element is
 *   bitwise equal to fp8bs_gemm on the transposed weight.  fp8bs_quantize of
 *   the [N, K] bf16 weight gives exactly the transposed codes and scale grid of
 *   quantizing its [K, N] transpose (blocks are 32x32 either way).
 *   a   [M, K] E4M3, 16-byte aligned      sa  [ceil(M/32), K/32] fp32
 *   bt  [N, K] E4M3, 16-byte aligned      sbt [N/32, K/32] fp32
 *   c   [M, N] bf16 out, 16-byte aligned
 *   Checks, errors and K == 0 as for fp8bs_gemm.
 */
fp8bs_status fp8bs_gemm_nt(const void* a, const float* sa, const void* bt, const float* sbt, void* c_bf16,
                           int64_t M, int64_t N, int64_t K, void* stream);

/*
 * fp8bs_grouped_gemm_nt - fp8bs_grouped_gemm with K-major weights [DG 4.1-4.2, 6]:
 *   bt [G, N, K] E4M3, sbt [G, N/32, K/32] fp32; everything else (offsets on
 *   the device, empty ranges, untouched rows, checks) as fp8bs_grouped_gemm.
 */
fp8bs_status fp8bs_grouped_gemm_nt(const void* a, const float* sa, const void* bt, const float* sbt,
                                   const int32_t* offsets_dev, int32_t G, void* c_bf16, int64_t M_total, int64_t N,
                                   int64_t K, void* stream);

/*
 * Per-token-group activation scales (one scale per row and 32 columns), the
 * activation-side granularity that the determinism article's RMSNorm part
 * (三, section 2, the vLLM table: per-token-group FP8 quantization fused with
 * the norm) lists; with it an element of C depends on its own row of the
 * bf16 activations only, so the quantize + GEMM chain is batch invariant end
 * to end [DET part 一, sections 6-7].  Weights keep 32x32 block scales.
 *
 * fp8bs_quantize_tg - as fp8bs_quantize, with groups of 1 row x 32 columns:
 *   group (r, cb) covers row r, columns [32cb, 32cb+32); amax, s = amax/448,
 *   codes exactly as fp8bs_quantize per group [DG 2.1, 5.2].
 *   x [rows, cols] bf16, q [rows, cols] E4M3 out, scales [rows, cols/32] fp32 out.
 *   Checks and errors as fp8bs_quantize.
 */
fp8bs_status fp8bs_quantize_tg(const void* x_bf16, int64_t rows, int64_t cols, void* q_e4m3, float* scales,
                               void* stream);

/*
 * fp8bs_gemm_tg / fp8bs_gemm_tg_nt - fp8bs_gemm / fp8bs_gemm_nt with A's
 *   scales per token group:
 *     C[i,j] = sum_kb  sa_rows[i, kb] * sb[kb, j/32] * sum_{k in kb} A[i,k] B[k,j]
 *   Each 32-deep partial is formed exactly, multiplied by the fp32 product
 *   sa_rows[i,kb]*sb (one rounding) and added into one fp32 accumulator, K-blocks
 *   ascending; C is rounded once to bf16.  Every kernel behind these two
 *   entry points forms its partials the same way, so results do not depend on
 *   M or on the kernel.
 *   a [M, K] E4M3, sa_rows [M, K/32] fp32 (4-byte aligned);
 *   fp8bs_gemm_tg:    b  [K, N] E4M3, sb  [K/32, N/32] fp32
 *   fp8bs_gemm_tg_nt: bt [N, K] E4M3, sbt [N/32, K/32] fp32
 *   c [M, N] bf16 out.  Checks, errors and K == 0 as for fp8bs_gemm.
 */
fp8bs_status fp8bs_gemm_tg(const void* a, const float* sa_rows, const void* b, const float* sb, void* c_bf16,
                           int64_t M, int64_t N, int64_t K, void* stream);
fp8bs_status fp8bs_gemm_tg_nt(const void* a, const float* sa_rows, const void* bt, const float* sbt, void* c_bf16,
                              int64_t M, int64_t N, int64_t K, void* stream);

/*
 * fp8bs_rmsnorm_quantize_tg - residual add + RMSNorm + per-token-group E4M3
 *   quantization in one pass over each row.  The norm is [DET part 三,
 *   section 1]: per row, y = x / sqrt(mean(x^2) + eps) * gamma; section 2 lists
 *   the residual ("fused add") form and the fusion of the norm with
 *   per-token-group FP8 quantization.  Per row of d columns:
 *     residual != NULL:  h = bf16(x + residual), written back to residual
 *                        (one round-to-nearest-even of the exact sum)
 *     residual == NULL:  h = x
 *     rinv = 1 / sqrt(sum(h^2) / d + eps)                       (fp32)
 *     y_i  = bf16((h_i * rinv) * gamma_i)                       (fp32, then RNE)
 *     q, scales = fp8bs_quantize_tg of y (1 x 32 groups, bit for bit)
 *   The sum of squares has a fixed order that depends on d only (never on
 *   rows), so each row's outputs depend on that row alone.
 *   x        [rows, d] bf16, 16-byte aligned
 *   residual [rows, d] bf16 in/out, or NULL; must not overlap x
 *   gamma    [d] bf16
 *   eps      finite, >= 0 (else FP8BS_EINVAL); eps == 0 with an all-zero row
 *            gives NaN scales (precondition: not both)
 *   q        [rows, d] E4M3 out; scales [rows, d/32] fp32 out
 *   y        [rows, d] bf16 out (the normalised rows), or NULL to skip it
 *   d % 32 == 0 and d <= 16384 (else FP8BS_ESHAPE); rows == 0 or d == 0: no-op.
 *   Outputs must not overlap inputs (residual is updated in place by design).
 */
fp8bs_status fp8bs_rmsnorm_quantize_tg(const void* x_bf16, void* residual_bf16, const void* gamma_bf16, float eps,
                                       int64_t rows, int64_t d, void* q_e4m3, float* scales, void* y_bf16,
                                       void* stream);

/*
 * Power-of-two (E8M0) block scales.  A separate contract: the DeepGEMM
 * write-up's 32x32 blocks [DG 2.2, 5.2] with each scale restricted to a power
 * of two 2^E, stored as one byte E + 127, so that gfx950's hardware-scaled
 * F8F6F4 MFMA applies it.  The pages describe no such variant.
 *
 * fp8bs_quantize_e8m0 - per 32x32 block: E = the smallest integer with
 *   448 * 2^E >= amax, clamped to [-127, 127] (-127 for an all-zero block);
 *   codes = E4M3(x * 2^-E) (exact scaling, then round half to even, sign
 *   kept; no value saturates).
 *   x [rows, cols] bf16, q [rows, cols] E4M3 out (both 16-byte aligned),
 *   e8m0 [ceil(rows/32), cols/32] bytes out.  Checks as fp8bs_quantize.
 */
fp8bs_status fp8bs_quantize_e8m0(const void* x_bf16, int64_t rows, int64_t cols, void* q_e4m3, void* e8m0,
                                 void* stream);

/*
 * fp8bs_gemm_e8m0_nt - C = sum_k dec(A) 2^Ea * dec(Bt) 2^Eb with the weight
 *   K-major [DG 6], on the hardware-scaled MFMA: 128-deep K steps in ascending
 *   order, accumulated by the instruction itself.  Results do not depend on M
 *   (every M runs the same instruction sequence per element).  The
 *   instruction's summation is not exact, so this entry point is not held to
 *   fp8bs_gemm's bound.  Its error bound (checked by the tests) follows from a
 *   model of one 128-deep step measured on the instruction: the 128 products
 *   fall into 16 groups of 8 consecutive K; with S = x(a) + x(b) + Ea + Eb
 *   (x = a code's exponent, its significand read in [0, 2), -6 for subnormal
 *   codes), each product of group g is cut toward zero to a multiple of
 *   2^(S_g - 13), S_g the group's largest S; each group and the accumulator
 *   input lose at most 2^(S_max - 23) more, S_max the step's largest S or
 *   the accumulator's exponent; the step's result is rounded to fp32, nearest
 *   even; C is rounded once to bf16, nearest even.  Per element,
 *   |C - exact| <= the sum over steps of those losses and half an fp32 ulp of
 *   each step's result, plus half a bf16 ulp of C.
 *   a  [M, K] E4M3, ea  [ceil(M/32), K/32] bytes (4-byte aligned)
 *   bt [N, K] E4M3, ebt [N/32, K/32] bytes (4-byte aligned)
 *   c  [M, N] bf16 out.  K % 128 == 0 and N % 32 == 0 (else FP8BS_ESHAPE);
 *   M == 0 or N == 0: no-op; K == 0: C is filled with +0.
 */
fp8bs_status fp8bs_gemm_e8m0_nt(const void* a, const void* ea, const void* bt, const void* ebt, void* c_bf16,
                                int64_t M, int64_t N, int64_t K, void* stream);

/* Human-readable name of a status code (static string, never NULL). */
const char* fp8bs_status_str(fp8bs_status status);

#ifdef __cplusplus
}
#endif

#endif /* FP8BS_H */
