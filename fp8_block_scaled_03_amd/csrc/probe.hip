// Measurement and test support for the E4M3 GEMM library: single gfx950
// instructions exposed for the tests and the bench.  Nothing of the GEMM
// path calls into this file, and it is built into its own library
// (libfp8bs_probe.so).
//
//  * fp8bs_probe_gemm: a plain block-scaled GEMM, one wave per 16x16 output
//    tile, fragments read straight from global memory.  Every 32-deep K-block
//    partial is formed by one MFMA, either v_mfma_f32_16x16x32_bf16 on exactly
//    decoded codes (what every kernel of the library does) or
//    v_mfma_f32_16x16x32_fp8_fp8 on the raw codes; promotion is the library's
//    (s = sa * sb, acc = fma(P, s, acc), K-blocks ascending; DeepGEMM
//    write-up on hncyxsy.com, sections 2.2-2.3).  The partials themselves can
//    be written out as well.
//  * fp8bs_probe_mfma_scale: a batch of independent single
//    v_mfma_scale_f32_16x16x128_f8f6f4 instructions on given codes, E8M0
//    scale bytes and accumulator input, to expose how the instruction sums.
//  * fp8bs_probe_promote_ceiling: a register-only loop of the exact recipe's
//    instruction mix (one 16x16x32 bf16 MFMA and four fp32 FMAs that promote
//    an earlier partial), the rate any kernel of this recipe can reach.
//  * fp8bs_probe_stream_read: a plain streaming read of a buffer, the HBM
//    read rate a memory-bound kernel can reach.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"

namespace fp8bs {
namespace probe {

typedef int v8i_t __attribute__((ext_vector_type(8)));

// One wave per 16x16 tile of C: tile t covers rows 16 * (t / (N/16)), columns
// 16 * (t % (N/16)).  Lane l reads row (l & 15) of A and column (l & 15) of B,
// K elements [8 (l >> 4), 8 (l >> 4) + 8) of each 32-deep block (the operand
// layout of both 16x16x32 MFMA forms); its four results are rows
// 4 (l >> 4) + r, column l & 15.
template <bool FP8_FORM>
__global__ void __launch_bounds__(256) probe_gemm_kernel(const uint8_t* __restrict__ a,
                                                         const float* __restrict__ sa,
                                                         const uint8_t* __restrict__ b,
                                                         const float* __restrict__ sb, uint16_t* __restrict__ c,
                                                         float* __restrict__ partials, int M, int N, int K) {
  const int lane = threadIdx.x & 63;
  const int64_t tile = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int tiles_n = N / 16;
  if (tile >= (int64_t)(M / 16) * tiles_n) return;
  const int r0 = (int)(tile / tiles_n) * 16, c0 = (int)(tile % tiles_n) * 16;
  const int lo = lane & 15, g = lane >> 4;
  const int KB = K / 32, NB = N / 32;
  const uint8_t* arow = a + (int64_t)(r0 + lo) * K + 8 * g;
  const uint8_t* bcol = b + (int64_t)(8 * g) * N + c0 + lo;
  v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int kb = 0; kb < KB; ++kb) {
    const uint2 aw = *reinterpret_cast<const uint2*>(arow + kb * 32);
    uint32_t bw[2] = {0u, 0u};
#pragma unroll
    for (int e = 0; e < 8; ++e) bw[e >> 2] |= (uint32_t)bcol[(int64_t)(kb * 32 + e) * N] << (8 * (e & 3));
    v4f p;
    if constexpr (FP8_FORM) {
      const long av = (long)(((uint64_t)aw.y << 32) | aw.x);
      const long bv = (long)(((uint64_t)bw[1] << 32) | bw[0]);
      const v4f z = {0.0f, 0.0f, 0.0f, 0.0f};
      p = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(av, bv, z, 0, 0, 0);
    } else {
      p = mfma_partial(e4m3x8_to_bf16x8(v2i{(int)aw.x, (int)aw.y}), e4m3x8_to_bf16x8(v2i{(int)bw[0], (int)bw[1]}));
    }
    if (partials) {
#pragma unroll
      for (int r = 0; r < 4; ++r) partials[((int64_t)kb * M + r0 + 4 * g + r) * N + c0 + lo] = p[r];
    }
    // the four rows of a lane lie in one 32-row block, its column in one
    // 32-column block: one scale product per lane and K-block
    const float s = sa[(int64_t)((r0 + 4 * g) >> 5) * KB + kb] * sb[(int64_t)kb * NB + ((c0 + lo) >> 5)];
    promote(acc, p, s);
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) c[(int64_t)(r0 + 4 * g + r) * N + c0 + lo] = (uint16_t)bf16_out(acc[r]);
}

// Problem q (one wave): D[m][n] = C[m][n] + sum_{k<128} dec(A[m][k]) 2^(ea[m][k/32]-127)
//                                          * dec(Bt[n][k]) 2^(eb[n][k/32]-127),
// m, n in [0, 16).  Lane l holds row l & 15 of A and of Bt: bytes 0-15 =
// K [16g, 16g+16), bytes 16-31 = K [64+16g, 80+16g), g = l >> 4; the scale
// byte of (row r, K-block kb) comes from lane 16 kb + r.  Lane l's results
// are D[4g + r][l & 15].
__global__ void __launch_bounds__(64) probe_mfma_scale_kernel(const uint8_t* __restrict__ a,
                                                              const uint8_t* __restrict__ bt,
                                                              const uint8_t* __restrict__ ea,
                                                              const uint8_t* __restrict__ eb,
                                                              const float* __restrict__ cin, float* __restrict__ d) {
  const int q = blockIdx.x;
  const int lane = threadIdx.x;
  const int lo = lane & 15, g = lane >> 4;
  const uint8_t* ar = a + ((int64_t)q * 16 + lo) * 128;
  const uint8_t* br = bt + ((int64_t)q * 16 + lo) * 128;
  const v4i a0 = *reinterpret_cast<const v4i*>(ar + 16 * g), a1 = *reinterpret_cast<const v4i*>(ar + 64 + 16 * g);
  const v4i b0 = *reinterpret_cast<const v4i*>(br + 16 * g), b1 = *reinterpret_cast<const v4i*>(br + 64 + 16 * g);
  const v8i_t av = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
  const v8i_t bv = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
  const int sca = ea[((int64_t)q * 16 + lo) * 4 + g];
  const int scb = eb[((int64_t)q * 16 + lo) * 4 + g];
  const float* cq = cin + (int64_t)q * 256;
  v4f cv;
#pragma unroll
  for (int r = 0; r < 4; ++r) cv[r] = cq[(4 * g + r) * 16 + lo];
  const v4f dv = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, cv, 0, 0, 0, sca, 0, scb);
  float* dq = d + (int64_t)q * 256;
#pragma unroll
  for (int r = 0; r < 4; ++r) dq[(4 * g + r) * 16 + lo] = dv[r];
}

// The exact recipe's instruction mix, registers only: per step one
// v_mfma_f32_16x16x32_bf16 with a zero accumulator input, and four fp32 FMAs
// that promote the partial formed RING steps earlier (so they never wait on
// the MFMA just issued).  MODE 1 keeps only the MFMAs, MODE 2 only the FMAs
// (the same count, on partials that are left as they were), so the three
// rates show how far the two kinds of work overlap on one SIMD; MODE 3 runs
// v_mfma_f32_16x16x32_fp8_fp8 alone instead of the bf16 form.  The eight
// steps of an iteration use eight different A operands and a B operand that
// is rotated every iteration, so no two MFMAs are alike and none is loop
// invariant; every MFMA result is read (by the FMAs, or by the final sum
// through its own slot), and each wave writes one value, so nothing is dead.
constexpr int RING = 4;
template <int MODE>
__global__ void __launch_bounds__(512) probe_promote_ceiling_kernel(float* __restrict__ out, int iters, float seed) {
  const int lane = threadIdx.x & 63;
  v8bf a[8], b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
#pragma unroll
    for (int u = 0; u < 8; ++u) a[u][e] = (__bf16)(seed * (float)(lane + e + 3 * u + 1));
    b[e] = (__bf16)(seed * (float)(lane - e + 3));
  }
  v4f acc[4];
  v4f ring[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int i = 0; i < 8; ++i) ring[i] = v4f{seed, seed, seed, seed};
  float s = seed;
  const v4f z = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if constexpr (MODE == 0) {
        const v4f p = mfma_partial(a[u], b);
        promote(acc[u & 3], ring[u % RING], s);
        ring[u % RING] = p;
      } else if constexpr (MODE == 1) {
        ring[u] = mfma_partial(a[u], b);
      } else if constexpr (MODE == 2) {
        promote(acc[u & 3], ring[u % RING], s);
      } else {
        // the FP8 form of a 32-deep partial, on the operands' raw bits
        const v4i ai = __builtin_bit_cast(v4i, a[u]), bi = __builtin_bit_cast(v4i, b);
        const long a8 = ((long)ai[0] << 32) | (unsigned)ai[1];
        const long b8 = ((long)bi[2] << 32) | (unsigned)bi[3];
        ring[u] = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(a8, b8, z, 0, 0, 0);
      }
    }
    s = s * 0.999f;
    b = __builtin_shufflevector(b, b, 1, 2, 3, 4, 5, 6, 7, 0);
  }
  float t = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) t += acc[i][0] + acc[i][1] + acc[i][2] + acc[i][3];
#pragma unroll
  for (int i = 0; i < 8; ++i) t += ring[i][0] + ring[i][1] + ring[i][2] + ring[i][3];
  if (lane == 0) out[(int64_t)blockIdx.x * 8 + (threadIdx.x >> 6)] = t;
}

// The same mix issued in bursts: BU MFMAs back to back, then the 4 BU FMAs
// that promote the previous burst's partials (a ring of 2 BU partials), 12
// steps per iteration (every BU used divides 12), iterations in pairs so that
// the two halves of the ring swap roles without register copies.  With two
// waves on a SIMD, the MFMA burst of one can overlap the FMA burst of the
// other.
template <int BU>
__global__ void __launch_bounds__(512) probe_promote_burst_kernel(float* __restrict__ out, int iters, float seed) {
  constexpr int H = 12;
  static_assert(H % BU == 0, "burst size divides the iteration");
  const int lane = threadIdx.x & 63;
  v8bf a[H], b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
#pragma unroll
    for (int u = 0; u < H; ++u) a[u][e] = (__bf16)(seed * (float)(lane + e + 3 * u + 1));
    b[e] = (__bf16)(seed * (float)(lane - e + 3));
  }
  v4f acc[4], r0[H], r1[H];
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int i = 0; i < H; ++i) r0[i] = r1[i] = v4f{seed, seed, seed, seed};
  float s = seed;
  for (int it = 0; it < iters; it += 2) {
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      v4f* older = half == 0 ? r0 : r1;  // partials promoted in this iteration
      v4f* newer = half == 0 ? r1 : r0;  // partials formed in this iteration
#pragma unroll
      for (int h = 0; h < H; h += BU) {
#pragma unroll
        for (int u = 0; u < BU; ++u) newer[h + u] = mfma_partial(a[h + u], b);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < BU; ++u) promote(acc[(h + u) & 3], older[h + u], s);
        __builtin_amdgcn_sched_barrier(0);
      }
      s = s * 0.999f;
      b = __builtin_shufflevector(b, b, 1, 2, 3, 4, 5, 6, 7, 0);
    }
  }
  float t = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) t += acc[i][0] + acc[i][1] + acc[i][2] + acc[i][3];
#pragma unroll
  for (int i = 0; i < H; ++i) t += r0[i][0] + r0[i][1] + r0[i][2] + r0[i][3] + r1[i][0] + r1[i][1] + r1[i][2] + r1[i][3];
  if (lane == 0) out[(int64_t)blockIdx.x * 8 + (threadIdx.x >> 6)] = t;
}

// The hardware-scaled MFMA alone: v_mfma_scale_f32_16x16x128_f8f6f4 on E4M3
// operands with unit scales (E8M0 127), eight accumulators, `iters` x 8
// instructions per wave; the rate the power-of-two-scale GEMM can reach.
__global__ void __launch_bounds__(512) probe_scaled_mfma_kernel(float* __restrict__ out, int iters, float seed) {
  const int lane = threadIdx.x & 63;
  const int bits = (int)(seed * 1024.0f);
  v8i_t a[4], b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
#pragma unroll
    for (int u = 0; u < 4; ++u) a[u][e] = 0x38383838 + bits * (lane + e + u);
    b[e] = 0x30303030 + bits * (lane - e);
  }
  v4f acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int u = 0; u < 8; ++u)
      acc[u] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a[u & 3], b, acc[u], 0, 0, 0, 127, 0, 127);
    b = __builtin_shufflevector(b, b, 1, 2, 3, 4, 5, 6, 7, 0);
  }
  float t = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) t += acc[i][0] + acc[i][1] + acc[i][2] + acc[i][3];
  if (lane == 0) out[(int64_t)blockIdx.x * 8 + (threadIdx.x >> 6)] = t;
}

// Streaming read of `n16` 16-byte words: every thread reads a grid-strided
// sequence, eight loads in flight, and folds them with xor; one word per wave
// is written so that nothing is dead.
__global__ void __launch_bounds__(512) probe_stream_read_kernel(const uint4* __restrict__ buf, int64_t n16,
                                                                uint32_t* __restrict__ out) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  uint32_t x = 0;
  for (; i + 7 * stride < n16; i += 8 * stride) {
    uint4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = buf[i + u * stride];
#pragma unroll
    for (int u = 0; u < 8; ++u) x ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const uint4 v = buf[i];
    x ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  // xor across the wave, then lane 0 writes
  for (int off = 32; off > 0; off >>= 1) x ^= (uint32_t)__shfl_xor((int)x, off, 64);
  if ((threadIdx.x & 63) == 0) out[(int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6)] = x;
}

}  // namespace probe
}  // namespace fp8bs

using namespace fp8bs::probe;

extern "C" {

int fp8bs_probe_gemm(const void* a, const float* sa, const void* b, const float* sb, void* c, float* partials,
                     int M, int N, int K, int fp8_form, void* stream) {
  if (!a || !sa || !b || !sb || !c) return 1;
  if (M <= 0 || N <= 0 || K <= 0 || M % 32 || N % 32 || K % 32) return 2;
  const int64_t tiles = (int64_t)(M / 16) * (N / 16);
  const unsigned grid = (unsigned)((tiles + 3) / 4);
  if (fp8_form)
    hipLaunchKernelGGL(probe_gemm_kernel<true>, dim3(grid), dim3(256), 0, (hipStream_t)stream, (const uint8_t*)a, sa,
                       (const uint8_t*)b, sb, (uint16_t*)c, partials, M, N, K);
  else
    hipLaunchKernelGGL(probe_gemm_kernel<false>, dim3(grid), dim3(256), 0, (hipStream_t)stream, (const uint8_t*)a,
                       sa, (const uint8_t*)b, sb, (uint16_t*)c, partials, M, N, K);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

int fp8bs_probe_mfma_scale(const void* a, const void* bt, const void* ea, const void* eb, const float* cin, float* d,
                           int count, void* stream) {
  if (!a || !bt || !ea || !eb || !cin || !d) return 1;
  if (count <= 0) return 2;
  hipLaunchKernelGGL(probe_mfma_scale_kernel, dim3((unsigned)count), dim3(64), 0, (hipStream_t)stream,
                     (const uint8_t*)a, (const uint8_t*)bt, (const uint8_t*)ea, (const uint8_t*)eb, cin, d);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

int fp8bs_probe_promote_ceiling(float* out, int workgroups, int iters, int mode, void* stream) {
  if (!out) return 1;
  if (workgroups <= 0 || iters <= 0 || mode < 0 || mode > 8) return 2;
  if (mode >= 4 && mode <= 7 && (iters & 1)) return 2;
  const dim3 grid((unsigned)workgroups), block(512);
  const hipStream_t st = (hipStream_t)stream;
  const float seed = 1.0f / 1024.0f;
  switch (mode) {
    case 0: hipLaunchKernelGGL(probe_promote_ceiling_kernel<0>, grid, block, 0, st, out, iters, seed); break;
    case 1: hipLaunchKernelGGL(probe_promote_ceiling_kernel<1>, grid, block, 0, st, out, iters, seed); break;
    case 2: hipLaunchKernelGGL(probe_promote_ceiling_kernel<2>, grid, block, 0, st, out, iters, seed); break;
    case 3: hipLaunchKernelGGL(probe_promote_ceiling_kernel<3>, grid, block, 0, st, out, iters, seed); break;
    case 4: hipLaunchKernelGGL(probe_promote_burst_kernel<2>, grid, block, 0, st, out, iters, seed); break;
    case 5: hipLaunchKernelGGL(probe_promote_burst_kernel<3>, grid, block, 0, st, out, iters, seed); break;
    case 6: hipLaunchKernelGGL(probe_promote_burst_kernel<4>, grid, block, 0, st, out, iters, seed); break;
    case 7: hipLaunchKernelGGL(probe_promote_burst_kernel<6>, grid, block, 0, st, out, iters, seed); break;
    default: hipLaunchKernelGGL(probe_scaled_mfma_kernel, grid, block, 0, st, out, iters, seed); break;
  }
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

int fp8bs_probe_stream_read(const void* buf, long long bytes, unsigned* out, int workgroups, void* stream) {
  if (!buf || !out) return 1;
  if (bytes <= 0 || bytes % 16 || workgroups <= 0) return 2;
  hipLaunchKernelGGL(probe_stream_read_kernel, dim3((unsigned)workgroups), dim3(512), 0, (hipStream_t)stream,
                     (const uint4*)buf, (int64_t)(bytes / 16), (uint32_t*)out);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

}  // extern "C"
