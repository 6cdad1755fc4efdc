// Shared device helpers for the gfx950 kernels of the E4M3 block-scaled GEMM.
//
// Numerics (identical in every kernel, so that results are batch invariant):
//   * an E4M3 byte is decoded exactly to bf16 by the hardware converter
//     (E4M3 values are a subset of bf16);
//   * one 32-deep K-block partial P = sum_{k in block} a_k b_k is one
//     v_mfma_f32_16x16x32_bf16 with a zero accumulator input (the bf16 MFMA
//     forms the partial at full fp32 precision; the FP8 MFMA forms drop
//     low-order product bits, which the accuracy bound does not allow);
//   * promotion: s = sa * sb (fp32, one rounding), acc = fma(P, s, acc),
//     K-blocks in ascending order into one fp32 accumulator
//     (DeepGEMM write-up on hncyxsy.com, sections 2.2-2.3: the block scales
//     enter during accumulation, not in a separate pass over C);
//   * C = bf16(acc), round to nearest even, once; an exact zero is stored as +0.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#pragma clang fp contract(off)

namespace fp8bs {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef short v4s __attribute__((ext_vector_type(4)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

typedef __attribute__((address_space(3))) v4s lds_v4s_t;
typedef __attribute__((address_space(3))) v2i lds_v2i_t;

// 4 E4M3 bytes (one dword) -> 4 bf16 (two dwords), exact.
__device__ __forceinline__ v2i e4m3x4_to_bf16x4(uint32_t w) {
  v2bf lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
  v2bf hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true);
  return v2i{__builtin_bit_cast(int, lo), __builtin_bit_cast(int, hi)};
}

// 8 E4M3 bytes -> the 8 bf16 operand of one MFMA lane.
__device__ __forceinline__ v8bf e4m3x8_to_bf16x8(v2i w) {
  v2i lo = e4m3x4_to_bf16x4((uint32_t)w[0]);
  v2i hi = e4m3x4_to_bf16x4((uint32_t)w[1]);
  return __builtin_bit_cast(v8bf, v4i{lo[0], lo[1], hi[0], hi[1]});
}

// 16 E4M3 bytes -> 16 bf16 (32 bytes).
__device__ __forceinline__ void e4m3x16_to_bf16x16(uint4 w, uint4& out0, uint4& out1) {
  v2i a = e4m3x4_to_bf16x4(w.x), b = e4m3x4_to_bf16x4(w.y);
  v2i c = e4m3x4_to_bf16x4(w.z), d = e4m3x4_to_bf16x4(w.w);
  out0 = make_uint4((uint32_t)a[0], (uint32_t)a[1], (uint32_t)b[0], (uint32_t)b[1]);
  out1 = make_uint4((uint32_t)c[0], (uint32_t)c[1], (uint32_t)d[0], (uint32_t)d[1]);
}

// One 32-deep K-block partial for a 16x16 output sub-tile.
__device__ __forceinline__ v4f mfma_partial(v8bf a, v8bf b) {
  v4f z = {0.0f, 0.0f, 0.0f, 0.0f};
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, z, 0, 0, 0);
}

// acc += P * s, element-wise, one rounding each.
__device__ __forceinline__ void promote(v4f& acc, v4f p, float s) {
  acc[0] = __builtin_fmaf(p[0], s, acc[0]);
  acc[1] = __builtin_fmaf(p[1], s, acc[1]);
  acc[2] = __builtin_fmaf(p[2], s, acc[2]);
  acc[3] = __builtin_fmaf(p[3], s, acc[3]);
}

// fp32 -> bf16 bits, round to nearest, ties to even (finite inputs).
__device__ __forceinline__ uint32_t bf16_rne(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// A GEMM output element: bf16(acc) with an exact zero stored as +0.  acc + 0
// turns -0 into +0 and leaves every other value unchanged, so the sign of a
// zero result never depends on which kernel formed it (a kernel that promotes
// an extra zero-scale K-block and one that does not may otherwise differ in
// the sign of an exact zero).
__device__ __forceinline__ uint32_t bf16_out(float acc) { return bf16_rne(acc + 0.0f); }

// ---- E4M3 quantizer steps shared by every kernel that writes codes --------------------
// Groups with amax at or above this value take the reciprocal path below.
constexpr float QUANT_RECIP_MIN_AMAX = 0x1p-60f;

// RN32(x / s) from r = RN32(1 / s): q0 = RN(x*r), e = x - s*q0 (exact), then
// RN(q0 + e*r) (Markstein, IBM J. Res. Dev. 34(1), 1990).  Valid when the
// group's amax >= QUANT_RECIP_MIN_AMAX (smaller |x| of such a group give
// quotients below 2^-33, a zero code whatever their last bits).  The sign is
// copied from x so that -0 stays -0.
__device__ __forceinline__ float quant_quotient_recip(float x, float s, float r) {
  const float q0 = x * r;
  const float e = __builtin_fmaf(-q0, s, x);
  return __builtin_copysignf(__builtin_fmaf(e, r, q0), x);
}
// The same by IEEE division, for groups with a tiny amax; s = 0 gives 0.
__device__ __forceinline__ float quant_quotient_div(float x, float s) { return s != 0.0f ? x / s : 0.0f; }
__device__ __forceinline__ float sat448(float t) { return fminf(fmaxf(t, -448.0f), 448.0f); }
// Four quotients (already within +-448) -> four E4M3FN bytes, round to nearest even.
__device__ __forceinline__ uint32_t pack_e4m3x4(float t0, float t1, float t2, float t3) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(t0, t1, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(t2, t3, w, true);
  return (uint32_t)w;
}

// Eight E4M3 codes (two dwords) stored with a non-temporal hint: the codes
// are read once, by the next GEMM, so they need not displace what the L2
// holds.  A quantize launched right after a 4096^3 GEMM took 12.8 against
// 14.1 us this way; with flushed caches the two are equal.
__device__ __forceinline__ void store_codes8(uint8_t* dst, uint32_t lo, uint32_t hi) {
  typedef unsigned v2u __attribute__((ext_vector_type(2)));
  __builtin_nontemporal_store(v2u{lo, hi}, reinterpret_cast<v2u*>(dst));
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xFFFF0000u); }

// Tile order: consecutive workgroup ids are dealt round-robin to the 8 XCDs, so
// ids are first re-dealt so that each XCD sees a contiguous run of tiles; the
// run is walked in groups of 4 M-tiles so that neighbours share A rows and B
// columns in that XCD's L2.
__device__ __forceinline__ void tile_coords(int64_t id, int64_t n_tiles, int64_t tiles_n, int64_t& tm, int64_t& tn) {
  const int64_t per_xcd = (n_tiles + 7) / 8;
  const int64_t lin = (id & 7) * per_xcd + (id >> 3);  // callers remap only when n_tiles % 8 == 0
  const int64_t GM = 4;
  const int64_t group = lin / (GM * tiles_n);
  const int64_t first_m = group * GM;
  const int64_t tiles_m_total = (n_tiles / tiles_n);
  const int64_t gm = (tiles_m_total - first_m) < GM ? (tiles_m_total - first_m) : GM;
  const int64_t r = lin - group * GM * tiles_n;
  tm = first_m + r % gm;
  tn = r / gm;
}

// ------------------------------------------------------------------------------------
// direct global->LDS loads
// ------------------------------------------------------------------------------------
// One direct global->LDS load of 16 bytes per lane (global_load_lds_dwordx4:
// lane l's bytes land at M0 + 16*l; M0 = LDS byte address of the wave's 1 KB
// destination).  Issued from inline asm so that the compiler does not drain
// every load before the next LDS read; the callers wait with explicit vmcnt
// counts (a wave's loads complete in issue order).  Nothing else in these
// kernels uses M0.
__device__ __forceinline__ void dma16(const void* gptr, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds_base), "v"(gptr)
               : "memory");
}
// The same with 4 bytes per lane (lane l's dword lands at M0 + 4*l).
__device__ __forceinline__ void dma4(const void* gptr, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, off" ::"s"(lds_base), "v"(gptr)
               : "memory");
}
// Workgroup barrier that orders LDS only: the direct loads in flight keep
// running (a plain __syncthreads would drain them).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__device__ __forceinline__ int wave_id_uniform() {
  return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
}

}  // namespace fp8bs
