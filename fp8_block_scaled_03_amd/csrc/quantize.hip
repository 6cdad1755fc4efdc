// bf16 -> E4M3 block quantizer for gfx950.
//
// DeepGEMM write-up (hncyxsy.com): section 2.2 - one scale per 32x32 block;
// section 5.2 - the scale comes from the block's absolute maximum; section
// 2.1 - E4M3 tops out at 448.  Per block: amax = max |x|, s = amax / 448 in
// fp32, each code = E4M3(x / s) with the quotient in fp32 (IEEE division,
// round to nearest even), rounded to E4M3 by the hardware converter
// (round to nearest even, E4M3FN) after clamping to +-448 (the converter would
// produce NaN above 464); an all-zero block gets s = 0 and 0x00 codes.
//
// The quotient.  x / s (IEEE, round to nearest even) costs about ten VALU
// instructions; instead each block forms r = RN(1/s) with one IEEE division and
// every element takes q0 = RN(x*r), e = x - s*q0 (exact, one fma), t =
// RN(q0 + e*r) (one fma).  With r the correctly rounded reciprocal and q0
// within an ulp of x/s this final correction returns RN(x/s) (Markstein's
// theorem, P. Markstein, IBM J. Res. Dev. 34(1), 1990), provided the remainder
// e does not underflow: that holds for |x| >= 2^-102, and blocks with
// amax >= 2^-60 send every smaller |x| to |x/s| < 2^-33, which becomes a zero
// code whatever its last bits.  Blocks with a smaller amax, where s is tiny,
// divide directly.  The sign is copied from x so that -0 stays -0.
//
// The kernel is bound by HBM traffic (2 bytes read + 1 byte written per
// element); the mapping below keeps 128 bytes per lane in flight.
#include "common.hpp"

#include <type_traits>

namespace fp8bs {

// Max over the 16 lanes that hold one block (lane bits 0, 1, 4, 5).
__device__ __forceinline__ float block_max(float v) {
  v = fmaxf(v, __shfl_xor(v, 1, 64));
  v = fmaxf(v, __shfl_xor(v, 2, 64));
  v = fmaxf(v, __shfl_xor(v, 16, 64));
  v = fmaxf(v, __shfl_xor(v, 32, 64));
  return v;
}

constexpr int Q_BLOCKS = 4;  // 32x32 blocks per wave region (32 rows x 128 columns)

// One wave per region of 32 rows x 128 columns (256 bytes of bf16 per row).
// Load k (0..7) of lane l reads 16 bytes: row 4k + (l>>4), byte 16*(l&15) of
// the region row, so one load instruction covers four whole region rows.  A
// lane therefore holds 8 rows x 8 columns of block b = (l>>2)&3, and a block's
// amax is a max over its 16 lanes.  All eight loads are in flight before any
// arithmetic.  Regions past the last column block hold fewer blocks; the
// missing ones load nothing and store nothing.
__global__ void __launch_bounds__(256) quantize_kernel(const uint16_t* __restrict__ x, int64_t rows, int64_t cols,
                                                       uint8_t* __restrict__ q, float* __restrict__ scales,
                                                       int64_t n_regions) {
  const int lane = threadIdx.x & 63;
  const int piece = lane & 15, rsub = lane >> 4;
  const int b = piece >> 2, cpart = piece & 3;
  const int64_t cb_count = cols >> 5;
  const int64_t rg_per_row = (cb_count + Q_BLOCKS - 1) / Q_BLOCKS;
  const int64_t waves_total = (int64_t)gridDim.x * 4;
  for (int64_t reg = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); reg < n_regions; reg += waves_total) {
    const int64_t rb = reg / rg_per_row, g = reg - rb * rg_per_row;
    const int64_t cb = g * Q_BLOCKS + b;
    const bool cb_ok = cb < cb_count;
    const int64_t col = (cb_ok ? cb : cb_count - 1) * 32 + cpart * 8;  // stays inside x
    uint4 w[8];
    bool ok[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int64_t row = rb * 32 + 4 * k + rsub;
      ok[k] = cb_ok && row < rows;
      const int64_t rc = row < rows ? row : rows - 1;
      w[k] = ok[k] ? *reinterpret_cast<const uint4*>(x + rc * cols + col) : make_uint4(0, 0, 0, 0);
    }
    // values are re-derived from the loaded words where needed, so only the
    // 32 dwords of raw bf16 stay live
    float m = 0.0f;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const uint32_t ws[4] = {w[k].x, w[k].y, w[k].z, w[k].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) m = fmaxf(m, fmaxf(fabsf(bf16_lo(ws[i])), fabsf(bf16_hi(ws[i]))));
    }
    const float amax = block_max(m);
    const float s = amax / 448.0f;
    const bool recip = amax >= QUANT_RECIP_MIN_AMAX;  // wave-uniform per block
    const float r = recip ? 1.0f / s : 0.0f;
    auto quotient = [&](float xv, auto FAST_) __attribute__((always_inline)) -> float {
      if (decltype(FAST_)::value || recip) return quant_quotient_recip(xv, s, r);
      return quant_quotient_div(xv, s);
    };
    auto encode_store = [&](auto FAST_) __attribute__((always_inline)) {
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const uint32_t ws[4] = {w[k].x, w[k].y, w[k].z, w[k].w};
        uint32_t packed[2];
#pragma unroll
        for (int i = 0; i < 2; ++i)
          packed[i] = pack_e4m3x4(sat448(quotient(bf16_lo(ws[2 * i]), FAST_)),
                                  sat448(quotient(bf16_hi(ws[2 * i]), FAST_)),
                                  sat448(quotient(bf16_lo(ws[2 * i + 1]), FAST_)),
                                  sat448(quotient(bf16_hi(ws[2 * i + 1]), FAST_)));
        if (ok[k]) {
          const int64_t row = rb * 32 + 4 * k + rsub;
          store_codes8(q + row * cols + col, packed[0], packed[1]);
        }
      }
    };
    // every block of the wave on the reciprocal path (the common case): no
    // per-element branches
    if (__all(recip)) encode_store(std::true_type{});
    else encode_store(std::false_type{});
    if (cpart == 0 && rsub == 0 && cb_ok) scales[rb * cb_count + cb] = s;
  }
}

// Per-token groups (1 row x 32 columns): the same region mapping, but each of
// a lane's 8 rows is a quarter of its own group (the 8 columns cpart*8.. of
// row 4k + rsub), so a group's amax is a max over the 4 lanes that differ in
// lane bits 0 and 1, and every (row, group) gets its own scale and reciprocal.
// The quotient and the E4M3 rounding are the block quantizer's.
__global__ void __launch_bounds__(256) quantize_tg_kernel(const uint16_t* __restrict__ x, int64_t rows,
                                                          int64_t cols, uint8_t* __restrict__ q,
                                                          float* __restrict__ scales, int64_t n_regions) {
  const int lane = threadIdx.x & 63;
  const int piece = lane & 15, rsub = lane >> 4;
  const int b = piece >> 2, cpart = piece & 3;
  const int64_t cb_count = cols >> 5;
  const int64_t rg_per_row = (cb_count + Q_BLOCKS - 1) / Q_BLOCKS;
  const int64_t waves_total = (int64_t)gridDim.x * 4;
  for (int64_t reg = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); reg < n_regions; reg += waves_total) {
    const int64_t rb = reg / rg_per_row, g = reg - rb * rg_per_row;
    const int64_t cb = g * Q_BLOCKS + b;
    const bool cb_ok = cb < cb_count;
    const int64_t col = (cb_ok ? cb : cb_count - 1) * 32 + cpart * 8;  // stays inside x
    uint4 w[8];
    bool ok[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int64_t row = rb * 32 + 4 * k + rsub;
      ok[k] = cb_ok && row < rows;
      const int64_t rc = row < rows ? row : rows - 1;
      w[k] = ok[k] ? *reinterpret_cast<const uint4*>(x + rc * cols + col) : make_uint4(0, 0, 0, 0);
    }
    float sk[8], rk[8];
    bool all_recip = true;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const uint32_t ws[4] = {w[k].x, w[k].y, w[k].z, w[k].w};
      float m = 0.0f;
#pragma unroll
      for (int i = 0; i < 4; ++i) m = fmaxf(m, fmaxf(fabsf(bf16_lo(ws[i])), fabsf(bf16_hi(ws[i]))));
      m = fmaxf(m, __shfl_xor(m, 1, 64));
      m = fmaxf(m, __shfl_xor(m, 2, 64));
      sk[k] = m / 448.0f;
      const bool recip = m >= QUANT_RECIP_MIN_AMAX;
      rk[k] = recip ? 1.0f / sk[k] : 0.0f;
      all_recip = all_recip && recip;
    }
    auto quotient = [&](float xv, int k, auto FAST_) __attribute__((always_inline)) -> float {
      if (decltype(FAST_)::value || rk[k] != 0.0f) return quant_quotient_recip(xv, sk[k], rk[k]);
      return quant_quotient_div(xv, sk[k]);
    };
    auto encode_store = [&](auto FAST_) __attribute__((always_inline)) {
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const uint32_t ws[4] = {w[k].x, w[k].y, w[k].z, w[k].w};
        uint32_t packed[2];
#pragma unroll
        for (int i = 0; i < 2; ++i)
          packed[i] = pack_e4m3x4(sat448(quotient(bf16_lo(ws[2 * i]), k, FAST_)),
                                  sat448(quotient(bf16_hi(ws[2 * i]), k, FAST_)),
                                  sat448(quotient(bf16_lo(ws[2 * i + 1]), k, FAST_)),
                                  sat448(quotient(bf16_hi(ws[2 * i + 1]), k, FAST_)));
        if (ok[k]) {
          const int64_t row = rb * 32 + 4 * k + rsub;
          store_codes8(q + row * cols + col, packed[0], packed[1]);
          if (cpart == 0) scales[row * cb_count + cb] = sk[k];
        }
      }
    };
    if (__all(all_recip)) encode_store(std::true_type{});
    else encode_store(std::false_type{});
  }
}

// Power-of-two (E8M0) scales: per 32x32 block E = the smallest integer with
// 448 * 2^E >= amax, clamped to [-127, 127] (-127 for a zero block), stored as
// the byte E + 127; codes E4M3(x * 2^-E), the scaling exact.  With amax =
// (1 + m) 2^L (L its exponent, m its mantissa fraction), 448 * 2^(L-8) =
// 1.75 * 2^L, so E = L - 8 when m <= 0.75 and L - 7 otherwise; a subnormal or
// zero amax (L < -126) lands on the clamp.
__device__ __forceinline__ int e8m0_exponent(float amax) {
  const uint32_t u = __builtin_bit_cast(uint32_t, amax);
  const int ef = (int)(u >> 23);
  if (ef == 0) return -127;
  const int e = ef - 127 - 8 + ((u & 0x7FFFFFu) > 0x600000u ? 1 : 0);
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}
// 2^k for k in [-127, 127] (2^-127 is an fp32 subnormal).
__device__ __forceinline__ float exp2_int(int k) {
  return k >= -126 ? __builtin_bit_cast(float, (uint32_t)(k + 127) << 23) : __builtin_bit_cast(float, 0x00400000u);
}

// The block quantizer's region mapping (one wave per 32 rows x 128 columns).
__global__ void __launch_bounds__(256) quantize_e8m0_kernel(const uint16_t* __restrict__ x, int64_t rows,
                                                            int64_t cols, uint8_t* __restrict__ q,
                                                            uint8_t* __restrict__ e8, int64_t n_regions) {
  const int lane = threadIdx.x & 63;
  const int piece = lane & 15, rsub = lane >> 4;
  const int b = piece >> 2, cpart = piece & 3;
  const int64_t cb_count = cols >> 5;
  const int64_t rg_per_row = (cb_count + Q_BLOCKS - 1) / Q_BLOCKS;
  const int64_t waves_total = (int64_t)gridDim.x * 4;
  for (int64_t reg = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); reg < n_regions; reg += waves_total) {
    const int64_t rb = reg / rg_per_row, g = reg - rb * rg_per_row;
    const int64_t cb = g * Q_BLOCKS + b;
    const bool cb_ok = cb < cb_count;
    const int64_t col = (cb_ok ? cb : cb_count - 1) * 32 + cpart * 8;
    uint4 w[8];
    bool ok[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int64_t row = rb * 32 + 4 * k + rsub;
      ok[k] = cb_ok && row < rows;
      const int64_t rc = row < rows ? row : rows - 1;
      w[k] = ok[k] ? *reinterpret_cast<const uint4*>(x + rc * cols + col) : make_uint4(0, 0, 0, 0);
    }
    float m = 0.0f;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const uint32_t ws[4] = {w[k].x, w[k].y, w[k].z, w[k].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) m = fmaxf(m, fmaxf(fabsf(bf16_lo(ws[i])), fabsf(bf16_hi(ws[i]))));
    }
    const int E = e8m0_exponent(block_max(m));
    const float r = exp2_int(-E);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const uint32_t ws[4] = {w[k].x, w[k].y, w[k].z, w[k].w};
      uint32_t packed[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        packed[i] = pack_e4m3x4(sat448(bf16_lo(ws[2 * i]) * r), sat448(bf16_hi(ws[2 * i]) * r),
                                sat448(bf16_lo(ws[2 * i + 1]) * r), sat448(bf16_hi(ws[2 * i + 1]) * r));
      if (ok[k]) {
        const int64_t row = rb * 32 + 4 * k + rsub;
        store_codes8(q + row * cols + col, packed[0], packed[1]);
      }
    }
    if (cpart == 0 && rsub == 0 && cb_ok) e8[rb * cb_count + cb] = (uint8_t)(E + 127);
  }
}

hipError_t launch_quantize_e8m0(const void* x, int64_t rows, int64_t cols, void* q, void* e8, hipStream_t stream) {
  const int64_t n_regions = ((rows + 31) / 32) * ((cols / 32 + Q_BLOCKS - 1) / Q_BLOCKS);
  int64_t grid = (n_regions + 3) / 4;
  if (grid > 65536) grid = 65536;
  hipLaunchKernelGGL(quantize_e8m0_kernel, dim3((unsigned)grid), dim3(256), 0, stream, (const uint16_t*)x, rows,
                     cols, (uint8_t*)q, (uint8_t*)e8, n_regions);
  return hipGetLastError();
}

hipError_t launch_quantize_tg(const void* x, int64_t rows, int64_t cols, void* q, float* scales,
                              hipStream_t stream) {
  const int64_t n_regions = ((rows + 31) / 32) * ((cols / 32 + Q_BLOCKS - 1) / Q_BLOCKS);
  int64_t grid = (n_regions + 3) / 4;
  if (grid > 65536) grid = 65536;
  hipLaunchKernelGGL(quantize_tg_kernel, dim3((unsigned)grid), dim3(256), 0, stream, (const uint16_t*)x, rows, cols,
                     (uint8_t*)q, scales, n_regions);
  return hipGetLastError();
}

hipError_t launch_quantize(const void* x, int64_t rows, int64_t cols, void* q, float* scales, hipStream_t stream) {
  const int64_t n_regions = ((rows + 31) / 32) * ((cols / 32 + Q_BLOCKS - 1) / Q_BLOCKS);
  int64_t grid = (n_regions + 3) / 4;
  if (grid > 65536) grid = 65536;
  hipLaunchKernelGGL(quantize_kernel, dim3((unsigned)grid), dim3(256), 0, stream, (const uint16_t*)x, rows, cols,
                     (uint8_t*)q, scales, n_regions);
  return hipGetLastError();
}

}  // namespace fp8bs
