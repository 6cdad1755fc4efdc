// Fused residual add + RMSNorm + per-token-group E4M3 quantizer for gfx950.
//
// "AI Infra 进阶：如何让大模型输出确定的结果" (aif.amtbbs.org), part 三:
// section 1 defines the norm per token, y = x / sqrt(mean(x^2) + eps) * gamma,
// and notes that one token's hidden vector must be reduced inside one thread
// block with a reduction shape that does not change with the number of
// tokens; section 2's table lists the serving forms, among them the residual
// ("fused add") form and the fusion of the norm with per-token-group FP8
// quantization in one kernel.  The quantizer is the one of quantize.hip with
// groups of 1 row x 32 columns (DeepGEMM write-up on hncyxsy.com, sections
// 2.1, 2.2, 5.2).
//
// Per row (all fp32, round to nearest even):
//   h_i = bf16(x_i + r_i)            residual form only; h is written back to r
//   ss  = sum_i h_i^2                fixed order, see below
//   rinv = 1 / sqrt(ss / d + eps)
//   y_i = bf16((h_i * rinv) * gamma_i)
//   per 32-column group: amax, s = amax / 448, codes E4M3(y / s)
// The reduction shape depends on d only.  A row belongs to WPR waves (1, 2
// or 4, from d); lane l of the row's wave k owns columns
// 512*(WPR*i + k) + 8*l .. +7 for i = 0, 1, ...; it sums its squares in that
// order (i ascending, then column), the 64 lane sums of a wave are combined by
// a butterfly over lane distances 32, 16, 8, 4, 2, 1 (the same bits in every
// lane), and the WPR wave sums are added in wave order through LDS.  So a
// row's outputs never depend on the other rows or on how many there are
// (batch invariance).
//
// 256-thread workgroups of 4 waves hold 4 / WPR rows.  The row stays in
// registers (h as packed bf16, 8*NL values per lane) between the reduction and
// the quantization, so x and the residual are read once.  The kernel is bound
// by HBM traffic.
#include "common.hpp"

#include <type_traits>

namespace fp8bs {

constexpr int RMS_NL = 8;  // 16-byte pieces per lane and wave (64 x 8 x 8 = 4096 columns)

template <int NL, int WPR>
__global__ void __launch_bounds__(256) rmsnorm_quant_tg_kernel(const uint16_t* __restrict__ x,
                                                               uint16_t* __restrict__ res,
                                                               const uint16_t* __restrict__ gamma, float eps,
                                                               int64_t rows, int64_t d, uint8_t* __restrict__ q,
                                                               float* __restrict__ scales, uint16_t* __restrict__ y) {
  constexpr int RPW = 4 / WPR;  // rows per workgroup
  __shared__ float part[2][4];  // wave sums, double-buffered by iteration
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int wk = w % WPR;       // this wave's share of its row
  const int64_t cb_count = d >> 5;
  const float d_f = (float)d;   // exact for d <= 2^24
  int iter = 0;
  // every wave runs the same number of iterations (the barrier below); rows
  // past the end load and store nothing
  for (int64_t base = (int64_t)blockIdx.x * RPW; base < rows; base += (int64_t)gridDim.x * RPW, ++iter) {
    const int64_t row = base + w / WPR;
    const bool row_ok = row < rows;
    const int64_t rrow = row_ok ? row : rows - 1;
    const uint16_t* xr = x + rrow * d;
    uint4 h[NL];
    bool ok[NL];
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int64_t col = (int64_t)(WPR * i + wk) * 512 + lane * 8;
      ok[i] = row_ok && col < d;
      h[i] = ok[i] ? *reinterpret_cast<const uint4*>(xr + col) : make_uint4(0, 0, 0, 0);
    }
    // gamma is loaded with the row, before the reduction: a row's latency then
    // holds one round trip to memory, not two
    uint4 gv[NL];
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int64_t col = (int64_t)(WPR * i + wk) * 512 + lane * 8;
      gv[i] = ok[i] ? *reinterpret_cast<const uint4*>(gamma + col) : make_uint4(0, 0, 0, 0);
    }
    if (res != nullptr) {
      uint16_t* rr = res + rrow * d;
      uint4 rv[NL];
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        const int64_t col = (int64_t)(WPR * i + wk) * 512 + lane * 8;
        rv[i] = ok[i] ? *reinterpret_cast<const uint4*>(rr + col) : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        // the fp32 sum of two bf16 values rounds to bf16 exactly as their exact sum does
        uint32_t* hw = reinterpret_cast<uint32_t*>(&h[i]);
        const uint32_t* rw = reinterpret_cast<const uint32_t*>(&rv[i]);
#pragma unroll
        for (int j = 0; j < 4; ++j)
          hw[j] = bf16_rne(bf16_lo(hw[j]) + bf16_lo(rw[j])) | (bf16_rne(bf16_hi(hw[j]) + bf16_hi(rw[j])) << 16);
        if (ok[i]) *reinterpret_cast<uint4*>(rr + (int64_t)(WPR * i + wk) * 512 + lane * 8) = h[i];
      }
    }

    // sum of squares: this lane's columns in order, the butterfly, then the row's waves in order
    float ss = 0.0f;
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const uint32_t* hw = reinterpret_cast<const uint32_t*>(&h[i]);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float a = bf16_lo(hw[j]), b = bf16_hi(hw[j]);
        ss = __builtin_fmaf(a, a, ss);
        ss = __builtin_fmaf(b, b, ss);
      }
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) ss = ss + __shfl_xor(ss, m, 64);
    if constexpr (WPR > 1) {
      float* pb = part[iter & 1];
      if (lane == 0) pb[w] = ss;
      __syncthreads();
      const int w0 = w - wk;
      ss = pb[w0];
#pragma unroll
      for (int k = 1; k < WPR; ++k) ss = ss + pb[w0 + k];
    }
    const float rinv = 1.0f / __builtin_sqrtf(ss / d_f + eps);

#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int64_t col = (int64_t)(WPR * i + wk) * 512 + lane * 8;
      const uint4 g = gv[i];
      const uint32_t* hw = reinterpret_cast<const uint32_t*>(&h[i]);
      const uint32_t gw[4] = {g.x, g.y, g.z, g.w};
      uint32_t yw[4];
      float m = 0.0f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t lo = bf16_rne((bf16_lo(hw[j]) * rinv) * bf16_lo(gw[j]));
        const uint32_t hi = bf16_rne((bf16_hi(hw[j]) * rinv) * bf16_hi(gw[j]));
        yw[j] = lo | (hi << 16);
        m = fmaxf(m, fmaxf(fabsf(bf16_lo(yw[j])), fabsf(bf16_hi(yw[j]))));
      }
      if (y != nullptr && ok[i])
        *reinterpret_cast<uint4*>(y + row * d + col) = make_uint4(yw[0], yw[1], yw[2], yw[3]);
      // a group is the 32 columns of four adjacent lanes
      m = fmaxf(m, __shfl_xor(m, 1, 64));
      m = fmaxf(m, __shfl_xor(m, 2, 64));
      const float s = m / 448.0f;
      const bool recip = m >= QUANT_RECIP_MIN_AMAX;
      const float r = recip ? 1.0f / s : 0.0f;
      auto encode = [&](auto FAST_) __attribute__((always_inline)) -> uint2 {
        auto quo = [&](float v) __attribute__((always_inline)) -> float {
          if (decltype(FAST_)::value || recip) return quant_quotient_recip(v, s, r);
          return quant_quotient_div(v, s);
        };
        uint32_t p[2];
#pragma unroll
        for (int k = 0; k < 2; ++k)
          p[k] = pack_e4m3x4(sat448(quo(bf16_lo(yw[2 * k]))), sat448(quo(bf16_hi(yw[2 * k]))),
                             sat448(quo(bf16_lo(yw[2 * k + 1]))), sat448(quo(bf16_hi(yw[2 * k + 1]))));
        return make_uint2(p[0], p[1]);
      };
      // lanes with nothing to store have m = 0 and would take the division
      // path; they only decide which path the wave takes
      const uint2 codes = __all(recip || !ok[i]) ? encode(std::true_type{}) : encode(std::false_type{});
      if (ok[i]) {
        *reinterpret_cast<uint2*>(q + row * d + col) = codes;
        if ((lane & 3) == 0) scales[row * cb_count + (col >> 5)] = s;
      }
    }
  }
}

template <int NL, int WPR>
static void launch_rms_t(const void* x, void* res, const void* gamma, float eps, int64_t rows, int64_t d, void* q,
                         float* scales, void* y, hipStream_t stream) {
  constexpr int RPW = 4 / WPR;
  int64_t grid = (rows + RPW - 1) / RPW;
  if (grid > 65536) grid = 65536;
  hipLaunchKernelGGL((rmsnorm_quant_tg_kernel<NL, WPR>), dim3((unsigned)grid), dim3(256), 0, stream,
                     (const uint16_t*)x, (uint16_t*)res, (const uint16_t*)gamma, eps, rows, d, (uint8_t*)q, scales,
                     (uint16_t*)y);
}

int rmsnorm_max_cols() { return 512 * RMS_NL * 4; }

hipError_t launch_rmsnorm_quantize_tg(const void* x, void* residual, const void* gamma, float eps, int64_t rows,
                                      int64_t d, void* q, float* scales, void* y, hipStream_t stream) {
  if (d <= 512) launch_rms_t<1, 1>(x, residual, gamma, eps, rows, d, q, scales, y, stream);
  else if (d <= 1024) launch_rms_t<2, 1>(x, residual, gamma, eps, rows, d, q, scales, y, stream);
  else if (d <= 2048) launch_rms_t<4, 1>(x, residual, gamma, eps, rows, d, q, scales, y, stream);
  else if (d <= 4096) launch_rms_t<RMS_NL, 1>(x, residual, gamma, eps, rows, d, q, scales, y, stream);
  else if (d <= 8192) launch_rms_t<RMS_NL, 2>(x, residual, gamma, eps, rows, d, q, scales, y, stream);
  else launch_rms_t<RMS_NL, 4>(x, residual, gamma, eps, rows, d, q, scales, y, stream);
  return hipGetLastError();
}

}  // namespace fp8bs
