// C ABI of the E4M3 block-scaled GEMM library (see include/fp8bs.h).
// Host-side argument checks, then one launch on the caller's stream.
#include "fp8bs.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <mutex>

#include "launch.hpp"

namespace {

constexpr int64_t MAX_DIM = int64_t(1) << 30;

bool aligned(const void* p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

// Kernel attributes (dynamic LDS above the default) are set once per process and
// per device the first time a GEMM is launched on it.
fp8bs_status ensure_attributes() {
  static std::mutex mu;
  static bool done[64] = {false};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return FP8BS_EHIP;
  if (dev < 0 || dev >= 64) return FP8BS_EHIP;
  std::lock_guard<std::mutex> lock(mu);
  if (!done[dev]) {
    if (fp8bs::set_gemm_attributes() != hipSuccess) return FP8BS_EHIP;
    if (fp8bs::set_gemm_e8m0_attributes() != hipSuccess) return FP8BS_EHIP;
    done[dev] = true;
  }
  return FP8BS_OK;
}

fp8bs_status from_hip(hipError_t e) { return e == hipSuccess ? FP8BS_OK : FP8BS_EHIP; }

fp8bs_status check_gemm_dims(int64_t M, int64_t N, int64_t K) {
  if (M < 0 || N < 0 || K < 0) return FP8BS_EINVAL;
  if (M > MAX_DIM || N > MAX_DIM || K > MAX_DIM) return FP8BS_ESHAPE;
  if (K % 32 || N % 32) return FP8BS_ESHAPE;
  return FP8BS_OK;
}

}  // namespace

extern "C" {

const char* fp8bs_status_str(fp8bs_status s) {
  switch (s) {
    case FP8BS_OK: return "FP8BS_OK";
    case FP8BS_EINVAL: return "FP8BS_EINVAL: invalid argument (null pointer, negative size or bad group count)";
    case FP8BS_ESHAPE: return "FP8BS_ESHAPE: a dimension is not a multiple of 32 or is too large";
    case FP8BS_EALIGN: return "FP8BS_EALIGN: matrix pointers must be 16-byte aligned, scales 4-byte aligned";
    case FP8BS_EHIP: return "FP8BS_EHIP: the HIP runtime reported an error";
    case FP8BS_ENOSYS: return "FP8BS_ENOSYS: not available on this device";
  }
  return "FP8BS: unknown status";
}

static fp8bs_status quantize_common(const void* x_bf16, int64_t rows, int64_t cols, void* q_e4m3, float* scales,
                                    bool token_groups, void* stream) {
  if (rows < 0 || cols < 0) return FP8BS_EINVAL;
  if (rows > MAX_DIM || cols > MAX_DIM) return FP8BS_ESHAPE;
  if (cols % 32) return FP8BS_ESHAPE;
  if (rows == 0 || cols == 0) return FP8BS_OK;
  if (!x_bf16 || !q_e4m3 || !scales) return FP8BS_EINVAL;
  if (!aligned(x_bf16, 16) || !aligned(q_e4m3, 16) || !aligned(scales, 4)) return FP8BS_EALIGN;
  if (token_groups)
    return from_hip(fp8bs::launch_quantize_tg(x_bf16, rows, cols, q_e4m3, scales, (hipStream_t)stream));
  return from_hip(fp8bs::launch_quantize(x_bf16, rows, cols, q_e4m3, scales, (hipStream_t)stream));
}

fp8bs_status fp8bs_quantize(const void* x_bf16, int64_t rows, int64_t cols, void* q_e4m3, float* scales,
                            void* stream) {
  return quantize_common(x_bf16, rows, cols, q_e4m3, scales, false, stream);
}

fp8bs_status fp8bs_quantize_tg(const void* x_bf16, int64_t rows, int64_t cols, void* q_e4m3, float* scales,
                               void* stream) {
  return quantize_common(x_bf16, rows, cols, q_e4m3, scales, true, stream);
}

fp8bs_status fp8bs_rmsnorm_quantize_tg(const void* x_bf16, void* residual_bf16, const void* gamma_bf16, float eps,
                                       int64_t rows, int64_t d, void* q_e4m3, float* scales, void* y_bf16,
                                       void* stream) {
  if (rows < 0 || d < 0) return FP8BS_EINVAL;
  if (!(eps >= 0.0f) || !std::isfinite(eps)) return FP8BS_EINVAL;
  if (rows > MAX_DIM || d % 32 || d > fp8bs::rmsnorm_max_cols()) return FP8BS_ESHAPE;
  if (rows == 0 || d == 0) return FP8BS_OK;
  if (!x_bf16 || !gamma_bf16 || !q_e4m3 || !scales) return FP8BS_EINVAL;
  if (!aligned(x_bf16, 16) || !aligned(gamma_bf16, 16) || !aligned(q_e4m3, 16) || !aligned(scales, 4) ||
      (residual_bf16 && !aligned(residual_bf16, 16)) || (y_bf16 && !aligned(y_bf16, 16)))
    return FP8BS_EALIGN;
  return from_hip(fp8bs::launch_rmsnorm_quantize_tg(x_bf16, residual_bf16, gamma_bf16, eps, rows, d, q_e4m3, scales,
                                                    y_bf16, (hipStream_t)stream));
}

fp8bs_status fp8bs_quantize_e8m0(const void* x_bf16, int64_t rows, int64_t cols, void* q_e4m3, void* e8m0,
                                 void* stream) {
  if (rows < 0 || cols < 0) return FP8BS_EINVAL;
  if (rows > MAX_DIM || cols > MAX_DIM) return FP8BS_ESHAPE;
  if (cols % 32) return FP8BS_ESHAPE;
  if (rows == 0 || cols == 0) return FP8BS_OK;
  if (!x_bf16 || !q_e4m3 || !e8m0) return FP8BS_EINVAL;
  if (!aligned(x_bf16, 16) || !aligned(q_e4m3, 16)) return FP8BS_EALIGN;
  return from_hip(fp8bs::launch_quantize_e8m0(x_bf16, rows, cols, q_e4m3, e8m0, (hipStream_t)stream));
}

fp8bs_status fp8bs_gemm_e8m0_nt(const void* a, const void* ea, const void* bt, const void* ebt, void* c_bf16,
                                int64_t M, int64_t N, int64_t K, void* stream) {
  fp8bs_status st = check_gemm_dims(M, N, K);
  if (st != FP8BS_OK) return st;
  if (K % 128) return FP8BS_ESHAPE;
  if (M == 0 || N == 0) return FP8BS_OK;
  if (!c_bf16) return FP8BS_EINVAL;
  if (K > 0 && (!a || !ea || !bt || !ebt)) return FP8BS_EINVAL;
  if (!aligned(c_bf16, 16) || (K > 0 && (!aligned(a, 16) || !aligned(bt, 16) || !aligned(ea, 4) || !aligned(ebt, 4))))
    return FP8BS_EALIGN;
  st = ensure_attributes();
  if (st != FP8BS_OK) return st;
  return from_hip(fp8bs::launch_gemm_e8m0_nt(a, ea, bt, ebt, c_bf16, M, N, K, (hipStream_t)stream));
}

static fp8bs_status gemm_common(const void* a, const float* sa, const void* b, const float* sb, void* c_bf16,
                                int64_t M, int64_t N, int64_t K, bool k_major_b, bool act_tg, void* stream) {
  fp8bs_status st = check_gemm_dims(M, N, K);
  if (st != FP8BS_OK) return st;
  if (M == 0 || N == 0) return FP8BS_OK;
  if (!c_bf16) return FP8BS_EINVAL;
  if (K > 0 && (!a || !sa || !b || !sb)) return FP8BS_EINVAL;
  if (!aligned(c_bf16, 16) || (K > 0 && (!aligned(a, 16) || !aligned(b, 16) || !aligned(sa, 4) || !aligned(sb, 4))))
    return FP8BS_EALIGN;
  st = ensure_attributes();
  if (st != FP8BS_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  if (M <= fp8bs::SMALL_M_MAX)
    return from_hip(fp8bs::launch_gemm_smallm(a, sa, b, sb, c_bf16, M, N, K, k_major_b, act_tg, s));
  return from_hip(fp8bs::launch_gemm_tile(a, sa, b, sb, c_bf16, M, N, K, k_major_b, act_tg, s));
}

static fp8bs_status grouped_common(const void* a, const float* sa, const void* b, const float* sb,
                                   const int32_t* offsets_dev, int32_t G, void* c_bf16, int64_t M_total, int64_t N,
                                   int64_t K, bool k_major_b, void* stream) {
  if (G < 1 || G > FP8BS_MAX_GROUPS) return FP8BS_EINVAL;
  fp8bs_status st = check_gemm_dims(M_total, N, K);
  if (st != FP8BS_OK) return st;
  if (M_total % 32) return FP8BS_ESHAPE;
  if (!offsets_dev) return FP8BS_EINVAL;
  if (!aligned(offsets_dev, 4)) return FP8BS_EALIGN;
  if (M_total == 0 || N == 0) return FP8BS_OK;
  if (!c_bf16) return FP8BS_EINVAL;
  if (K > 0 && (!a || !sa || !b || !sb)) return FP8BS_EINVAL;
  if (!aligned(c_bf16, 16) || (K > 0 && (!aligned(a, 16) || !aligned(b, 16) || !aligned(sa, 4) || !aligned(sb, 4))))
    return FP8BS_EALIGN;
  st = ensure_attributes();
  if (st != FP8BS_OK) return st;
  return from_hip(fp8bs::launch_gemm_grouped(a, sa, b, sb, offsets_dev, G, c_bf16, M_total, N, K, k_major_b,
                                             (hipStream_t)stream));
}

fp8bs_status fp8bs_gemm(const void* a, const float* sa, const void* b, const float* sb, void* c_bf16, int64_t M,
                        int64_t N, int64_t K, void* stream) {
  return gemm_common(a, sa, b, sb, c_bf16, M, N, K, false, false, stream);
}

fp8bs_status fp8bs_gemm_nt(const void* a, const float* sa, const void* bt, const float* sbt, void* c_bf16,
                           int64_t M, int64_t N, int64_t K, void* stream) {
  return gemm_common(a, sa, bt, sbt, c_bf16, M, N, K, true, false, stream);
}

fp8bs_status fp8bs_gemm_tg(const void* a, const float* sa_rows, const void* b, const float* sb, void* c_bf16,
                           int64_t M, int64_t N, int64_t K, void* stream) {
  return gemm_common(a, sa_rows, b, sb, c_bf16, M, N, K, false, true, stream);
}

fp8bs_status fp8bs_gemm_tg_nt(const void* a, const float* sa_rows, const void* bt, const float* sbt, void* c_bf16,
                              int64_t M, int64_t N, int64_t K, void* stream) {
  return gemm_common(a, sa_rows, bt, sbt, c_bf16, M, N, K, true, true, stream);
}

fp8bs_status fp8bs_grouped_gemm(const void* a, const float* sa, const void* b, const float* sb,
                                const int32_t* offsets_dev, int32_t G, void* c_bf16, int64_t M_total, int64_t N,
                                int64_t K, void* stream) {
  return grouped_common(a, sa, b, sb, offsets_dev, G, c_bf16, M_total, N, K, false, stream);
}

fp8bs_status fp8bs_grouped_gemm_nt(const void* a, const float* sa, const void* bt, const float* sbt,
                                   const int32_t* offsets_dev, int32_t G, void* c_bf16, int64_t M_total, int64_t N,
                                   int64_t K, void* stream) {
  return grouped_common(a, sa, bt, sbt, offsets_dev, G, c_bf16, M_total, N, K, true, stream);
}

}  // extern "C"
