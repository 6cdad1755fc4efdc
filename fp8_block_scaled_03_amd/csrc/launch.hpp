// Internal launcher declarations (not part of the public ABI).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8bs {
hipError_t launch_quantize(const void* x, int64_t rows, int64_t cols, void* q, float* scales, hipStream_t stream);
// per-token groups (1 x 32): scales [rows, cols/32]
hipError_t launch_quantize_tg(const void* x, int64_t rows, int64_t cols, void* q, float* scales,
                              hipStream_t stream);
// k_major_b: the weight is B^T [N, K] with scales [N/32, K/32] instead of
// B [K, N] with scales [K/32, N/32] (for grouped calls, per group).
// act_tg: A's scales are per token group, [M, K/32] (one per row and K-block).
hipError_t launch_gemm_tile(const void* a, const float* sa, const void* b, const float* sb, void* c, int64_t M,
                            int64_t N, int64_t K, bool k_major_b, bool act_tg, hipStream_t stream);
hipError_t launch_gemm_smallm(const void* a, const float* sa, const void* b, const float* sb, void* c, int64_t M,
                              int64_t N, int64_t K, bool k_major_b, bool act_tg, hipStream_t stream);
hipError_t launch_gemm_grouped(const void* a, const float* sa, const void* b, const float* sb,
                               const int32_t* offsets, int G, void* c, int64_t M_total, int64_t N, int64_t K,
                               bool k_major_b, hipStream_t stream);
hipError_t set_gemm_attributes();
// residual add (residual may be null) + RMSNorm + per-token-group quantizer;
// y (the bf16 normalised rows) may be null.  d <= rmsnorm_max_cols().
hipError_t launch_rmsnorm_quantize_tg(const void* x, void* residual, const void* gamma, float eps, int64_t rows,
                                      int64_t d, void* q, float* scales, void* y, hipStream_t stream);
int rmsnorm_max_cols();
// power-of-two (E8M0) block scales: one byte E + 127 per 32x32 block
hipError_t launch_quantize_e8m0(const void* x, int64_t rows, int64_t cols, void* q, void* e8, hipStream_t stream);
hipError_t launch_gemm_e8m0_nt(const void* a, const void* ea, const void* bt, const void* ebt, void* c, int64_t M,
                               int64_t N, int64_t K, hipStream_t stream);
hipError_t set_gemm_e8m0_attributes();

// M at or below which the bandwidth-oriented small-M kernel runs.  Both kernels
// follow the same per-element recipe, so the switch never changes a result.
constexpr int64_t SMALL_M_MAX = 64;
}  // namespace fp8bs
