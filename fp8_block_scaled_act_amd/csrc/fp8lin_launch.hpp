// fp8lin_launch.hpp -- internal launchers behind the C ABI (not exported).
// Every launcher only enqueues on `st`; arguments were validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8lin {

void launch_quant_rowgroup(const void* x, int64_t ngroups, uint8_t* q, float* s, hipStream_t st);
void launch_quant_block(const void* w, int64_t N, int64_t K, uint8_t* q, float* s, hipStream_t st);
void launch_quant_transpose_bf16(const void* x, int64_t T, int64_t C, uint8_t* qT, float* sT,
                                 uint8_t* qrow, float* srow, hipStream_t st);
void launch_quant_transpose_fp8(const uint8_t* src, const float* srow, int64_t T, int64_t C,
                                uint8_t* qT, float* sT, hipStream_t st);
void launch_transpose_codes(const uint8_t* src, const float* s, int64_t R, int64_t C, uint8_t* dst, float* sT,
                            hipStream_t st);
// Diagnostic: the block-scaled forward product on FP8 MFMA form `form` (0..3)
// or the fp16 control (4), fp32 output [M][N]; N % 128 == 0, K % 128 == 0, M >= 1.
int mfma_probe_tile(int form);
void launch_gemm_fwd_mfma_probe(const uint8_t* xq, const float* sx, const uint8_t* wq, const float* sw, int64_t M,
                                int64_t N, int64_t K, float* y, int form, hipStream_t st);
void launch_encode_probe(const float* in, int64_t n, uint8_t* out, int method, hipStream_t st);
void launch_decode_probe(const uint8_t* in, int64_t n, float* out, int method, hipStream_t st);
void launch_math_probe(const float* in, int64_t n, float* out, int fn, hipStream_t st);
void launch_flag_probe(const float* v, int64_t n, float lim, float* out, hipStream_t st);

// Producer operators fused with 1x128 quantization (K <= 16384 for RMSNorm).
void launch_rmsnorm_quant(const void* x, const void* gamma, int64_t M, int64_t K, float eps, uint8_t* q,
                          float* s, float* rstd, hipStream_t st);
// RMSNorm backward: dx, and dgamma (when non-NULL) through ws [ceil(M/128)][K] fp64.
void launch_rmsnorm_bwd(const void* x, const void* gamma, const float* rstd, const void* dy, int64_t M, int64_t K,
                        void* dx, float* dgamma, double* ws, hipStream_t st);
void launch_swiglu_quant(const void* gate, const void* up, int64_t ld, int64_t M, int64_t F, uint8_t* q,
                         float* s, hipStream_t st);
void launch_swiglu_bwd(const void* gate, const void* up, int64_t ld, const void* dh, int64_t M, int64_t F,
                       void* dgu, hipStream_t st);
void launch_swiglu_bwd_quant(const void* gate, const void* up, int64_t ld, const void* dh, int64_t T, int64_t F,
                             uint8_t* q, float* s, uint8_t* qT, float* sT, hipStream_t st);

void launch_fill_zero_bf16(void* c, int64_t n, hipStream_t st);
void launch_gemm_fwd(const uint8_t* xq, const float* sx, const uint8_t* wq, const float* sw,
                     int64_t M, int64_t N, int64_t K, void* y, hipStream_t st);
// The forward GEMM on one kernel for every M (rows bit-identical across calls).
void launch_gemm_fwd_unified(const uint8_t* xq, const float* sx, const uint8_t* wq, const float* sw,
                             int64_t M, int64_t N, int64_t K, void* y, hipStream_t st);
// Decode layout of W (fp8_weight_pack) and the forward GEMM on it
// (M <= 64, K % 256 == 0, K <= 16384).
void launch_pack_decode(const uint8_t* wq, int64_t N, int64_t K, uint8_t* wqp, hipStream_t st);
void launch_gemm_fwd_packed(const uint8_t* xq, const float* sx, const uint8_t* wqp, const float* sw,
                            int64_t M, int64_t N, int64_t K, void* y, hipStream_t st);
// Split-K variant for few output columns: S = splitk_splits(N, K) workgroups
// per 64-column block, fp32 partials in ws [S][M][N] (unused when S == 1).
int64_t splitk_splits(int64_t N, int64_t K);
void launch_gemm_fwd_packed_splitk(const uint8_t* xq, const float* sx, const uint8_t* wqp, const float* sw,
                                   int64_t M, int64_t N, int64_t K, void* y, float* ws, hipStream_t st);
// Size of the per-GPU device array behind the allocation-free split-K entry
// point, and its device address on the current device (looked up once per
// device).
constexpr int64_t kSplitkScratchBytes = int64_t(4) << 20;
hipError_t splitk_scratch(void** out);
void launch_gemm_dgrad(const uint8_t* dyq, const float* sdy, const uint8_t* wq, const float* sw,
                       int64_t T, int64_t N, int64_t K, void* dx, hipStream_t st);
void launch_gemm_wgrad(const uint8_t* dyTq, const float* sdyT, const uint8_t* xTq, const float* sxT,
                       int64_t N, int64_t K, int64_t T, void* dw, hipStream_t st);

// 4-bit (MXFP4) weights: quantization (K % 32 == 0) and the rollout GEMM
// (K % 128 == 0, K <= gemm_w4_max_k(), M, N >= 1).
void launch_mxfp4_quant(const void* w, int64_t N, int64_t K, uint8_t* codes, uint8_t* scales, hipStream_t st);
int64_t gemm_w4_max_k();
void launch_gemm_fwd_w4(const uint8_t* xq, const float* sx, const uint8_t* w4, const uint8_t* s4, int64_t M,
                        int64_t N, int64_t K, void* y, hipStream_t st);

}  // namespace fp8lin
