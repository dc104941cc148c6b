// Internal launchers: called by the C ABI layer after it has validated every
// argument.  Each enqueues its kernels on `stream` and returns the HIP status
// of the launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace coda {

constexpr int kRmsTileWidth = 128;  // features per partial sum-of-squares tile
constexpr int kLseTileWidth = 128;  // vocabulary entries per log-sum-exp tile

// Compute units of the current device (persistent GEMM grids launch one
// workgroup per compute unit); queried once per device.
int cu_count();

hipError_t launch_residual_partialrms_bf16(const uint16_t* A, const uint16_t* W,
                                           const uint16_t* res, uint16_t* h, float* psum, int M,
                                           int N, int K, hipStream_t stream);
hipError_t launch_rowscale_swiglu_bf16(const uint16_t* X, const uint16_t* Wg, const uint16_t* Wu,
                                       const float* r, uint16_t* out, int M, int N, int K,
                                       hipStream_t stream);
hipError_t launch_rowscale_swiglu_save_bf16(const uint16_t* X, const uint16_t* Wg,
                                            const uint16_t* Wu, const float* r, uint16_t* out,
                                            uint16_t* gu, int M, int N, int K, hipStream_t stream);
hipError_t launch_swiglu_bwd_bf16(const uint16_t* dY, const uint16_t* WdT, const uint16_t* gu,
                                  uint16_t* dz, float* pdot, int M, int N, int K,
                                  hipStream_t stream);
hipError_t launch_rmsnorm_bwd_bf16(const uint16_t* dz, const uint16_t* W2T, const uint16_t* h,
                                   const uint16_t* dY, const float* r, const float* c,
                                   uint16_t* dh, int M, int N, int K, hipStream_t stream);
hipError_t launch_gemm_wgrad_gamma_bf16(const uint16_t* A, const uint16_t* B, const uint16_t* W,
                                       const float* gamma, uint16_t* dW, float* pdg, int M, int N,
                                       int K, hipStream_t stream);
hipError_t launch_dgamma_reduce(const float* pdg, int P, int N, const float* gamma_div,
                                float* dgamma, hipStream_t stream);
hipError_t launch_col_dot_partial(const uint16_t* X, const uint16_t* Y, int M, int N, float* pdg,
                                  hipStream_t stream);
hipError_t launch_rms_bwd_reduce(const float* pdot, int T, int M, const float* r, int N, float* c,
                                 hipStream_t stream);
hipError_t launch_swiglu_bwd(const uint16_t* dout, const uint16_t* gu, uint16_t* dz, int M, int N,
                             hipStream_t stream);
hipError_t launch_rmsnorm_bwd(const uint16_t* G, const uint16_t* h, const uint16_t* dY, float eps,
                              uint16_t* dh, int M, int N, hipStream_t stream);
hipError_t launch_rope_bf16(const uint16_t* X, const uint16_t* W, const float* r,
                            const float* rcos, const float* rsin, const int* pos, int max_pos,
                            uint16_t* out, int M, int K, int n_q, int n_kv, int head_dim,
                            hipStream_t stream);
// plain bf16 GEMM on the 128 x 384 block tile, and whether a shape should use it
hipError_t launch_gemm_plain_bf16_wide(const uint16_t* A, const uint16_t* W, uint16_t* C, int M,
                                       int N, int K, hipStream_t stream);
bool prefer_wide_tile(int M, int N);
// Plain GEMM with the reduction split in `parts` ranges of K / parts columns:
// fp32 partial products to ws [parts, M, N], then C = bf16 of their sum.
hipError_t launch_gemm_splitk_bf16(const uint16_t* A, const uint16_t* W, uint16_t* C, float* ws,
                                   int M, int N, int K, int parts, hipStream_t stream);
// same operation on the 128 x 384 block tile (QKV width a multiple of 384)
hipError_t launch_rope_bf16_wide(const uint16_t* X, const uint16_t* W, const float* r,
                                 const float* rcos, const float* rsin, const int* pos, int max_pos,
                                 uint16_t* out, int M, int K, int n_q, int n_kv,
                                 hipStream_t stream);
hipError_t launch_rope_tables(double theta, int max_pos, int head_dim, float* rcos, float* rsin,
                              hipStream_t stream);
hipError_t launch_attention_fwd(const uint16_t* qkv, uint16_t* o, int M, int L, int nq, int nkv,
                                int head_dim, hipStream_t stream);
hipError_t launch_block_lse_bf16(const uint16_t* X, const uint16_t* W, const float* r,
                                 const int* labels, float* tmax, float* tsum, float* label_logit,
                                 int M, int V, int K, hipStream_t stream);
hipError_t launch_lse_merge(const float* tmax, const float* tsum, const float* label_logit,
                            const int* labels, int T, int M, int V, float* lse, float* loss,
                            hipStream_t stream);
hipError_t launch_gemm_plain_bf16(const uint16_t* A, const uint16_t* W, uint16_t* C, int M, int N,
                                  int K, hipStream_t stream);

hipError_t launch_residual_partialrms_fp8(const uint8_t* A, const uint8_t* W, const float* a_scale,
                                          const float* w_scale, const uint16_t* res, uint16_t* h,
                                          float* psum, const float* h8_scale, uint8_t* h8,
                                          float* pamax, int M, int N, int K, hipStream_t stream);
hipError_t launch_rowscale_swiglu_fp8(const uint8_t* X, const float* x_scale, const uint8_t* Wg,
                                      const uint8_t* Wu, const float* wg_scale,
                                      const float* wu_scale, const float* r, uint16_t* out, int M,
                                      int N, int K, hipStream_t stream);

hipError_t launch_rms_reduce(const float* psum, const float* pamax, int T, int M, int N, float eps,
                             float* r, float* h_amax, float* h8_scale_out, hipStream_t stream);
hipError_t launch_transpose_bf16(const uint16_t* src, const float* row_scale, int rows, int cols,
                                 uint16_t* dst, int ld_dst, hipStream_t stream);
hipError_t launch_fold_gamma(const uint16_t* W, const float* gamma, uint16_t* W_out, int N, int K,
                             hipStream_t stream);
hipError_t launch_residual_add(const uint16_t* y, const uint16_t* res, uint16_t* h, int64_t count,
                               hipStream_t stream);
hipError_t launch_rmsnorm(const uint16_t* h, const float* gamma, float eps, uint16_t* out, int M,
                          int N, hipStream_t stream);
hipError_t launch_swiglu(const uint16_t* gu, uint16_t* out, int M, int N, hipStream_t stream);
hipError_t launch_rope_apply(uint16_t* qkv, const float* rcos, const float* rsin, const int* pos,
                             int max_pos, int M, int n_q, int n_kv, int head_dim,
                             hipStream_t stream);
hipError_t launch_gemm_plain_fp8(const uint8_t* A, const uint8_t* W, const float* a_scale,
                                 const float* w_scale, uint16_t* C, int M, int N, int K, int ldc,
                                 hipStream_t stream);
hipError_t launch_quantize_e4m3(const uint16_t* x, const float* s_in, uint8_t* out, int64_t count,
                                float* amax, float* s_out, hipStream_t stream);
hipError_t launch_ce_rows(const uint16_t* z, const int* labels, float* lse, float* loss, int M,
                          int V, hipStream_t stream);

}  // namespace coda
