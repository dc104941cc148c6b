// C ABI of libcoda (declared in include/coda.h): argument validation, the
// gfx950 device check, and the launches.  Validation runs before any HIP
// runtime call, so every argument error is reported without touching a GPU.
// No C++ exception crosses the boundary.

#include "coda.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstring>

#include "launch.hpp"

namespace {

constexpr int kAbiVersion = 1;
constexpr int kMaxDevices = 64;
// 0 = unknown, 1 = gfx950, 2 = other / error
std::atomic<int> g_arch_state[kMaxDevices];
std::atomic<int> g_cu_count[kMaxDevices];

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Elements of a matrix must stay below 2^30 so byte offsets fit the 32-bit
// buffer addressing of the GEMM loads.
bool small_enough(int64_t rows, int64_t cols) { return rows * cols < (int64_t(1) << 30); }

int check_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return CODA_ERR_DEVICE;
  if (dev >= kMaxDevices) return CODA_ERR_DEVICE;
  int st = g_arch_state[dev].load(std::memory_order_acquire);
  if (st == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
      st = 2;
    } else {
      st = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
      g_cu_count[dev].store(prop.multiProcessorCount > 0 ? prop.multiProcessorCount : 1,
                            std::memory_order_release);
    }
    g_arch_state[dev].store(st, std::memory_order_release);
  }
  return st == 1 ? CODA_OK : CODA_ERR_DEVICE;
}

int launched(hipError_t e) { return e == hipSuccess ? CODA_OK : CODA_ERR_LAUNCH; }

// Scratch of the entry point that allocates nothing (coda_gemm_block_lse_noalloc).
// Host code never uses the array's name as an address: each device's copy is
// located once with hipGetSymbolAddress and that pointer is used.
constexpr size_t kScratchBytes = size_t(64) << 20;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::atomic<int> g_scratch_state[kMaxDevices];  // 0 unknown, 1 ready, 2 failed

}  // namespace

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

// This device's scratch pointer (the current device has passed check_device).
void* device_scratch() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  int st = g_scratch_state[dev].load(std::memory_order_acquire);
  if (st == 0) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e == hipSuccess && ptr) g_scratch_ptr[dev].store(ptr, std::memory_order_release);
    st = (e == hipSuccess && ptr) ? 1 : 2;
    g_scratch_state[dev].store(st, std::memory_order_release);
  }
  return st == 1 ? g_scratch_ptr[dev].load(std::memory_order_acquire) : nullptr;
}

size_t round256(size_t b) { return (b + 255) & ~size_t(255); }

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

int check_gemm_shape(int M, int N, int K, int kmul) {
  if (M < 1 || N < 16 || K < 64) return CODA_ERR_SHAPE;
  if (N % 16 != 0 || K % kmul != 0) return CODA_ERR_SHAPE;
  if (!small_enough(M, K) || !small_enough(N, K) || !small_enough(M, N)) return CODA_ERR_SHAPE;
  return CODA_OK;
}

}  // namespace

namespace coda {
// Only called after check_device() succeeded on the current device.
int cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
  const int n = g_cu_count[dev].load(std::memory_order_acquire);
  return n > 0 ? n : 256;
}
}  // namespace coda

extern "C" {

int coda_abi_version(void) { return kAbiVersion; }

const char* coda_status_string(int status) {
  switch (status) {
    case CODA_OK: return "ok";
    case CODA_ERR_NULL: return "a required pointer is NULL";
    case CODA_ERR_SHAPE: return "a size is out of range or not a required multiple";
    case CODA_ERR_DTYPE: return "unknown or unsupported number format";
    case CODA_ERR_ALIGN: return "a pointer is not aligned as required";
    case CODA_ERR_DEVICE: return "current device is not gfx950 or cannot be queried";
    case CODA_ERR_LAUNCH: return "the HIP runtime reported an error at launch";
    default: return "unknown status";
  }
}

int coda_rms_tile_width(void) { return coda::kRmsTileWidth; }
int coda_rms_tiles(int N) { return N <= 0 ? 0 : (N + coda::kRmsTileWidth - 1) / coda::kRmsTileWidth; }
int coda_lse_tile_width(void) { return coda::kLseTileWidth; }
int coda_lse_tiles(int V) { return V <= 0 ? 0 : (V + coda::kLseTileWidth - 1) / coda::kLseTileWidth; }

int coda_gemm_residual_partialrms(int dtype, const void* A, const void* W, const float* a_scale,
                                  const float* w_scale, const void* residual, void* h,
                                  float* partial_sumsq, const float* h8_scale, void* h8,
                                  float* partial_amax, int M, int N, int K, void* stream) {
  try {
    if (dtype != CODA_BF16 && dtype != CODA_FP8_E4M3) return CODA_ERR_DTYPE;
    if (!A || !W || !residual || !h || !partial_sumsq) return CODA_ERR_NULL;
    const bool fp8 = dtype == CODA_FP8_E4M3;
    if (fp8) {
      if (!a_scale || !w_scale || (h8 && !h8_scale)) return CODA_ERR_NULL;
    } else if (a_scale || w_scale || h8_scale || h8 || partial_amax) {
      return CODA_ERR_DTYPE;
    }
    if (int st = check_gemm_shape(M, N, K, fp8 ? 128 : 64)) return st;
    if (!aligned(A, 16) || !aligned(W, 16) || !aligned(residual, 16) || !aligned(h, 16) ||
        !aligned(partial_sumsq, 4) || (h8 && !aligned(h8, 16)) ||
        (partial_amax && !aligned(partial_amax, 4)) || (a_scale && !aligned(a_scale, 4)) ||
        (w_scale && !aligned(w_scale, 4)) || (h8_scale && !aligned(h8_scale, 4)))
      return CODA_ERR_ALIGN;
    if (int st = check_device()) return st;
    if (fp8)
      return launched(coda::launch_residual_partialrms_fp8(
          static_cast<const uint8_t*>(A), static_cast<const uint8_t*>(W), a_scale, w_scale,
          static_cast<const uint16_t*>(residual), static_cast<uint16_t*>(h), partial_sumsq,
          h8_scale, static_cast<uint8_t*>(h8), partial_amax, M, N, K, as_stream(stream)));
    return launched(coda::launch_residual_partialrms_bf16(
        static_cast<const uint16_t*>(A), static_cast<const uint16_t*>(W),
        static_cast<const uint16_t*>(residual), static_cast<uint16_t*>(h), partial_sumsq, M, N, K,
        as_stream(stream)));
  } catch (...) {
    return CODA_ERR_LAUNCH;
  }
}

int coda_rms_reduce(const float* partial_sumsq, const float* partial_amax, int T, int M, int N,
                    float eps, float* r, float* h_amax, float* h8_scale_out, void* stream) {
  try {
    if (!partial_sumsq || !r) return CODA_ERR_NULL;
    if (partial_amax && (!h_amax || !h8_scale_out)) return CODA_ERR_NULL;
    if (T < 1 || M < 1 || N < 1 || !(eps >= 0.f)) return CODA_ERR_SHAPE;
    if (!small_enough(T, M)) return CODA_ERR_SHAPE;
    if (!aligned(partial_sumsq, 4) || !aligned(r, 4) || (partial_amax && !aligned(partial_amax, 4)) ||
        (h_amax && !aligned(h_amax, 4)) || (h8_scale_out && !aligned(h8_scale_out, 4)))
      return CODA_ERR_ALIGN;
    if (int st = check_device()) return st;
    return launched(coda::launch_rms_reduce(partial_sumsq, partial_amax, T, M, N, eps, r,
                                            partial_amax ? h_amax : nullptr,
                                            partial_amax ? h8_scale_out : nullptr,
                                            as_stream(stream)));
  } catch (...) {
    return CODA_ERR_LAUNCH;
  }
}

int coda_gemm_rowscale_swiglu(int dtype, const void* X, const float* x_scale, const void* Wg,
                              const void* Wu, const float* wg_scale, const float* wu_scale,
                              const float* r, void* out, int M, int N, int K, void* stream) {
  try {
    if (dtype != CODA_BF16 && dtype != CODA_FP8_E4M3) return CODA_ERR_DTYPE;
    if (!X || !Wg || !Wu || !r || !out) return CODA_ERR_NULL;
    const bool fp8 = dtype == CODA_FP8_E4M3;
    if (fp8) {
      if (!x_scale || !wg_scale || !wu_scale) return CODA_ERR_NULL;
    } else if (x_scale || wg_scale || wu_scale) {
      return CODA_ERR_DTYPE;
    }
    if (int st = check_gemm_shape(M, N, K, fp8 ? 128 : 64)) return st;
    if (!aligned(X, 16) || !aligned(Wg, 16) || !aligned(Wu, 16) || !aligned(out, 16) ||
        !aligned(r, 4) || (x_scale && !aligned(x_scale, 4)) ||
        (wg_scale && !aligned(wg_scale, 4)) || (wu_scale && !aligned(wu_scale, 4)))
      return CODA_ERR_ALIGN;
    if (int st = check_device()) return st;
    if (fp8)
      return launched(coda::launch_rowscale_swiglu_fp8(
          static_cast<const uint8_t*>(X), x_scale, static_cast<const uint8_t*>(Wg),
          static_cast<const uint8_t*>(Wu), wg_scale, wu_scale, r, static_cast<uint16_t*>(out), M,
          N, K, as_stream(stream)));
    return launched(coda::launch_rowscale_swiglu_bf16(
        static_cast<const uint16_t*>(X), static_cast<const uint16_t*>(Wg),
        static_cast<const uint16_t*>(Wu), r, static_cast<uint16_t*>(out), M, N, K,
        as_stream(stream)));
  } catch (...) {
    return CODA_ERR_LAUNCH;
  }
}

int coda_gemm_rowscale_swiglu_save(const void* X, const void* Wg, const void* Wu, const float* r,
                                   void* out, void* gu, int M, int N, int K, void* stream) {
  try {
    if (!X || !Wg || !Wu || !r || !out || !gu) return CODA_ERR_NULL;
    if (int st = check_gemm_shape(M, N, K, 64)) return st;
    if (!small_enough(M, 2 * (int64_t)N)) return CODA_ERR_SHAPE;
    if (!aligned(X, 16) || !aligned(Wg, 16) || !aligned(Wu, 16) || !aligned(out, 16) ||
        !aligned(gu, 16) || !aligned(r, 4))
      return CODA_ERR_ALIGN;
    if (int st = check_device()) return st;
    return launched(coda::launch_rowscale_swiglu_save_bf16(
        static_cast<const uint16_t*>(X), static_cast<const uint16_t*>(Wg),
        static_cast<const uint16_t*>(Wu), r, static_cast<uint16_t*>(out),
        static_cast<uint16_t*>(gu), M, N, K, as_stream(stream)));
  } catch (...) {
    return CODA_ERR_LAUNCH;
  }
}

int coda_gemm_swiglu_bwd(const void* dY, const void* WdT, const void* gu, void* dz,
                         float* partial_dot, int M, int N, int K, void* stream) {
  try {
    if (!dY || !WdT || !gu || !dz || !partial_dot) return CODA_ERR_NULL;
    if (int st = check_gemm_shape(M, N, K, 64)) return st;
    if (!small_enough(M, 2 * (int64_t)N)) return CODA_ERR_SHAPE;
    if (!aligned(dY, 16) || !aligned(WdT, 16) || !aligned(gu, 16) || !aligned(dz, 16) ||
        !aligned(partial_dot, 4))
      return CODA_ERR_ALIGN;
    if (int st = check_device()) return st;
    return launched(coda::launch_swiglu_bwd_bf16(
        static_cast<const uint16_t*>(dY), static_cast<const uint16_t*>(WdT),
        static_cast<const uint16_t*>(gu), static_cast<uint16_t*>(dz), partial_dot, M, N, K,
        as_stream(stream)));
  } catch (...) {
    return CODA_ERR_LAUNCH;
  }
}

int coda_dgamma_slices(int M) { return M <= 0 ? 0 : (M + 127) / 128; }

int coda_gemm_wgrad_gamma(const void* A, const void* B, const void* W, const float* gamma,
                          void* dW, float* partial_dgamma, int M, int N, int K, void* stream) {
  try {
    if (!A || !B || !W || !gamma || !dW || !partial_dgamma) return CODA_ERR_NULL;
    if (int st = check_gemm_shape(M, N, K, 64)) return st;
    if (!small_enough(coda_dgamma_slices(M), N)) return CODA_ERR_SHAPE;
    if (!aligned(A, 16) || !aligned(B, 16) || !aligned(W, 16) || !aligned(dW, 16) ||
        !aligned(gamma, 16) || !aligned(partial_dgamma, 16))
      return CODA_ERR_ALIGN;
    if (int st = check_device()) return st;
    return launched(coda::launch_gemm_wgrad_gamma_bf16(
        static_cast<const uint16_t*>(A), static_cast<const uint16_t*>(B),
        static_cast<const uint16_t*>(W), gamma, static_cast<uint16_t*>(dW), partial_dgamma, M, N,
        K, as_stream(stream)));
  } catch (...) {
    return CODA_ERR_LAUNCH;
  }
}

int coda_dgamma_reduce(const float* partial, int P, int N, const float* gamma_div, float* dgamma,
                       void* stream) {
  try {
    if (!partial || !dgamma) return CODA_ERR_NULL;
    if (P < 1 || N < 1 || !small_enough(P, N)) return CODA_ERR_SHAPE;
    if (!aligned(partial, 4) || !aligned(dgamma, 4) || (gamma_div && !aligned(gamma_div, 4)))
      return CODA_ERR_ALIGN;
    if (int st = check_device()) return st;
    return launched(coda::launch_dgamma_reduce(partial, P, N, gamma_div, dgamma,
                                               as_stream(stream)));
  } catch (...) {
    return CODA_ERR_LAUNCH;
  }
}

int coda_col_dot_partial(const void* X, const void* Y, int M, int N, float* partial,
                         void* stream) {
  try {
    if (!X || !Y || !partial) return CODA_ERR_NULL;
    if (M < 1 || N < 8 || N % 8 != 0 || !small_enough(M, N)) return CODA_ERR_SHAPE;
    if (!aligned(X, 16) || !aligned(Y, 16) || !aligned(partial, 4)) return CODA_ERR_ALIGN;
    if (int st = check_device()) return st;
    return launched(coda::launch_col_dot_partial(static_cast<const uint16_t*>(X),
                                                 static_cast<const uint16_t*>(Y), M, N, partial,
                                                 as_stream(stream)));
  } catch (...) {
    return CODA_ERR_LAUNCH;
  }
}

int coda_rms_bwd_reduce(const float* partial_dot, int T, int M, const float* r, int N, float* c,
                        void* stream) {
  try {
    if (!partial_dot || !r || !c) return CODA_ERR_NULL;
    if (T < 1 || M < 1 || N < 1 || !small_enough(T, M)) return CODA_ERR_SHAPE;
    if (!aligned(partial_dot, 4) || !aligned(r, 4) || !aligned(c, 4)) return CODA_ERR_ALIGN;
    if (int st = check_device()) return st;
    return launched(coda::launch_rms_bwd_reduce(partial_dot, T, M, r, N, c, as_stream(stream)));
  } catch (...) {
    return CODA_ERR_LAUNCH;
  }
}

int coda_gemm_rmsnorm_bwd(const void* dz, const void* W2T, const void* h, const void* dY,
                          const float* r, const float* c, void* dh, int M, int N, int K,
                          void* stream) {
  try {
    if (!dz || !W2T || !h || !dY || !r || !c || !dh) return CODA_ERR_NULL;
    if (int st = check_gemm_shape(M, N, K, 64)) return st;
    if (!aligned(dz, 16) || !aligned(W2T, 16) || !aligned(h, 16) || !aligned(dY, 16) ||
        !aligned(dh, 16) || !aligned(r, 4) || !aligned(c, 4))
      return CODA_ERR_ALIGN;
    if (int st = check_device()) return st;
    return launched(coda::launch_rmsnorm_bwd_bf16(
        static_cast<const uint16_t*>(dz), static_cast<const uint16_t*>(W2T),
        static_cast<const uint16_t*>(h), static_cast<const uint16_t*>(dY), r, c,
        static_cast<uint16_t*>(dh), M, N, K, as_stream(stream)));
  } catch (...) {
    return CODA_ERR_LAUNCH;
  }
}

int coda_transpose_bf16(const void* src, const float* row_scale, int rows, int cols, void* dst,
                        int ld_dst, void* stream) {
  try {
    if (!src || !dst) return CODA_ERR_NULL;
    if (rows < 1 || cols < 1 || ld_dst < rows || (int64_t)rows * cols >= (int64_t(1) << 31) ||
        (int64_t)cols * ld_dst >= (int64_t(1) << 31) || cols > 65535 * 64 || rows > 65535 * 64)
      return CODA_ERR_SHAPE;
    if (!aligned(src, 2) || !aligned(dst, 2) || (row_scale && !aligned(row_scale, 4)))
      return CODA_ERR_ALIGN;
    if (int st = check_device()) return st;
    return launched(coda::launch_transpose_bf16(static_cast<const uint16_t*>(src), row_scale,
                                                rows, cols, static_cast<uint16_t*>(dst), ld_dst,
                                                as_stream(stream)));
  } catch (...) {
    return CODA_ERR_LAUNCH;
  }
}

int coda_gemm_rope(const void* h, const void* Wqkv, const float* r, const float* rope_cos,
                   const float* rope_sin, const int32_t* pos, int max_pos, void* qkv, int M, int K,
                   int n_q_heads, int n_kv_heads, int head_dim, void* stream) {
  try {
    if (!h || !Wqkv || !r || !rope_cos || !rope_sin || !pos || !qkv) return CODA_ERR_NULL;
    if ((head_dim != 64 && head_dim != 128) || n_q_heads < 1 || n_kv_heads < 1 || max_pos < 1)
      return CODA_ERR_SHAPE;
    const int64_t N = (int64_t)(n_q_heads + 2 * n_kv_heads) * head_dim;
    if (N > (int64_t(1) << 24)) return CODA_ERR_SHAPE;
    if (int st = check_gemm_shape(M, (int)N, K, 64)) return st;
    if (!aligned(h, 16) || !aligned(Wqkv, 16) || !aligned(qkv, 16) || !aligned(r, 4) ||
        !aligned(rope_cos, 16) || !aligned(rope_sin, 16) || !aligned(pos, 4))
      return CODA_ERR_ALIGN;
    if (int st = check_device()) return st;
    const uint16_t* hx = static_cast<const uint16_t*>(h);
    const uint16_t* wx = static_cast<const uint16_t*>(Wqkv);
    uint16_t* out = static_cast<uint16_t*>(qkv);
    // 64-wide heads whose count is a multiple of six (384 columns) run on the
    // 128 x 384 block tile, which fills whole rounds of compute units where
    // the 256 x 256 tile would leave the last round partly idle
    if (head_dim == 64 && (n_q_heads + 2 * n_kv_heads) % 6 == 0)
      return launched(coda::launch_rope_bf16_wide(hx, wx, r, rope_cos, rope_sin, pos, max_pos, out,
                                                  M, K, n_q_heads, n_kv_heads,
                                                  as_stream(stream)));
    return launched(coda::launch_rope_bf16(hx, wx, r, rope_cos, rope_sin, pos, max_pos, out, M, K,
                                           n_q_heads, n_kv_heads, head_dim, as_stream(stream)));
  } catch (...) {
    return CODA_ERR_LAUNCH;
  }
}

int coda_gemm_block_lse(const void* X, const void* W, const float* r, const int32_t* labels,
                        float* tile_max, float* tile_sumexp, float* label_logit, float* lse,
                        float* loss, int M, int V, int K, void* stream) {
  try {
    if (!X || !W || !labels || !tile_max || !tile_sumexp || !label_logit || !loss)
      return CODA_ERR_NULL;
    if (int st = check_gemm_shape(M, V, K, 64)) return st;
    if (!aligned(X, 16) || !aligned(W, 16) || !aligned(labels, 4) || !aligned(tile_max, 4) ||
        !aligned(tile_sumexp, 4) || !aligned(label_logit, 4) || !aligned(loss, 4) ||
        (r && !aligned(r, 4)) || (lse && !aligned(lse, 4)))
      return CODA_ERR_ALIGN;
    if (int st = check_device()) return st;
    hipStream_t s = as_stream(stream);
    if (hipError_t e = coda::launch_block_lse_bf16(static_cast<const uint16_t*>(X),
                                                   static_cast<const uint16_t*>(W), r, labels,
                                                   tile_max, tile_sumexp, label_logit, M, V, K, s))
      return launched(e);
    return launched(coda::launch_lse_merge(tile_max, tile_sumexp, label_logit, labels,
                                           coda_lse_tiles(V), M, V, lse, loss, s));
  } catch (...) {
    return CODA_ERR_LAUNCH;
  }
}

int coda_attention_fwd(const void* qkv, void* o, int M, int seq_len, int n_q_heads,
                       int n_kv_heads, int head_dim, void* stream) {
  try {
    if (!qkv || !o) return CODA_ERR_NULL;
    if ((head_dim != 64 && head_dim != 128) || n_q_heads < 1 || n_kv_heads < 1 ||
        n_q_heads % n_kv_heads != 0)
      return CODA_ERR_SHAPE;
    if (seq_len < 128 || seq_len % 128 != 0 || M < seq_len || M % seq_len != 0)
      return CODA_ERR_SHAPE;
    const int64_t C = (int64_t)(n_q_heads + 2 * n_kv_heads) * head_dim;
    if (!small_enough(M, C) || !small_enough(M, (int64_t)n_q_heads * head_dim))
      return CODA_ERR_SHAPE;
    if (!aligned(qkv, 16) || !aligned(o, 16)) return CODA_ERR_ALIGN;
    if (int st = check_device()) return st;
    return launched(coda::launch_attention_fwd(static_cast<const uint16_t*>(qkv),
                                               static_cast<uint16_t*>(o), M, seq_len, n_q_heads,
                                               n_kv_heads, head_dim, as_stream(stream)));
  } catch (...) {
    return CODA_ERR_LAUNCH;
  }
}

size_t coda_lse_noalloc_max_bytes(void) { return kScratchBytes; }

int coda_gemm_block_lse_noalloc(const void* X, const void* W, const float* r,
                                const int32_t* labels, float* lse, float* loss, int M, int V,
                                int K, void* stream) {
  try {
    if (!X || !W || !labels || !loss) return CODA_ERR_NULL;
    if (int st = check_gemm_shape(M, V, K, 64)) return st;
    const size_t T = (size_t)coda_lse_tiles(V);
    const size_t part = round256(T * (size_t)M * 4);
    if (2 * part + round256((size_t)M * 4) > kScratchBytes) return CODA_ERR_SHAPE;
    if (!aligned(X, 16) || !aligned(W, 16) || !aligned(labels, 4) || !aligned(loss, 4) ||
        (r && !aligned(r, 4)) || (lse && !aligned(lse, 4)))
      return CODA_ERR_ALIGN;
    if (int st = check_device()) return st;
    char* base = static_cast<char*>(device_scratch());
    if (!base) return CODA_ERR_DEVICE;
    float* tmax = reinterpret_cast<float*>(base);
    float* tsum = reinterpret_cast<float*>(base + part);
    float* zl = reinterpret_cast<float*>(base + 2 * part);
    hipStream_t s = as_stream(stream);
    if (hipError_t e = coda::launch_block_lse_bf16(static_cast<const uint16_t*>(X),
                                                   static_cast<const uint16_t*>(W), r, labels,
                                                   tmax, tsum, zl, M, V, K, s))
      return launched(e);
    return launched(coda::launch_lse_merge(tmax, tsum, zl, labels, (int)T, M, V, lse, loss, s));
  } catch (...) {
    return CODA_ERR_LAUNCH;
  }
}

int coda_fold_gamma(const void* W, const float* gamma, void* W_out, int N, int K, void* stream) {
  try {
    if (!W || !gamma || !W_out) return CODA_ERR_NULL;
    if (N < 1 || K < 8 || K % 8 != 0 || !small_enough(N, K)) return CODA_ERR_SHAPE;
    if (!aligned(W, 16) || !aligned(W_out, 16) || !aligned(gamma, 4)) return CODA_ERR_ALIGN;
    if (int st = check_device()) return st;
    return launched(coda::launch_fold_gamma(static_cast<const uint16_t*>(W), gamma,
                                            static_cast<uint16_t*>(W_out), N, K,
                                            as_stream(stream)));
  } catch (...) {
    return CODA_ERR_LAUNCH;
  }
}

int coda_rope_tables(double theta, int max_pos, int head_dim, float* rope_cos, float* rope_sin,
                     void* stream) {
  try {
    if (!rope_cos || !rope_sin) return CODA_ERR_NULL;
    if (!(theta > 0.0) || max_pos < 1 || head_dim < 2 || head_dim % 2 != 0 ||
        !small_enough(max_pos, head_dim))
      return CODA_ERR_SHAPE;
    if (!aligned(rope_cos, 4) || !aligned(rope_sin, 4)) return CODA_ERR_ALIGN;
    if (int st = check_device()) return st;
    return launched(coda::launch_rope_tables(theta, max_pos, head_dim, rope_cos, rope_sin,
                                             as_stream(stream)));
  } catch (...) {
    return CODA_ERR_LAUNCH;
  }
}

int coda_gemm_bf16(const void* A, const void* W, void* C, int M, int N, int K, void* stream) {
  try {
    if (!A || !W || !C) return CODA_ERR_NULL;
    if (int st = check_gemm_shape(M, N, K, 64)) return st;
    if (!aligned(A, 16) || !aligned(W, 16) || !aligned(C, 16)) return CODA_ERR_ALIGN;
    if (int st = check_device()) return st;
    // the 128 x 384 tile where it fills the rounds of compute units better
    const auto launch = coda::prefer_wide_tile(M, N) ? coda::launch_gemm_plain_bf16_wide
                                                     : coda::launch_gemm_plain_bf16;
    return launched(launch(static_cast<const uint16_t*>(A), static_cast<const uint16_t*>(W),
                           static_cast<uint16_t*>(C), M, N, K, as_stream(stream)));
  } catch (...) {
    return CODA_ERR_LAUNCH;
  }
}

int coda_gemm_bf16_splitk(const void* A, const void* W, void* C, float* workspace, int M, int N,
                          int K, int parts, void* stream) {
  try {
    if (!A || !W || !C || !workspace) return CODA_ERR_NULL;
    if (parts < 1 || parts > 16) return CODA_ERR_SHAPE;
    if (int st = check_gemm_shape(M, N, K, 64 * parts)) return st;
    // one block's workspace rows (up to 256 x N fp32) stay below 2 GiB
    if ((int64_t)std::min(M, 256) * N * 4 >= (int64_t(1) << 31)) return CODA_ERR_SHAPE;
    if (!aligned(A, 16) || !aligned(W, 16) || !aligned(C, 16) || !aligned(workspace, 16))
      return CODA_ERR_ALIGN;
    if (int st = check_device()) return st;
    return launched(coda::launch_gemm_splitk_bf16(
        static_cast<const uint16_t*>(A), static_cast<const uint16_t*>(W),
        static_cast<uint16_t*>(C), workspace, M, N, K, parts, as_stream(stream)));
  } catch (...) {
    return CODA_ERR_LAUNCH;
  }
}

int coda_residual_add(const void* y, const void* res, void* h, int64_t count, void* stream) {
  try {
    if (!y || !res || !h) return CODA_ERR_NULL;
    if (count < 8 || count % 8 != 0) return CODA_ERR_SHAPE;
    if (!aligned(y, 16) || !aligned(res, 16) || !aligned(h, 16)) return CODA_ERR_ALIGN;
    if (int st = check_device()) return st;
    return launched(coda::launch_residual_add(static_cast<const uint16_t*>(y),
                                              static_cast<const uint16_t*>(res),
                                              static_cast<uint16_t*>(h), count,
                                              as_stream(stream)));
  } catch (...) {
    return CODA_ERR_LAUNCH;
  }
}

int coda_rmsnorm(const void* h, const float* gamma, float eps, void* out, int M, int N,
                 void* stream) {
  try {
    if (!h || !gamma || !out) return CODA_ERR_NULL;
    if (M < 1 || N < 8 || N % 8 != 0 || N > 16384 || !(eps >= 0.f) || !small_enough(M, N))
      return CODA_ERR_SHAPE;
    if (!aligned(h, 16) || !aligned(out, 16) || !aligned(gamma, 4)) return CODA_ERR_ALIGN;
    if (int st = check_device()) return st;
    return launched(coda::launch_rmsnorm(static_cast<const uint16_t*>(h), gamma, eps,
                                         static_cast<uint16_t*>(out), M, N, as_stream(stream)));
  } catch (...) {
    return CODA_ERR_LAUNCH;
  }
}

int coda_swiglu(const void* gu, void* out, int M, int N, void* stream) {
  try {
    if (!gu || !out) return CODA_ERR_NULL;
    if (M < 1 || N < 8 || N % 8 != 0 || !small_enough(M, 2 * (int64_t)N)) return CODA_ERR_SHAPE;
    if (!aligned(gu, 16) || !aligned(out, 16)) return CODA_ERR_ALIGN;
    if (int st = check_device()) return st;
    return launched(coda::launch_swiglu(static_cast<const uint16_t*>(gu),
                                        static_cast<uint16_t*>(out), M, N, as_stream(stream)));
  } catch (...) {
    return CODA_ERR_LAUNCH;
  }
}

int coda_swiglu_bwd(const void* dout, const void* gu, void* dz, int M, int N, void* stream) {
  try {
    if (!dout || !gu || !dz) return CODA_ERR_NULL;
    if (M < 1 || N < 8 || N % 8 != 0 || !small_enough(M, 2 * (int64_t)N)) return CODA_ERR_SHAPE;
    if (!aligned(dout, 16) || !aligned(gu, 16) || !aligned(dz, 16)) return CODA_ERR_ALIGN;
    if (int st = check_device()) return st;
    return launched(coda::launch_swiglu_bwd(static_cast<const uint16_t*>(dout),
                                            static_cast<const uint16_t*>(gu),
                                            static_cast<uint16_t*>(dz), M, N, as_stream(stream)));
  } catch (...) {
    return CODA_ERR_LAUNCH;
  }
}

int coda_rmsnorm_bwd(const void* G, const void* h, const void* dY, float eps, void* dh, int M,
                     int N, void* stream) {
  try {
    if (!G || !h || !dY || !dh) return CODA_ERR_NULL;
    if (M < 1 || N < 8 || N % 8 != 0 || N > 16384 || !(eps >= 0.f) || !small_enough(M, N))
      return CODA_ERR_SHAPE;
    if (!aligned(G, 16) || !aligned(h, 16) || !aligned(dY, 16) || !aligned(dh, 16))
      return CODA_ERR_ALIGN;
    if (int st = check_device()) return st;
    return launched(coda::launch_rmsnorm_bwd(
        static_cast<const uint16_t*>(G), static_cast<const uint16_t*>(h),
        static_cast<const uint16_t*>(dY), eps, static_cast<uint16_t*>(dh), M, N,
        as_stream(stream)));
  } catch (...) {
    return CODA_ERR_LAUNCH;
  }
}

int coda_gemm_fp8(const void* A, const void* W, const float* a_scale, const float* w_scale,
                  void* C, int ldc, int M, int N, int K, void* stream) {
  try {
    if (!A || !W || !a_scale || !w_scale || !C) return CODA_ERR_NULL;
    if (int st = check_gemm_shape(M, N, K, 128)) return st;
    if (ldc < N || ldc % 8 != 0 || !small_enough(M, ldc)) return CODA_ERR_SHAPE;
    if (!aligned(A, 16) || !aligned(W, 16) || !aligned(C, 16) || !aligned(a_scale, 4) ||
        !aligned(w_scale, 4))
      return CODA_ERR_ALIGN;
    if (int st = check_device()) return st;
    return launched(coda::launch_gemm_plain_fp8(
        static_cast<const uint8_t*>(A), static_cast<const uint8_t*>(W), a_scale, w_scale,
        static_cast<uint16_t*>(C), M, N, K, ldc, as_stream(stream)));
  } catch (...) {
    return CODA_ERR_LAUNCH;
  }
}

int coda_quantize_e4m3(const void* x, int64_t count, const float* s_in, void* out, float* amax,
                       float* s_out, void* stream) {
  try {
    if (!x || !s_in || !out || !amax || !s_out) return CODA_ERR_NULL;
    if (count < 8 || count % 8 != 0 || count >= (int64_t(1) << 34)) return CODA_ERR_SHAPE;
    if (!aligned(x, 16) || !aligned(out, 8) || !aligned(s_in, 4) || !aligned(amax, 4) ||
        !aligned(s_out, 4))
      return CODA_ERR_ALIGN;
    if (int st = check_device()) return st;
    return launched(coda::launch_quantize_e4m3(static_cast<const uint16_t*>(x), s_in,
                                               static_cast<uint8_t*>(out), count, amax, s_out,
                                               as_stream(stream)));
  } catch (...) {
    return CODA_ERR_LAUNCH;
  }
}

int coda_rope_apply(void* qkv, const float* rope_cos, const float* rope_sin, const int32_t* pos,
                    int max_pos, int M, int n_q_heads, int n_kv_heads, int head_dim, void* stream) {
  try {
    if (!qkv || !rope_cos || !rope_sin || !pos) return CODA_ERR_NULL;
    if ((head_dim != 64 && head_dim != 128) || n_q_heads < 1 || n_kv_heads < 1 || max_pos < 1 ||
        M < 1)
      return CODA_ERR_SHAPE;
    const int64_t N = (int64_t)(n_q_heads + 2 * n_kv_heads) * head_dim;
    if (N > (int64_t(1) << 24) || !small_enough(M, N)) return CODA_ERR_SHAPE;
    if (!aligned(qkv, 16) || !aligned(rope_cos, 16) || !aligned(rope_sin, 16) || !aligned(pos, 4))
      return CODA_ERR_ALIGN;
    if (int st = check_device()) return st;
    return launched(coda::launch_rope_apply(static_cast<uint16_t*>(qkv), rope_cos, rope_sin, pos,
                                            max_pos, M, n_q_heads, n_kv_heads, head_dim,
                                            as_stream(stream)));
  } catch (...) {
    return CODA_ERR_LAUNCH;
  }
}

int coda_cross_entropy_rows(const void* logits, const int32_t* labels, float* lse, float* loss,
                            int M, int V, void* stream) {
  try {
    if (!logits || !labels || !lse || !loss) return CODA_ERR_NULL;
    if (M < 1 || V < 8 || V % 8 != 0 || !small_enough(M, V)) return CODA_ERR_SHAPE;
    if (!aligned(logits, 16) || !aligned(labels, 4) || !aligned(lse, 4) || !aligned(loss, 4))
      return CODA_ERR_ALIGN;
    if (int st = check_device()) return st;
    return launched(coda::launch_ce_rows(static_cast<const uint16_t*>(logits), labels, lse, loss,
                                         M, V, as_stream(stream)));
  } catch (...) {
    return CODA_ERR_LAUNCH;
  }
}

}  // extern "C"
