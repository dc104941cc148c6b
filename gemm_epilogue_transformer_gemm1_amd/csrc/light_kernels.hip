// Light (bandwidth- or latency-bound) kernels: the RMS reduction between the
// two GEMMs, weight preparation, and the unfused baseline's elementwise ops.
//
// Citations name sections of the news page "CODA: New Research Optimizes
// Transformer Training with GEMM-Epilogue Programming" (KuCoin news flash).

#include <algorithm>

#include "coda_device.hpp"
#include "launch.hpp"

namespace coda {

static inline int cdiv(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }

// 8 bf16 (16 bytes) <-> 8 floats
__device__ __forceinline__ void load8(const uint16_t* p, float* f) {
  const i32x4_t raw = *(const i32x4_t*)p;
  unpack_bf16x4(u32x2_t{(unsigned)raw.x, (unsigned)raw.y}, f);
  unpack_bf16x4(u32x2_t{(unsigned)raw.z, (unsigned)raw.w}, f + 4);
}

__device__ __forceinline__ void store8(uint16_t* p, const float* f) {
  const u32x2_t lo = pack_bf16x4(f[0], f[1], f[2], f[3]);
  const u32x2_t hi = pack_bf16x4(f[4], f[5], f[6], f[7]);
  *(i32x4_t*)p = i32x4_t{(int)lo.x, (int)lo.y, (int)hi.x, (int)hi.y};
}


// ---------------------------------------------------------------------------
// The light reduction (section "CODA: the secret in the epilogue": a light
// reduction kernel aggregates the partial RMS values).  Four lanes per token
// row: lane = 16 * g + (row % 16) sums tiles g, g + 4, g + 8, ... with all of
// its loads issued before the first add (the kernel is latency-bound: a row
// has only T values), then the four partial sums meet through two lane
// exchanges.  The 16 lanes of one tile read 16 consecutive rows, so loads are
// coalesced.  Optionally a global amax over the partial amax tiles (fp8
// delayed scaling): one atomicMax per block on the non-negative float's bit
// pattern, which orders like the float.
// ---------------------------------------------------------------------------
constexpr int kReduceRowsPerBlock = 64;  // 4 waves x 16 rows

__global__ __launch_bounds__(256) void k_rms_reduce(const float* __restrict__ psum,
                                                    const float* __restrict__ pamax, int T, int M,
                                                    float inv_n, float eps, float* __restrict__ r,
                                                    unsigned int* __restrict__ amax_bits) {
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4;
  const int m = blockIdx.x * kReduceRowsPerBlock + (threadIdx.x >> 6) * 16 + (lane & 15);
  const bool row_ok = m < M;
  float s = 0.f, mx = 0.f;
  if (row_ok) {
    int t = g;
    for (; t + 12 < T; t += 16) {  // four tiles per round, loads first
      const float a0 = psum[(size_t)t * M + m], a1 = psum[(size_t)(t + 4) * M + m];
      const float a2 = psum[(size_t)(t + 8) * M + m], a3 = psum[(size_t)(t + 12) * M + m];
      s += (a0 + a1) + (a2 + a3);
    }
    for (; t < T; t += 4) s += psum[(size_t)t * M + m];
    if (pamax)
      for (int u = g; u < T; u += 4) mx = fmaxf(mx, pamax[(size_t)u * M + m]);
  }
  s += __shfl_xor(s, 16, 64);
  s += __shfl_xor(s, 32, 64);
  if (row_ok && g == 0) r[m] = 1.0f / sqrtf(s * inv_n + eps);
  if (pamax) {
    __shared__ float red[4];
    for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = mx;
    __syncthreads();
    if (threadIdx.x == 0) {
      mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
      atomicMax(amax_bits, __float_as_uint(mx));
    }
  }
}

// Backward row coefficient: the SwiGLU-backward GEMM's epilogue leaves partial
// sums of dz * z per (row, 128-feature tile), combined here into
//   c[m] = r[m]^2 / N * sum_t pdot[t, m]
// (N = the normalised width d), the coefficient of h in the RMSNorm backward
// dh = r G - c h + dY.  Same 4-lanes-per-row split as k_rms_reduce.
__global__ __launch_bounds__(256) void k_rms_bwd_reduce(const float* __restrict__ pdot, int T,
                                                        int M, const float* __restrict__ r,
                                                        float inv_n, float* __restrict__ c) {
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4;
  const int m = blockIdx.x * kReduceRowsPerBlock + (threadIdx.x >> 6) * 16 + (lane & 15);
  const bool row_ok = m < M;
  float s = 0.f;
  if (row_ok) {
    int t = g;
    for (; t + 12 < T; t += 16) {
      const float a0 = pdot[(size_t)t * M + m], a1 = pdot[(size_t)(t + 4) * M + m];
      const float a2 = pdot[(size_t)(t + 8) * M + m], a3 = pdot[(size_t)(t + 12) * M + m];
      s += (a0 + a1) + (a2 + a3);
    }
    for (; t < T; t += 4) s += pdot[(size_t)t * M + m];
  }
  s += __shfl_xor(s, 16, 64);
  s += __shfl_xor(s, 32, 64);
  if (row_ok && g == 0) {
    const float rm = r[m];
    c[m] = (rm * rm) * (s * inv_n);
  }
}

hipError_t launch_rms_bwd_reduce(const float* pdot, int T, int M, const float* r, int N, float* c,
                                 hipStream_t stream) {
  hipLaunchKernelGGL(k_rms_bwd_reduce, dim3(cdiv(M, kReduceRowsPerBlock)), dim3(256), 0, stream,
                     pdot, T, M, r, 1.0f / (float)N, c);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Gradient of the RMSNorm gain.  The fused weight-gradient GEMM leaves partial
// column sums pdg [P, N] (one row per 128-row slice of the gate|up weight);
// the light reduction sums them in slice order (deterministic):
//   dgamma[k] = sum_p pdg[p, k]          (divided by gamma[k] if gamma_div).
// A 512-thread block owns 64 columns; wave w sums slices w, w + 8, ... with
// four loads in flight, the eight partial sums meet in LDS.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(512) void k_dgamma_reduce(const float* __restrict__ pdg, int P,
                                                       int N, const float* __restrict__ gamma_div,
                                                       float* __restrict__ dgamma) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = blockIdx.x * 64 + lane;
  const int cc = min(col, N - 1);
  float s = 0.f;
  int p = wave;
  for (; p + 24 < P; p += 32) {
    const float a0 = pdg[(size_t)p * N + cc], a1 = pdg[(size_t)(p + 8) * N + cc];
    const float a2 = pdg[(size_t)(p + 16) * N + cc], a3 = pdg[(size_t)(p + 24) * N + cc];
    s += (a0 + a1) + (a2 + a3);
  }
  for (; p < P; p += 8) s += pdg[(size_t)p * N + cc];
  __shared__ float red[8][64];
  red[wave][lane] = s;
  __syncthreads();
  if (wave == 0 && col < N) {
    float t = 0.f;
#pragma unroll
    for (int w = 0; w < 8; ++w) t += red[w][lane];
    dgamma[col] = gamma_div ? t / gamma_div[col] : t;
  }
}

hipError_t launch_dgamma_reduce(const float* pdg, int P, int N, const float* gamma_div,
                                float* dgamma, hipStream_t stream) {
  hipLaunchKernelGGL(k_dgamma_reduce, dim3(cdiv(N, 64)), dim3(512), 0, stream, pdg, P, N,
                     gamma_div, dgamma);
  return hipGetLastError();
}

// Unfused counterpart of the weight-gradient epilogue: per 128-row slice p,
//   pdg[p, k] = sum over rows n of the slice of X[n, k] Y[n, k]   (bf16 in)
// e.g. X = the stored unfolded-weight gradient dW, Y = W (then dgamma is that
// sum divided by gamma).  A 256-thread block covers 512 columns of one slice:
// each wave 32 of its rows, 8 columns per lane with 16-byte loads, the four
// waves' sums meet in LDS.
__global__ __launch_bounds__(256) void k_col_dot_partial(const uint16_t* __restrict__ X,
                                                         const uint16_t* __restrict__ Y, int M,
                                                         int N, float* __restrict__ pdg) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c0 = blockIdx.x * 512 + lane * 8;
  const int r0 = blockIdx.y * 128 + wave * 32;
  float acc[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) acc[q] = 0.f;
  if (c0 < N) {
    const int rn = max(0, min(32, M - r0));
    int k = 0;
    for (; k + 4 <= rn; k += 4) {
      float xv[4][8], yv[4][8];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        load8(X + (size_t)(r0 + k + u) * N + c0, xv[u]);
        load8(Y + (size_t)(r0 + k + u) * N + c0, yv[u]);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[q] = __builtin_fmaf(xv[u][q], yv[u][q], acc[q]);
    }
    for (; k < rn; ++k) {
      float xv[8], yv[8];
      load8(X + (size_t)(r0 + k) * N + c0, xv);
      load8(Y + (size_t)(r0 + k) * N + c0, yv);
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[q] = __builtin_fmaf(xv[q], yv[q], acc[q]);
    }
  }
  __shared__ float red[4][512];
#pragma unroll
  for (int q = 0; q < 8; ++q) red[wave][lane * 8 + q] = acc[q];
  __syncthreads();
  for (int c = threadIdx.x; c < 512; c += 256) {
    const int col = blockIdx.x * 512 + c;
    if (col < N)
      pdg[(size_t)blockIdx.y * N + col] = (red[0][c] + red[1][c]) + (red[2][c] + red[3][c]);
  }
}

hipError_t launch_col_dot_partial(const uint16_t* X, const uint16_t* Y, int M, int N, float* pdg,
                                  hipStream_t stream) {
  hipLaunchKernelGGL(k_col_dot_partial, dim3(cdiv(N, 512), cdiv(M, 128)), dim3(256), 0, stream, X,
                     Y, M, N, pdg);
  return hipGetLastError();
}

__global__ void k_zero_u32(unsigned int* p) { *p = 0u; }

__global__ void k_amax_to_scale(const unsigned int* amax_bits, float* h_amax, float* scale_out) {
  const float a = __uint_as_float(*amax_bits);
  *h_amax = a;
  *scale_out = a > 0.f ? a * (1.0f / 448.0f) : 1.0f;
}

hipError_t launch_rms_reduce(const float* psum, const float* pamax, int T, int M, int N, float eps,
                             float* r, float* h_amax, float* h8_scale_out, hipStream_t stream) {
  unsigned int* bits = reinterpret_cast<unsigned int*>(h_amax);
  if (pamax) hipLaunchKernelGGL(k_zero_u32, dim3(1), dim3(1), 0, stream, bits);
  hipLaunchKernelGGL(k_rms_reduce, dim3(cdiv(M, kReduceRowsPerBlock)), dim3(256), 0, stream, psum,
                     pamax, T, M, 1.0f / (float)N, eps, r, bits);
  if (pamax)
    hipLaunchKernelGGL(k_amax_to_scale, dim3(1), dim3(1), 0, stream, bits, h_amax, h8_scale_out);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Weight preparation: fold the RMSNorm gain (it lies along GEMM2's K axis)
// into the weight columns, W'[n,k] = bf16(W[n,k] * gamma[k]).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_fold_gamma(const uint16_t* __restrict__ W,
                                                    const float* __restrict__ gamma,
                                                    uint16_t* __restrict__ out, int64_t total8,
                                                    int K) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;  // group of 8 elements
  if (idx >= total8) return;
  const int64_t e = idx * 8;
  const int k = (int)(e % K);
  const i32x4_t raw = *(const i32x4_t*)(W + e);
  const u32x2_t lo = {(unsigned)raw.x, (unsigned)raw.y}, hi = {(unsigned)raw.z, (unsigned)raw.w};
  float f[8];
  unpack_bf16x4(lo, f);
  unpack_bf16x4(hi, f + 4);
#pragma unroll
  for (int q = 0; q < 8; ++q) f[q] *= gamma[k + q];
  const u32x2_t plo = pack_bf16x4(f[0], f[1], f[2], f[3]);
  const u32x2_t phi = pack_bf16x4(f[4], f[5], f[6], f[7]);
  *(i32x4_t*)(out + e) = i32x4_t{(int)plo.x, (int)plo.y, (int)phi.x, (int)phi.y};
}

// Transposed copies for the backward GEMMs, which reduce along what the
// forward keeps in rows (weights with the output features along K; token-major
// activations for the weight gradients):
//   dst[c * ld_dst + r] = src[r * cols + c]                       (row_scale NULL)
//   dst[c * ld_dst + r] = bf16(src[r * cols + c] * row_scale[r])  (one rounding)
// The second form carries the RMS row scale into the gradient of the folded
// GEMM2 weight, dW' = dz^T (r h), whose reduction runs over the token rows.
// 64 x 64 tiles through LDS (one padding column against bank conflicts), so
// both the reads and the writes are row-contiguous.
__global__ __launch_bounds__(256) void k_transpose_bf16(const uint16_t* __restrict__ src,
                                                        const float* __restrict__ row_scale,
                                                        int rows, int cols,
                                                        uint16_t* __restrict__ dst, int ld_dst) {
  __shared__ uint16_t tile[64][65];
  const int r0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const int r = r0 + ty * 16 + k, c = c0 + tx;
    if (r < rows && c < cols) {
      uint16_t v = src[(size_t)r * cols + c];
      if (row_scale) v = __builtin_bit_cast(uint16_t, (__bf16)(bf16_to_f32(v) * row_scale[r]));
      tile[ty * 16 + k][tx] = v;
    }
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const int c = c0 + ty * 16 + k, r = r0 + tx;
    if (r < rows && c < cols) dst[(size_t)c * ld_dst + r] = tile[tx][ty * 16 + k];
  }
}

// The same with 16-byte accesses on both sides and no LDS, for rows % 8 ==
// cols % 8 == ld_dst % 8 == 0 and 16-byte aligned pointers.  A lane loads an
// 8 x 8 block (8 source rows of 16 bytes), transposes it in registers and
// stores 8 destination rows of 16 bytes.  Lane L of a wave takes row group
// L / 8 and column chunk L % 8 of a 64 x 64 wave tile, so each load reads 8
// runs of 128 bytes (8 lanes along a source row) and each store writes 8 runs
// of 128 bytes (8 lanes along a destination row); the four waves of a block
// cover 128 x 128.  Every block is either wholly inside or wholly outside
// the matrix per lane (both sizes are multiples of 8).
__global__ __launch_bounds__(256) void k_transpose_bf16_r8(const uint16_t* __restrict__ src,
                                                           const float* __restrict__ row_scale,
                                                           int rows, int cols,
                                                           uint16_t* __restrict__ dst,
                                                           int ld_dst) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = blockIdx.y * 128 + (wave >> 1) * 64 + (lane >> 3) * 8;
  const int c = blockIdx.x * 128 + (wave & 1) * 64 + (lane & 7) * 8;
  if (r >= rows || c >= cols) return;
  u32x4_t v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = *(const u32x4_t*)(src + (size_t)(r + i) * cols + c);
  if (row_scale) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float sc = row_scale[r + i];
      float f[8];
      unpack_bf16x4(u32x2_t{v[i].x, v[i].y}, f);
      unpack_bf16x4(u32x2_t{v[i].z, v[i].w}, f + 4);
      const u32x2_t lo = pack_bf16x4(f[0] * sc, f[1] * sc, f[2] * sc, f[3] * sc);
      const u32x2_t hi = pack_bf16x4(f[4] * sc, f[5] * sc, f[6] * sc, f[7] * sc);
      v[i] = u32x4_t{lo.x, lo.y, hi.x, hi.y};
    }
  }
  // destination row c + j holds element j of source rows r .. r + 7: element
  // j of row i is half j & 1 of word j / 2 of v[i]
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    uint32_t w[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) w[i] = v[i][j >> 1];
    uint32_t o[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      o[e] = (j & 1) ? ((w[2 * e] >> 16) | (w[2 * e + 1] & 0xffff0000u))
                     : ((w[2 * e] & 0xffffu) | (w[2 * e + 1] << 16));
    *(u32x4_t*)(dst + (size_t)(c + j) * ld_dst + r) = u32x4_t{o[0], o[1], o[2], o[3]};
  }
}

hipError_t launch_transpose_bf16(const uint16_t* src, const float* row_scale, int rows, int cols,
                                 uint16_t* dst, int ld_dst, hipStream_t stream) {
  const bool v8 = rows % 8 == 0 && cols % 8 == 0 && ld_dst % 8 == 0 &&
                  (reinterpret_cast<uintptr_t>(src) & 15) == 0 &&
                  (reinterpret_cast<uintptr_t>(dst) & 15) == 0;
  if (v8)
    hipLaunchKernelGGL(k_transpose_bf16_r8, dim3(cdiv(cols, 128), cdiv(rows, 128)), dim3(256), 0,
                       stream, src, row_scale, rows, cols, dst, ld_dst);
  else
    hipLaunchKernelGGL(k_transpose_bf16, dim3(cdiv(cols, 64), cdiv(rows, 64)), dim3(256), 0,
                       stream, src, row_scale, rows, cols, dst, ld_dst);
  return hipGetLastError();
}

hipError_t launch_fold_gamma(const uint16_t* W, const float* gamma, uint16_t* W_out, int N, int K,
                             hipStream_t stream) {
  const int64_t total8 = (int64_t)N * K / 8;
  hipLaunchKernelGGL(k_fold_gamma, dim3(cdiv(total8, 256)), dim3(256), 0, stream, W, gamma, W_out,
                     total8, K);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Log-sum-exp merge of the per-tile (max, sum-exp) pairs (section "Five
// building blocks and a LEGO language": the running max / sum-exp statistics
// of online normalisation).  A 1024-thread block owns 32 token rows and
// splits each row's tiles over 32 lanes: lane l of wave w takes row
// 32*block + l%32 and tiles s, s+32, s+64, ... with s = 2w + l/32, so every
// load instruction reads two 128-byte runs (32 consecutive rows of two
// tiles).  A lane merges four tiles per step (one new max, five exponentials)
// and issues the next step's eight loads before it merges the current four,
// so each lane keeps up to sixteen loads in flight; the two halves of a wave
// meet through one lane exchange and the sixteen waves through LDS.
//   lse = Mx + ln sum_t s_t e^(m_t - Mx);  loss = lse - label_logit,
// and loss = 0 for a label outside [0, V) (a row that carries no loss; its
// label logit is never read).
// ---------------------------------------------------------------------------
__device__ __forceinline__ void lse_combine(float& m, float& s, float m2, float s2) {
  const float nm = fmaxf(m, m2);
  if (nm == -INFINITY) return;  // both empty
  const float k = 1.4426950408889634f;
  s = s * __builtin_amdgcn_exp2f((m - nm) * k) + s2 * __builtin_amdgcn_exp2f((m2 - nm) * k);
  m = nm;
}

constexpr int kMergeRows = 32;    // token rows per block
constexpr int kMergeSlices = 32;  // lanes sharing one row (16 waves x 2 halves)
constexpr int kMergeWaves = 16;

__global__ __launch_bounds__(1024) void k_lse_merge(const float* __restrict__ tmax,
                                                    const float* __restrict__ tsum,
                                                    const float* __restrict__ label_logit,
                                                    const int* __restrict__ labels, int T, int M,
                                                    int V, float* __restrict__ lse,
                                                    float* __restrict__ loss) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int row = lane & (kMergeRows - 1);
  const int m = blockIdx.x * kMergeRows + row;
  const size_t mc = (size_t)min(m, M - 1);
  const float k = 1.4426950408889634f;
  constexpr int S = kMergeSlices;
  float rm = -INFINITY, rs = 0.f;
  int t = wave * 2 + (lane >> 5);
  auto load4 = [&](int t0, float (&a)[4], float (&b)[4]) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      a[q] = tmax[(size_t)(t0 + q * S) * M + mc];
      b[q] = tsum[(size_t)(t0 + q * S) * M + mc];
    }
  };
  float a[4], b[4];
  bool have = t + 3 * S < T;
  if (have) load4(t, a, b);
  while (have) {
    const int tn = t + 4 * S;
    const bool nhave = tn + 3 * S < T;
    float na[4], nb[4];
    if (nhave) load4(tn, na, nb);  // in flight while this step merges
    const float nm = fmaxf(fmaxf(fmaxf(a[0], a[1]), fmaxf(a[2], a[3])), rm);
    if (nm != -INFINITY) {
      float acc = rs * __builtin_amdgcn_exp2f((rm - nm) * k);
#pragma unroll
      for (int q = 0; q < 4; ++q) acc += b[q] * __builtin_amdgcn_exp2f((a[q] - nm) * k);
      rs = acc;
      rm = nm;
    }
    t = tn;
    have = nhave;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      a[q] = na[q];
      b[q] = nb[q];
    }
  }
  for (; t < T; t += S) lse_combine(rm, rs, tmax[(size_t)t * M + mc], tsum[(size_t)t * M + mc]);
  lse_combine(rm, rs, __shfl_xor(rm, 32, 64), __shfl_xor(rs, 32, 64));
  __shared__ float pm[kMergeWaves][kMergeRows], ps[kMergeWaves][kMergeRows];
  if (lane < kMergeRows) {
    pm[wave][lane] = rm;
    ps[wave][lane] = rs;
  }
  __syncthreads();
  if (wave == 0 && lane < kMergeRows && m < M) {
#pragma unroll
    for (int w = 1; w < kMergeWaves; ++w) lse_combine(rm, rs, pm[w][lane], ps[w][lane]);
    const float l = rm + logf(rs);
    if (lse) lse[m] = l;
    const int lab = labels[m];
    loss[m] = (lab >= 0 && lab < V) ? l - label_logit[m] : 0.f;
  }
}

hipError_t launch_lse_merge(const float* tmax, const float* tsum, const float* label_logit,
                            const int* labels, int T, int M, int V, float* lse, float* loss,
                            hipStream_t stream) {
  hipLaunchKernelGGL(k_lse_merge, dim3(cdiv(M, kMergeRows)), dim3(64 * kMergeWaves), 0, stream,
                     tmax, tsum, label_logit, labels, T, M, V, lse, loss);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Rotary tables: cos / sin of p * theta^(-2i/hd), angles and trigonometry in
// fp64, stored fp32, [max_pos, hd/2].
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_rope_tables(double theta, int max_pos, int half,
                                                     float* __restrict__ rcos,
                                                     float* __restrict__ rsin) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)max_pos * half) return;
  const int p = (int)(idx / half), i = (int)(idx % half);
  const double ang = (double)p * pow(theta, -2.0 * (double)i / (double)(2 * half));
  rcos[idx] = (float)cos(ang);
  rsin[idx] = (float)sin(ang);
}

hipError_t launch_rope_tables(double theta, int max_pos, int head_dim, float* rcos, float* rsin,
                              hipStream_t stream) {
  const int half = head_dim / 2;
  hipLaunchKernelGGL(k_rope_tables, dim3(cdiv((int64_t)max_pos * half, 256)), dim3(256), 0, stream,
                     theta, max_pos, half, rcos, rsin);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Unfused baseline ops: each reads its inputs from HBM and writes its output
// back (section "The cost of laziness in large-model training": every
// operator boundary is a write-back to GPU memory).  16 B per lane accesses.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_residual_add(const uint16_t* __restrict__ y,
                                                      const uint16_t* __restrict__ res,
                                                      uint16_t* __restrict__ h, int64_t total8) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= total8) return;
  float a[8], b[8];
  load8(y + idx * 8, a);
  load8(res + idx * 8, b);
#pragma unroll
  for (int q = 0; q < 8; ++q) a[q] += b[q];
  store8(h + idx * 8, a);
}

hipError_t launch_residual_add(const uint16_t* y, const uint16_t* res, uint16_t* h, int64_t count,
                               hipStream_t stream) {
  const int64_t total8 = count / 8;
  hipLaunchKernelGGL(k_residual_add, dim3(cdiv(total8, 256)), dim3(256), 0, stream, y, res, h,
                     total8);
  return hipGetLastError();
}

// RMSNorm of one row per 256-thread block; each thread owns 8-element groups
// strided by 256*8, kept in registers between the two passes (N <= 16384).
constexpr int kNormMaxGroups = 8;
__global__ __launch_bounds__(256) void k_rmsnorm(const uint16_t* __restrict__ h,
                                                 const float* __restrict__ gamma, float eps,
                                                 uint16_t* __restrict__ out, int N) {
  const int m = blockIdx.x;
  const uint16_t* row = h + (size_t)m * N;
  float v[kNormMaxGroups][8];
  float ss = 0.f;
#pragma unroll
  for (int g = 0; g < kNormMaxGroups; ++g) {
    const int n = (g * 256 + threadIdx.x) * 8;
    if (n < N) {
      load8(row + n, v[g]);
#pragma unroll
      for (int q = 0; q < 8; ++q) ss += v[g][q] * v[g][q];
    }
  }
  __shared__ float red[4];
  for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float tot = red[0] + red[1] + red[2] + red[3];
  const float rr = 1.0f / sqrtf(tot / (float)N + eps);
#pragma unroll
  for (int g = 0; g < kNormMaxGroups; ++g) {
    const int n = (g * 256 + threadIdx.x) * 8;
    if (n < N) {
      float o[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) o[q] = v[g][q] * rr * gamma[n + q];
      store8(out + (size_t)m * N + n, o);
    }
  }
}

hipError_t launch_rmsnorm(const uint16_t* h, const float* gamma, float eps, uint16_t* out, int M,
                          int N, hipStream_t stream) {
  hipLaunchKernelGGL(k_rmsnorm, dim3(M), dim3(256), 0, stream, h, gamma, eps, out, N);
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void k_swiglu(const uint16_t* __restrict__ gu,
                                                uint16_t* __restrict__ out, int M, int N) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int n8 = N / 8;
  if (idx >= (int64_t)M * n8) return;
  const int64_t m = idx / n8;
  const int n = (int)(idx - m * n8) * 8;
  float g[8], u[8];
  load8(gu + (size_t)m * 2 * N + n, g);
  load8(gu + (size_t)m * 2 * N + N + n, u);
#pragma unroll
  for (int q = 0; q < 8; ++q) g[q] = silu_f32(g[q]) * u[q];
  store8(out + (size_t)m * N + n, g);
}

hipError_t launch_swiglu(const uint16_t* gu, uint16_t* out, int M, int N, hipStream_t stream) {
  hipLaunchKernelGGL(k_swiglu, dim3(cdiv((int64_t)M * (N / 8), 256)), dim3(256), 0, stream, gu,
                     out, M, N);
  return hipGetLastError();
}

// Unfused backward pieces (the passes the fused backward epilogues replace).
// SwiGLU backward from a stored dout [M, N] and the saved gu = [g | u]:
// dz = [dg | du], 8 features per thread.
__global__ __launch_bounds__(256) void k_swiglu_bwd(const uint16_t* __restrict__ dout,
                                                    const uint16_t* __restrict__ gu,
                                                    uint16_t* __restrict__ dz, int M, int N) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int n8 = N / 8;
  if (idx >= (int64_t)M * n8) return;
  const int64_t m = idx / n8;
  const int n = (int)(idx - m * n8) * 8;
  float d[8], g[8], u[8], dg[8], du[8];
  load8(dout + (size_t)m * N + n, d);
  load8(gu + (size_t)m * 2 * N + n, g);
  load8(gu + (size_t)m * 2 * N + N + n, u);
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const float sg = 1.0f / (1.0f + __expf(-g[q]));
    const float sl = g[q] * sg;
    du[q] = d[q] * sl;
    dg[q] = d[q] * u[q] * (sg + sl * (1.0f - sg));
  }
  store8(dz + (size_t)m * 2 * N + n, dg);
  store8(dz + (size_t)m * 2 * N + N + n, du);
}

hipError_t launch_swiglu_bwd(const uint16_t* dout, const uint16_t* gu, uint16_t* dz, int M, int N,
                             hipStream_t stream) {
  hipLaunchKernelGGL(k_swiglu_bwd, dim3(cdiv((int64_t)M * (N / 8), 256)), dim3(256), 0, stream,
                     dout, gu, dz, M, N);
  return hipGetLastError();
}

// RMSNorm backward from a stored G = dz W' [M, N] (gamma folded into W'),
// one block per row; the row scale is recomputed from h in the same pass:
//   r = 1 / sqrt(mean h^2 + eps),  dh = r G - (r^3 / N) (sum_j h_j G_j) h + dY.
__global__ __launch_bounds__(256) void k_rmsnorm_bwd(const uint16_t* __restrict__ G,
                                                     const uint16_t* __restrict__ h,
                                                     const uint16_t* __restrict__ dY, float eps,
                                                     uint16_t* __restrict__ dh, int N) {
  const int m = blockIdx.x;
  const size_t row = (size_t)m * N;
  float gv[kNormMaxGroups][8], hv[kNormMaxGroups][8];
  float dot = 0.f, ss = 0.f;
#pragma unroll
  for (int g = 0; g < kNormMaxGroups; ++g) {
    const int n = (g * 256 + threadIdx.x) * 8;
    if (n < N) {
      load8(G + row + n, gv[g]);
      load8(h + row + n, hv[g]);
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        dot += gv[g][q] * hv[g][q];
        ss += hv[g][q] * hv[g][q];
      }
    }
  }
  __shared__ float red[2][4];
  for (int o = 32; o > 0; o >>= 1) {
    dot += __shfl_xor(dot, o, 64);
    ss += __shfl_xor(ss, o, 64);
  }
  if ((threadIdx.x & 63) == 0) {
    red[0][threadIdx.x >> 6] = dot;
    red[1][threadIdx.x >> 6] = ss;
  }
  __syncthreads();
  const float inv_n = 1.0f / (float)N;
  const float rr = 1.0f / sqrtf((red[1][0] + red[1][1] + red[1][2] + red[1][3]) * inv_n + eps);
  const float cm = rr * rr * rr * ((red[0][0] + red[0][1] + red[0][2] + red[0][3]) * inv_n);
#pragma unroll
  for (int g = 0; g < kNormMaxGroups; ++g) {
    const int n = (g * 256 + threadIdx.x) * 8;
    if (n < N) {
      float y[8], o[8];
      load8(dY + row + n, y);
#pragma unroll
      for (int q = 0; q < 8; ++q) o[q] = rr * gv[g][q] - cm * hv[g][q] + y[q];
      store8(dh + row + n, o);
    }
  }
}

hipError_t launch_rmsnorm_bwd(const uint16_t* G, const uint16_t* h, const uint16_t* dY, float eps,
                              uint16_t* dh, int M, int N, hipStream_t stream) {
  hipLaunchKernelGGL(k_rmsnorm_bwd, dim3(M), dim3(256), 0, stream, G, h, dY, eps, dh, N);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Unfused baseline pieces for the attention-input and LM-head workloads (the
// sequences the fused epilogues replace; not on the hot path).
// ---------------------------------------------------------------------------

// In-place rotate-half RoPE on the first n_rot heads (q, then k) of a stored
// qkv tensor [M, N], heads of hd (64 or 128): one thread per (row, head, 4
// pairs).  Positions outside the table are clamped into it, as in the fused
// kernel.
__global__ __launch_bounds__(256) void k_rope_apply(uint16_t* __restrict__ qkv,
                                                    const float* __restrict__ rcos,
                                                    const float* __restrict__ rsin,
                                                    const int* __restrict__ pos, int max_pos,
                                                    int M, int N, int n_rot, int hd) {
  const int half = hd / 2, quads = half / 4;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t per_row = (int64_t)n_rot * quads;
  if (idx >= (int64_t)M * per_row) return;
  const int64_t m = idx / per_row;
  const int rem = (int)(idx - m * per_row);
  const int q4 = (rem % quads) * 4;
  uint16_t* base = qkv + m * N + (int64_t)(rem / quads) * hd;
  const size_t p = (size_t)min(max(pos[m], 0), max_pos - 1) * half + q4;
  const f32x4_t c = *(const f32x4_t*)(rcos + p), sn = *(const f32x4_t*)(rsin + p);
  float a[4], b[4], ra[4], rb[4];
  unpack_bf16x4(*(const u32x2_t*)(base + q4), a);
  unpack_bf16x4(*(const u32x2_t*)(base + half + q4), b);
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    ra[v] = a[v] * c[v] - b[v] * sn[v];
    rb[v] = b[v] * c[v] + a[v] * sn[v];
  }
  *(u32x2_t*)(base + q4) = pack_bf16x4(ra[0], ra[1], ra[2], ra[3]);
  *(u32x2_t*)(base + half + q4) = pack_bf16x4(rb[0], rb[1], rb[2], rb[3]);
}

hipError_t launch_rope_apply(uint16_t* qkv, const float* rcos, const float* rsin, const int* pos,
                             int max_pos, int M, int n_q, int n_kv, int head_dim,
                             hipStream_t stream) {
  const int N = (n_q + 2 * n_kv) * head_dim, n_rot = n_q + n_kv;
  hipLaunchKernelGGL(k_rope_apply, dim3(cdiv((int64_t)M * n_rot * (head_dim / 8), 256)),
                     dim3(256), 0, stream, qkv, rcos, rsin, pos, max_pos, M, N, n_rot, head_dim);
  return hipGetLastError();
}

// loss[m] = logsumexp_n z[m, n] - z[m, label[m]] over stored bf16 logits
// [M, V]: one block per row; each thread keeps a running (max, sum exp) over
// its chunks of 8 logits, then the 256 pairs are merged.  A label outside
// [0, V) gives loss 0, as in the fused merge.
__global__ __launch_bounds__(256) void k_ce_rows(const uint16_t* __restrict__ z,
                                                 const int* __restrict__ labels,
                                                 float* __restrict__ lse, float* __restrict__ loss,
                                                 int V) {
  __shared__ float pm[4], ps[4];
  const int m = blockIdx.x;
  const uint16_t* row = z + (size_t)m * V;
  float mx = -INFINITY, se = 0.f;
  for (int c = threadIdx.x * 8; c < V; c += 256 * 8) {
    float f[8];
    load8(row + c, f);
    float cm = f[0];
#pragma unroll
    for (int q = 1; q < 8; ++q) cm = fmaxf(cm, f[q]);
    if (cm > mx) {
      se = mx == -INFINITY ? 0.f : se * __expf(mx - cm);
      mx = cm;
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) se += __expf(f[q] - mx);
  }
  for (int o = 32; o > 0; o >>= 1) {
    const float m2 = __shfl_xor(mx, o, 64), s2 = __shfl_xor(se, o, 64);
    lse_combine(mx, se, m2, s2);
  }
  if ((threadIdx.x & 63) == 0) {
    pm[threadIdx.x >> 6] = mx;
    ps[threadIdx.x >> 6] = se;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < 4; ++w) lse_combine(mx, se, pm[w], ps[w]);
    const float l = mx + logf(se);
    const int lab = labels[m];
    lse[m] = l;
    loss[m] = (lab >= 0 && lab < V) ? l - bf16_to_f32(row[lab]) : 0.f;
  }
}

// e4m3 quantisation for the unfused fp8 baseline (delayed scaling):
// out = E4M3_sat(x / s_in) with s_in the previous scale, and the amax of |x|
// for the next one.  A grid of a few blocks per compute unit walks the
// tensor in 8-element groups (four groups in flight per lane), keeps the
// lane's running amax in a register, and each block issues one atomicMax
// (on the non-negative float's bit pattern, which orders like the float).
__device__ __forceinline__ float quantize8(const uint16_t* __restrict__ x, uint8_t* __restrict__ out,
                                           int64_t g, float inv, float mx) {
  float f[8];
  load8(x + g * 8, f);
#pragma unroll
  for (int q = 0; q < 8; ++q) mx = fmaxf(mx, fabsf(f[q]));
  const uint32_t lo = pack_e4m3x4_sat(f[0] * inv, f[1] * inv, f[2] * inv, f[3] * inv);
  const uint32_t hi = pack_e4m3x4_sat(f[4] * inv, f[5] * inv, f[6] * inv, f[7] * inv);
  *(u32x2_t*)(out + g * 8) = u32x2_t{lo, hi};
  return mx;
}

__global__ __launch_bounds__(256) void k_quantize_e4m3(const uint16_t* __restrict__ x,
                                                       const float* __restrict__ s_in,
                                                       uint8_t* __restrict__ out, int64_t total8,
                                                       unsigned int* __restrict__ amax_bits) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const float inv = 1.0f / s_in[0];
  float mx = 0.f;
  for (; g + 3 * stride < total8; g += 4 * stride) {
    i32x4_t raw[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) raw[u] = *(const i32x4_t*)(x + (g + u * stride) * 8);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      float f[8];
      unpack_bf16x4(u32x2_t{(unsigned)raw[u].x, (unsigned)raw[u].y}, f);
      unpack_bf16x4(u32x2_t{(unsigned)raw[u].z, (unsigned)raw[u].w}, f + 4);
#pragma unroll
      for (int q = 0; q < 8; ++q) mx = fmaxf(mx, fabsf(f[q]));
      const uint32_t lo = pack_e4m3x4_sat(f[0] * inv, f[1] * inv, f[2] * inv, f[3] * inv);
      const uint32_t hi = pack_e4m3x4_sat(f[4] * inv, f[5] * inv, f[6] * inv, f[7] * inv);
      *(u32x2_t*)(out + (g + u * stride) * 8) = u32x2_t{lo, hi};
    }
  }
  for (; g < total8; g += stride) mx = quantize8(x, out, g, inv, mx);
  __shared__ float red[4];
  for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = mx;
  __syncthreads();
  if (threadIdx.x == 0)
    atomicMax(amax_bits, __float_as_uint(fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]))));
}

hipError_t launch_quantize_e4m3(const uint16_t* x, const float* s_in, uint8_t* out, int64_t count,
                                float* amax, float* s_out, hipStream_t stream) {
  unsigned int* bits = reinterpret_cast<unsigned int*>(amax);
  const int64_t total8 = count / 8;
  const int blocks = (int)std::min<int64_t>(cdiv(total8, 256), (int64_t)cu_count() * 8);
  hipLaunchKernelGGL(k_zero_u32, dim3(1), dim3(1), 0, stream, bits);
  hipLaunchKernelGGL(k_quantize_e4m3, dim3(blocks), dim3(256), 0, stream, x, s_in, out, total8,
                     bits);
  hipLaunchKernelGGL(k_amax_to_scale, dim3(1), dim3(1), 0, stream, bits, amax, s_out);
  return hipGetLastError();
}

hipError_t launch_ce_rows(const uint16_t* z, const int* labels, float* lse, float* loss, int M,
                          int V, hipStream_t stream) {
  hipLaunchKernelGGL(k_ce_rows, dim3(M), dim3(256), 0, stream, z, labels, lse, loss, V);
  return hipGetLastError();
}

}  // namespace coda
