// e4m3 (OCP E4M3FN) GEMM kernels with epilogue programs, on the fp8 mainloop
// of gemm_core_fp8.hpp.
//
// Citations name sections of the news page "CODA: New Research Optimizes
// Transformer Training with GEMM-Epilogue Programming" (KuCoin news flash).
// Section "The cost of laziness in large-model training" notes that FP8 makes
// the matrix products faster while the data movement around them does not
// shrink, which is what fusing the epilogues removes.
//
// The mainloop is gemm_core_fp8.hpp's mainloop_fp8 (v_mfma_f32_16x16x128_f8f6f4),
// whose accumulators have the bf16 kernels' layout: lane L = 16 gq + r,
// register v of the 16x16 tile (j, i) holds feature nbase + 16 j + 4 gq + v
// of token mbase + 16 i + r.  A run of 4 consecutive features is 8 bytes of
// bf16 or 4 bytes of e4m3, and a per-token sum over the wave's features is a
// lane-local sum plus exchanges between lanes 16 and 32 apart.

#include "gemm_core_fp8.hpp"
#include "launch.hpp"

namespace coda {

// ---------------------------------------------------------------------------
// GEMM1 (fp8 operands): h = residual + acc * sa * sw, stored bf16; partial
// sums of squares and partial amax of the unrounded h (features at or past N
// left out); optionally h8 = E4M3(h / s_h) for the fp8 second GEMM (delayed
// scaling: s_h is a device scalar written by the previous reduction).
//   residual: 16 bytes per lane at the start of the epilogue; for a pair of
//     subtiles (2 p, 2 p + 1), lanes of even gq load subtile 2 p at features
//     8 (gq / 2) + 0..7 and lanes of odd gq subtile 2 p + 1, then lanes 16
//     apart swap one run (32 loads per lane);
//   h: lanes 16 apart exchange one run per pair of subtiles, one 16-byte
//     store of 8 features (as the bf16 GEMM1);
//   h8: the 4-byte e4m3 runs of four subtiles go through two exchanges
//     (lanes 16 apart, then 32 apart) so that each lane stores one whole
//     16-feature subtile row, 16 bytes.
// ---------------------------------------------------------------------------
// At least this many vector memory operations per lane follow a tile's
// prefetch of the next tile (the residual loads and the 16-byte h stores; h8
// and partial stores come on top), so the next tile waits for its stage 0
// without draining them.
constexpr int kGemm1Stores8 = 32;

__global__ __launch_bounds__(kThreads, 1) void k_residual_partialrms_fp8(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ W, const float* __restrict__ a_scale,
    const float* __restrict__ w_scale, const uint16_t* __restrict__ res, uint16_t* __restrict__ h,
    float* __restrict__ psum, const float* __restrict__ h8_scale, uint8_t* __restrict__ h8,
    float* __restrict__ pamax, int M, int N, int K, int gm, int gn) {
  __shared__ __attribute__((aligned(1024))) char smem[kSmemBytes];
  const float scale = a_scale[0] * w_scale[0];
  const float inv_s8 = h8 ? 1.0f / h8_scale[0] : 1.0f;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int gq = lane >> 4;
  const bool godd = (gq & 1) != 0, ghi = gq >= 2;
  const int nt = gm * gn;
  bool prefetched = false;
  for (int t = blockIdx.x; t < nt; t += gridDim.x) {
    const TileCoord tc = map_tile(t, gm, gn, 8);
    const int m0 = tc.tm * kBM, n0 = tc.tn * kBN;
    TileChain ch;
    ch.prefetched = prefetched;
    const bool has_next = t + (int)gridDim.x < nt;
    const TileCoord nc = has_next ? map_tile(t + gridDim.x, gm, gn, 8) : tc;
    ch.next = MainloopSrc{A, W, nullptr, M, N, K, nc.tm * kBM, nc.tn * kBN};
    const int nw0 = n0 + wn * 128;
    const uint32_t rows_here = (uint32_t)min(kBM, M - m0);
    const __amdgpu_buffer_rsrc_t rrsrc = make_rsrc(res + (size_t)m0 * N, rows_here * (uint32_t)N * 2u);
    const __amdgpu_buffer_rsrc_t hrsrc = make_rsrc(h + (size_t)m0 * N, rows_here * (uint32_t)N * 2u);
    const __amdgpu_buffer_rsrc_t qrsrc =
        make_rsrc(h8 ? h8 + (size_t)m0 * N : nullptr, h8 ? rows_here * (uint32_t)N : 0u);
    Acc acc;
    mainloop_fp8<false, kGemm1Stores8>(acc, smem, MainloopSrc{A, W, nullptr, M, N, K, m0, n0},
                                          ch, [] {}, [] {});
    u32x4_t rq[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t ml = (uint32_t)(wm * 128 + i * 16 + (lane & 15));
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const int n = nw0 + 16 * (2 * p + (godd ? 1 : 0));
        const uint32_t off = n < N ? (ml * (uint32_t)N + (uint32_t)(n + 8 * (gq >> 1))) * 2u : kOobOffset;
        rq[i][p] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rrsrc, off, 0, 0));
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int ml = wm * 128 + i * 16 + (lane & 15);
      const bool mv = m0 + ml < M;
      float ss = 0.f, amax = 0.f;
      uint32_t q8[8];  // e4m3 runs of subtiles 0..7
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        // this lane's residual runs of subtiles 2p (rr[0]) and 2p + 1 (rr[1])
        u32x2_t rr[2];
        {
          const u32x4_t& v = rq[i][p];
          const u32x2_t lo = {v.x, v.y}, hi = {v.z, v.w};
          const u32x2_t sd = godd ? lo : hi;
          const u32x2_t rx = {(unsigned)__shfl_xor((int)sd.x, 16, 64),
                              (unsigned)__shfl_xor((int)sd.y, 16, 64)};
          rr[0] = godd ? rx : lo;
          rr[1] = godd ? hi : rx;
        }
        u32x2_t pk[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int j = 2 * p + u;
          const bool nv = nw0 + 16 * j + 4 * gq < N;
          float rv[4], hv[4];
          unpack_bf16x4(rr[u], rv);
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            hv[v] = rv[v] + acc.v[j][i][v] * scale;
            const float hm = nv ? hv[v] : 0.f;
            ss = __builtin_fmaf(hm, hm, ss);
            asm("v_max_f32_e64 %0, %1, |%2|" : "=v"(amax) : "v"(amax), "v"(hm));
          }
          pk[u] = pack_bf16x4(hv[0], hv[1], hv[2], hv[3]);
          q8[j] = pack_e4m3x4_sat(hv[0] * inv_s8, hv[1] * inv_s8, hv[2] * inv_s8, hv[3] * inv_s8);
        }
        const int n = nw0 + 16 * (2 * p + (godd ? 1 : 0)) + 8 * (gq >> 1);
        store16_exchanged(hrsrc, pk, godd,
                          (mv && n < N) ? ((uint32_t)ml * (uint32_t)N + (uint32_t)n) * 2u
                                        : kOobOffset);
      }
      if (h8) {
#pragma unroll
        for (int b = 0; b < 2; ++b) {  // subtiles 4b .. 4b + 3
          // step 1 (lanes 16 apart): runs of subtiles 4b + s (s = 0, 1 for even
          // gq; s = 1 for odd) -> 8 bytes of subtile 4b + (gq & 1) and of
          // 4b + 2 + (gq & 1), at features 8 (gq / 2) + 0..7
          uint32_t e8[2][2];  // [subtile pair][run]
#pragma unroll
          for (int pr = 0; pr < 2; ++pr) {
            const uint32_t a0 = q8[4 * b + 2 * pr], a1 = q8[4 * b + 2 * pr + 1];
            const uint32_t sd = godd ? a0 : a1;
            const uint32_t rx = (unsigned)__shfl_xor((int)sd, 16, 64);
            e8[pr][0] = godd ? rx : a0;  // lower 4 features of the lane's 8
            e8[pr][1] = godd ? a1 : rx;
          }
          // step 2 (lanes 32 apart): gq < 2 keeps pair 0 (features 0..7 of
          // its subtile) and receives features 8..15 of it; gq >= 2 keeps
          // pair 1 (features 8..15) and receives features 0..7
          const uint32_t s0 = ghi ? e8[0][0] : e8[1][0], s1 = ghi ? e8[0][1] : e8[1][1];
          const uint32_t x0 = (unsigned)__shfl_xor((int)s0, 32, 64);
          const uint32_t x1 = (unsigned)__shfl_xor((int)s1, 32, 64);
          const u32x4_t v = ghi ? u32x4_t{x0, x1, e8[1][0], e8[1][1]}
                                : u32x4_t{e8[0][0], e8[0][1], x0, x1};
          const int sub = 4 * b + (godd ? 1 : 0) + (ghi ? 2 : 0);
          const int n = nw0 + 16 * sub;
          store16(qrsrc, v, (mv && n < N) ? (uint32_t)ml * (uint32_t)N + (uint32_t)n : kOobOffset);
        }
      }
      ss = sum_over_lane_groups(ss);
      amax = max_over_lane_groups(amax);
      if (mv && lane < 16 && nw0 < N) {
        const size_t tt = (size_t)(nw0 / kRmsTileWidth);
        psum[tt * M + m0 + ml] = ss;
        if (pamax) pamax[tt * M + m0 + ml] = amax;
      }
    }
    prefetched = has_next;
  }
  wait_vm0();  // the last tile's unused prefetch into LDS lands before the block ends
}

// ---------------------------------------------------------------------------
// GEMM2 (fp8 operands): g = r * acc_g * sx * sg, u = r * acc_u * sx * su,
// out = silu(g) * u (stored bf16).  Output tile 256 tokens x 128 features.
// ---------------------------------------------------------------------------
constexpr int kSwigluStores8 = 16;  // 16-byte stores per lane per tile

// Gate subtile j and up subtile j + 4 sit in the same lane and register (as
// in the bf16 GEMM2); lanes 16 apart exchange one 4-feature run per 16-byte
// store.
__global__ __launch_bounds__(kThreads, 1) void k_rowscale_swiglu_fp8(
    const uint8_t* __restrict__ X, const float* __restrict__ x_scale,
    const uint8_t* __restrict__ Wg, const uint8_t* __restrict__ Wu,
    const float* __restrict__ wg_scale, const float* __restrict__ wu_scale,
    const float* __restrict__ r, uint16_t* __restrict__ out, int M, int N, int K, int gm, int gn) {
  __shared__ __attribute__((aligned(1024))) char smem[kSmemBytes];
  const float sg = x_scale[0] * wg_scale[0];
  const float sgu = sg * (x_scale[0] * wu_scale[0]);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int gq = lane >> 4;
  const bool godd = (gq & 1) != 0;
  const int nt = gm * gn;
  bool prefetched = false;
  for (int t = blockIdx.x; t < nt; t += gridDim.x) {
    const TileCoord tc = map_tile(t, gm, gn, 8);
    const int m0 = tc.tm * kBM, n0 = tc.tn * (kBN / 2);
    TileChain ch;
    ch.prefetched = prefetched;
    const bool has_next = t + (int)gridDim.x < nt;
    const TileCoord nc = has_next ? map_tile(t + gridDim.x, gm, gn, 8) : tc;
    ch.next = MainloopSrc{X, Wg, Wu, M, N, K, nc.tm * kBM, nc.tn * (kBN / 2)};
    float rr[8];
    auto pre = [&]() {
#pragma unroll
      for (int i = 0; i < 8; ++i) rr[i] = r[min(m0 + wm * 128 + i * 16 + (lane & 15), M - 1)];
    };
    Acc acc;
    mainloop_fp8<true, kSwigluStores8>(acc, smem, MainloopSrc{X, Wg, Wu, M, N, K, m0, n0}, ch,
                                          pre, [] {});
    const __amdgpu_buffer_rsrc_t orsrc =
        make_rsrc(out + (size_t)m0 * N, (uint32_t)min(kBM, M - m0) * (uint32_t)N * 2u);
    const int nw0 = n0 + wn * 64;
    const float kNegLog2e = -1.4426950408889634f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int ml = wm * 128 + i * 16 + (lane & 15);
      const bool mv = m0 + ml < M;
      // silu(g) u = (a b sx^2 sg su r^2) / (1 + 2^(-log2e sx sg r a))
      const float c1 = kNegLog2e * sg * rr[i], k = sgu * rr[i] * rr[i];
#pragma unroll
      for (int j0 = 0; j0 < 4; j0 += 2) {
        u32x2_t pk[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int j = j0 + u;
          float o[4];
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const float a = acc.v[j][i][v], b = acc.v[j + 4][i][v];
            const float e = __builtin_amdgcn_exp2f(a * c1);
            o[v] = (a * k) * b * __builtin_amdgcn_rcpf(1.0f + e);
          }
          pk[u] = pack_bf16x4(o[0], o[1], o[2], o[3]);
        }
        const int n = nw0 + 16 * (j0 + (godd ? 1 : 0)) + 8 * (gq >> 1);
        store16_exchanged(orsrc, pk, godd,
                          (mv && n < N) ? ((uint32_t)ml * (uint32_t)N + (uint32_t)n) * 2u
                                        : kOobOffset);
      }
    }
    prefetched = has_next;
  }
  wait_vm0();  // the last tile's unused prefetch into LDS lands before the block ends
}

// ---------------------------------------------------------------------------
// Plain fp8 GEMM for the unfused baseline: C[m, n] = bf16(A[m,:] . W[n,:] *
// sa * sw), C with row stride ldc (so two GEMMs with different weight scales
// can fill the two halves of one [M, 2N] buffer).  Stores as in the plain
// bf16 GEMM (lanes 16 apart exchange a 4-feature run; 16 bytes per store).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads, 1) void k_gemm_plain_fp8(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ W, const float* __restrict__ a_scale,
    const float* __restrict__ w_scale, uint16_t* __restrict__ C, int M, int N, int K, int ldc,
    int gm, int gn) {
  __shared__ __attribute__((aligned(1024))) char smem[kSmemBytes];
  const float scale = a_scale[0] * w_scale[0];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int gq = lane >> 4;
  const bool godd = (gq & 1) != 0;
  const int nt = gm * gn;
  bool prefetched = false;
  for (int t = blockIdx.x; t < nt; t += gridDim.x) {
    const TileCoord tc = map_tile(t, gm, gn, 8);
    const int m0 = tc.tm * kBM, n0 = tc.tn * kBN;
    TileChain ch;
    ch.prefetched = prefetched;
    const bool has_next = t + (int)gridDim.x < nt;
    const TileCoord nc = has_next ? map_tile(t + gridDim.x, gm, gn, 8) : tc;
    ch.next = MainloopSrc{A, W, nullptr, M, N, K, nc.tm * kBM, nc.tn * kBN};
    Acc acc;
    mainloop_fp8<false, 32>(acc, smem, MainloopSrc{A, W, nullptr, M, N, K, m0, n0}, ch,
                               [] {}, [] {});
    const int nw0 = n0 + wn * 128;
    const __amdgpu_buffer_rsrc_t crsrc =
        make_rsrc(C + (size_t)m0 * ldc, (uint32_t)min(kBM, M - m0) * (uint32_t)ldc * 2u);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int ml = wm * 128 + i * 16 + (lane & 15);
      const bool mv = m0 + ml < M;
#pragma unroll
      for (int j0 = 0; j0 < 8; j0 += 2) {
        u32x2_t pk[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const f32x4_t& a = acc.v[j0 + u][i];
          pk[u] = pack_bf16x4(a[0] * scale, a[1] * scale, a[2] * scale, a[3] * scale);
        }
        const int n = nw0 + 16 * (j0 + (godd ? 1 : 0)) + 8 * (gq >> 1);
        store16_exchanged(crsrc, pk, godd,
                          (mv && n < N) ? ((uint32_t)ml * (uint32_t)ldc + (uint32_t)n) * 2u
                                        : kOobOffset);
      }
    }
    prefetched = has_next;
  }
  wait_vm0();  // the last tile's unused prefetch into LDS lands before the block ends
}

static inline int cdiv(int a, int b) { return (a + b - 1) / b; }

hipError_t launch_gemm_plain_fp8(const uint8_t* A, const uint8_t* W, const float* a_scale,
                                 const float* w_scale, uint16_t* C, int M, int N, int K, int ldc,
                                 hipStream_t stream) {
  const int gm = cdiv(M, kBM), gn = cdiv(N, kBN);
  hipLaunchKernelGGL(k_gemm_plain_fp8, dim3(min(gm * gn, cu_count())), dim3(kThreads), 0,
                     stream, A, W, a_scale, w_scale, C, M, N, K, ldc, gm, gn);
  return hipGetLastError();
}

hipError_t launch_residual_partialrms_fp8(const uint8_t* A, const uint8_t* W, const float* a_scale,
                                          const float* w_scale, const uint16_t* res, uint16_t* h,
                                          float* psum, const float* h8_scale, uint8_t* h8,
                                          float* pamax, int M, int N, int K, hipStream_t stream) {
  const int gm = cdiv(M, kBM), gn = cdiv(N, kBN);
  hipLaunchKernelGGL(k_residual_partialrms_fp8, dim3(min(gm * gn, cu_count())), dim3(kThreads), 0,
                     stream, A, W,
                     a_scale, w_scale, res, h, psum, h8_scale, h8, pamax, M, N, K, gm, gn);
  return hipGetLastError();
}

hipError_t launch_rowscale_swiglu_fp8(const uint8_t* X, const float* x_scale, const uint8_t* Wg,
                                      const uint8_t* Wu, const float* wg_scale,
                                      const float* wu_scale, const float* r, uint16_t* out, int M,
                                      int N, int K, hipStream_t stream) {
  const int gm = cdiv(M, kBM), gn = cdiv(N, kBN / 2);
  hipLaunchKernelGGL(k_rowscale_swiglu_fp8, dim3(min(gm * gn, cu_count())), dim3(kThreads), 0,
                     stream, X, x_scale,
                     Wg, Wu, wg_scale, wu_scale, r, out, M, N, K, gm, gn);
  return hipGetLastError();
}

}  // namespace coda
