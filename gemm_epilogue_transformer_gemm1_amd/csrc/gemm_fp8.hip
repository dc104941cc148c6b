// e4m3 (OCP E4M3FN) GEMM kernels with epilogue programs, on the fp8 mainloop
// of gemm_core.hpp.
//
// Citations name sections of the news page "CODA: New Research Optimizes
// Transformer Training with GEMM-Epilogue Programming" (KuCoin news flash).
// Section "The cost of laziness in large-model training" notes that FP8 makes
// the matrix products faster while the data movement around them does not
// shrink, which is what fusing the epilogues removes.
//
// Accumulator layout (32x32 tiles): lane L, register r of tile (j, i) holds
// feature nbase + 32j + 8(r/4) + 4(L/32) + r%4 of token mbase + 32i + L%32.
// Each group g = r/4 is a run of 4 consecutive features (8 bytes of bf16, 4
// bytes of e4m3), and a per-token sum over the wave's features is a
// lane-local sum plus one exchange between lanes L and L^32.

#include "gemm_core.hpp"
#include "launch.hpp"

namespace coda {

// ---------------------------------------------------------------------------
// GEMM1 (fp8 operands): h = residual + acc * sa * sw, stored bf16; partial
// sums of squares and partial amax of the unrounded h; optionally
// h8 = E4M3(h / s_h) for the fp8 second GEMM (delayed scaling: s_h is a
// device scalar written by the previous reduction).
// ---------------------------------------------------------------------------
// At least this many vector memory operations per lane follow a tile's
// prefetch of the next tile (the 16-byte h stores; the residual loads, h8
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
  const int g4 = (lane >> 5) * 4;
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
    // The residual tile is loaded at the start of the epilogue into the
    // registers the fragments used (loaded during the last stages it would
    // make their waits longer and push the mainloop into spills).  Lanes L
    // and L + 32 hold the runs 8g + 0..3 and 8g + 4..7 of one row in each
    // 32-feature block; for a pair of runs (gp, gp + 1) lane L loads the 16
    // bytes of run gp (its own half and lane L + 32's) and lane L + 32 those
    // of run gp + 1, and `res_runs` swaps the foreign halves: 32 loads of 16
    // bytes per lane instead of 64 of 8.  Column starts are clamped to N - 8
    // and rows to M - 1 (those values are never used).
    u32x4_t rq[4][8];
    const bool hi = lane >= 32;
    auto load_res = [&](int i0) {
#pragma unroll
      for (int i = i0; i < i0 + 2; ++i) {
        const size_t row = (size_t)min(m0 + wm * 128 + i * 32 + (lane & 31), M - 1) * (size_t)N;
#pragma unroll
        for (int q = 0; q < 8; ++q) {  // q = 2 j + gp / 2
          const int n = min(nw0 + (q >> 1) * 32 + ((q & 1) * 2 + (hi ? 1 : 0)) * 8, N - 8);
          rq[i][q] = *(const u32x4_t*)(res + row + n);
        }
      }
    };
    // this lane's runs gp (out[0]) and gp + 1 (out[1]) from its 16 bytes;
    // all 64 lanes take part (lane shuffle)
    auto res_runs = [&](const u32x4_t& v, u32x2_t (&out)[2]) {
      const u32x2_t lo2 = {v.x, v.y}, hi2 = {v.z, v.w};
      const u32x2_t sd = hi ? lo2 : hi2;
      const u32x2_t rx = {(unsigned)__shfl_xor((int)sd.x, 32, 64),
                          (unsigned)__shfl_xor((int)sd.y, 32, 64)};
      out[0] = hi ? rx : lo2;
      out[1] = hi ? hi2 : rx;
    };
    Acc8 acc;
    mainloop_fp8<false, kGemm1Stores8>(acc, smem, MainloopSrc{A, W, nullptr, M, N, K, m0, n0},
                                       ch, [] {}, [] {});
    load_res(0);
    load_res(2);

    // Lanes L and L + 32 hold the runs 8g + 0..3 and 8g + 4..7 (g = 0..3) of
    // the same row in each 32-feature block j.  Exchanges between them give
    // every lane contiguous output: for h, one whole 8-feature run per pair
    // of runs (two 16-byte stores per block); for h8, features 0..15 (lane L)
    // or 16..31 (lane L + 32) of the block (one 16-byte store).  Each store
    // then covers 32 rows with 32 contiguous bytes a row, instead of 8 or 4
    // bytes from each of two lanes: the store path pays per row touched.
    // Buffers start at the tile's first row; masked lanes store out of range.
    const uint32_t rows_here = (uint32_t)min(kBM, M - m0);
    const __amdgpu_buffer_rsrc_t hrsrc = make_rsrc(h + (size_t)m0 * N, rows_here * (uint32_t)N * 2u);
    const __amdgpu_buffer_rsrc_t qrsrc =
        make_rsrc(h8 ? h8 + (size_t)m0 * N : nullptr, h8 ? rows_here * (uint32_t)N : 0u);
    // Partial statistics leave out features at or past N (one select per
    // value; a branch to a mask-free copy of this code for full-width waves
    // makes the register allocator copy the accumulators).
    {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int ml = wm * 128 + i * 32 + (lane & 31);  // row within the tile
        const bool mv = m0 + ml < M;
        const uint32_t erow = (uint32_t)ml * (uint32_t)N;
        float ss = 0.f, amax = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          u32x2_t hb[4], rr[2][2];  // rr[gp / 2][g - gp]: residual run g
          uint32_t qb[4];
          res_runs(rq[i][2 * j], rr[0]);
          res_runs(rq[i][2 * j + 1], rr[1]);
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const bool nv = nw0 + j * 32 + g * 8 + g4 < N;
            float rv[4], hv[4];
            unpack_bf16x4(rr[g >> 1][g & 1], rv);
#pragma unroll
            for (int v = 0; v < 4; ++v) {
              hv[v] = rv[v] + acc.v[j][i][g * 4 + v] * scale;
              const float hm = nv ? hv[v] : 0.f;
              ss = __builtin_fmaf(hm, hm, ss);
              // max(amax, |hm|) in one instruction (fmaxf would first
              // canonicalise both operands)
              asm("v_max_f32_e64 %0, %1, |%2|" : "=v"(amax) : "v"(amax), "v"(hm));
            }
            hb[g] = pack_bf16x4(hv[0], hv[1], hv[2], hv[3]);
            qb[g] = pack_e4m3x4_sat(hv[0] * inv_s8, hv[1] * inv_s8, hv[2] * inv_s8, hv[3] * inv_s8);
          }
#pragma unroll
          for (int gp = 0; gp < 4; gp += 2) {  // h: runs gp (lane L) and gp + 1 (lane L + 32)
            const int n = nw0 + j * 32 + (gp + (hi ? 1 : 0)) * 8;
            const u32x2_t hs = hi ? hb[gp] : hb[gp + 1];
            const u32x2_t hr = {(unsigned)__shfl_xor((int)hs.x, 32, 64),
                                (unsigned)__shfl_xor((int)hs.y, 32, 64)};
            store16(hrsrc,
                    hi ? u32x4_t{hr.x, hr.y, hb[gp + 1].x, hb[gp + 1].y}
                       : u32x4_t{hb[gp].x, hb[gp].y, hr.x, hr.y},
                    (mv && n < N) ? (erow + (uint32_t)n) * 2u : kOobOffset);
          }
          if (h8) {  // lane L: features 0..15 of the block, lane L + 32: 16..31
            const int n = nw0 + j * 32 + (hi ? 16 : 0);
            const uint32_t q0 = hi ? qb[0] : qb[2], q1 = hi ? qb[1] : qb[3];
            const uint32_t r0 = (unsigned)__shfl_xor((int)q0, 32, 64);
            const uint32_t r1 = (unsigned)__shfl_xor((int)q1, 32, 64);
            store16(qrsrc, hi ? u32x4_t{r0, qb[2], r1, qb[3]} : u32x4_t{qb[0], r0, qb[1], r1},
                    (mv && n < N) ? erow + (uint32_t)n : kOobOffset);
          }
        }
        ss += __shfl_xor(ss, 32, 64);
        amax = fmaxf(amax, __shfl_xor(amax, 32, 64));
        if (mv && lane < 32 && nw0 < N) {
          const size_t tt = (size_t)(nw0 / kRmsTileWidth);
          psum[tt * M + m0 + ml] = ss;
          if (pamax) pamax[tt * M + m0 + ml] = amax;
        }
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
    float rr[4];
    auto pre = [&]() {
#pragma unroll
      for (int i = 0; i < 4; ++i) rr[i] = r[min(m0 + wm * 128 + i * 32 + (lane & 31), M - 1)];
    };
    Acc8 acc;
    mainloop_fp8<true, kSwigluStores8>(acc, smem, MainloopSrc{X, Wg, Wu, M, N, K, m0, n0}, ch,
                                       pre, [] {});

    // 16 stores per lane (masked ones at an out-of-range offset of a buffer
    // starting at row m0); lanes L and L + 32 exchange halves of their 4-run
    // pairs so that each stores a whole 8-feature run (see GEMM1 above).
    const __amdgpu_buffer_rsrc_t orsrc =
        make_rsrc(out + (size_t)m0 * N, (uint32_t)min(kBM, M - m0) * (uint32_t)N * 2u);
    const int nw0 = n0 + wn * 64;
    const bool hi = lane >= 32;
    const float kNegLog2e = -1.4426950408889634f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ml = wm * 128 + i * 32 + (lane & 31);
      const bool mv = m0 + ml < M;
      // silu(g) u = (a b sx^2 sg su r^2) / (1 + 2^(-log2e sx sg r a))
      const float c1 = kNegLog2e * sg * rr[i], k = sgu * rr[i] * rr[i];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
#pragma unroll
        for (int gp = 0; gp < 4; gp += 2) {
          u32x2_t ob[2];
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const int g = gp + u;
            float o[4];
#pragma unroll
            for (int v = 0; v < 4; ++v) {
              const float a = acc.v[j][i][g * 4 + v], b = acc.v[j + 2][i][g * 4 + v];
              const float e = __builtin_amdgcn_exp2f(a * c1);
              o[v] = (a * k) * b * __builtin_amdgcn_rcpf(1.0f + e);
            }
            ob[u] = pack_bf16x4(o[0], o[1], o[2], o[3]);
          }
          const int n = nw0 + j * 32 + (gp + (hi ? 1 : 0)) * 8;
          const u32x2_t os = hi ? ob[0] : ob[1];
          const u32x2_t orx = {(unsigned)__shfl_xor((int)os.x, 32, 64),
                               (unsigned)__shfl_xor((int)os.y, 32, 64)};
          const uint32_t off = (mv && n < N) ? ((uint32_t)ml * (uint32_t)N + (uint32_t)n) * 2u
                                             : kOobOffset;
          store16(orsrc, hi ? u32x4_t{orx.x, orx.y, ob[1].x, ob[1].y}
                            : u32x4_t{ob[0].x, ob[0].y, orx.x, orx.y}, off);
        }
      }
    }
    prefetched = has_next;
  }
  wait_vm0();  // the last tile's unused prefetch into LDS lands before the block ends
}

// ---------------------------------------------------------------------------
// Plain fp8 GEMM for the unfused baseline: C[m, n] = bf16(A[m,:] . W[n,:] *
// sa * sw), C with row stride ldc (so two GEMMs with different weight scales
// can fill the two halves of one [M, 2N] buffer).  Stores as in GEMM1: lanes
// L and L + 32 exchange halves of their run pairs, 16 bytes per store.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads, 1) void k_gemm_plain_fp8(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ W, const float* __restrict__ a_scale,
    const float* __restrict__ w_scale, uint16_t* __restrict__ C, int M, int N, int K, int ldc,
    int gm, int gn) {
  __shared__ __attribute__((aligned(1024))) char smem[kSmemBytes];
  const float scale = a_scale[0] * w_scale[0];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int nt = gm * gn;
  const bool hi = lane >= 32;
  bool prefetched = false;
  for (int t = blockIdx.x; t < nt; t += gridDim.x) {
    const TileCoord tc = map_tile(t, gm, gn, 8);
    const int m0 = tc.tm * kBM, n0 = tc.tn * kBN;
    TileChain ch;
    ch.prefetched = prefetched;
    const bool has_next = t + (int)gridDim.x < nt;
    const TileCoord nc = has_next ? map_tile(t + gridDim.x, gm, gn, 8) : tc;
    ch.next = MainloopSrc{A, W, nullptr, M, N, K, nc.tm * kBM, nc.tn * kBN};
    Acc8 acc;
    mainloop_fp8<false>(acc, smem, MainloopSrc{A, W, nullptr, M, N, K, m0, n0}, ch, [] {}, [] {});
    const __amdgpu_buffer_rsrc_t crsrc =
        make_rsrc(C + (size_t)m0 * ldc, (uint32_t)min(kBM, M - m0) * (uint32_t)ldc * 2u);
    const int nw0 = n0 + wn * 128;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ml = wm * 128 + i * 32 + (lane & 31);
      const bool mv = m0 + ml < M;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        u32x2_t pk[4];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x16_t& a = acc.v[j][i];
          pk[g] = pack_bf16x4(a[g * 4] * scale, a[g * 4 + 1] * scale, a[g * 4 + 2] * scale,
                              a[g * 4 + 3] * scale);
        }
#pragma unroll
        for (int gp = 0; gp < 4; gp += 2) {
          const int n = nw0 + j * 32 + (gp + (hi ? 1 : 0)) * 8;
          const u32x2_t sd = hi ? pk[gp] : pk[gp + 1];
          const u32x2_t rx = {(unsigned)__shfl_xor((int)sd.x, 32, 64),
                              (unsigned)__shfl_xor((int)sd.y, 32, 64)};
          store16(crsrc,
                  hi ? u32x4_t{rx.x, rx.y, pk[gp + 1].x, pk[gp + 1].y}
                     : u32x4_t{pk[gp].x, pk[gp].y, rx.x, rx.y},
                  (mv && n < N) ? ((uint32_t)ml * (uint32_t)ldc + (uint32_t)n) * 2u : kOobOffset);
        }
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
  hipLaunchKernelGGL(k_gemm_plain_fp8, dim3(min(gm * gn, cu_count())), dim3(kThreads), 0, stream,
                     A, W, a_scale, w_scale, C, M, N, K, ldc, gm, gn);
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
