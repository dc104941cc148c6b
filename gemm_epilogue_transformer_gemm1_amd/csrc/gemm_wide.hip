// Kernels on the 128 x 384 block tile of gemm_core_wide.hpp: the QKV GEMM with
// the row-scale + RoPE epilogue for QKV widths that are a multiple of 384 (six
// heads of 64), and the plain GEMM for shapes whose 256 x 256 tiles would
// leave the last round of compute units partly idle.
//
// QKV + RoPE: same arithmetic per output as k_rope_bf16 (section "CODA: the secret in
// the epilogue": RoPE re-parameterised into the epilogue; section "Five
// building blocks and a LEGO language": RoPE is an elementwise transform and
// the cos/sin rows are vector loads).
//
// Citations name sections of the news page "CODA: New Research Optimizes
// Transformer Training with GEMM-Epilogue Programming" (KuCoin news flash).
//
// A wave's 192 features are three whole 64-wide heads; the rotate-half partner
// of feature c (< 32) of a head, c + 32, is weight subtile j + 2 in the same
// lane and register, so the rotation needs no data exchange.

#include "gemm_core_wide.hpp"
#include "launch.hpp"

namespace coda {

__global__ __launch_bounds__(kThreads, 1) void k_rope_bf16_wide(
    const uint16_t* __restrict__ X, const uint16_t* __restrict__ W, const float* __restrict__ r,
    const float* __restrict__ rcos, const float* __restrict__ rsin, const int* __restrict__ pos,
    int max_pos, uint16_t* __restrict__ out, int M, int N, int K, int rot_features, int gm,
    int gn) {
  __shared__ __attribute__((aligned(1024))) char smem[kSmemBytes];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int gq = lane >> 4;
  const int nt = gm * gn;
  bool prefetched = false;
  for (int t = blockIdx.x; t < nt; t += gridDim.x) {
    const TileCoord tc = map_tile(t, gm, gn, 8);
    const int m0 = tc.tm * kBMw, n0 = tc.tn * kBNw;
    TileChain ch;
    ch.prefetched = prefetched;
    const bool has_next = t + (int)gridDim.x < nt;
    const TileCoord nc = has_next ? map_tile(t + gridDim.x, gm, gn, 8) : tc;
    ch.next = MainloopSrc{X, W, nullptr, M, N, K, nc.tm * kBMw, nc.tn * kBNw};
    float rr[4];
    int pp[4];
    auto pre = [&]() {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int mc = min(m0 + wm * 64 + i * 16 + (lane & 15), M - 1);
        rr[i] = r[mc];
        pp[i] = pos[mc];
      }
    };
    AccW acc;
    mainloop_bf16_wide(acc, smem, MainloopSrc{X, W, nullptr, M, N, K, m0, n0}, ch, pre, [] {});

    const int nw0 = n0 + wn * 192;  // multiple of 64: three whole heads
    // cos/sin of the 4 token subtiles, loaded before the first use; positions
    // outside the table are clamped into it (memory safety).  Angle index of
    // subtile jj (0, 1) of a head: 16 jj + 4 gq + v.
    f32x4_t ct[4][2], st[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const size_t p = (size_t)min(max(pp[i], 0), max_pos - 1) * 32 + 4 * gq;
      ct[i][0] = *(const f32x4_t*)(rcos + p);
      ct[i][1] = *(const f32x4_t*)(rcos + p + 16);
      st[i][0] = *(const f32x4_t*)(rsin + p);
      st[i][1] = *(const f32x4_t*)(rsin + p + 16);
    }
    // Stores: lanes gq and gq ^ 1 exchange one run of each pair of subtiles
    // (jj = 0, 1 of a half-head), so each 16-byte store writes 64 contiguous
    // bytes of 16 rows; masked lanes store out of range of a buffer that
    // starts at the tile's first row.
    const __amdgpu_buffer_rsrc_t orsrc =
        make_rsrc(out + (size_t)m0 * N, (uint32_t)min(kBMw, M - m0) * (uint32_t)N * 2u);
    const bool godd = (gq & 1) != 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ml = wm * 64 + i * 16 + (lane & 15);  // row within the tile
      const bool mv = m0 + ml < M;
      const float rr_i = rr[i];
#pragma unroll
      for (int hh = 0; hh < 3; ++hh) {
        const int hbase = nw0 + hh * 64;
        const bool rot = hbase < rot_features;
        u32x2_t plo[2], phi[2];
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
          const int ja = hh * 4 + jj, jb = ja + 2;
          const f32x4_t cs = ct[i][jj], sn = st[i][jj];
          float lo[4], hi[4];
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const float a = acc.v[ja][i][v] * rr_i, b = acc.v[jb][i][v] * rr_i;
            lo[v] = rot ? a * cs[v] - b * sn[v] : a;
            hi[v] = rot ? b * cs[v] + a * sn[v] : b;
          }
          plo[jj] = pack_bf16x4(lo[0], lo[1], lo[2], lo[3]);
          phi[jj] = pack_bf16x4(hi[0], hi[1], hi[2], hi[3]);
        }
#pragma unroll
        for (int half = 0; half < 2; ++half) {  // features [0,32) and [32,64) of the head
          const int n = hbase + 32 * half + 16 * (godd ? 1 : 0) + 8 * (gq >> 1);
          store16_exchanged(orsrc, half ? phi : plo, godd,
                            (mv && n < N) ? ((uint32_t)ml * (uint32_t)N + (uint32_t)n) * 2u
                                          : kOobOffset);
        }
      }
    }
    prefetched = has_next;
  }
  wait_vm0();  // the last tile's unused prefetch into LDS lands before the block ends
}

// Plain GEMM (unfused baseline) on the wide tile: C = bf16(A W^T), stores as
// in the plain bf16 GEMM.
__global__ __launch_bounds__(kThreads, 1) void k_gemm_plain_bf16_wide(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ W, uint16_t* __restrict__ C,
    int M, int N, int K, int gm, int gn) {
  __shared__ __attribute__((aligned(1024))) char smem[kSmemBytes];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int gq = lane >> 4;
  const bool godd = (gq & 1) != 0;
  const int nt = gm * gn;
  bool prefetched = false;
  for (int t = blockIdx.x; t < nt; t += gridDim.x) {
    const TileCoord tc = map_tile(t, gm, gn, 8);
    const int m0 = tc.tm * kBMw, n0 = tc.tn * kBNw;
    TileChain ch;
    ch.prefetched = prefetched;
    const bool has_next = t + (int)gridDim.x < nt;
    const TileCoord nc = has_next ? map_tile(t + gridDim.x, gm, gn, 8) : tc;
    ch.next = MainloopSrc{A, W, nullptr, M, N, K, nc.tm * kBMw, nc.tn * kBNw};
    AccW acc;
    mainloop_bf16_wide(acc, smem, MainloopSrc{A, W, nullptr, M, N, K, m0, n0}, ch, [] {}, [] {});
    const int nw0 = n0 + wn * 192;
    const __amdgpu_buffer_rsrc_t crsrc =
        make_rsrc(C + (size_t)m0 * N, (uint32_t)min(kBMw, M - m0) * (uint32_t)N * 2u);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ml = wm * 64 + i * 16 + (lane & 15);
      const bool mv = m0 + ml < M;
#pragma unroll
      for (int j0 = 0; j0 < 12; j0 += 2) {
        u32x2_t pk[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const f32x4_t& a = acc.v[j0 + u][i];
          pk[u] = pack_bf16x4(a[0], a[1], a[2], a[3]);
        }
        const int n = nw0 + 16 * (j0 + (godd ? 1 : 0)) + 8 * (gq >> 1);
        store16_exchanged(crsrc, pk, godd,
                          (mv && n < N) ? ((uint32_t)ml * (uint32_t)N + (uint32_t)n) * 2u
                                        : kOobOffset);
      }
    }
    prefetched = has_next;
  }
  wait_vm0();  // the last tile's unused prefetch into LDS lands before the block ends
}

static inline int cdiv_w(int a, int b) { return (a + b - 1) / b; }

hipError_t launch_rope_bf16_wide(const uint16_t* X, const uint16_t* W, const float* r,
                                 const float* rcos, const float* rsin, const int* pos,
                                 int max_pos, uint16_t* out, int M, int K, int n_q, int n_kv,
                                 hipStream_t stream) {
  const int N = (n_q + 2 * n_kv) * 64;
  const int gm = cdiv_w(M, kBMw), gn = cdiv_w(N, kBNw);
  hipLaunchKernelGGL(k_rope_bf16_wide, dim3(min(gm * gn, cu_count())), dim3(kThreads), 0, stream,
                     X, W, r, rcos, rsin, pos, max_pos, out, M, N, K, (n_q + n_kv) * 64, gm, gn);
  return hipGetLastError();
}


hipError_t launch_gemm_plain_bf16_wide(const uint16_t* A, const uint16_t* W, uint16_t* C, int M,
                                       int N, int K, hipStream_t stream) {
  const int gm = cdiv_w(M, kBMw), gn = cdiv_w(N, kBNw);
  hipLaunchKernelGGL(k_gemm_plain_bf16_wide, dim3(min(gm * gn, cu_count())), dim3(kThreads), 0,
                     stream, A, W, C, M, N, K, gm, gn);
  return hipGetLastError();
}

// A 128 x 384 tile carries 3/4 of a 256 x 256 tile's work at about 10 % lower
// efficiency per MFMA: pick it when its rounds over the compute units, so
// weighted, are fewer.
bool prefer_wide_tile(int M, int N) {
  const long cus = cu_count();
  const long r256 = (((long)cdiv_w(M, 256) * cdiv_w(N, 256)) + cus - 1) / cus;
  const long rw = (((long)cdiv_w(M, kBMw) * cdiv_w(N, kBNw)) + cus - 1) / cus;
  return N % 64 == 0 && 33 * rw < 40 * r256;
}

}  // namespace coda
