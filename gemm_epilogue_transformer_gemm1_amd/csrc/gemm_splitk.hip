// Plain GEMM with its reduction split in `parts` column ranges, for outputs
// too small to give every compute unit a tile: the weight gradients of the
// backward pass reduce over all tokens into a d x d matrix (page section "CODA:
// the secret in the epilogue": the backward pass inherits the forward's
// structure; section "Experimental results": backward kernels).  At d = 2048,
// K = 8192 tokens, 64 output tiles leave three quarters of 256 compute units
// idle; four parts give 256 work units of a quarter of the reduction each.
//
// Citations name sections of the news page "CODA: New Research Optimizes
// Transformer Training with GEMM-Epilogue Programming" (KuCoin news flash).
//
//   k_gemm_splitk_bf16: unit (p, tile) runs the mainloop of gemm_core.hpp over
//     columns [p*Kp, (p+1)*Kp) of A and W (row pitch K) and stores its fp32
//     accumulators to workspace part p (no atomics; every element of every
//     part is written);
//   k_splitk_reduce_bf16: C = bf16(((part 0 + part 1) + part 2) + ...), the
//     same order for every element, so results do not depend on scheduling.

#include "gemm_core.hpp"
#include "launch.hpp"

namespace coda {

constexpr int kSplitStores = 64;  // 16-byte fp32 stores per lane per tile

__global__ __launch_bounds__(kThreads, 1) void k_gemm_splitk_bf16(const uint16_t* __restrict__ A,
                                                                  const uint16_t* __restrict__ W,
                                                                  float* __restrict__ ws, int M,
                                                                  int N, int K, int parts, int gm,
                                                                  int gn) {
  __shared__ __attribute__((aligned(1024))) char smem[kSmemBytes];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int nt = gm * gn * parts;
  const int kp = K / parts;
  // Units form a (parts * gm) x gn grid of tiles, part-major along the rows,
  // walked in the XCD-aware order: each XCD's units then share one part's
  // operand slabs through its L2 (dWo: one part and 8 x 4 tiles per XCD,
  // 12 MiB of operands, instead of one tile column of every part, 36 MiB).
  auto unit = [&](int t, int& p) {
    const TileCoord c = map_tile(t, gm * parts, gn, 8);
    p = c.tm / gm;
    return TileCoord{c.tm - p * gm, c.tn};
  };
  auto src = [&](int t) {
    int p;
    const TileCoord c = unit(t, p);
    return MainloopSrc{A + (size_t)p * kp, W + (size_t)p * kp, nullptr, M, N, kp,
                       c.tm * kBM, c.tn * kBN, K};
  };
  bool prefetched = false;
  for (int t = blockIdx.x; t < nt; t += gridDim.x) {
    const MainloopSrc cur = src(t);
    TileChain ch;
    ch.prefetched = prefetched;
    const bool has_next = t + (int)gridDim.x < nt;
    ch.next = src(has_next ? t + (int)gridDim.x : t);
    Acc acc;
    mainloop_bf16<false, kSplitStores>(acc, smem, cur, ch, [] {}, [] {});

    // lane L of a 16 x 16 subtile holds 4 consecutive features of one row:
    // each store writes 64 contiguous bytes of 16 rows
    const int m0 = cur.m0, n0 = cur.n0;
    int p;
    unit(t, p);
    const int nw0 = n0 + wn * 128 + 4 * (lane >> 4);
    const __amdgpu_buffer_rsrc_t wsrc =
        make_rsrc(ws + ((size_t)p * M + m0) * N, (uint32_t)min(kBM, M - m0) * (uint32_t)N * 4u);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int ml = wm * 128 + i * 16 + (lane & 15);
      const bool mv = m0 + ml < M;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int n = nw0 + 16 * j;
        store16(wsrc, __builtin_bit_cast(u32x4_t, acc.v[j][i]),
                (mv && n < N) ? ((uint32_t)ml * (uint32_t)N + (uint32_t)n) * 4u : kOobOffset);
      }
    }
    prefetched = has_next;
  }
  wait_vm0();  // the last tile's unused prefetch into LDS lands before the block ends
}

// 8 outputs per thread and step: two 16-byte loads per part, one 16-byte store.
__global__ __launch_bounds__(256) void k_splitk_reduce_bf16(const float* __restrict__ ws,
                                                            uint16_t* __restrict__ C,
                                                            int64_t count, int parts) {
  const int64_t n8 = count / 8;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; v < n8; v += stride) {
    const f32x4_t* q = reinterpret_cast<const f32x4_t*>(ws) + 2 * v;
    f32x4_t a = __builtin_nontemporal_load(q), b = __builtin_nontemporal_load(q + 1);
    for (int p = 1; p < parts; ++p) {
      q += count / 4;
      a += __builtin_nontemporal_load(q);
      b += __builtin_nontemporal_load(q + 1);
    }
    const u32x2_t lo = pack_bf16x4(a[0], a[1], a[2], a[3]);
    const u32x2_t hi = pack_bf16x4(b[0], b[1], b[2], b[3]);
    reinterpret_cast<u32x4_t*>(C)[v] = u32x4_t{lo.x, lo.y, hi.x, hi.y};
  }
}

hipError_t launch_gemm_splitk_bf16(const uint16_t* A, const uint16_t* W, uint16_t* C, float* ws,
                                   int M, int N, int K, int parts, hipStream_t stream) {
  const int gm = (M + kBM - 1) / kBM, gn = (N + kBN - 1) / kBN;
  hipLaunchKernelGGL(k_gemm_splitk_bf16, dim3(min(gm * gn * parts, cu_count())), dim3(kThreads),
                     0, stream, A, W, ws, M, N, K, parts, gm, gn);
  if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  const int64_t count = (int64_t)M * N;
  const int64_t blocks = (count / 8 + 255) / 256, cap = 8 * (int64_t)cu_count();
  hipLaunchKernelGGL(k_splitk_reduce_bf16, dim3((unsigned)(blocks < cap ? blocks : cap)), dim3(256),
                     0, stream, ws, C, count, parts);
  return hipGetLastError();
}

}  // namespace coda
