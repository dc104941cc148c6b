// bf16 GEMM kernels with epilogue programs, on the mainloop of gemm_core.hpp.
//
// Citations name sections of the news page "CODA: New Research Optimizes
// Transformer Training with GEMM-Epilogue Programming" (KuCoin news flash).
//
// Accumulator layout reminder (see gemm_core.hpp): lane L, register v of the
// 16x16 tile (j, i) holds output feature  nbase + j*16 + 4*(L/16) + v  of
// token  mbase + i*16 + L%16.  So each lane stores 4 consecutive features
// (8 bytes of bf16) of one token, and a per-token sum over the wave's
// features is a lane-local sum followed by one reduction over the 4 lane
// groups.

#include "gemm_core.hpp"
#include "launch.hpp"

namespace coda {

// ---------------------------------------------------------------------------
// GEMM1: residual add + partial sums of squares (section "CODA: the secret in
// the epilogue": the first GEMM's epilogue computes only a partial RMS).
// Output tile 256 tokens x 256 features; each wave's 128 features form one
// partial tile, so T = ceil(N / 128).
// ---------------------------------------------------------------------------
// The thread index as an opaque value: lane/wave arithmetic derived from it
// is recomputed in each tile body instead of being kept live (or spilled)
// across the phases of a kernel that runs several kinds of tiles.
__device__ __forceinline__ int tile_tid() {
  int t = (int)threadIdx.x;
  asm volatile("" : "+v"(t));
  return t;
}

struct Gemm1Args {
  const uint16_t* A;    // [M, K]
  const uint16_t* W;    // [N, K]
  const uint16_t* res;  // [M, N]
  uint16_t* h;          // [M, N]
  float* psum;          // [T, M]
  int M, N, K;
};

__device__ __forceinline__ void gemm1_tile(const Gemm1Args& g, char* smem, int m0, int n0,
                                           const TileChain& ch) {
  const int tid = tile_tid();
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int gq = lane >> 4;
  const int M = g.M, N = g.N;
  const int nw0 = n0 + wn * 128;  // first feature of this wave = partial tile start
  // Residual and h go through buffers that start at the tile's first row
  // (offsets below 256 * N * 2 bytes; out-of-range loads return zero and
  // out-of-range stores are dropped).  Lane L = 16 gq + r, run j: features
  // nw0 + 16 j + 4 gq + 0..3 of row r.
  const uint32_t rows_here = (uint32_t)min(kBM, M - m0);
  const __amdgpu_buffer_rsrc_t rrsrc = make_rsrc(g.res + (size_t)m0 * N, rows_here * (uint32_t)N * 2u);
  const __amdgpu_buffer_rsrc_t hrsrc = make_rsrc(g.h + (size_t)m0 * N, rows_here * (uint32_t)N * 2u);
  auto row_off = [&](int i) {  // byte offset of this lane's row i at feature nw0 + 4 gq
    const int ml = wm * 128 + i * 16 + (lane & 15);
    return ((uint32_t)ml * (uint32_t)N + (uint32_t)(nw0 + 4 * gq)) * 2u;
  };
  // the residual tile (4 features x 8 x 8 token subtiles per lane) is
  // loaded during the last two stages, ahead of the next tile's loads:
  // token subtiles 0, 1 in stage nk-2 (both fragment sets still live), 2..7
  // in the last stage
  u32x2_t rv[8][8];
  auto load_res = [&](int i0, int i1) {
#pragma unroll
    for (int i = i0; i < i1; ++i) {
      const uint32_t o = row_off(i);
#pragma unroll
      for (int j = 0; j < 8; ++j)
        rv[i][j] = __builtin_amdgcn_raw_buffer_load_b64(rrsrc, o + (uint32_t)j * 32u, 0, 0);
    }
  };
  Acc acc;
  mainloop_bf16<false>(acc, smem, MainloopSrc{g.A, g.W, nullptr, M, N, g.K, m0, n0}, ch,
                       [&] { load_res(0, 2); }, [&] { load_res(2, 8); });

  // h stores: lanes gq and gq ^ 1 exchange one run per pair of subtiles (as in
  // GEMM2), so each 16-byte store writes 64 contiguous bytes of 16 rows.
  const bool godd = (gq & 1) != 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int m = m0 + wm * 128 + i * 16 + (lane & 15);
    const bool mv = m < M;
    const int ml = m - m0;
    float ss = 0.f;
#pragma unroll
    for (int j0 = 0; j0 < 8; j0 += 2) {
      u32x2_t pk[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int j = j0 + u;
        const bool nv = nw0 + j * 16 + 4 * gq < N;
        float r4[4];
        unpack_bf16x4(rv[i][j], r4);
        float hv[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          hv[v] = acc.v[j][i][v] + r4[v];
          ss += nv ? hv[v] * hv[v] : 0.f;
        }
        pk[u] = pack_bf16x4(hv[0], hv[1], hv[2], hv[3]);
      }
      const u32x2_t sd = godd ? pk[0] : pk[1];
      const u32x2_t rx = {(unsigned)__shfl_xor((int)sd.x, 16, 64),
                          (unsigned)__shfl_xor((int)sd.y, 16, 64)};
      const int n = nw0 + 16 * (j0 + (godd ? 1 : 0)) + 8 * (gq >> 1);
      const uint32_t off = (mv && n < N) ? ((uint32_t)ml * (uint32_t)N + (uint32_t)n) * 2u
                                         : kOobOffset;
      store16(hrsrc, godd ? u32x4_t{rx.x, rx.y, pk[1].x, pk[1].y}
                          : u32x4_t{pk[0].x, pk[0].y, rx.x, rx.y}, off);
    }
    ss = sum_over_lane_groups(ss);
    if (mv && lane < 16 && nw0 < N) g.psum[(size_t)(nw0 / kRmsTileWidth) * M + m] = ss;
  }
}

__global__ __launch_bounds__(kThreads, 1) void k_residual_partialrms_bf16(Gemm1Args g, int gm,
                                                                          int gn) {
  __shared__ __attribute__((aligned(1024))) char smem[kSmemBytes];
  const int nt = gm * gn;
  bool prefetched = false;
  for (int t = blockIdx.x; t < nt; t += gridDim.x) {
    const TileCoord tc = map_tile(t, gm, gn, 8);
    TileChain ch;
    ch.prefetched = prefetched;
    const bool has_next = t + (int)gridDim.x < nt;
    const TileCoord nc = has_next ? map_tile(t + gridDim.x, gm, gn, 8) : tc;
    ch.next = MainloopSrc{g.A, g.W, nullptr, g.M, g.N, g.K, nc.tm * kBM, nc.tn * kBN};
    gemm1_tile(g, smem, tc.tm * kBM, tc.tn * kBN, ch);
    prefetched = has_next;
  }
  wait_vm0();  // the last tile's unused prefetch into LDS lands before the block ends
}

// ---------------------------------------------------------------------------
// GEMM2: row scale + SwiGLU (section "CODA: the secret in the epilogue": the
// row scale r commutes with the second GEMM and is applied at its end; SwiGLU
// is re-parameterised the same way).  Output tile 256 tokens x 128 features:
// the block's LDS weight tile holds 128 gate rows and the same 128 up rows.
// ---------------------------------------------------------------------------
constexpr int kSwigluStores = 16;  // 16-byte stores per lane per tile
// ... when the pre-activations are saved too (out, g and u)
constexpr int kSwigluSaveStores = 48;

struct Gemm2Args {
  const uint16_t* X;   // [M, K]
  const uint16_t* Wg;  // [N, K]
  const uint16_t* Wu;  // [N, K]
  const float* r;      // [M]
  uint16_t* out;       // [M, N]
  uint16_t* gu;        // [M, 2N] g | u for the backward pass, or unused
  int M, N, K;
};

__device__ __forceinline__ MainloopSrc gemm2_src(const Gemm2Args& g, TileCoord c) {
  return MainloopSrc{g.X, g.Wg, g.Wu, g.M, g.N, g.K, c.tm * kBM, c.tn * (kBN / 2)};
}

// kSave: also store the pre-activations g = r a and u = r b (bf16) into
// gu[m, n] and gu[m, N + n] (section "Five building blocks and a LEGO
// language": tile stores that keep intermediate activations for the backward
// pass).
template <bool kSave>
__device__ __forceinline__ void gemm2_tile(const Gemm2Args& g, char* smem, int m0, int n0,
                                           const TileChain& ch) {
  const int tid = tile_tid();
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int M = g.M, N = g.N;
  float rr[8];
  auto pre = [&]() {
#pragma unroll
    for (int i = 0; i < 8; ++i) rr[i] = g.r[min(m0 + wm * 128 + i * 16 + (lane & 15), M - 1)];
  };
  Acc acc;
  mainloop_bf16<true, kSave ? kSwigluSaveStores : kSwigluStores>(
      acc, smem, MainloopSrc{g.X, g.Wg, g.Wu, M, N, g.K, m0, n0}, ch, pre, [] {});

  // Lane L = 16 g + r holds the run of 4 features 16 j + 4 g of token r
  // for each subtile j.  For a pair of subtiles (j0, j0 + 1), lanes g and
  // g ^ 1 exchange one run, so that every lane holds 8 contiguous features
  // and one 16-byte store writes 64 contiguous bytes of each of 16 rows
  // (instead of 4 runs of 8 bytes): the store path pays per row touched.
  // Every lane issues the same 16 stores (masked ones at an out-of-range
  // offset), which the next tile's first wait counts on.  The buffer starts
  // at the tile's first row, so offsets stay below 256 * N * 2 bytes.
  const __amdgpu_buffer_rsrc_t orsrc =
      make_rsrc(g.out + (size_t)m0 * N, (uint32_t)min(kBM, M - m0) * (uint32_t)N * 2u);
  __amdgpu_buffer_rsrc_t zrsrc;
  if constexpr (kSave)
    zrsrc = make_rsrc(g.gu + (size_t)m0 * 2 * N, (uint32_t)min(kBM, M - m0) * (uint32_t)N * 4u);
  const int nw0 = n0 + wn * 64;
  const int gq = lane >> 4;
  const bool godd = (gq & 1) != 0;
  const float kNegLog2e = -1.4426950408889634f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int ml = wm * 128 + i * 16 + (lane & 15);  // row within the tile
    const bool mv = m0 + ml < M;
    // silu(g) u with g = r a, u = r b:  a b / ((1 + 2^(-log2e r a)) / r^2),
    // the denominator one fma with 1/r^2 = mean(h^2) + eps (finite)
    const float s2 = __builtin_amdgcn_rcpf(rr[i] * rr[i]), c1 = rr[i] * kNegLog2e;
#pragma unroll
    for (int j0 = 0; j0 < 4; j0 += 2) {
      u32x2_t pk[2], pg[2], pu[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int j = j0 + u;
        float o[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float a = acc.v[j][i][v], b = acc.v[j + 4][i][v];
          const float e = __builtin_amdgcn_exp2f(a * c1);
          o[v] = (a * b) * __builtin_amdgcn_rcpf(__builtin_fmaf(e, s2, s2));
        }
        pk[u] = pack_bf16x4(o[0], o[1], o[2], o[3]);
        if constexpr (kSave) {
          const f32x4_t& a = acc.v[j][i];
          const f32x4_t& b = acc.v[j + 4][i];
          const float q = rr[i];
          pg[u] = pack_bf16x4(a[0] * q, a[1] * q, a[2] * q, a[3] * q);
          pu[u] = pack_bf16x4(b[0] * q, b[1] * q, b[2] * q, b[3] * q);
        }
      }
      const u32x2_t sd = godd ? pk[0] : pk[1];
      const u32x2_t rv = {(unsigned)__shfl_xor((int)sd.x, 16, 64),
                          (unsigned)__shfl_xor((int)sd.y, 16, 64)};
      // even g: features 16 j0 + 8 (g/2) + 0..7; odd g: the same in j0 + 1
      const int n = nw0 + 16 * (j0 + (godd ? 1 : 0)) + 8 * (gq >> 1);
      const uint32_t off = (mv && n < N) ? ((uint32_t)ml * (uint32_t)N + (uint32_t)n) * 2u
                                         : kOobOffset;
      store16(orsrc, godd ? u32x4_t{rv.x, rv.y, pk[1].x, pk[1].y}
                          : u32x4_t{pk[0].x, pk[0].y, rv.x, rv.y}, off);
      if constexpr (kSave) {
        const bool ok = mv && n < N;
        const uint32_t og = ok ? ((uint32_t)ml * (uint32_t)(2 * N) + (uint32_t)n) * 2u : kOobOffset;
        const uint32_t ou = ok ? og + (uint32_t)N * 2u : kOobOffset;
        store16_exchanged(zrsrc, pg, godd, og);
        store16_exchanged(zrsrc, pu, godd, ou);
      }
    }
  }
}

template <bool kSave>
__global__ __launch_bounds__(kThreads, 1) void k_rowscale_swiglu_bf16(Gemm2Args g, int gm,
                                                                      int gn) {
  __shared__ __attribute__((aligned(1024))) char smem[kSmemBytes];
  const int nt = gm * gn;
  bool prefetched = false;
  for (int t = blockIdx.x; t < nt; t += gridDim.x) {
    const TileCoord tc = map_tile(t, gm, gn, 8);
    TileChain ch;
    ch.prefetched = prefetched;
    const bool has_next = t + (int)gridDim.x < nt;
    ch.next = gemm2_src(g, has_next ? map_tile(t + gridDim.x, gm, gn, 8) : tc);
    gemm2_tile<kSave>(g, smem, tc.tm * kBM, tc.tn * (kBN / 2), ch);
    prefetched = has_next;
  }
  wait_vm0();  // the last tile's unused prefetch into LDS lands before the block ends
}

// ---------------------------------------------------------------------------
// QKV GEMM: row scale + rotary position embedding (section "CODA: the secret
// in the epilogue": RoPE re-parameterised into the epilogue; section "Five
// building blocks and a LEGO language": RoPE is an elementwise transform and
// the cos/sin rows are vector loads).  Output tile 256 tokens x 256 features;
// a wave's 128 features are whole heads (two of 64, or one of 128), and the
// rotate-half partner of feature c < kHd / 2 of a head, c + kHd / 2, is
// subtile j + kHd / 32 in the same lane and register, so the rotation needs
// no data exchange.
// ---------------------------------------------------------------------------
template <int kHd>
__global__ __launch_bounds__(kThreads, 1) void k_rope_bf16(
    const uint16_t* __restrict__ X, const uint16_t* __restrict__ W, const float* __restrict__ r,
    const float* __restrict__ rcos, const float* __restrict__ rsin, const int* __restrict__ pos,
    int max_pos, uint16_t* __restrict__ out, int M, int N, int K, int rot_features, int gm,
    int gn) {
  static_assert(kHd == 64 || kHd == 128, "head size");
  constexpr int kHalf = kHd / 2;          // rotate-half pair distance
  constexpr int kSub = kHalf / 16;        // subtiles per half head (2 or 4)
  constexpr int kHeads = 128 / kHd;       // heads per wave (2 or 1)
  __shared__ __attribute__((aligned(1024))) char smem[kSmemBytes];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int gq = lane >> 4;
  const int nt = gm * gn;
  bool prefetched = false;
  for (int t = blockIdx.x; t < nt; t += gridDim.x) {
    const TileCoord tc = map_tile(t, gm, gn, 8);
    const int m0 = tc.tm * kBM, n0 = tc.tn * kBN;
    TileChain ch;
    ch.prefetched = prefetched;
    const bool has_next = t + (int)gridDim.x < nt;
    const TileCoord nc = has_next ? map_tile(t + gridDim.x, gm, gn, 8) : tc;
    ch.next = MainloopSrc{X, W, nullptr, M, N, K, nc.tm * kBM, nc.tn * kBN};
    float rr[8];
    int pp[8];
    auto pre = [&]() {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int mc = min(m0 + wm * 128 + i * 16 + (lane & 15), M - 1);
        rr[i] = r[mc];
        pp[i] = pos[mc];
      }
    };
    Acc acc;
    mainloop_bf16<false>(acc, smem, MainloopSrc{X, W, nullptr, M, N, K, m0, n0}, ch, pre, [] {});

    const int nw0 = n0 + wn * 128;  // multiple of 128: whole heads
    // cos/sin rows: angle index of subtile jj (< kSub) of a half head is
    // 16 jj + 4 gq + v.  Positions outside the table are clamped into it
    // (memory safety).  With 64-wide heads the rows of all 8 token subtiles
    // are loaded before the first use (one latency instead of eight); with
    // 128-wide heads (twice the registers) token subtile i + 1's rows are
    // loaded while subtile i is processed.
    constexpr int kPre = kHd == 64 ? 8 : 2;
    f32x4_t ct[kPre][kSub], st[kPre][kSub];
    auto load_cs = [&](int i, int slot) {
      const size_t p = (size_t)min(max(pp[i], 0), max_pos - 1) * kHalf + 4 * gq;
#pragma unroll
      for (int jj = 0; jj < kSub; ++jj) {
        ct[slot][jj] = *(const f32x4_t*)(rcos + p + 16 * jj);
        st[slot][jj] = *(const f32x4_t*)(rsin + p + 16 * jj);
      }
    };
    if constexpr (kHd == 64) {
#pragma unroll
      for (int i = 0; i < 8; ++i) load_cs(i, i);
    } else {
      load_cs(0, 0);
    }
    // Stores as in GEMM2: lanes gq and gq ^ 1 exchange one run of each pair of
    // subtiles of a half head, so each 16-byte store writes 64 contiguous
    // bytes of 16 rows; masked lanes store out of range of a buffer that
    // starts at the tile's first row.
    const __amdgpu_buffer_rsrc_t orsrc =
        make_rsrc(out + (size_t)m0 * N, (uint32_t)min(kBM, M - m0) * (uint32_t)N * 2u);
    const bool godd = (gq & 1) != 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int cur = kHd == 64 ? i : (i & 1);
      if constexpr (kHd != 64) {
        if (i + 1 < 8) load_cs(i + 1, (i + 1) & 1);
      }
      const int ml = wm * 128 + i * 16 + (lane & 15);  // row within the tile
      const bool mv = m0 + ml < M;
      const float rr_i = rr[i];
#pragma unroll
      for (int hh = 0; hh < kHeads; ++hh) {
        const int hbase = nw0 + hh * kHd;
        const bool rot = hbase < rot_features;
        u32x2_t plo[kSub], phi[kSub];
#pragma unroll
        for (int jj = 0; jj < kSub; ++jj) {
          const int ja = hh * 2 * kSub + jj, jb = ja + kSub;
          const f32x4_t cs = ct[cur][jj], sn = st[cur][jj];
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
        for (int half = 0; half < 2; ++half) {  // features [0, kHalf) and [kHalf, kHd) of the head
#pragma unroll
          for (int jp = 0; jp < kSub / 2; ++jp) {  // subtile pairs (2 jp, 2 jp + 1)
            const u32x2_t* pk = (half ? phi : plo) + 2 * jp;
            const u32x2_t sd = godd ? pk[0] : pk[1];
            const u32x2_t rx = {(unsigned)__shfl_xor((int)sd.x, 16, 64),
                                (unsigned)__shfl_xor((int)sd.y, 16, 64)};
            const int n = hbase + kHalf * half + 16 * (2 * jp + (godd ? 1 : 0)) + 8 * (gq >> 1);
            const uint32_t off = (mv && n < N) ? ((uint32_t)ml * (uint32_t)N + (uint32_t)n) * 2u
                                               : kOobOffset;
            store16(orsrc, godd ? u32x4_t{rx.x, rx.y, pk[1].x, pk[1].y}
                                : u32x4_t{pk[0].x, pk[0].y, rx.x, rx.y}, off);
          }
        }
      }
    }
    prefetched = has_next;
  }
  wait_vm0();  // the last tile's unused prefetch into LDS lands before the block ends
}

// ---------------------------------------------------------------------------
// LM head: block log-sum-exp (section "Five building blocks and a LEGO
// language": block reduction "block log-sum-exp" and the stateful max /
// sum-exp statistics of online normalisation; section "CODA: the secret in the
// epilogue": cross-entropy re-parameterised into the epilogue).  The logits
// z = r * X W^T never leave registers: each wave reduces its 128 vocabulary
// entries per token to (max, sum exp(z - max)) and the lane that holds the
// label's logit writes it, taken from the fp32 accumulator.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads, 1) void k_block_lse_bf16(
    const uint16_t* __restrict__ X, const uint16_t* __restrict__ W, const float* __restrict__ r,
    const int* __restrict__ labels, float* __restrict__ tmax, float* __restrict__ tsum,
    float* __restrict__ label_logit, int M, int V, int K, int gm, int gn) {
  __shared__ __attribute__((aligned(1024))) char smem[kSmemBytes];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int g4 = (lane >> 4) * 4;
  const float kLog2e = 1.4426950408889634f;
  const int nt = gm * gn;
  bool prefetched = false;
  for (int t = blockIdx.x; t < nt; t += gridDim.x) {
    const TileCoord tc = map_tile(t, gm, gn, 8);
    const int m0 = tc.tm * kBM, n0 = tc.tn * kBN;
    TileChain ch;
    ch.prefetched = prefetched;
    const bool has_next = t + (int)gridDim.x < nt;
    const TileCoord nc = has_next ? map_tile(t + gridDim.x, gm, gn, 8) : tc;
    ch.next = MainloopSrc{X, W, nullptr, M, V, K, nc.tm * kBM, nc.tn * kBN};
    float rr[8];
    int lab[8];
    auto pre = [&]() {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int mc = min(m0 + wm * 128 + i * 16 + (lane & 15), M - 1);
        rr[i] = r ? r[mc] : 1.0f;
        lab[i] = labels[mc];
      }
    };
    Acc acc;
    mainloop_bf16<false>(acc, smem, MainloopSrc{X, W, nullptr, M, V, K, m0, n0}, ch, pre, [] {});

    const int nw0 = n0 + wn * kLseTileWidth;
    // Per token row i (the lane's 32 logits of it): the max is taken on the
    // raw accumulators and scaled once (r > 0 and rounding r z is monotonic
    // in z, so max(r z) = r max(z) exactly).  Entries past V need no mask in
    // the max: their weight rows are clamped copies of row V - 1, so their
    // logits repeat a valid one; only the sum of a ragged last tile masks
    // them.  The label logit lies in this wave's 128 entries for about one
    // tile in a thousand, so one wave-wide vote decides whether to look.
    const bool full = nw0 + kLseTileWidth <= V;
    const int lim = V - nw0 - g4;  // entry 16 j + v of this lane exists iff 16 j + v < lim
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int m = m0 + wm * 128 + i * 16 + (lane & 15);
      const bool mv = m < M;
      float mxr = acc.v[0][i][0];
#pragma unroll
      for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int v = 0; v < 4; ++v) mxr = fmaxf(mxr, acc.v[j][i][v]);
      const float mx = max_over_lane_groups(mxr) * rr[i];
      const float rr2 = rr[i] * kLog2e, mx2 = mx * kLog2e;
      float se = 0.f;
      if (full) {
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
          for (int v = 0; v < 4; ++v) se += __builtin_amdgcn_exp2f(acc.v[j][i][v] * rr2 - mx2);
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const float e = __builtin_amdgcn_exp2f(acc.v[j][i][v] * rr2 - mx2);
            se += (j * 16 + v < lim) ? e : 0.f;
          }
      }
      se = sum_over_lane_groups(se);
      // label's entry within this wave's window; labels at or past V (rows
      // that carry no loss) match nothing, not even the padding of the last tile
      const int loff = lab[i] < V ? lab[i] - nw0 : -1;
      if (__any((unsigned)loff < (unsigned)kLseTileWidth)) {
        float zl = 0.f;
        bool has = false;
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const bool hit = loff == j * 16 + g4 + v;
            zl = hit ? acc.v[j][i][v] : zl;
            has = has || hit;
          }
        if (mv && has) label_logit[m] = zl * rr[i];
      }
      if (mv && lane < 16 && nw0 < V) {
        const size_t tt = (size_t)(nw0 / kLseTileWidth);
        tmax[tt * M + m] = mx;
        tsum[tt * M + m] = se;
      }
    }
    prefetched = has_next;
  }
  wait_vm0();  // the last tile's unused prefetch into LDS lands before the block ends
}

// ---------------------------------------------------------------------------
// Plain GEMM (unfused baseline): the same mainloop, epilogue = convert + store.
// ---------------------------------------------------------------------------
constexpr int kPlainStores = 32;  // 16-byte stores per lane per tile

__global__ __launch_bounds__(kThreads, 1) void k_gemm_plain_bf16(const uint16_t* __restrict__ A,
                                                                 const uint16_t* __restrict__ W,
                                                                 uint16_t* __restrict__ C, int M,
                                                                 int N, int K, int gm, int gn) {
  __shared__ __attribute__((aligned(1024))) char smem[kSmemBytes];
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
    mainloop_bf16<false, kPlainStores>(acc, smem, MainloopSrc{A, W, nullptr, M, N, K, m0, n0},
                                       ch, [] {}, [] {});

    // 16-byte stores of exchanged runs, as in the fused epilogues
    const int nw0 = n0 + wn * 128;
    const __amdgpu_buffer_rsrc_t crsrc =
        make_rsrc(C + (size_t)m0 * N, (uint32_t)min(kBM, M - m0) * (uint32_t)N * 2u);
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

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
static inline int cdiv(int a, int b) { return (a + b - 1) / b; }

hipError_t launch_residual_partialrms_bf16(const uint16_t* A, const uint16_t* W,
                                           const uint16_t* res, uint16_t* h, float* psum, int M,
                                           int N, int K, hipStream_t stream) {
  const int gm = cdiv(M, kBM), gn = cdiv(N, kBN);
  hipLaunchKernelGGL(k_residual_partialrms_bf16, dim3(min(gm * gn, cu_count())), dim3(kThreads), 0,
                     stream, Gemm1Args{A, W, res, h, psum, M, N, K}, gm, gn);
  return hipGetLastError();
}

hipError_t launch_rowscale_swiglu_bf16(const uint16_t* X, const uint16_t* Wg, const uint16_t* Wu,
                                       const float* r, uint16_t* out, int M, int N, int K,
                                       hipStream_t stream) {
  const int gm = cdiv(M, kBM), gn = cdiv(N, kBN / 2);
  hipLaunchKernelGGL(k_rowscale_swiglu_bf16<false>, dim3(min(gm * gn, cu_count())),
                     dim3(kThreads), 0, stream, Gemm2Args{X, Wg, Wu, r, out, nullptr, M, N, K},
                     gm, gn);
  return hipGetLastError();
}

hipError_t launch_rowscale_swiglu_save_bf16(const uint16_t* X, const uint16_t* Wg,
                                            const uint16_t* Wu, const float* r, uint16_t* out,
                                            uint16_t* gu, int M, int N, int K,
                                            hipStream_t stream) {
  const int gm = cdiv(M, kBM), gn = cdiv(N, kBN / 2);
  hipLaunchKernelGGL(k_rowscale_swiglu_bf16<true>, dim3(min(gm * gn, cu_count())),
                     dim3(kThreads), 0, stream, Gemm2Args{X, Wg, Wu, r, out, gu, M, N, K}, gm,
                     gn);
  return hipGetLastError();
}


hipError_t launch_rope_bf16(const uint16_t* X, const uint16_t* W, const float* r,
                            const float* rcos, const float* rsin, const int* pos, int max_pos,
                            uint16_t* out, int M, int K, int n_q, int n_kv, int head_dim,
                            hipStream_t stream) {
  const int N = (n_q + 2 * n_kv) * head_dim;
  const int gm = cdiv(M, kBM), gn = cdiv(N, kBN);
  const auto kern = head_dim == 128 ? k_rope_bf16<128> : k_rope_bf16<64>;
  hipLaunchKernelGGL(kern, dim3(min(gm * gn, cu_count())), dim3(kThreads), 0, stream, X, W, r,
                     rcos, rsin, pos, max_pos, out, M, N, K, (n_q + n_kv) * head_dim, gm, gn);
  return hipGetLastError();
}

hipError_t launch_block_lse_bf16(const uint16_t* X, const uint16_t* W, const float* r,
                                 const int* labels, float* tmax, float* tsum, float* label_logit,
                                 int M, int V, int K, hipStream_t stream) {
  const int gm = cdiv(M, kBM), gn = cdiv(V, kBN);
  hipLaunchKernelGGL(k_block_lse_bf16, dim3(min(gm * gn, cu_count())), dim3(kThreads), 0, stream, X, W, r, labels,
                     tmax, tsum, label_logit, M, V, K, gm, gn);
  return hipGetLastError();
}

hipError_t launch_gemm_plain_bf16(const uint16_t* A, const uint16_t* W, uint16_t* C, int M, int N,
                                  int K, hipStream_t stream) {
  const int gm = cdiv(M, kBM), gn = cdiv(N, kBN);
  hipLaunchKernelGGL(k_gemm_plain_bf16, dim3(min(gm * gn, cu_count())), dim3(kThreads), 0, stream, A, W, C, M, N,
                     K, gm, gn);
  return hipGetLastError();
}

}  // namespace coda
