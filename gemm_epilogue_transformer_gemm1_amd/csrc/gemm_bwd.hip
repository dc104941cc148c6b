// bf16 backward GEMMs of the MLP sub-layer with epilogue programs, on the
// mainloop of gemm_core.hpp.
//
// Citations name sections of the news page "CODA: New Research Optimizes
// Transformer Training with GEMM-Epilogue Programming" (KuCoin news flash).
// Section "CODA: the secret in the epilogue" states that a block-local forward
// tail gives a backward pass of the same structure; section "Experimental results" reports
// backward kernels for SwiGLU and for GEMM-Residual-PartialRMS-GEMM.  The page
// prints no formulas; the ones below are the chain rule of the forward
//   h = res + x Wo^T,  z = [g | u] = r h W'^T (W' = [Wg; Wu] diag(gamma)),
//   out = silu(g) u,   next = h + out Wd^T,
// given dY = dL/dnext.  With dz = [dg | du] and G = dz W':
//   dh = r G - c h + dY,  c = (r^3 / d) sum_j h_j G_j = (r^2 / d) sum_n dz_n z_n
// (sum_j h_j G_j = sum_n dz_n (h W'^T)_n = sum_n dz_n z_n / r).  The second
// form of c needs only values the SwiGLU-backward epilogue already holds, so
// that epilogue emits it as per-(row, tile) partial sums -- the same partial
// reduction the forward GEMM1 epilogue does for the RMS -- and the GEMM that
// forms G applies the whole RMSNorm backward and the skip connection at its
// end.
//
// Accumulator layout: lane L, register v of the 16x16 tile (j, i) holds
// output feature nbase + 16 j + 4 (L / 16) + v of token mbase + 16 i + L % 16.

#include <type_traits>

#include "gemm_core.hpp"
#include "gemm_core8.hpp"
#include "launch.hpp"

namespace coda {

// The thread index as an opaque value (lane/wave arithmetic is recomputed in
// each tile body instead of being kept live across phases).
__device__ __forceinline__ int bwd_tile_tid() {
  int t = (int)threadIdx.x;
  asm volatile("" : "+v"(t));
  return t;
}

// Vector memory operations each epilogue below issues per lane after the next
// tile's loads (operand loads of token subtiles 3..7 plus the stores) is well
// above 47, so the next tile's first wait is vmcnt(63).
constexpr int kBwdEpiVmem = 47;

// The RMSNorm-backward epilogue's two operand tiles (h and dY, [M, ld] each),
// loaded with 8-byte loads (one 4-feature run per lane, the accumulator layout
// itself; a 16-byte form with a lane exchange needs temporaries that push
// this kernel past the register file).  Its epilogue is small next to its
// mainloop (K = 2 ffn).  Token subtiles 0..2 are loaded during the last two
// stages of the mainloop, subtile i + 3 while subtile i is processed; rows
// past M lie beyond the buffers, which start at the tile's first row.
struct EpiPairNarrow {
  __amdgpu_buffer_rsrc_t rs_a, rs_b;
  uint32_t ld;
  int nw0, N, wm, lane;
  u32x2_t a[8][8], b[8][8];

  __device__ __forceinline__ uint32_t off(int i, int j) const {
    const int n = nw0 + 16 * j;
    if (n >= N) return kOobOffset;  // wave-uniform
    const uint32_t ml = (uint32_t)(wm * 128 + i * 16 + (lane & 15));
    return (ml * ld + (uint32_t)(n + 4 * (lane >> 4))) * 2u;
  }
  __device__ __forceinline__ void load(int i) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t o = off(i, j);
      a[i][j] = __builtin_amdgcn_raw_buffer_load_b64(rs_a, o, 0, 0);
      b[i][j] = __builtin_amdgcn_raw_buffer_load_b64(rs_b, o, 0, 0);
    }
  }
};

// ---------------------------------------------------------------------------
// SwiGLU backward: dout = dY Wd (weight passed as WdT = Wd^T, [N = ffn, K = d]);
// epilogue with the saved pre-activations g = gu[:, :N], u = gu[:, N:]:
//   s = sigmoid(g), du = dout silu(g), dg = dout u (s + silu(g) (1 - s)),
// stores dz = [dg | du] and the partial sums  sum (dg g + du u)  over each
// wave's 128 features (T = ceil(N / 128) tiles, [T, M]).
//
// This GEMM runs on the two-waves-per-SIMD mainloop (gemm_core8.hpp): its
// epilogue reads 256 KiB (g | u) and writes 256 KiB (dz) per 256 x 256 tile
// and is bound by the loads the waves keep in flight, which eight waves
// double; the mainloop itself is not faster with eight waves.  Each lane
// loads its operands 16 bytes at a time (8 features of one row): for the
// feature subtile pair (2 jp, 2 jp + 1), lanes of even 16-lane groups g read
// subtile 2 jp at features 8 (g / 2) .. + 7 (their own 4-feature run and that
// of group g + 1), odd groups subtile 2 jp + 1, and `runs` swaps the foreign
// halves between lanes 16 apart.  Subtile 0 is loaded in the last stage of
// the mainloop, subtile i + 1 while subtile i is processed (more ahead would
// not fit the 128 registers a wave has beside its accumulators).  Feature
// runs at or past N read at an out-of-range offset (zeros); rows past M lie
// beyond the buffer, which starts at the tile's first row.
// ---------------------------------------------------------------------------
struct SwigluBwdArgs {
  const uint16_t* dY;   // [M, K]
  const uint16_t* WdT;  // [N, K]
  const uint16_t* gu;   // [M, 2N]
  uint16_t* dz;         // [M, 2N]
  float* pdot;          // [T, M]
  int M, N, K;
};

// vector memory operations per lane the epilogue issues after the next
// tile's loads: at least 3 x 8 operand loads and 4 x 8 stores
constexpr int kSwigluBwdEpiVmem = 47;

struct EpiGU {
  __amdgpu_buffer_rsrc_t rs;
  uint32_t ld, col_b;
  int nw0, N, wm, lane;
  u32x4_t a[4][4], b[4][4];

  __device__ __forceinline__ uint32_t off(int i, int jp, uint32_t col) const {
    const int gq = lane >> 4;
    const int n = nw0 + 16 * (2 * jp + (gq & 1));
    const uint32_t ml = (uint32_t)(wm * 64 + i * 16 + (lane & 15));
    return n < N ? (ml * ld + col + (uint32_t)(n + 8 * (gq >> 1))) * 2u : kOobOffset;
  }
  __device__ __forceinline__ void load(int i) {
#pragma unroll
    for (int jp = 0; jp < 4; ++jp) {
      a[i][jp] = __builtin_bit_cast(
          u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, off(i, jp, 0), 0, 0));
      b[i][jp] = __builtin_bit_cast(
          u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, off(i, jp, col_b), 0, 0));
    }
  }
  // This lane's runs of subtiles 2 jp (out[0]) and 2 jp + 1 (out[1]) from the
  // 16 bytes it loaded; all 64 lanes must take part (lane shuffle).
  __device__ __forceinline__ static void runs(const u32x4_t& v, bool godd, u32x2_t (&out)[2]) {
    const u32x2_t lo = {v.x, v.y}, hi = {v.z, v.w};
    const u32x2_t sd = godd ? lo : hi;
    const u32x2_t rx = {(unsigned)__shfl_xor((int)sd.x, 16, 64),
                        (unsigned)__shfl_xor((int)sd.y, 16, 64)};
    out[0] = godd ? rx : lo;
    out[1] = godd ? hi : rx;
  }
};

__device__ __forceinline__ void swiglu_bwd_tile(const SwigluBwdArgs& g, char* smem, int m0, int n0,
                                                const TileChain& ch) {
  const int tid = bwd_tile_tid();
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int gq = lane >> 4;
  const int M = g.M, N = g.N;
  const uint32_t ld = 2u * (uint32_t)N;
  const int nw0 = n0 + wn * 128;
  const uint32_t rows_here = (uint32_t)min(kBM, M - m0);
  EpiGU z;
  z.rs = make_rsrc(g.gu + (size_t)m0 * ld, rows_here * ld * 2u);
  z.ld = ld;
  z.col_b = (uint32_t)N;
  z.nw0 = nw0;
  z.N = N;
  z.wm = wm;
  z.lane = lane;
  const __amdgpu_buffer_rsrc_t drsrc = make_rsrc(g.dz + (size_t)m0 * ld, rows_here * ld * 2u);
  Acc8 acc;
  mainloop8_bf16<false, kSwigluBwdEpiVmem>(
      acc, smem, MainloopSrc{g.dY, g.WdT, nullptr, M, N, g.K, m0, n0}, ch, [] {},
      [&] { z.load(0); });

  const bool godd = (gq & 1) != 0;
  const float kNegLog2e = -1.4426950408889634f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (i + 1 < 4) z.load(i + 1);
    const int ml = wm * 64 + i * 16 + (lane & 15);
    const bool mv = m0 + ml < M;
    float ps = 0.f;
#pragma unroll
    for (int j0 = 0; j0 < 8; j0 += 2) {
      u32x2_t pg[2], pu[2], ga[2], ub[2];
      EpiGU::runs(z.a[i][j0 / 2], godd, ga);
      EpiGU::runs(z.b[i][j0 / 2], godd, ub);
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int j = j0 + u;
        float gv[4], uv[4], dg[4], du[4];
        unpack_bf16x4(ga[u], gv);
        unpack_bf16x4(ub[u], uv);
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float d = acc.v[j][i][v];
          // s = 1 / (1 + 2^(-log2e g)): 0 for very negative g (2^x = inf)
          const float s = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(gv[v] * kNegLog2e));
          const float sl = gv[v] * s;
          du[v] = d * sl;
          dg[v] = (d * uv[v]) * __builtin_fmaf(sl, 1.0f - s, s);
          ps += dg[v] * gv[v] + du[v] * uv[v];
        }
        pg[u] = pack_bf16x4(dg[0], dg[1], dg[2], dg[3]);
        pu[u] = pack_bf16x4(du[0], du[1], du[2], du[3]);
      }
      const int n = nw0 + 16 * (j0 + (godd ? 1 : 0)) + 8 * (gq >> 1);
      const bool ok = mv && n < N;
      const uint32_t og = ok ? ((uint32_t)ml * ld + (uint32_t)n) * 2u : kOobOffset;
      const uint32_t ou = ok ? og + (uint32_t)N * 2u : kOobOffset;
      store16_exchanged(drsrc, pg, godd, og);
      store16_exchanged(drsrc, pu, godd, ou);
    }
    ps = sum_over_lane_groups(ps);
    if (mv && lane < 16 && nw0 < N) g.pdot[(size_t)(nw0 / kRmsTileWidth) * M + m0 + ml] = ps;
  }
}

__global__ __launch_bounds__(kThreads8, 1) void k_swiglu_bwd_bf16(SwigluBwdArgs g, int gm, int gn) {
  __shared__ __attribute__((aligned(1024))) char smem[kSmemBytes];
  const int nt = gm * gn;
  bool prefetched = false;
  for (int t = blockIdx.x; t < nt; t += gridDim.x) {
    const TileCoord tc = map_tile(t, gm, gn, 8);
    TileChain ch;
    ch.prefetched = prefetched;
    const bool has_next = t + (int)gridDim.x < nt;
    const TileCoord nc = has_next ? map_tile(t + gridDim.x, gm, gn, 8) : tc;
    ch.next = MainloopSrc{g.dY, g.WdT, nullptr, g.M, g.N, g.K, nc.tm * kBM, nc.tn * kBN};
    swiglu_bwd_tile(g, smem, tc.tm * kBM, tc.tn * kBN, ch);
    prefetched = has_next;
  }
  wait_vm0();  // the last tile's unused prefetch into LDS lands before the block ends
}

// ---------------------------------------------------------------------------
// RMSNorm backward through GEMM2: G = dz W' (weight passed as W2T = W'^T,
// [N = d, K = 2 ffn], gamma folded in), epilogue
//   dh = r G - c h + dY
// with the forward row scale r, the row coefficient c, the forward h and the
// gradient dY arriving through the skip connection.
// ---------------------------------------------------------------------------
struct RmsBwdArgs {
  const uint16_t* dz;   // [M, K]
  const uint16_t* W2T;  // [N, K]
  const uint16_t* h;    // [M, N]
  const uint16_t* dY;   // [M, N]
  const float* r;       // [M]
  const float* c;       // [M]
  uint16_t* dh;         // [M, N]
  int M, N, K;
};

__device__ __forceinline__ void rmsnorm_bwd_tile(const RmsBwdArgs& g, char* smem, int m0, int n0,
                                                 const TileChain& ch) {
  const int tid = bwd_tile_tid();
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int gq = lane >> 4;
  const int M = g.M, N = g.N;
  const int nw0 = n0 + wn * 128;
  const uint32_t rows_here = (uint32_t)min(kBM, M - m0);
  // h and dY are separate [M, N] matrices: one pair, two buffers
  EpiPairNarrow hy;
  hy.rs_a = make_rsrc(g.h + (size_t)m0 * N, rows_here * (uint32_t)N * 2u);
  hy.rs_b = make_rsrc(g.dY + (size_t)m0 * N, rows_here * (uint32_t)N * 2u);
  hy.ld = (uint32_t)N;
  hy.nw0 = nw0;
  hy.N = N;
  hy.wm = wm;
  hy.lane = lane;
  auto load = [&](int i) { hy.load(i); };
  float rr[8], cc[8];
  auto pre = [&] {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int mc = min(m0 + wm * 128 + i * 16 + (lane & 15), M - 1);
      rr[i] = g.r[mc];
      cc[i] = g.c[mc];
    }
    load(0);
  };
  const __amdgpu_buffer_rsrc_t orsrc = make_rsrc(g.dh + (size_t)m0 * N, rows_here * (uint32_t)N * 2u);
  Acc acc;
  mainloop_bf16<false, kBwdEpiVmem>(acc, smem, MainloopSrc{g.dz, g.W2T, nullptr, M, N, g.K, m0, n0},
                                    ch, pre, [&] { load(1); load(2); });

  const bool godd = (gq & 1) != 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    if (i + 3 < 8) load(i + 3);
    const int ml = wm * 128 + i * 16 + (lane & 15);
    const bool mv = m0 + ml < M;
#pragma unroll
    for (int j0 = 0; j0 < 8; j0 += 2) {
      u32x2_t pk[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int j = j0 + u;
        float hv[4], yv[4], o[4];
        unpack_bf16x4(hy.a[i][j], hv);
        unpack_bf16x4(hy.b[i][j], yv);
#pragma unroll
        for (int v = 0; v < 4; ++v)
          o[v] = __builtin_fmaf(rr[i], acc.v[j][i][v], __builtin_fmaf(-cc[i], hv[v], yv[v]));
        pk[u] = pack_bf16x4(o[0], o[1], o[2], o[3]);
      }
      const int n = nw0 + 16 * (j0 + (godd ? 1 : 0)) + 8 * (gq >> 1);
      store16_exchanged(orsrc, pk, godd,
                        (mv && n < N) ? ((uint32_t)ml * (uint32_t)N + (uint32_t)n) * 2u
                                      : kOobOffset);
    }
  }
}

__global__ __launch_bounds__(kThreads, 1) void k_rmsnorm_bwd_bf16(RmsBwdArgs g, int gm, int gn) {
  __shared__ __attribute__((aligned(1024))) char smem[kSmemBytes];
  const int nt = gm * gn;
  bool prefetched = false;
  for (int t = blockIdx.x; t < nt; t += gridDim.x) {
    const TileCoord tc = map_tile(t, gm, gn, 8);
    TileChain ch;
    ch.prefetched = prefetched;
    const bool has_next = t + (int)gridDim.x < nt;
    const TileCoord nc = has_next ? map_tile(t + gridDim.x, gm, gn, 8) : tc;
    ch.next = MainloopSrc{g.dz, g.W2T, nullptr, g.M, g.N, g.K, nc.tm * kBM, nc.tn * kBN};
    rmsnorm_bwd_tile(g, smem, tc.tm * kBM, tc.tn * kBN, ch);
    prefetched = has_next;
  }
  wait_vm0();  // the last tile's unused prefetch into LDS lands before the block ends
}

// ---------------------------------------------------------------------------
// Weight gradient of the gamma-folded gate|up weight W' = W diag(gamma), with
// the gradient of the RMSNorm gain as its epilogue (section "What CODA can
// do": RMSNorm gradients; section "Five building blocks and a LEGO language":
// block reduction).  The GEMM reduces over the tokens,
//   G[n,k] = A[n,:] . B[k,:]    (A = dz^T [M, K], B = (r h)^T [N, K]; G = dW'),
// and its epilogue reads the unfolded weight W [M, N] and gamma [N]:
//   dW[n,k]   = bf16(G[n,k] gamma[k])                      (gradient of W)
//   pdg[p, k] = sum over the 128 rows n of slice p of G[n,k] W[n,k]
// so that dgamma[k] = sum_p pdg[p, k] (from W'[n,k] = W[n,k] gamma[k]).  A
// wave's slice is its 128 rows; its 32 column sums per lane meet over the 16
// rows of a lane group in four halving exchange steps, after which each lane
// holds two adjacent columns.
// ---------------------------------------------------------------------------
struct WgradGammaArgs {
  const uint16_t* A;      // [M, K]
  const uint16_t* B;      // [N, K]
  const uint16_t* W;      // [M, N]
  const float* gamma;     // [N]
  uint16_t* dW;           // [M, N]
  float* pdg;             // [ceil(M / 128), N]
  int M, N, K;
};

// One bf16 operand tile of the epilogue in the accumulator layout (a 4-feature
// run per lane, 8-byte loads), loaded per token subtile as in EpiPairNarrow.
struct EpiOne {
  __amdgpu_buffer_rsrc_t rs;
  uint32_t ld;
  int nw0, N, wm, lane;
  u32x2_t a[8][8];

  __device__ __forceinline__ void load(int i) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int n = nw0 + 16 * j;
      const uint32_t ml = (uint32_t)(wm * 128 + i * 16 + (lane & 15));
      const uint32_t o = n < N ? (ml * ld + (uint32_t)(n + 4 * (lane >> 4))) * 2u : kOobOffset;
      a[i][j] = __builtin_amdgcn_raw_buffer_load_b64(rs, o, 0, 0);
    }
  }
};

// Value of the lane given by a DPP row pattern (all lanes take part).
template <int kCtrl>
__device__ __forceinline__ float dpp_f32(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), kCtrl, 0xF, 0xF, false));
}

// Sum of v over the 16 lanes of each 16-lane group (lane bits 0..3), the
// values kept per lane halving each step: on return lane L holds, in v[0] and
// v[1], the sums of its group's values 2 (8 b3 + 4 b2 + 2 b1 + b0) + 0 and + 1,
// b_k the bits of L.  Step s pairs each lane with a partner that differs in
// bit 3 - s and agrees in the bits decided before (partners L ^ 8, L ^ 7,
// L ^ 2, L ^ 1: a row rotation by 8, the half-row mirror and two quad
// permutations, all DPP moves rather than LDS-crossbar shuffles); the lane
// with that bit set keeps the upper half of the values.
__device__ __forceinline__ void rows16_halving_sum(float (&v)[32], int lane) {
  auto step = [&](auto ctrl_tag, int half, int bit) {
    constexpr int kCtrl = decltype(ctrl_tag)::value;
    const bool hi = (lane & bit) != 0;
#pragma unroll
    for (int c = 0; c < 16; ++c) {
      if (c < half) {
        const float send = hi ? v[c] : v[c + half];
        const float keep = hi ? v[c + half] : v[c];
        v[c] = keep + dpp_f32<kCtrl>(send);
      }
    }
  };
  step(std::integral_constant<int, 0x128>{}, 16, 8);  // row_ror:8        (L ^ 8)
  step(std::integral_constant<int, 0x141>{}, 8, 4);   // row_half_mirror  (L ^ 7)
  step(std::integral_constant<int, 0x4E>{}, 4, 2);    // quad_perm 2,3,0,1 (L ^ 2)
  step(std::integral_constant<int, 0xB1>{}, 2, 1);    // quad_perm 1,0,3,2 (L ^ 1)
}

__device__ __forceinline__ void wgrad_gamma_tile(const WgradGammaArgs& g, char* smem, int m0,
                                                 int n0, const TileChain& ch) {
  const int tid = bwd_tile_tid();
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int gq = lane >> 4;
  const int M = g.M, N = g.N;
  const int nw0 = n0 + wn * 128;
  const uint32_t rows_here = (uint32_t)min(kBM, M - m0);
  EpiOne wt;
  wt.rs = make_rsrc(g.W + (size_t)m0 * N, rows_here * (uint32_t)N * 2u);
  wt.ld = (uint32_t)N;
  wt.nw0 = nw0;
  wt.N = N;
  wt.wm = wm;
  wt.lane = lane;
  // gamma of the lane's 32 columns nw0 + 16 j + 4 gq + 0..3 (zero past N)
  const __amdgpu_buffer_rsrc_t grs = make_rsrc(g.gamma, (uint32_t)N * 4u);
  f32x4_t gm[8];
  auto pre = [&] {
#pragma unroll
    for (int j = 0; j < 8; ++j)
      gm[j] = __builtin_bit_cast(
          f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                       grs, (uint32_t)(nw0 + 16 * j + 4 * gq) * 4u, 0, 0));
    wt.load(0);
  };
  const __amdgpu_buffer_rsrc_t orsrc =
      make_rsrc(g.dW + (size_t)m0 * N, rows_here * (uint32_t)N * 2u);
  Acc acc;
  mainloop_bf16<false, kBwdEpiVmem>(acc, smem, MainloopSrc{g.A, g.B, nullptr, M, N, g.K, m0, n0},
                                    ch, pre, [&] { wt.load(1); wt.load(2); });

  const bool godd = (gq & 1) != 0;
  float ds[32];
#pragma unroll
  for (int c = 0; c < 32; ++c) ds[c] = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    if (i + 3 < 8) wt.load(i + 3);
    const int ml = wm * 128 + i * 16 + (lane & 15);
    const bool mv = m0 + ml < M;
#pragma unroll
    for (int j0 = 0; j0 < 8; j0 += 2) {
      u32x2_t pk[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int j = j0 + u;
        float wv[4], o[4];
        unpack_bf16x4(wt.a[i][j], wv);  // zero past M or N
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float gv = acc.v[j][i][v];
          ds[4 * j + v] = __builtin_fmaf(gv, wv[v], ds[4 * j + v]);
          o[v] = gv * gm[j][v];
        }
        pk[u] = pack_bf16x4(o[0], o[1], o[2], o[3]);
      }
      const int n = nw0 + 16 * (j0 + (godd ? 1 : 0)) + 8 * (gq >> 1);
      store16_exchanged(orsrc, pk, godd,
                        (mv && n < N) ? ((uint32_t)ml * (uint32_t)N + (uint32_t)n) * 2u
                                      : kOobOffset);
    }
  }
  rows16_halving_sum(ds, lane);
  // lane holds columns c0, c0 + 1 of its 4-wide runs: c = 2 (8 b3 + 4 b2 + 2 b1 + b0)
  // indexes 4 j + v, so j = 4 b3 + 2 b2 + b1 and v = 2 b0
  const int b = lane & 15;
  const int col = nw0 + 16 * (b >> 1) + 4 * gq + 2 * (b & 1);
  if (col < N && m0 + wm * 128 < M) {
    const size_t p = (size_t)((m0 + wm * 128) / 128);
    *(float2*)(g.pdg + p * N + col) = make_float2(ds[0], ds[1]);
  }
}

__global__ __launch_bounds__(kThreads, 1) void k_gemm_wgrad_gamma_bf16(WgradGammaArgs g, int gm,
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
    ch.next = MainloopSrc{g.A, g.B, nullptr, g.M, g.N, g.K, nc.tm * kBM, nc.tn * kBN};
    wgrad_gamma_tile(g, smem, tc.tm * kBM, tc.tn * kBN, ch);
    prefetched = has_next;
  }
  wait_vm0();  // the last tile's unused prefetch into LDS lands before the block ends
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
static inline int cdiv_b(int a, int b) { return (a + b - 1) / b; }

hipError_t launch_swiglu_bwd_bf16(const uint16_t* dY, const uint16_t* WdT, const uint16_t* gu,
                                  uint16_t* dz, float* pdot, int M, int N, int K,
                                  hipStream_t stream) {
  const int gm = cdiv_b(M, kBM), gn = cdiv_b(N, kBN);
  hipLaunchKernelGGL(k_swiglu_bwd_bf16, dim3(min(gm * gn, cu_count())), dim3(kThreads8), 0,
                     stream, SwigluBwdArgs{dY, WdT, gu, dz, pdot, M, N, K}, gm, gn);
  return hipGetLastError();
}

hipError_t launch_rmsnorm_bwd_bf16(const uint16_t* dz, const uint16_t* W2T, const uint16_t* h,
                                   const uint16_t* dY, const float* r, const float* c,
                                   uint16_t* dh, int M, int N, int K, hipStream_t stream) {
  const int gm = cdiv_b(M, kBM), gn = cdiv_b(N, kBN);
  hipLaunchKernelGGL(k_rmsnorm_bwd_bf16, dim3(min(gm * gn, cu_count())), dim3(kThreads), 0, stream,
                     RmsBwdArgs{dz, W2T, h, dY, r, c, dh, M, N, K}, gm, gn);
  return hipGetLastError();
}

hipError_t launch_gemm_wgrad_gamma_bf16(const uint16_t* A, const uint16_t* B, const uint16_t* W,
                                       const float* gamma, uint16_t* dW, float* pdg, int M, int N,
                                       int K, hipStream_t stream) {
  const int gm = cdiv_b(M, kBM), gn = cdiv_b(N, kBN);
  hipLaunchKernelGGL(k_gemm_wgrad_gamma_bf16, dim3(min(gm * gn, cu_count())), dim3(kThreads), 0,
                     stream, WgradGammaArgs{A, B, W, gamma, dW, pdg, M, N, K}, gm, gn);
  return hipGetLastError();
}

}  // namespace coda
