// bf16 mainloop with a 128-token x 384-weight-row block tile (page section
// "CODA: the secret in the epilogue": the mainloop is fixed and the epilogue
// programs run on its output tile in registers).
//
// For weight widths that are a multiple of 384 but not of 256 x CUs, the
// 256 x 256 tile of gemm_core.hpp leaves a last round with idle compute units
// (the QKV projection, 3072 wide at M = 8192, is 384 tiles, 1.5 rounds); this
// tile gives 512 tiles, two full rounds.
//   * 4 waves in a 2 x 2 grid, each owning 64 tokens x 192 weight rows:
//     4 token subtiles x 12 weight subtiles of 16 x 16, 192 fp32
//     accumulators per lane pinned to AGPRs; a wave's 192 features are three
//     whole 64-wide heads;
//   * LDS stage: 128 token rows (16 KiB) + 384 weight rows (48 KiB) of 128
//     reduction bytes, 64 KiB as in gemm_core.hpp, the same chunk swizzle
//     (chunk c of row r at slot c ^ (r & 7)), two slots;
//   * the same stage schedule as mainloop_bf16 with 48 MFMAs per k32 step
//     (groups of three): R1 {fragment reads of step 1, MFMAs of step 0},
//     barrier, {loads of stage kt+2, MFMAs}, R2 {MFMAs of the first half of
//     step 1, last loads}, wait for stage kt+1 + barrier, R3 {fragment reads
//     of step 0 of kt+1, second half of step 1}; tile chaining and the
//     epilogue hooks as there.
#pragma once

#include "gemm_core.hpp"

namespace coda {

constexpr int kBMw = 128;                     // token rows per block
constexpr int kBNw = 384;                     // weight rows per block
constexpr int kXBytesW = kBMw * kRowBytes;    // 16 KiB
static_assert(kXBytesW + kBNw * kRowBytes == kStageBytes, "same 64 KiB stage");

// Accumulators of one wave: v[j][i] is the 16x16 tile of weight subtile j
// (0..11) and token subtile i (0..3).  Lane L, register r holds feature
// 16j + 4(L/16) + r of token 16i + L%16 (relative to the wave's corner).
struct AccW {
  f32x4_t v[12][4];
};

// Global -> LDS: wave w fills token rows [w*32, +32) (4 instructions) and
// weight rows [w*96, +96) (12 instructions), 8 rows x 128 B per instruction.
// Rows past the matrix are clamped to its last row (never stored).
struct LoadPlanW {
  __amdgpu_buffer_rsrc_t xr, wr;
  uint32_t off[16];
  char* lds[16];

  __device__ __forceinline__ LoadPlanW(const MainloopSrc& s, char* smem, int wave, int lane) {
    const uint32_t row_bytes = (uint32_t)(s.ld > 0 ? s.ld : s.K) * 2u;
    const uint32_t tail = (uint32_t)s.K * 2u;  // ranges end at the last row's K-th element
    xr = make_rsrc(s.X, (uint32_t)(s.M - 1) * row_bytes + tail);
    wr = make_rsrc(s.W0, (uint32_t)(s.Nw - 1) * row_bytes + tail);
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const bool isx = q < 4;
      const int lr = isx ? wave * 32 + q * 8 + (lane >> 3) : wave * 96 + (q - 4) * 8 + (lane >> 3);
      const int lc = (lane & 7) ^ (lr & 7);
      const int g = isx ? min(s.m0 + lr, s.M - 1) : min(s.n0 + lr, s.Nw - 1);
      off[q] = (uint32_t)g * row_bytes + (uint32_t)lc * 16u;
      lds[q] = smem + (isx ? 0 : kXBytesW) + (isx ? wave * 32 + q * 8 : wave * 96 + (q - 4) * 8) * kRowBytes;
    }
  }
  __device__ __forceinline__ void issue(int slot, int kt, int q) const {
    load16_to_lds(q < 4 ? xr : wr, lds[q] + slot * kStageBytes, off[q], (uint32_t)kt * kRowBytes);
  }
  __device__ __forceinline__ void issue_all(int slot, int kt) const {
#pragma unroll
    for (int q = 0; q < 16; ++q) issue(slot, kt, q);
  }
};

struct FragsW {
  bf16x8_t a[4];   // token subtiles
  bf16x8_t b[12];  // weight subtiles
};

template <int kEpiVmem = -1, class Pre, class PreLast>
__device__ __forceinline__ void mainloop_bf16_wide(AccW& acc, char* smem, const MainloopSrc& s,
                                                   const TileChain& chain, Pre&& pre,
                                                   PreLast&& pre_last) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const LoadPlanW lp(s, smem, wave, lane);

  // lane reads row base + lane%16, logical chunk 4*step + lane/16 at slot
  // chunk ^ (row & 7), row & 7 == lane & 7 (subtile bases are multiples of 16)
  const int r16 = lane & 15;
  uint32_t xo[2], wo[2];
#pragma unroll
  for (int st = 0; st < 2; ++st) {
    const uint32_t slot = (uint32_t)(((st * 4) + (lane >> 4)) ^ (lane & 7)) * 16u;
    xo[st] = (uint32_t)(wm * 64 + r16) * kRowBytes + slot;
    wo[st] = (uint32_t)kXBytesW + (uint32_t)(wn * 192 + r16) * kRowBytes + slot;
  }
  auto rd = [&](FragsW& f, int q, const char* stage, int st) {  // q: 0..3 token, 4..15 weight
    if (q < 4)
      f.a[q] = *(const bf16x8_t*)(stage + xo[st] + q * 16 * kRowBytes);
    else
      f.b[q - 4] = *(const bf16x8_t*)(stage + wo[st] + (q - 4) * 16 * kRowBytes);
  };
  // MFMA m (0..47) of a step: weight subtile m / 4, token subtile m % 4
  auto mma = [&](const FragsW& f, int m) {
    mfma16x16x32_acc(acc.v[m >> 2][m & 3], f.b[m >> 2], f.a[m & 3]);
  };

  const int nk = s.K / 64;
  FragsW fa, fb;
  if (!chain.prefetched) {
    lp.issue_all(0, 0);
    if (nk > 1) {
      lp.issue_all(1, 1);
      wait_vm16();
    } else {
      wait_vm0();
    }
    __syncthreads();
  } else {
    if constexpr (kEpiVmem >= 0)
      wait_vm<(kEpiVmem + 16 < 63 ? kEpiVmem + 16 : 63)>();
    else
      wait_vm0();
    __syncthreads();
  }
#pragma unroll
  for (int j = 0; j < 12; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc.v[j][i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int q = 0; q < 16; ++q) rd(fa, q, smem, 0);

  auto stage = [&](int kt, auto load_tag, auto next_tag) {
    constexpr bool load2 = decltype(load_tag)::value;
    constexpr bool next = decltype(next_tag)::value;
    constexpr bool last = !load2 && !next;
    const int cur = kt & 1;
    const char* base = smem + cur * kStageBytes;
    const char* nbase = smem + (cur ^ 1) * kStageBytes;
    __builtin_amdgcn_sched_barrier(0);
    // R1a: the 16 step-1 fragment reads, 4 per group of 3 MFMAs on fa
#pragma unroll
    for (int g = 0; g < 4; ++g) {
#pragma unroll
      for (int r = 0; r < 4; ++r) rd(fb, 4 * g + r, base, 1);
#pragma unroll
      for (int m = 3 * g; m < 3 * g + 3; ++m) mma(fa, m);
      __builtin_amdgcn_sched_barrier(0);
    }
    // R1b: two more groups while the reads drain
#pragma unroll
    for (int g = 4; g < 6; ++g) {
#pragma unroll
      for (int m = 3 * g; m < 3 * g + 3; ++m) mma(fa, m);
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (load2) {  // B1: slot kt&1 fully read by every wave
      wait_lgkm0();
      bare_barrier();
      __builtin_amdgcn_sched_barrier(0);
    }
    // R1c: the rest of fa's MFMAs with the first 10 loads of stage kt+2
#pragma unroll
    for (int g = 6; g < 16; ++g) {
      if constexpr (load2) lp.issue(cur, kt + 2, g - 6);
#pragma unroll
      for (int m = 3 * g; m < 3 * g + 3; ++m) mma(fa, m);
      __builtin_amdgcn_sched_barrier(0);
    }
    // R2: first half of fb's MFMAs with the last 6 loads (in a tile's last
    // stage: after a barrier, the next tile's stages 0 and 1)
    auto r2 = [&](auto chain_tag) {
      constexpr bool chained = decltype(chain_tag)::value;
      if constexpr (chained) {
        wait_lgkm0();
        bare_barrier();
        __builtin_amdgcn_sched_barrier(0);
      }
      const LoadPlanW nlp(chain.next, smem, wave, lane);
#pragma unroll
      for (int g = 0; g < 8; ++g) {
        if constexpr (load2) {
          if (g < 6) lp.issue(cur, kt + 2, 10 + g);
        }
        if constexpr (chained) {  // all of stage 0, then all of stage 1
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int q = 4 * g + u;  // 0..31
            nlp.issue(q >> 4, q >> 4, q & 15);
          }
        }
#pragma unroll
        for (int m = 3 * g; m < 3 * g + 3; ++m) mma(fb, m);
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    if constexpr (last) {
      if (nk == 1) pre();
      pre_last();
      __builtin_amdgcn_sched_barrier(0);
      r2(std::true_type{});
    } else {
      r2(std::false_type{});
    }
    if constexpr (next) {  // B2
      if constexpr (load2)
        wait_vm16();
      else
        wait_vm0();
      bare_barrier();
    }
    if constexpr (!load2 && next) pre();
    __builtin_amdgcn_sched_barrier(0);
    // R3: second half of fb's MFMAs with the 16 fa reads of step 0 of kt+1
#pragma unroll
    for (int g = 8; g < 16; ++g) {
      if constexpr (next) {
        rd(fa, 2 * (g - 8), nbase, 0);
        rd(fa, 2 * (g - 8) + 1, nbase, 0);
      }
#pragma unroll
      for (int m = 3 * g; m < 3 * g + 3; ++m) mma(fb, m);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  for (int kt = 0; kt < nk - 2; ++kt) stage(kt, std::true_type{}, std::true_type{});
  if (nk >= 2) stage(nk - 2, std::false_type{}, std::true_type{});
  stage(nk - 1, std::false_type{}, std::false_type{});
  settle_accumulators<AccW, 12, 4>(acc);
}

}  // namespace coda
