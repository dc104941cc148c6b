// The bf16 GEMM mainloop with two waves per SIMD (page section "Five building
// blocks and a LEGO language": one fixed mainloop under every epilogue
// program; this is the same block tile as gemm_core.hpp's mainloop_bf16 with
// twice the waves).
//
// gfx950 design (one 512-thread workgroup per CU, 8 waves in a 4 x 2 grid):
//   * block tile 256 token rows x 256 weight rows, two 64 KiB LDS stages of
//     128 reduction bytes per row, the same chunk swizzle and the same
//     buffer_load ... lds global -> LDS plan as mainloop_bf16 (each wave now
//     fills 32 rows of each operand tile per stage: 8 instructions);
//   * wave w owns token rows 64 (w / 2) .. + 63 and weight rows 128 (w % 2) ..
//     + 127 (gated: 64 gate rows and the matching 64 up rows), 128 fp32
//     accumulators per lane pinned to AGPRs: 4 token x 8 weight subtiles of
//     16 x 16, the accumulator layout of mainloop_bf16 restricted to 4 token
//     subtiles (lane L, register v of tile (j, i): feature 16 j + 4 (L / 16)
//     + v of token 16 i + L % 16 relative to the wave's corner);
//   * per k32 step a wave reads 12 fragments (4 token, 8 weight) for 32
//     MFMAs.  That is 1.5 times the LDS reads per MFMA of the one-wave-per-
//     SIMD loop, but with two waves per SIMD the LDS serves them faster
//     (measured on gfx950: ~183 B/clk per CU with 8 waves issuing 16-byte
//     reads against ~110 with 4), and while one wave of a SIMD waits for its
//     fragments, a barrier or its epilogue operands, the other one can issue
//     MFMAs.  Measured, the mainloop itself is no faster than
//     mainloop_bf16's (equal at K = 2048, slower at K = 8192); what gains is
//     an epilogue bound by memory operations in flight;
//   * pipeline per stage kt (slot kt & 1; fa = the step-0 fragments, already
//     in registers):
//       R1: 8 groups of 4 MFMAs on fa; the 12 step-1 fragment reads (fb)
//           within the first kRdGroups groups (default 3), B1 after group
//           kB1 - 1 (default 4: reads drained + barrier, slot kt & 1 is free
//           everywhere), the 8 loads of stage kt+2 into that slot in the
//           groups after it (later barriers and other read spreads measured
//           equal or slower);
//       R2: 8 groups of 2 MFMAs on fb (weight subtiles 0..3);
//       B2: this wave's stage kt+1 loads landed (kt+2 stays in flight), barrier;
//       R3: 16 single MFMAs on fb (weight subtiles 4..7), the 12 step-0
//           fragment reads of stage kt+1 in the first 12;
//   * tile chaining, the epilogue-operand hooks and the accumulator settling
//     work as in mainloop_bf16.
#pragma once

#include <type_traits>

#include "gemm_core.hpp"

namespace coda {

constexpr int kThreads8 = 512;

// v[j][i]: weight subtile j (0..7), token subtile i (0..3)
struct Acc8 {
  f32x4_t v[8][4];
};

// Global -> LDS plan: wave w fills LDS rows [w*32, w*32+32) of both tiles with
// 4 instructions each.  Gated blocks: LDS weight rows [0,128) hold gate rows
// (waves 0..3 load them), [128,256) the up rows (waves 4..7).  Rows past the
// matrix are clamped to its last row (their results are never stored).
template <bool kGated>
struct LoadPlan8 {
  __amdgpu_buffer_rsrc_t xr, wr;
  uint32_t xoff[4], woff[4];
  char* x_lds;
  char* w_lds;

  __device__ __forceinline__ LoadPlan8(const MainloopSrc& s, char* smem, int wave, int lane,
                                       int esize) {
    const uint32_t row_bytes = (uint32_t)(s.ld > 0 ? s.ld : s.K) * (uint32_t)esize;
    const uint32_t tail = (uint32_t)s.K * (uint32_t)esize;
    xr = make_rsrc(s.X, (uint32_t)(s.M - 1) * row_bytes + tail);
    const void* wsrc = (kGated && wave >= 4) ? s.W1 : s.W0;
    wr = make_rsrc(wsrc, (uint32_t)(s.Nw - 1) * row_bytes + tail);
    const int wrow_shift = (kGated && wave >= 4) ? 128 : 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int lr = wave * 32 + q * 8 + (lane >> 3);
      const int lc = (lane & 7) ^ (lr & 7);
      const int gx = min(s.m0 + lr, s.M - 1);
      const int gw = min(s.n0 + lr - wrow_shift, s.Nw - 1);
      xoff[q] = (uint32_t)gx * row_bytes + (uint32_t)lc * 16u;
      woff[q] = (uint32_t)gw * row_bytes + (uint32_t)lc * 16u;
    }
    x_lds = smem + wave * 32 * kRowBytes;
    w_lds = smem + kXBytes + wave * 32 * kRowBytes;
  }

  // q in [0,8): instruction q of stage kt into LDS slot `slot`
  __device__ __forceinline__ void issue(int slot, int kt, int q) const {
    const uint32_t soff = (uint32_t)kt * kRowBytes;
    if (q < 4)
      load16_to_lds(xr, x_lds + slot * kStageBytes + q * 8 * kRowBytes, xoff[q], soff);
    else
      load16_to_lds(wr, w_lds + slot * kStageBytes + (q - 4) * 8 * kRowBytes, woff[q - 4], soff);
  }

  __device__ __forceinline__ void issue_all(int slot, int kt) const {
#pragma unroll
    for (int q = 0; q < 8; ++q) issue(slot, kt, q);
  }
};

struct Frags8 {
  bf16x8_t a[4];  // token subtiles i = 0..3
  bf16x8_t b[8];  // weight subtiles j = 0..7
};

// fragment q (0..3 token, 4..11 weight) of one step
template <bool kGated>
__device__ __forceinline__ void read_frag8(Frags8& f, int q, const char* stage, uint32_t xo,
                                           uint32_t wo) {
  if (q < 4)
    f.a[q] = *(const bf16x8_t*)(stage + xo + q * 16 * kRowBytes);
  else
    f.b[q - 4] = *(const bf16x8_t*)(stage + wo + wrow_of_subtile<kGated>(q - 4) * kRowBytes);
}

// `pre` and `pre_last` as in mainloop_bf16; kEpiVmem = vector memory
// operations the epilogue issues per lane after the next tile's loads (or
// -1: unknown), so the next tile waits only for its own stage 0.
template <bool kGated, int kEpiVmem = -1, int kRdGroups = 3, int kB1 = 4, class Pre,
          class PreLast>
__device__ __forceinline__ void mainloop8_bf16(Acc8& acc, char* smem, const MainloopSrc& s,
                                               const TileChain& chain, Pre&& pre,
                                               PreLast&& pre_last) {
  static_assert(kRdGroups >= 1 && kRdGroups <= kB1 && kB1 >= 1 && kB1 < 8, "R1 schedule");
  // the thread index as an opaque value: the lane-derived addresses below are
  // recomputed for every tile instead of being kept live (or spilled) across
  // the tiles of a persistent kernel
  int tid = (int)threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int wm = wave >> 1, wn = wave & 1;
  const LoadPlan8<kGated> lp(s, smem, wave, lane, 2);

  // LDS -> register plan (as mainloop_bf16): lane reads row base + lane % 16,
  // logical chunk 4 step + lane / 16, stored at chunk ^ (row & 7).
  const int r16 = lane & 15;
  uint32_t xfrag[2], wfrag[2];
#pragma unroll
  for (int st = 0; st < 2; ++st) {
    const uint32_t slot = (uint32_t)(((st * 4) + (lane >> 4)) ^ (lane & 7)) * 16u;
    xfrag[st] = (uint32_t)(wm * 64 + r16) * kRowBytes + slot;
    wfrag[st] = (uint32_t)kXBytes + (uint32_t)(wave_wrow_base<kGated>(wn) + r16) * kRowBytes + slot;
  }

  const int nk = s.K / 64;
  Frags8 fa, fb;
  if (!chain.prefetched) {
    lp.issue_all(0, 0);
    if (nk > 1) {
      lp.issue_all(1, 1);
      wait_vm<8>();
    } else {
      wait_vm0();
    }
    __syncthreads();
  } else {
    // stage 0 was issued during the previous tile, before stage 1 and that
    // tile's epilogue operations
    if constexpr (kEpiVmem >= 0)
      wait_vm<(kEpiVmem + 8 < 63 ? kEpiVmem + 8 : 63)>();
    else
      wait_vm0();
    __syncthreads();
  }
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc.v[j][i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int q = 0; q < 12; ++q) read_frag8<kGated>(fa, q, smem, xfrag[0], wfrag[0]);

  auto stage = [&](int kt, auto load_tag, auto next_tag) {
    constexpr bool load2 = decltype(load_tag)::value;  // stage kt+2 exists
    constexpr bool next = decltype(next_tag)::value;   // stage kt+1 exists
    constexpr bool last = !load2 && !next;
    const int cur = kt & 1;
    const char* base = smem + cur * kStageBytes;
    const char* nbase = smem + (cur ^ 1) * kStageBytes;
    __builtin_amdgcn_sched_barrier(0);
    // R1: 8 groups of 4 MFMAs on fa (weight subtile q).  The 12 step-1
    // fragment reads go out in the first kRdGroups groups (weight fragments
    // first: the previous stage's last MFMAs read fb.a[*]); after group
    // kB1 - 1, B1 (reads drained + barrier: slot kt & 1 is free everywhere);
    // the 8 loads of stage kt+2 into that slot spread over the groups after it.
    constexpr int kRdPer = (12 + kRdGroups - 1) / kRdGroups;
    constexpr int kLdPer = (8 + (8 - kB1) - 1) / (8 - kB1);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      if (q < kRdGroups) {
#pragma unroll
        for (int r = 0; r < kRdPer; ++r)
          if (q * kRdPer + r < 12)
            read_frag8<kGated>(fb, (q * kRdPer + r + 4) % 12, base, xfrag[1], wfrag[1]);
      }
      if constexpr (load2) {
        if (q >= kB1) {
#pragma unroll
          for (int r = 0; r < kLdPer; ++r)
            if ((q - kB1) * kLdPer + r < 8) lp.issue(cur, kt + 2, (q - kB1) * kLdPer + r);
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) mfma16x16x32_acc(acc.v[q][i], fa.b[q], fa.a[i]);
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (load2) {
        if (q == kB1 - 1) {  // B1
          wait_lgkm0();
          bare_barrier();
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
    // R2: fb's weight subtiles 0..3; in the last stage of a tile, after a
    // barrier (both slots free), the next tile's stages 0 and 1
    auto r2 = [&](auto chain_tag) {
      constexpr bool chained = decltype(chain_tag)::value;
      if constexpr (chained) {
        wait_lgkm0();
        bare_barrier();
        __builtin_amdgcn_sched_barrier(0);
      }
      const LoadPlan8<kGated> nlp(chain.next, smem, wave, lane, 2);
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        if constexpr (chained) {
          // stage 1 is loaded even when K has one stage (never read then),
          // so the count of operations in flight behind the epilogue is the
          // same on every path
          if (q < 4) {
            nlp.issue(0, 0, 2 * q);
            nlp.issue(0, 0, 2 * q + 1);
          } else {
            nlp.issue(1, 1, 2 * q - 8);
            nlp.issue(1, 1, 2 * q - 7);
          }
        }
        const int j = q >> 1, i0 = (q & 1) * 2;
#pragma unroll
        for (int i = i0; i < i0 + 2; ++i) mfma16x16x32_acc(acc.v[j][i], fb.b[j], fb.a[i]);
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    if constexpr (last) {
      if (nk == 1) pre();  // otherwise already issued in stage nk-2
      pre_last();
      __builtin_amdgcn_sched_barrier(0);
      r2(std::true_type{});
    } else {
      r2(std::false_type{});
    }
    if constexpr (next) {  // B2
      if constexpr (load2)
        wait_vm<8>();
      else
        wait_vm0();
      bare_barrier();
    }
    if constexpr (!load2 && next) pre();
    __builtin_amdgcn_sched_barrier(0);
    // R3: fb's weight subtiles 4..7, with the step-0 fragments of stage kt+1
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      if constexpr (next) {
        if (q < 12) read_frag8<kGated>(fa, q, nbase, xfrag[0], wfrag[0]);
      }
      const int j = 4 + (q >> 2), i = q & 3;
      mfma16x16x32_acc(acc.v[j][i], fb.b[j], fb.a[i]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  for (int kt = 0; kt < nk - 2; ++kt) stage(kt, std::true_type{}, std::true_type{});
  if (nk >= 2) stage(nk - 2, std::false_type{}, std::true_type{});
  stage(nk - 1, std::false_type{}, std::false_type{});
  settle_accumulators<Acc8, 8, 4>(acc);
}

}  // namespace coda
