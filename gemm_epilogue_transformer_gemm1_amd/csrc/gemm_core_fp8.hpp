// The e4m3 mainloop every fp8 epilogue program runs on (page section "CODA:
// the secret in the epilogue": a GEMM is a blocked multiply-accumulate
// mainloop followed by an epilogue that still holds the output tile in
// registers).  It shares the bf16 mainloop's LDS layout, load plan, tile
// chaining and epilogue hooks (gemm_core.hpp).
#pragma once

#include "gemm_core.hpp"

namespace coda {

// ===========================================================================
// e4m3 mainloop on v_mfma_f32_16x16x128_f8f6f4: one 128-deep reduction step
// per stage, accumulators in the bf16 layout (struct Acc).  Under the power
// limit this MFMA form keeps a higher clock than the 32x32x64 one.  A
// fragment is 32 bytes of one row (two 16-byte chunks): lane L reads row
// base + L % 16, logical chunks L / 16 and L / 16 + 4.  Each of the two
// 16-byte reads then has the bf16 loop's pattern (the four lane groups read
// four consecutive chunks), which is free of LDS bank conflicts; chunks 2 g
// and 2 g + 1 instead conflict on about half the cycles.  Both operands use
// the same lane -> chunk map, so every product pairs equal k.
//
// Registers: token fragments A[0..7] and weight fragments B[0..7] of one
// stage (128 VGPRs).  Per stage kt (slot kt & 1), with A[0..3] and B of kt
// already loaded:
//   P1a: token subtile 0 (8 MFMAs) with the reads of A[4..7] of kt
//   B1:  slot kt & 1 read by every wave (only when stage kt+2 exists)
//   P1b: token subtiles 1..3 (24 MFMAs) with the 16 loads of stage kt+2
//   B2:  this wave's stage kt+1 loads landed, barrier
//   P2:  token subtiles 4..7 weight-subtile-major: 8 groups of 4 MFMAs on
//        B[j]; after group j the next stage's B[j-1] is read into the
//        registers group j-1 used (one group of distance), and in groups
//        0..3 the next stage's A[j] (free since P1b)
// Tile chaining, the epilogue operand hooks and the vector memory accounting
// are as in mainloop_bf16: `pre` after B2 of stage nk-2 (in the last stage
// if there is only one), `pre_last` in the last stage before the next
// tile's loads, which start after a barrier at the head of P1b there.
// ===========================================================================
template <bool kGated, int kEpiVmem = -1, class Pre, class PreLast>
__device__ __forceinline__ void mainloop_fp8(Acc& acc, char* smem, const MainloopSrc& s,
                                                const TileChain& chain, Pre&& pre,
                                                PreLast&& pre_last) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const LoadPlan<kGated> lp(s, smem, wave, lane, 1);

  // row base + lane % 16 has row & 7 == lane & 7 (every subtile base is a
  // multiple of 16)
  uint32_t xo[2], wo[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint32_t slot = (uint32_t)((4 * h + (lane >> 4)) ^ (lane & 7)) * 16u;
    xo[h] = (uint32_t)(wm * 128 + (lane & 15)) * kRowBytes + slot;
    wo[h] = (uint32_t)kXBytes + (uint32_t)(wave_wrow_base<kGated>(wn) + (lane & 15)) * kRowBytes + slot;
  }
  auto rd = [&](const char* stage, const uint32_t (&o)[2], int rowoff) {
    const i32x4_t lo = *(const i32x4_t*)(stage + o[0] + rowoff);
    const i32x4_t hi = *(const i32x4_t*)(stage + o[1] + rowoff);
    return i32x8_t{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
  };
  auto rd_a = [&](const char* stage, int i) { return rd(stage, xo, i * 16 * kRowBytes); };
  auto rd_b = [&](const char* stage, int j) {
    return rd(stage, wo, wrow_of_subtile<kGated>(j) * kRowBytes);
  };

  const int nk = s.K / 128;
  i32x8_t A[8], B[8];
  if (!chain.prefetched) {
    prologue(lp, nk);
  } else {
    if constexpr (kEpiVmem >= 0)
      wait_vm<(kEpiVmem + 16 < 63 ? kEpiVmem + 16 : 63)>();
    else
      wait_vm0();
    __syncthreads();
  }
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int i = 0; i < 8; ++i) acc.v[j][i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < 4; ++i) A[i] = rd_a(smem, i);
#pragma unroll
  for (int j = 0; j < 8; ++j) B[j] = rd_b(smem, j);

  auto stage = [&](int kt, auto load_tag, auto next_tag) {
    constexpr bool load2 = decltype(load_tag)::value;
    constexpr bool next = decltype(next_tag)::value;
    constexpr bool last = !load2 && !next;
    const int cur = kt & 1;
    const char* base = smem + cur * kStageBytes;
    const char* nbase = smem + (cur ^ 1) * kStageBytes;
    __builtin_amdgcn_sched_barrier(0);
    // P1a: token subtile 0 with the reads of A[4..7]
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      A[4 + q] = rd_a(base, 4 + q);
      mfma16x16x128_f8_acc(acc.v[2 * q][0], B[2 * q], A[0]);
      mfma16x16x128_f8_acc(acc.v[2 * q + 1][0], B[2 * q + 1], A[0]);
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (load2) {  // B1
      wait_lgkm0();
      bare_barrier();
      __builtin_amdgcn_sched_barrier(0);
    }
    const LoadPlan<kGated> nlp(chain.next, smem, wave, lane, 1);
    if constexpr (last) {
      if (nk == 1) pre();
      pre_last();
      // every wave holds all fragments of both slots: both are free for the
      // next tile's stages 0 and 1 (stage 1 is loaded even when K has one
      // stage, as in mainloop_bf16)
      wait_lgkm0();
      bare_barrier();
      __builtin_amdgcn_sched_barrier(0);
    }
    // P1b: token subtiles 1..3 with the stage loads
#pragma unroll
    for (int q = 0; q < 24; ++q) {
      if constexpr (load2) {
        if (q < 16) lp.issue(cur, kt + 2, q);
      }
      if constexpr (last) {  // next tile: all of stage 0 (slot 0), then stage 1 (slot 1)
        if (q < 16) {
          nlp.issue(q >> 3, q >> 3, 2 * (q & 7));
          nlp.issue(q >> 3, q >> 3, 2 * (q & 7) + 1);
        }
      }
      const int i = 1 + q / 8, j = q % 8;
      mfma16x16x128_f8_acc(acc.v[j][i], B[j], A[i]);
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (next) {  // B2
      if constexpr (load2)
        wait_vm16();
      else
        wait_vm0();
      bare_barrier();
    }
    if constexpr (!load2 && next) pre();  // stage nk-2, as in mainloop_bf16
    __builtin_amdgcn_sched_barrier(0);
    // P2: token subtiles 4..7, weight-subtile-major, refilling the fragments
#pragma unroll
    for (int j = 0; j < 8; ++j) {
#pragma unroll
      for (int i = 4; i < 8; ++i) mfma16x16x128_f8_acc(acc.v[j][i], B[j], A[i]);
      if constexpr (next) {
        if (j >= 1) B[j - 1] = rd_b(nbase, j - 1);
        if (j < 4) A[j] = rd_a(nbase, j);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (next) B[7] = rd_b(nbase, 7);
  };
  for (int kt = 0; kt < nk - 2; ++kt) stage(kt, std::true_type{}, std::true_type{});
  if (nk >= 2) stage(nk - 2, std::false_type{}, std::true_type{});
  stage(nk - 1, std::false_type{}, std::false_type{});
  settle_accumulators<Acc, 8, 8>(acc);
}

}  // namespace coda
