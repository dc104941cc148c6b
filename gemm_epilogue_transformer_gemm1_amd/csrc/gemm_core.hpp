// The fixed GEMM mainloops every epilogue program runs on (page section
// "CODA: the secret in the epilogue": a GEMM is a blocked multiply-accumulate
// mainloop followed by an epilogue that still holds the output tile in
// registers; section "Five building blocks and a LEGO language": the mainloop
// stays fixed and epilogue primitives are composed on top of it).
//
// gfx950 design (one 256-thread workgroup per CU, 4 waves in a 2x2 grid):
//   * block tile 256 token rows x 256 weight rows; each stage covers 128 bytes
//     of reduction per row (64 bf16 or 128 e4m3 values); two LDS stages of
//     64 KiB (token tile 32 KiB + weight tile 32 KiB);
//   * global -> LDS with buffer_load ... lds (16 B per lane, no VGPR staging);
//     each 128 B LDS row is 8 chunks of 16 B, chunk c of row r stored at slot
//     c ^ (r & 7), so the lanes reading one MFMA fragment hit distinct banks;
//   * the WEIGHT fragment is the MFMA's first operand and the TOKEN fragment
//     its second, so the accumulator is C^T and a lane holds runs of 4
//     consecutive output features of one token: per-token reductions (RMS
//     partials, log-sum-exp) are mostly lane-local;
//   * each wave owns a 128-token x 128-weight-row quarter, 256 fp32
//     accumulators per lane, pinned to AGPRs;
//   * bf16: v_mfma_f32_16x16x32_bf16, e4m3: v_mfma_f32_16x16x128_f8f6f4;
//     8x8 tiles of 16x16 per wave in both;
//   * pipeline (bf16): the reduction of a stage is two MFMA steps with
//     fragment sets fa / fb; a stage's LDS slot is refilled as soon as every
//     wave holds its second step's fragments, so each stage's loads are
//     issued about one and a half stages of MFMA work before they are needed.
//     The e4m3 loop (one 128-deep step per stage) is gemm_core_fp8.hpp's
//     mainloop_fp8, on the same load plan, tile chaining and LDS layout.
#pragma once

#include <type_traits>

#include "coda_device.hpp"

namespace coda {

constexpr int kThreads = 256;
constexpr int kBM = 256;                      // token rows per block
constexpr int kBN = 256;                      // weight rows per block
constexpr int kRowBytes = 128;                // reduction bytes per row per stage
constexpr int kXBytes = kBM * kRowBytes;      // 32 KiB token tile
constexpr int kWBytes = kBN * kRowBytes;      // 32 KiB weight tile
constexpr int kStageBytes = kXBytes + kWBytes;
constexpr int kSmemBytes = 2 * kStageBytes;   // 128 KiB

// bf16 accumulators of one wave: v[j][i] is the 16x16 tile of weight subtile
// j and token subtile i.  Lane L, register r holds feature 16j + 4(L/16) + r
// of token 16i + L%16 (relative to the wave's corner).
struct Acc {
  f32x4_t v[8][8];
};

struct TileCoord {
  int tm, tn;
};

// Workgroup -> output tile.  Workgroups are handed to the 8 XCDs round robin
// (workgroup b runs on XCD b % 8), so first give each XCD a contiguous range
// of tile ids, then walk tiles in groups of `group_m` token tiles so the
// blocks running together on one XCD share token rows and weight rows in its
// L2.  Both steps are bijections on [0, gm*gn).
__device__ __forceinline__ TileCoord map_tile(int b, int gm, int gn, int group_m) {
  const int nb = gm * gn;
  const int q = nb >> 3, rem = nb & 7;
  const int xcd = b & 7, local = b >> 3;
  const int t = xcd * q + (xcd < rem ? xcd : rem) + local;
  const int group_size = group_m * gn;
  const int g = t / group_size;
  const int first_m = g * group_m;
  const int rows = min(gm - first_m, group_m);
  const int in_g = t - g * group_size;
  TileCoord c;
  c.tm = first_m + in_g % rows;
  c.tn = in_g / rows;
  return c;
}

// Operand sources of one block.
struct MainloopSrc {
  const void* X;   // token operand [M, K]
  const void* W0;  // weight rows for LDS rows [0,256) (plain) or [0,128) (gated)
  const void* W1;  // gated only: weight rows for LDS rows [128,256)
  int M;           // token rows of X
  int Nw;          // rows of each weight matrix
  int K;           // reduction length in elements
  int m0;          // first token row of the block
  int n0;          // first weight row of the block (per weight matrix)
  int ld = 0;      // row pitch of X and the weights in elements (0: K); a pitch
                   // above K reads a column slice, e.g. one part of a split
                   // reduction with X and the weights offset to its first column
};

// Persistent kernels walk several tiles per workgroup.  While a tile's last
// stage runs, both LDS slots are refilled with the first two stages of the
// workgroup's next tile, so that tile's loads are in flight during this
// tile's epilogue and its stores drain while the next tile computes.  The
// last tile of a workgroup names itself as `next`: the loads are then
// harmless re-reads that nobody consumes, and the MFMA code has no branch
// (a branch there makes the register allocator copy accumulators).
//
// The next tile's stage-0 loads are issued first, then its stage-1 loads,
// then the epilogue's own vector memory operations.  Those retire in issue
// order, so if the epilogue issues at least E of them per wave
// (kEpiVmem = E), the next tile waits for its stage 0 alone with
// vmcnt(min(16 + E, 63)) instead of draining the stores too; kEpiVmem < 0
// means no such bound and waits for everything.
struct TileChain {
  bool prefetched;   // stages 0 and 1 of this tile are already in flight
  MainloopSrc next;  // the workgroup's next tile, or this tile if none
};

// Gated (SwiGLU) blocks: LDS weight rows [0,128) hold gate rows n0.. and
// [128,256) the same up rows, and a wave owns gate rows [wn*64, +64) and the
// matching up rows, so gate and up values of one output element sit in the
// same lane and register.  Plain blocks: the wave owns rows [wn*128, +128).
template <bool kGated>
__device__ __forceinline__ int wave_wrow_base(int wn) {
  return kGated ? wn * 64 : wn * 128;
}

// Global -> LDS load plan: wave w fills LDS rows [w*64, w*64+64) of both
// tiles with 8 instructions each (8 rows x 128 B per instruction).  Rows past
// the matrix are clamped to its last row (their results are never stored).
template <bool kGated>
struct LoadPlan {
  __amdgpu_buffer_rsrc_t xr, wr;
  uint32_t xoff[8], woff[8];
  char* x_lds;
  char* w_lds;

  __device__ __forceinline__ LoadPlan(const MainloopSrc& s, char* smem, int wave, int lane,
                                      int esize) {
    const uint32_t row_bytes = (uint32_t)(s.ld > 0 ? s.ld : s.K) * (uint32_t)esize;
    // ranges end at the last row's K-th element (the whole matrix for ld = K)
    const uint32_t tail = (uint32_t)s.K * (uint32_t)esize;
    xr = make_rsrc(s.X, (uint32_t)(s.M - 1) * row_bytes + tail);
    const void* wsrc = (kGated && wave >= 2) ? s.W1 : s.W0;
    wr = make_rsrc(wsrc, (uint32_t)(s.Nw - 1) * row_bytes + tail);
    const int wrow_shift = (kGated && wave >= 2) ? 128 : 0;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int lr = wave * 64 + q * 8 + (lane >> 3);
      const int lc = (lane & 7) ^ (lr & 7);
      const int gx = min(s.m0 + lr, s.M - 1);
      const int gw = min(s.n0 + lr - wrow_shift, s.Nw - 1);
      xoff[q] = (uint32_t)gx * row_bytes + (uint32_t)lc * 16u;
      woff[q] = (uint32_t)gw * row_bytes + (uint32_t)lc * 16u;
    }
    x_lds = smem + wave * 64 * kRowBytes;
    w_lds = smem + kXBytes + wave * 64 * kRowBytes;
  }

  // q in [0,16): instruction q of stage kt into LDS slot `slot`
  __device__ __forceinline__ void issue(int slot, int kt, int q) const {
    const uint32_t soff = (uint32_t)kt * kRowBytes;
    if (q < 8)
      load16_to_lds(xr, x_lds + slot * kStageBytes + q * 8 * kRowBytes, xoff[q], soff);
    else
      load16_to_lds(wr, w_lds + slot * kStageBytes + (q - 8) * 8 * kRowBytes, woff[q - 8], soff);
  }

  __device__ __forceinline__ void issue_all(int slot, int kt) const {
#pragma unroll
    for (int q = 0; q < 16; ++q) issue(slot, kt, q);
  }
};

// s_waitcnt vmcnt(n) (n < 64; expcnt and lgkmcnt not waited for)
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}
__device__ __forceinline__ void wait_vm0() { wait_vm<0>(); }
__device__ __forceinline__ void wait_vm16() { wait_vm<16>(); }
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }  // lgkmcnt(0)

// Barrier without the release fence of __syncthreads (which would also drain
// the loads still in flight).  The signal fences keep the compiler from
// moving LDS accesses across it.
__device__ __forceinline__ void bare_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Prologue: stages 0 and 1 in flight, wait for stage 0.
template <bool kGated>
__device__ __forceinline__ void prologue(const LoadPlan<kGated>& lp, int nk) {
  lp.issue_all(0, 0);
  if (nk > 1) {
    lp.issue_all(1, 1);
    wait_vm16();
  } else {
    wait_vm0();
  }
  __syncthreads();
}

// The MFMAs are inline asm, so the compiler's hazard recognizer does not see
// their accumulator writes and could read an accumulator right after the MFMA
// that writes it.  Give the last MFMAs time to retire, then re-define every
// accumulator with an empty asm statement ordered after the wait states: every
// epilogue read depends on it and so comes later.
template <class AccT, int NJ, int NI>
__device__ __forceinline__ void settle_accumulators(AccT& acc) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
  for (int j = 0; j < NJ; ++j)
#pragma unroll
    for (int i = 0; i < NI; ++i) asm volatile("" : "+a"(acc.v[j][i]));
  __builtin_amdgcn_sched_barrier(0);
}

// ===========================================================================
// bf16 mainloop: v_mfma_f32_16x16x32_bf16, two k32 steps per stage.
// ===========================================================================
struct Frags {
  bf16x8_t a[8];  // token subtiles i = 0..7
  bf16x8_t b[8];  // weight subtiles j = 0..7
};

template <bool kGated>
__device__ __forceinline__ constexpr int wrow_of_subtile(int j) {
  return kGated ? (j < 4 ? j * 16 : 128 + (j - 4) * 16) : j * 16;
}

// fragment q (0..7 token, 8..15 weight) of one step
template <bool kGated>
__device__ __forceinline__ void read_frag(Frags& f, int q, const char* stage, uint32_t xo,
                                          uint32_t wo) {
  if (q < 8)
    f.a[q] = *(const bf16x8_t*)(stage + xo + q * 16 * kRowBytes);
  else
    f.b[q - 8] = *(const bf16x8_t*)(stage + wo + wrow_of_subtile<kGated>(q - 8) * kRowBytes);
}

// `pre` runs once, in the second-to-last stage after its end-of-stage wait
// (in the last stage if there is only one), and `pre_last` in the last stage,
// both before the next tile's loads are issued: epilogue operands loaded
// there arrive during the last stages and are not queued behind those loads
// (vector memory operations complete in order), and no stage wait includes
// them.
template <bool kGated, int kEpiVmem = -1, class Pre, class PreLast>
__device__ __forceinline__ void mainloop_bf16(Acc& acc, char* smem, const MainloopSrc& s,
                                              const TileChain& chain, Pre&& pre,
                                              PreLast&& pre_last) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int wm = wave >> 1, wn = wave & 1;
  const LoadPlan<kGated> lp(s, smem, wave, lane, 2);

  // LDS -> register plan: lane reads row (base + lane%16), logical chunk
  // 4*step + lane/16, stored at slot chunk ^ (row & 7) with row & 7 == lane & 7.
  const int r16 = lane & 15;
  uint32_t xfrag[2], wfrag[2];
#pragma unroll
  for (int st = 0; st < 2; ++st) {
    const uint32_t slot = (uint32_t)(((st * 4) + (lane >> 4)) ^ (lane & 7)) * 16u;
    xfrag[st] = (uint32_t)(wm * 128 + r16) * kRowBytes + slot;
    wfrag[st] = (uint32_t)kXBytes + (uint32_t)(wave_wrow_base<kGated>(wn) + r16) * kRowBytes + slot;
  }

  // Per stage kt (slot kt & 1), with fa = step 0 of kt already in registers:
  //   R1: the 16 fb fragment reads (step 1 of kt) in the first 4 groups of 4
  //       MFMAs on fa, 2 more groups, then B1 (reads drained + barrier: slot
  //       kt&1 is free everywhere), then fa's last 10 groups with the first
  //       10 loads of stage kt+2 into slot kt&1
  //   R2: 16 x {2 MFMAs on fb}, the last 6 loads in its first groups
  //   B2: this wave's stage kt+1 loads landed (kt+2 stays in flight), barrier
  //   R3: 16 x {one fa fragment read (step 0 of kt+1), 2 MFMAs on fb}
  // Every group is fenced with sched_barrier(0) so the compiler keeps this
  // interleaving; it still inserts the exact waitcnts the reads need.
  const int nk = s.K / 64;
  Frags fa, fb;
  if (!chain.prefetched) {
    prologue(lp, nk);
  } else {
    // stage 0, issued during the previous tile before stage 1 and that
    // tile's epilogue operations
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
  for (int q = 0; q < 16; ++q) read_frag<kGated>(fa, q, smem, xfrag[0], wfrag[0]);

  auto stage = [&](int kt, auto load_tag, auto next_tag) {
    constexpr bool load2 = decltype(load_tag)::value;  // stage kt+2 exists
    constexpr bool next = decltype(next_tag)::value;   // stage kt+1 exists
    constexpr bool last = !load2 && !next;             // last stage of the tile
    const int cur = kt & 1;
    const char* base = smem + cur * kStageBytes;
    const char* nbase = smem + (cur ^ 1) * kStageBytes;
    __builtin_amdgcn_sched_barrier(0);
    // R1a: all 16 step-1 fragment reads up front (4 per group of 4 MFMAs on fa)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
#pragma unroll
      for (int r = 0; r < 4; ++r) read_frag<kGated>(fb, 4 * q + r, base, xfrag[1], wfrag[1]);
      const int j = q >> 1, i0 = (q & 1) * 4;
#pragma unroll
      for (int i = i0; i < i0 + 4; ++i) mfma16x16x32_acc(acc.v[j][i], fa.b[j], fa.a[i]);
      __builtin_amdgcn_sched_barrier(0);
    }
    // R1b: two more groups while the reads drain
#pragma unroll
    for (int q = 4; q < 6; ++q) {
      const int j = q >> 1, i0 = (q & 1) * 4;
#pragma unroll
      for (int i = i0; i < i0 + 4; ++i) mfma16x16x32_acc(acc.v[j][i], fa.b[j], fa.a[i]);
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (load2) {  // B1: slot kt&1 fully read by every wave
      wait_lgkm0();
      bare_barrier();
      __builtin_amdgcn_sched_barrier(0);
    }
    // R1c: rest of fa's MFMAs, with the first 10 loads of stage kt+2
#pragma unroll
    for (int q = 6; q < 16; ++q) {
      if constexpr (load2) lp.issue(cur, kt + 2, q - 6);
      const int j = q >> 1, i0 = (q & 1) * 4;
#pragma unroll
      for (int i = i0; i < i0 + 4; ++i) mfma16x16x32_acc(acc.v[j][i], fa.b[j], fa.a[i]);
      __builtin_amdgcn_sched_barrier(0);
    }
    // R2: first half of fb's MFMAs, with the last 6 loads
    auto r2 = [&](auto chain_tag) {
      constexpr bool chained = decltype(chain_tag)::value;
      if constexpr (chained) {
        // every wave holds its step-1 fragments, so both slots are free
        wait_lgkm0();
        bare_barrier();
        __builtin_amdgcn_sched_barrier(0);
      }
      const LoadPlan<kGated> nlp(chain.next, smem, wave, lane, 2);
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        if constexpr (load2) {
          if (q < 6) lp.issue(cur, kt + 2, 10 + q);
        }
        if constexpr (chained) {
          // all of stage 0, then all of stage 1.  Stage 1 is loaded even
          // when K has one stage (slot 1 is then never read; past the end of
          // the buffer the loads return zeros), so the count of operations
          // in flight behind the epilogue's operand loads is the same on
          // every path and the compiler's waits for them do not stall.
          if (q < 8) {
            nlp.issue(0, 0, 2 * q);
            nlp.issue(0, 0, 2 * q + 1);
          } else {
            nlp.issue(1, 1, 2 * q - 16);
            nlp.issue(1, 1, 2 * q - 15);
          }
        }
        const int j = q >> 2, i0 = (q & 3) * 2;
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
        wait_vm16();
      else
        wait_vm0();
      bare_barrier();
    }
    // stage nk-2 (no stage loads of its own): the epilogue operand loads go
    // out after B2's wait, so that wait does not include them
    if constexpr (!load2 && next) pre();
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int q = 0; q < 16; ++q) {  // R3
      if constexpr (next) read_frag<kGated>(fa, q, nbase, xfrag[0], wfrag[0]);
      const int j = 4 + (q >> 2), i0 = (q & 3) * 2;
#pragma unroll
      for (int i = i0; i < i0 + 2; ++i) mfma16x16x32_acc(acc.v[j][i], fb.b[j], fb.a[i]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  for (int kt = 0; kt < nk - 2; ++kt) stage(kt, std::true_type{}, std::true_type{});
  if (nk >= 2) stage(nk - 2, std::false_type{}, std::true_type{});
  stage(nk - 1, std::false_type{}, std::false_type{});
  settle_accumulators<Acc, 8, 8>(acc);
}

}  // namespace coda
