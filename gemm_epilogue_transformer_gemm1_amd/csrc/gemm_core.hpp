// The fixed GEMM mainloop every epilogue program runs on (page section
// "CODA: the secret in the epilogue": a GEMM is a blocked multiply-accumulate
// mainloop followed by an epilogue that still holds the output tile in
// registers; section "Five building blocks and a LEGO language": the mainloop
// stays fixed and epilogue primitives are composed on top of it).
//
// gfx950 design (one 256-thread workgroup per CU, 4 waves in a 2x2 grid):
//   * block tile 256 token rows x 256 weight rows, reduction depth 64 per
//     stage; two LDS stages of 64 KiB (token tile 32 KiB + weight tile 32 KiB);
//   * global -> LDS with buffer_load ... lds (16 B per lane, no VGPR staging);
//     each LDS row holds 64 bf16 (128 B) as 8 chunks of 16 B, chunk c of row r
//     stored at chunk slot c ^ (r & 7) so that the 16 lanes reading one MFMA
//     fragment hit distinct banks;
//   * v_mfma_f32_16x16x32_bf16 with the WEIGHT fragment as the first operand
//     and the TOKEN fragment as the second, so the accumulator is C^T: lane L,
//     register v of a 16x16 tile holds output feature 4*(L/16)+v of token L%16.
//     A lane therefore owns 4 consecutive features of one token, which makes
//     per-token reductions (RMS partials, log-sum-exp) mostly lane-local;
//   * each wave owns a 128-token x 128-weight-row quarter: 8x8 tiles of 16x16,
//     256 fp32 accumulators per lane.
#pragma once

#include <type_traits>

#include "coda_device.hpp"

namespace coda {

constexpr int kThreads = 256;
constexpr int kBM = 256;                      // token rows per block
constexpr int kBN = 256;                      // weight rows per block
constexpr int kBK = 64;                       // bf16 reduction depth per stage
constexpr int kRowBytes = kBK * 2;            // 128 B per LDS row
constexpr int kXBytes = kBM * kRowBytes;      // 32 KiB token tile
constexpr int kWBytes = kBN * kRowBytes;      // 32 KiB weight tile
constexpr int kStageBytes = kXBytes + kWBytes;
constexpr int kSmemBytes = 2 * kStageBytes;   // 128 KiB

// Accumulators of one wave: acc[j][i] is the 16x16 tile of weight-row
// subtile j and token subtile i.
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

// Weight-tile row (within the 256-row LDS weight tile) of this wave's
// n-subtile j.  Plain GEMMs: the wave owns rows [wn*128, wn*128+128).  Gated
// (SwiGLU) GEMMs: LDS rows [0,128) hold gate rows and [128,256) the matching
// up rows, and the wave owns gate rows [wn*64, +64) (subtiles 0..3) and the
// same up rows (subtiles 4..7), so gate and up values of one output element
// sit in the same lane and register.
template <bool kGated>
__device__ __forceinline__ constexpr int wrow_of_subtile(int j) {
  return kGated ? (j < 4 ? j * 16 : 128 + (j - 4) * 16) : j * 16;
}

template <bool kGated>
__device__ __forceinline__ int wave_wrow_base(int wn) {
  return kGated ? wn * 64 : wn * 128;
}

// Operand sources of one block.
struct MainloopSrc {
  const uint16_t* X;   // token operand [M, K] bf16
  const uint16_t* W0;  // weight rows for LDS rows [0,256) (plain) or [0,128) (gated)
  const uint16_t* W1;  // gated only: weight rows for LDS rows [128,256)
  int M;               // token rows of X
  int Nw;              // rows of each weight matrix
  int K;               // reduction length, multiple of 64
  int m0;              // first token row of the block
  int n0;              // first weight row of the block (per weight matrix)
};

// One k32 step's MFMA operands for a wave: 8 token fragments and 8 weight
// fragments (16 B per lane each).
struct Frags {
  bf16x8_t a[8];  // token subtiles i = 0..7
  bf16x8_t b[8];  // weight subtiles j = 0..7
};

template <bool kGated>
__device__ __forceinline__ void read_frags(Frags& f, const char* stage, uint32_t xo, uint32_t wo) {
#pragma unroll
  for (int i = 0; i < 8; ++i) f.a[i] = *(const bf16x8_t*)(stage + xo + i * 16 * kRowBytes);
#pragma unroll
  for (int j = 0; j < 8; ++j)
    f.b[j] = *(const bf16x8_t*)(stage + wo + wrow_of_subtile<kGated>(j) * kRowBytes);
}

template <int J0, int J1>
__device__ __forceinline__ void mfma_rows(Acc& acc, const Frags& f) {
#pragma unroll
  for (int j = J0; j < J1; ++j)
#pragma unroll
    for (int i = 0; i < 8; ++i) acc.v[j][i] = mfma16x16x32(f.b[j], f.a[i], acc.v[j][i]);
}

// Scheduling masks of __builtin_amdgcn_sched_group_barrier.
constexpr int kSchedMfma = 0x008;
constexpr int kSchedVmem = 0x010;
constexpr int kSchedDsRead = 0x100;

template <bool kGated>
__device__ __forceinline__ void mainloop_bf16(Acc& acc, char* smem, const MainloopSrc& s) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int wm = wave >> 1, wn = wave & 1;

  // ---- global -> LDS load plan: wave w fills LDS rows [w*64, w*64+64) of
  // both tiles with 8 instructions each (8 rows x 128 B per instruction).
  const uint32_t xbytes = (uint32_t)s.M * (uint32_t)s.K * 2u;
  const uint32_t wbytes = (uint32_t)s.Nw * (uint32_t)s.K * 2u;
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(s.X, xbytes);
  const uint16_t* wsrc = (kGated && wave >= 2) ? s.W1 : s.W0;
  const __amdgpu_buffer_rsrc_t wr = make_rsrc(wsrc, wbytes);
  const int wrow_shift = (kGated && wave >= 2) ? 128 : 0;
  uint32_t xoff[8], woff[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int lr = wave * 64 + q * 8 + (lane >> 3);
    const int lc = (lane & 7) ^ (lr & 7);
    const int gx = min(s.m0 + lr, s.M - 1);
    const int gw = min(s.n0 + lr - wrow_shift, s.Nw - 1);
    xoff[q] = (uint32_t)gx * (uint32_t)s.K * 2u + (uint32_t)lc * 16u;
    woff[q] = (uint32_t)gw * (uint32_t)s.K * 2u + (uint32_t)lc * 16u;
  }
  char* x_lds_wave = smem + wave * 64 * kRowBytes;
  char* w_lds_wave = smem + kXBytes + wave * 64 * kRowBytes;

  auto issue_stage = [&](int stage, int kt) {  // prologue only
    const uint32_t soff = (uint32_t)kt * kRowBytes;
    char* xs = x_lds_wave + stage * kStageBytes;
    char* ws = w_lds_wave + stage * kStageBytes;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      load16_to_lds(xr, xs + q * 8 * kRowBytes, xoff[q], soff);
      load16_to_lds(wr, ws + q * 8 * kRowBytes, woff[q], soff);
    }
  };

  // ---- LDS -> register fragment plan.  Lane reads row (base + lane%16),
  // logical chunk 4*step + lane/16, stored at slot chunk ^ (row & 7) where
  // row & 7 == lane & 7 because every fragment base is a multiple of 16.
  const int r16 = lane & 15;
  uint32_t xfrag[2], wfrag[2];
#pragma unroll
  for (int st = 0; st < 2; ++st) {
    const uint32_t slot = (uint32_t)(((st * 4) + (lane >> 4)) ^ (lane & 7)) * 16u;
    xfrag[st] = (uint32_t)(wm * 128 + r16) * kRowBytes + slot;
    wfrag[st] = (uint32_t)kXBytes + (uint32_t)(wave_wrow_base<kGated>(wn) + r16) * kRowBytes + slot;
  }

#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int i = 0; i < 8; ++i) acc.v[j][i] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // Software pipeline over stages kt (two k32 steps each; fragment register
  // sets fa / fb; LDS stages alternate, stage kt lives in slot kt & 1):
  //   [fa = step 0 of kt already in registers; slot kt&1 holds kt, the other
  //    slot is receiving kt+1]
  //   R1: 16 x {one fb fragment read (step 1 of kt), 4 MFMAs on fa}
  //   B1: barrier -- every wave has its step-1 fragments, so slot kt&1 is free
  //   R2: 16 x {one 1 KiB load of stage kt+2 into slot kt&1, 2 MFMAs on fb}
  //   B2: wait for this wave's stage kt+1 loads only (those of kt+2 stay in
  //       flight), barrier (stage kt+1 complete everywhere)
  //   R3: 16 x {one fa fragment read (step 0 of kt+1), 2 MFMAs on fb}
  // A stage's loads are therefore issued about one and a half stages of MFMA
  // work before they are needed.  Every group is fenced with
  // sched_barrier(0) so the compiler keeps this interleaving; the barriers are
  // plain s_barrier (no release fence, which would also drain the loads still
  // in flight) after the explicit LDS-read wait they need.
  const int nk = s.K / kBK;
  Frags fa, fb;
  issue_stage(0, 0);
  if (nk > 1) {
    issue_stage(1, 1);
    __builtin_amdgcn_s_waitcnt(0x4F70);  // vmcnt(16): stage 0 landed
  } else {
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  }
  __syncthreads();
  read_frags<kGated>(fa, smem, xfrag[0], wfrag[0]);

  auto stage = [&](int kt, auto load_tag, auto next_tag) {
    constexpr bool load2 = decltype(load_tag)::value;  // stage kt+2 exists
    constexpr bool next = decltype(next_tag)::value;   // stage kt+1 exists
    const int cur = kt & 1;
    const char* base = smem + cur * kStageBytes;
    const char* nbase = smem + (cur ^ 1) * kStageBytes;
    const uint32_t soff = (uint32_t)(kt + 2) * kRowBytes;
    char* xs = x_lds_wave + cur * kStageBytes;
    char* ws = w_lds_wave + cur * kStageBytes;
    __builtin_amdgcn_sched_barrier(0);
    // R1
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      if (q < 8)
        fb.a[q] = *(const bf16x8_t*)(base + xfrag[1] + q * 16 * kRowBytes);
      else
        fb.b[q - 8] =
            *(const bf16x8_t*)(base + wfrag[1] + wrow_of_subtile<kGated>(q - 8) * kRowBytes);
      const int j = q >> 1, i0 = (q & 1) * 4;
#pragma unroll
      for (int i = i0; i < i0 + 4; ++i) mfma16x16x32_acc(acc.v[j][i], fa.b[j], fa.a[i]);
      __builtin_amdgcn_sched_barrier(0);
    }
    // B1
    if constexpr (load2) {
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): own step-1 reads done
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      __builtin_amdgcn_s_barrier();
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      __builtin_amdgcn_sched_barrier(0);
    }
    // R2
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      if constexpr (load2) {
        if (q < 8)
          load16_to_lds(xr, xs + q * 8 * kRowBytes, xoff[q], soff);
        else
          load16_to_lds(wr, ws + (q - 8) * 8 * kRowBytes, woff[q - 8], soff);
      }
      const int j = q >> 2, i0 = (q & 3) * 2;
#pragma unroll
      for (int i = i0; i < i0 + 2; ++i) mfma16x16x32_acc(acc.v[j][i], fb.b[j], fb.a[i]);
      __builtin_amdgcn_sched_barrier(0);
    }
    // B2
    if constexpr (next) {
      if constexpr (load2)
        __builtin_amdgcn_s_waitcnt(0x4F70);  // vmcnt(16): stage kt+1 landed, kt+2 in flight
      else
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      __builtin_amdgcn_s_barrier();
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
    }
    __builtin_amdgcn_sched_barrier(0);
    // R3
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      if constexpr (next) {
        if (q < 8)
          fa.a[q] = *(const bf16x8_t*)(nbase + xfrag[0] + q * 16 * kRowBytes);
        else
          fa.b[q - 8] =
              *(const bf16x8_t*)(nbase + wfrag[0] + wrow_of_subtile<kGated>(q - 8) * kRowBytes);
      }
      const int j = 4 + (q >> 2), i0 = (q & 3) * 2;
#pragma unroll
      for (int i = i0; i < i0 + 2; ++i) mfma16x16x32_acc(acc.v[j][i], fb.b[j], fb.a[i]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  for (int kt = 0; kt < nk - 2; ++kt) stage(kt, std::true_type{}, std::true_type{});
  if (nk >= 2) stage(nk - 2, std::false_type{}, std::true_type{});
  stage(nk - 1, std::false_type{}, std::false_type{});
  // The MFMAs are inline asm, so the compiler's hazard recognizer does not
  // see their accumulator writes and would happily read an accumulator right
  // after the MFMA that writes it.  Give the last MFMAs time to retire, then
  // re-define every accumulator with an empty asm statement ordered after the
  // wait states: every epilogue read depends on it and so comes later.
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int i = 0; i < 8; ++i) asm volatile("" : "+a"(acc.v[j][i]));
  __builtin_amdgcn_sched_barrier(0);
}

}  // namespace coda
