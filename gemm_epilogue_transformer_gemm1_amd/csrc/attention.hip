// Causal grouped-query attention forward: the attention core of the full
// transformer-layer forward.  The page's method re-parameterises every
// operator of the layer except attention (section "What CODA can do"); this
// kernel is the plain attention between the QKV+RoPE GEMM and the output
// projection GEMM, written for gfx950.  Its running statistics are the
// page's stateful max / sum-exp transform (section "Five building blocks and
// a LEGO language"), the same ones as the LM head's block log-sum-exp.
//
//   o_i = sum_{j <= i} softmax_j(q_i . k_j / sqrt(64)) v_j   per q head,
//   keys and values of kv head h / (n_q / n_kv), within one sequence.
//
// Design (one workgroup per (sequence, q head, 128 queries); heads of 64 or
// 128 features):
//   * each wave owns kQW queries of the block (64 with heads of 64, 32 with
//     heads of 128, so 2 or 4 waves) in 16-query subtiles; its q fragments stay
//     in registers, so every K and V fragment read from LDS feeds kQW / 16
//     MFMAs;
//   * key steps of 64 through two LDS stages: the K and V rows of a step are
//     loaded straight into LDS (buffer_load ... lds, no register staging),
//     row-major with a 16-byte chunk swizzle (chunk c of row r at slot
//     c ^ (r mod chunks per row)); the step after next is in flight while a
//     step computes, with one barrier per step;
//   * S^T = K Q^T on v_mfma_f32_16x16x32_bf16 with K as the first operand:
//     lane L holds the scores of keys 4 (L / 16) + r of query L % 16, so a
//     query's row max is a lane-local max and two lane-group exchanges
//     (v_permlane32_swap, v_permlane16_swap);
//   * P V as O^T = V^T P^T: lane L's eight P values (keys 4 g .. 4 g + 3 and
//     16 + 4 g .. 16 + 4 g + 3 of a 32-key chunk, g = L / 16) are exactly the
//     second operand of the MFMA for its query, so P never leaves the lane;
//     the V^T operand comes from the row-major V rows through the transposing
//     LDS read ds_read_b64_tr_b16 (per 16-lane group, result lane i, element j
//     is element i % 4 of source lane 4 j + i / 4), in the same key order;
//   * online softmax in base 2 with the scale folded into one FMA:
//     p = 2^(s log2(e) / sqrt(hd) - m).  The reference m is raised only when a
//     row's max exceeds it by more than 2^8 (one wave-uniform test per step),
//     so the rescale of O and of the sums by 2^(m_old - m_new) is rare; p stays
//     below 2^8, well inside bf16 and fp32 range, and O / sum does not depend
//     on m;
//   * causal: a wave skips the key steps after its queries; the step that
//     holds them masks keys past each query to -inf;
//   * workgroups are launched longest first (the query blocks with the most
//     key steps), all heads and sequences of a block position together, the
//     q heads that share a kv head on one XCD.
#include "coda_device.hpp"
#include "launch.hpp"

namespace coda {

constexpr int kAttnQB = 128;              // queries per workgroup
constexpr int kAttnKB = 64;               // keys per step
constexpr float kLazyGrow = 8.0f;         // log2 headroom before the reference max is raised

typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;

struct AttnArgs {
  const uint16_t* qkv;  // [M, C], C = (n_q + 2 n_kv) hd, q | k | v
  uint16_t* o;          // [M, n_q hd]
  int M, L, nq, nkv;
};

// max over lanes l, l ^ 16, l ^ 32, l ^ 48
__device__ __forceinline__ float max_lane_groups(float v) {
  const uint32_t b = __builtin_bit_cast(uint32_t, v);
  const auto x = __builtin_amdgcn_permlane32_swap(b, b, false, false);
  v = fmaxf(__builtin_bit_cast(float, x[0]), __builtin_bit_cast(float, x[1]));
  const uint32_t c = __builtin_bit_cast(uint32_t, v);
  const auto y = __builtin_amdgcn_permlane16_swap(c, c, false, false);
  return fmaxf(__builtin_bit_cast(float, y[0]), __builtin_bit_cast(float, y[1]));
}

// s_waitcnt vmcnt(n), expcnt and lgkmcnt not waited for
template <int N>
__device__ __forceinline__ void attn_wait_vm() {
  static_assert(N >= 0 && N < 16, "small counts only");
  __builtin_amdgcn_s_waitcnt(0x0F70 | N);
}

// Barrier without the release fence of __syncthreads, which would also wait
// for the loads of the step after next; the signal fences keep the compiler
// from moving LDS accesses across it.
__device__ __forceinline__ void attn_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

template <int kHd>
struct AttnShape {
  static constexpr int kQW = kHd == 64 ? 64 : 32;          // queries per wave
  static constexpr int kQS = kQW / 16;                     // query subtiles per wave
  static constexpr int kWaves = kAttnQB / kQW;             // waves per workgroup
  static constexpr int kRowB = 2 * kHd;                    // bytes per K / V row
  static constexpr int kChunks = kRowB / 16;               // 16-byte chunks per row
  static constexpr int kBlock = kAttnKB * kRowB;           // K (or V) rows of one step
  static constexpr int kStage = 2 * kBlock;                // K rows, then V rows
  static constexpr int kRowsPerLoad = 1024 / kRowB;        // rows per wave instruction
  static constexpr int kLoads = kBlock / 1024 / kWaves;    // K (and V) instructions per wave
  static_assert(kLoads == 4, "each wave moves four K and four V instructions per step");
};

template <int kHd>
__device__ __forceinline__ int attn_swz(int row, int chunk) {
  return row * AttnShape<kHd>::kRowB + ((chunk ^ (row & (AttnShape<kHd>::kChunks - 1))) << 4);
}

template <int kHd>
__global__ __launch_bounds__(64 * AttnShape<kHd>::kWaves, 2) void k_attention_fwd(AttnArgs a) {
  using S = AttnShape<kHd>;
  constexpr int kQS = S::kQS, kQW = S::kQW;
  __shared__ __attribute__((aligned(1024))) char smem[2 * S::kStage];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int g4 = lane >> 4, r16 = lane & 15;
  const int nqb = a.L / kAttnQB;
  const int grp = a.nq / a.nkv;             // q heads per kv head
  const int npairs = a.nkv * (a.M / a.L);   // (kv head, sequence) pairs
  const int units = npairs * grp;           // workgroups per query-block position
  // longest first: every (q head, sequence) of the last query block, then
  // the next-to-last, ...  When the pairs split evenly over the 8 XCDs
  // (workgroup i runs on XCD i % 8), XCD x takes the pairs p = x mod 8 with
  // all their q heads at every block position, so the K and V rows of a pair
  // are read through one L2.
  const int qb = nqb - 1 - (int)blockIdx.x / units;
  const int t = (int)blockIdx.x % units;
  int pair, gi;
  if (npairs % 8 == 0) {
    pair = ((t >> 3) / grp) * 8 + (t & 7);
    gi = (t >> 3) % grp;
  } else {
    pair = t / grp;
    gi = t % grp;
  }
  const int kvh = pair % a.nkv, seq = pair / a.nkv;
  const int h = kvh * grp + gi;
  const int C = (a.nq + 2 * a.nkv) * kHd;
  const size_t row0 = (size_t)seq * a.L;  // first row of the sequence
  const int q0 = qb * kAttnQB;            // first query of the block (sequence position)
  const int qmin = q0 + kQW * wave;       // this wave's first query

  // q fragments: subtile qs, 32-feature chunk c: query qmin + 16 qs + L % 16,
  // features 32 c + 8 (L / 16) .. + 7
  bf16x8_t qf[kQS][kHd / 32];
#pragma unroll
  for (int qs = 0; qs < kQS; ++qs)
#pragma unroll
    for (int c = 0; c < kHd / 32; ++c)
      qf[qs][c] = *(const bf16x8_t*)(a.qkv + (row0 + qmin + 16 * qs + r16) * C +
                                     (size_t)h * kHd + 32 * c + 8 * g4);

  // loads of one step: wave w fills rows 64 w / kWaves .. of the K and of the
  // V block, kRowsPerLoad rows (1 KiB) per instruction; the lane writing LDS
  // slot s of row r fetches chunk s ^ (r mod kChunks) of that row
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(a.qkv + row0 * C, (uint32_t)a.L * C * 2u);
  uint32_t koff[4], voff[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int lr = (kAttnKB / S::kWaves) * wave + S::kRowsPerLoad * q + lane / S::kChunks;
    const int c = (lane % S::kChunks) ^ (lr & (S::kChunks - 1));
    koff[q] = (uint32_t)(lr * C + (a.nq + kvh) * kHd) * 2u + 16u * c;
    voff[q] = (uint32_t)(lr * C + (a.nq + a.nkv + kvh) * kHd) * 2u + 16u * c;
  }
  auto issue = [&](int slot, int kb) {
    const uint32_t soff = (uint32_t)kb * kAttnKB * C * 2u;
    char* kl = smem + slot * S::kStage + wave * (kAttnKB / S::kWaves) * S::kRowB;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      load16_to_lds(rs, kl + q * 1024, koff[q], soff);
      load16_to_lds(rs, kl + S::kBlock + q * 1024, voff[q], soff);
    }
  };
  // transposing-read address (bytes into a V block) of this lane for feature
  // subtile dt and 32-key chunk c, half hf (keys +0 / +16): source lane
  // 4 j + q of group g points at row 32 c + 16 hf + 4 g + j, features
  // 16 dt + 4 q .. + 3
  const int tr_j = r16 >> 2, tr_q = lane & 3;
  auto tr_off = [&](int dt, int c, int hf) {
    const int row = 32 * c + 16 * hf + 4 * g4 + tr_j;
    const int byte = 32 * dt + 8 * tr_q;
    return attn_swz<kHd>(row, byte >> 4) | (byte & 15);
  };

  // log2(e) / sqrt(hd)
  const float kC = 1.4426950408889634f * (kHd == 64 ? 0.125f : 0.08838834764831845f);
  float mref[kQS], lrun[kQS];  // reference max (base-2 units), this lane's share of the sum
  f32x4_t ot[kHd / 16][kQS];   // O^T: feature subtile dt, query subtile qs
#pragma unroll
  for (int qs = 0; qs < kQS; ++qs) {
    mref[qs] = -INFINITY;
    lrun[qs] = 0.f;
#pragma unroll
    for (int dt = 0; dt < kHd / 16; ++dt) ot[dt][qs] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  const int nkb = (q0 + kAttnQB) / kAttnKB;  // key steps up to the block's last query
  issue(0, 0);
  if (nkb > 1) {
    issue(1, 1);
    attn_wait_vm<8>();
  } else {
    attn_wait_vm<0>();
  }
  attn_barrier();
  for (int kb = 0; kb < nkb; ++kb) {
    const int k0 = kb * kAttnKB;
    if (k0 <= qmin + kQW - 1) {  // wave-uniform: steps after the wave's queries are skipped
      const char* ks = smem + (kb & 1) * S::kStage;
      __attribute__((address_space(3))) char* vs =
          (__attribute__((address_space(3))) char*)(ks + S::kBlock);
      // S^T = K Q^T: st[kt][qs] lane L, register r: key k0 + 16 kt + 4 g + r,
      // query qmin + 16 qs + L % 16 (raw scores)
      f32x4_t st[4][kQS];
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        const int row = 16 * kt + r16;
#pragma unroll
        for (int qs = 0; qs < kQS; ++qs) st[kt][qs] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < kHd / 32; ++c) {
          const bf16x8_t kf = *(const bf16x8_t*)(ks + attn_swz<kHd>(row, 4 * c + g4));
#pragma unroll
          for (int qs = 0; qs < kQS; ++qs) st[kt][qs] = mfma16x16x32(kf, qf[qs][c], st[kt][qs]);
        }
      }
      if (k0 + kAttnKB - 1 > qmin) {  // the step holds the wave's queries: mask later keys
#pragma unroll
        for (int qs = 0; qs < kQS; ++qs) {
          const int rel = qmin + 16 * qs + r16 - k0 - 4 * g4;  // key offset limit in this lane
#pragma unroll
          for (int kt = 0; kt < 4; ++kt)
#pragma unroll
            for (int r = 0; r < 4; ++r)
              if (16 * kt + r > rel) st[kt][qs][r] = -INFINITY;
        }
      }
      float mnew[kQS];
      bool grow = false;
#pragma unroll
      for (int qs = 0; qs < kQS; ++qs) {
        float mx = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int r = 0; r < 4; ++r) mx = fmaxf(mx, st[kt][qs][r]);
        mnew[qs] = max_lane_groups(mx) * kC;
        grow |= mnew[qs] > mref[qs] + kLazyGrow;
      }
      if (__builtin_amdgcn_ballot_w64(grow) != 0) {  // wave-uniform: raise the reference
#pragma unroll
        for (int qs = 0; qs < kQS; ++qs) {
          const float m = fmaxf(mref[qs], mnew[qs]);
          const float alpha = __builtin_amdgcn_exp2f(mref[qs] - m);
          mref[qs] = m;
          lrun[qs] *= alpha;
#pragma unroll
          for (int dt = 0; dt < kHd / 16; ++dt) ot[dt][qs] *= alpha;
        }
      }
#pragma unroll
      for (int qs = 0; qs < kQS; ++qs) {
        const float nm = -mref[qs];
        float ls = 0.f;
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(st[kt][qs][r], kC, nm));
            st[kt][qs][r] = p;
            ls += p;
          }
        lrun[qs] += ls;
      }
      // O^T += V^T P^T over two 32-key chunks
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        bf16x8_t pf[kQS];
#pragma unroll
        for (int qs = 0; qs < kQS; ++qs) {
          const f32x4_t& lo = st[2 * c][qs];
          const f32x4_t& hi = st[2 * c + 1][qs];
          pf[qs] = bf16x8_t{(__bf16)lo[0], (__bf16)lo[1], (__bf16)lo[2], (__bf16)lo[3],
                            (__bf16)hi[0], (__bf16)hi[1], (__bf16)hi[2], (__bf16)hi[3]};
        }
#pragma unroll
        for (int dt = 0; dt < kHd / 16; ++dt) {
          const i16x4_t va = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(vs + tr_off(dt, c, 0)));
          const i16x4_t vb = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(vs + tr_off(dt, c, 1)));
          const u32x2_t wa = __builtin_bit_cast(u32x2_t, va), wb = __builtin_bit_cast(u32x2_t, vb);
          const bf16x8_t vf = __builtin_bit_cast(bf16x8_t, u32x4_t{wa.x, wa.y, wb.x, wb.y});
#pragma unroll
          for (int qs = 0; qs < kQS; ++qs) ot[dt][qs] = mfma16x16x32(vf, pf[qs], ot[dt][qs]);
        }
      }
    }
    if (kb + 1 < nkb) attn_wait_vm<0>();  // this wave's part of the next step has landed
    attn_barrier();                       // ... every wave's, and this step's slot is free
    if (kb + 2 < nkb) issue(kb & 1, kb + 2);
  }

  // o[query][h hd + 16 dt + 4 g + r] = O^T / sum
#pragma unroll
  for (int qs = 0; qs < kQS; ++qs) {
    const float inv = 1.0f / sum_over_lane_groups(lrun[qs]);
    uint16_t* orow = a.o + (row0 + qmin + 16 * qs + r16) * (size_t)(a.nq * kHd) +
                     (size_t)h * kHd + 4 * g4;
#pragma unroll
    for (int dt = 0; dt < kHd / 16; ++dt) {
      const f32x4_t& v = ot[dt][qs];
      *(u32x2_t*)(orow + 16 * dt) = pack_bf16x4(v[0] * inv, v[1] * inv, v[2] * inv, v[3] * inv);
    }
  }
}

hipError_t launch_attention_fwd(const uint16_t* qkv, uint16_t* o, int M, int L, int nq, int nkv,
                                int head_dim, hipStream_t stream) {
  const int blocks = (L / kAttnQB) * nq * (M / L);
  const AttnArgs args{qkv, o, M, L, nq, nkv};
  if (head_dim == 128)
    hipLaunchKernelGGL(k_attention_fwd<128>, dim3(blocks), dim3(64 * AttnShape<128>::kWaves), 0,
                       stream, args);
  else
    hipLaunchKernelGGL(k_attention_fwd<64>, dim3(blocks), dim3(64 * AttnShape<64>::kWaves), 0,
                       stream, args);
  return hipGetLastError();
}

}  // namespace coda
