// Device helpers shared by the gfx950 kernels of libcoda.
//
// Citations name sections of the news page "CODA: New Research Optimizes
// Transformer Training with GEMM-Epilogue Programming" (KuCoin news flash).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace coda {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

typedef __attribute__((address_space(3))) void lds_void_t;

// Raw buffer resource over `bytes` bytes starting at `base` (gfx9 family
// descriptor: stride 0, raw addressing).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

// 16 bytes per lane from global memory straight into LDS.  The LDS
// destination of lane L is lds_base + 16 * L (the wave writes 1 KiB
// contiguously); the global source is rsrc + voffset + soffset.
__device__ __forceinline__ void load16_to_lds(__amdgpu_buffer_rsrc_t rsrc, void* lds_base,
                                              uint32_t voffset, uint32_t soffset) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void_t*)lds_base, 16, voffset, soffset, 0,
                                           0);
}

// Offset that is out of range of every buffer built by make_rsrc (all are
// smaller than 2 GiB): a raw-buffer store at this offset is dropped by the
// hardware range check, so masked lanes can issue the same store
// instructions as the others.
constexpr uint32_t kOobOffset = 0x80000000u;

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// 16 bytes per lane to rsrc + voffset (dropped if out of range).
__device__ __forceinline__ void store16(__amdgpu_buffer_rsrc_t rsrc, u32x4_t v, uint32_t voffset) {
  __builtin_amdgcn_raw_buffer_store_b128(v, rsrc, voffset, 0, 0);
}

// A lane of 16-lane group g holds, for one token row, the runs of 4 features
// 16 j0 + 4 g + 0..3 (pk[0]) and 16 (j0 + 1) + 4 g + 0..3 (pk[1]).  Groups g
// and g ^ 1 swap one run, so each lane stores 8 contiguous features with one
// 16-byte store: features 16 j0 + 8 (g / 2) + 0..7 for even g, the same in
// subtile j0 + 1 for odd g.  `voffset` is the byte offset of that run (or
// kOobOffset).  All 64 lanes must take part (the swap is a lane shuffle).
__device__ __forceinline__ void store16_exchanged(__amdgpu_buffer_rsrc_t rsrc, const u32x2_t (&pk)[2],
                                                  bool godd, uint32_t voffset) {
  const u32x2_t sd = godd ? pk[0] : pk[1];
  const u32x2_t rx = {(unsigned)__shfl_xor((int)sd.x, 16, 64),
                      (unsigned)__shfl_xor((int)sd.y, 16, 64)};
  store16(rsrc, godd ? u32x4_t{rx.x, rx.y, pk[1].x, pk[1].y} : u32x4_t{pk[0].x, pk[0].y, rx.x, rx.y},
          voffset);
}

// 8 bytes per lane to rsrc + voffset (dropped if voffset + 8 > the range).
__device__ __forceinline__ void store8(__amdgpu_buffer_rsrc_t rsrc, u32x2_t v, uint32_t voffset) {
  __builtin_amdgcn_raw_buffer_store_b64(v, rsrc, voffset, 0, 0);
}

__device__ __forceinline__ f32x4_t mfma16x16x32(const bf16x8_t& a, const bf16x8_t& b,
                                                const f32x4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// In-place accumulate with the accumulator pinned to AGPRs (tied operand), so
// the register allocator cannot rename accumulators across loop iterations.
__device__ __forceinline__ void mfma16x16x32_acc(f32x4_t& c, const bf16x8_t& a,
                                                 const bf16x8_t& b) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
}

// e4m3 MFMA with a 16x16 output tile and a 128-deep reduction (32 bytes of
// each operand per lane); same output layout as the 16x16 bf16 form.
__device__ __forceinline__ void mfma16x16x128_f8_acc(f32x4_t& c, const i32x8_t& a,
                                                    const i32x8_t& b) {
  asm volatile("v_mfma_f32_16x16x128_f8f6f4 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
}

// Round-to-nearest-even float -> bf16 bits for four values, packed in 8 bytes.
__device__ __forceinline__ u32x2_t pack_bf16x4(float a, float b, float c, float d) {
  bf16x4_t v = {(__bf16)a, (__bf16)b, (__bf16)c, (__bf16)d};
  return __builtin_bit_cast(u32x2_t, v);
}

// Four floats -> four OCP E4M3FN codes (round to nearest even), saturating:
// magnitudes above 448 are clamped to 448 first; NaN stays NaN.
__device__ __forceinline__ uint32_t pack_e4m3x4_sat(float a, float b, float c, float d) {
  const float lim = 448.0f;
  a = __builtin_fminf(__builtin_fmaxf(a, -lim), lim);
  b = __builtin_fminf(__builtin_fmaxf(b, -lim), lim);
  c = __builtin_fminf(__builtin_fmaxf(c, -lim), lim);
  d = __builtin_fminf(__builtin_fmaxf(d, -lim), lim);
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

__device__ __forceinline__ float bf16_to_f32(uint16_t bits) {
  return __builtin_bit_cast(float, (uint32_t)bits << 16);
}

// Unpack 4 bf16 (8 bytes) to floats.
__device__ __forceinline__ void unpack_bf16x4(u32x2_t v, float* f) {
  f[0] = __builtin_bit_cast(float, v.x << 16);
  f[1] = __builtin_bit_cast(float, v.x & 0xffff0000u);
  f[2] = __builtin_bit_cast(float, v.y << 16);
  f[3] = __builtin_bit_cast(float, v.y & 0xffff0000u);
}

// Sum over the four 16-lane groups of a wave (lanes l, l^16, l^32, l^48).
__device__ __forceinline__ float sum_over_lane_groups(float v) {
  v += __shfl_xor(v, 16, 64);
  v += __shfl_xor(v, 32, 64);
  return v;
}

__device__ __forceinline__ float max_over_lane_groups(float v) {
  v = fmaxf(v, __shfl_xor(v, 16, 64));
  v = fmaxf(v, __shfl_xor(v, 32, 64));
  return v;
}

// silu(z) = z / (1 + e^-z), with the hardware exp and reciprocal; for very
// negative z, e^-z = inf and the reciprocal gives 0.
__device__ __forceinline__ float silu_f32(float z) {
  return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z));
}

}  // namespace coda
