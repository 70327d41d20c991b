// Device helpers: fp16 bit conversions, the exact group decode, dot products
// and wavefront reductions for gfx950 (wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "aqlm_internal.hpp"

namespace aqlm {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef uint16_t u16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef float float16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// Streaming 16-byte accesses that bypass cache retention (data used once).
__device__ __forceinline__ uint4 load_nt16(const void *p) {
  const u32x4_t v = __builtin_nontemporal_load(static_cast<const u32x4_t *>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void store_nt16(void *p, const uint4 &w) {
  u32x4_t v = {w.x, w.y, w.z, w.w};
  __builtin_nontemporal_store(v, static_cast<u32x4_t *>(p));
}

// Raw buffer resources (gfx9 descriptor word 3 = 0x00020000): loads at
// offsets outside [0, num_records) return zero instead of faulting, which lets
// bounds-checked loads stay branch-free.
typedef __amdgpu_buffer_rsrc_t Rsrc;
__device__ __forceinline__ Rsrc make_rsrc(const void *base, uint32_t num_bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)num_bytes,
                                           0x00020000);
}
// a 2-byte store; dropped by the hardware where off is out of range
__device__ __forceinline__ void buf_store_u16(Rsrc r, uint32_t off, uint16_t v) {
  __builtin_amdgcn_raw_buffer_store_b16(v, r, off, 0, 0);
}
__device__ __forceinline__ uint4 buf_load16(Rsrc r, uint32_t off) {
  const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}
// streaming variant (non-temporal: data read once)
__device__ __forceinline__ uint4 buf_load16_nt(Rsrc r, uint32_t off) {
  const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 2);
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 buf_load8(Rsrc r, uint32_t off) {
  typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
  const u32x2_t v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
  return make_uint2(v.x, v.y);
}
__device__ __forceinline__ uint32_t buf_load4(Rsrc r, uint32_t off) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}
// 16-bit load zero-extended into its own 32-bit register (kept unpacked so a
// refill never has to merge into a register another value lives in).
__device__ __forceinline__ uint32_t buf_load_u16(Rsrc r, uint32_t off) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
}
// fp16 bits in the low half of a register -> float, without masking the
// register first (the conversion reads only bits 0..15).
__device__ __forceinline__ float low_half_to_float(uint32_t reg) {
  float f;
  asm("v_cvt_f32_f16 %0, %1" : "=v"(f) : "v"(reg));
  return f;
}

__device__ __forceinline__ float h2f(uint32_t bits16) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(bits16)));
}

// float32 -> float16, round to nearest even, subnormals kept, overflow to inf
// (v_cvt_f16_f32 under the default rounding and denormal modes).
__device__ __forceinline__ uint32_t f2h(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<_Float16>(f));
}

// Two fp16 products accumulated into float32: c + a.lo*b.lo + a.hi*b.hi.
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, a), __builtin_bit_cast(half2_t, b), c,
                                false);
}

__device__ __forceinline__ float dot8(const uint4 &a, const uint4 &b, float c) {
  c = dot2(a.x, b.x, c);
  c = dot2(a.y, b.y, c);
  c = dot2(a.z, b.z, c);
  c = dot2(a.w, b.w, c);
  return c;
}

// Packed fp16 add of two codewords (8 halves each): the on-chip tile form used
// by the matrix-core product, where the row scale is applied in the epilogue.
__device__ __forceinline__ uint32_t hadd2(uint32_t a, uint32_t b) {
  half2_t r = __builtin_bit_cast(half2_t, a) + __builtin_bit_cast(half2_t, b);
  return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ uint4 hadd8(const uint4 &a, const uint4 &b) {
  return make_uint4(hadd2(a.x, b.x), hadd2(a.y, b.y), hadd2(a.z, b.z), hadd2(a.w, b.w));
}

// Overflow guard of the fp16 codeword sum in the 2x8 matrix-core tiles.
// Those tiles feed fp16(C_0[c_0] + C_1[c_1]) to the matrix cores and apply the
// row scale to the float32 total. The fp16 sum overflows when both codewords
// are large (|C_0 + C_1| > 65504) even where the decoded weight
// s * (C_0 + C_1) is finite (|s| < 1); it cannot when every codebook half is
// below 2^15 in magnitude, since the largest such value is 32752 and
// 2 * 32752 = 65504. A workgroup whose staged codebooks hold a half of
// magnitude >= 2^15 (infinities and NaNs included) halves every codeword in
// its table (exact for normal values; subnormal halves round to nearest
// even) and doubles its float32 partial sums before the scale (exact).
//
// True when some fp16 half of v has magnitude >= 2^15: (bits & 0x7FFF) +
// 0x0800 reaches bit 15 exactly then, with no carry between the halves.
__device__ __forceinline__ bool has_large_half(const uint4 &v) {
  const uint32_t m = 0x7FFF7FFFu, k = 0x08000800u;
  return ((((v.x & m) + k) | ((v.y & m) + k) | ((v.z & m) + k) | ((v.w & m) + k)) &
          0x80008000u) != 0;
}
// Every half of a codeword times 0.5 (packed fp16 multiplies, round to
// nearest even).
__device__ __forceinline__ uint32_t hhalf2(uint32_t a) {
  const half2_t h = {(_Float16)0.5f, (_Float16)0.5f};
  return __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, a) * h);
}
__device__ __forceinline__ uint4 hhalf8(const uint4 &a) {
  return make_uint4(hhalf2(a.x), hhalf2(a.y), hhalf2(a.z), hhalf2(a.w));
}
// Workgroup OR of a per-thread flag around a barrier the caller already has:
// publish_flag before it (one LDS word per wavefront, flags[wave]), read_flag
// after it. The result is uniform across the workgroup.
__device__ __forceinline__ void publish_flag(uint32_t *flags, bool mine) {
  const uint64_t b = __ballot(mine);
  if ((threadIdx.x & 63) == 0) flags[threadIdx.x >> 6] = b != 0 ? 1u : 0u;
}
__device__ __forceinline__ bool read_flag(const uint32_t *flags, int waves) {
  uint32_t f = 0;
  for (int w = 0; w < waves; ++w) f |= flags[w];
  return __builtin_amdgcn_readfirstlane(f) != 0;
}

// Pins a float32 value in a register: the optimiser may not fold the
// operation that produced it into a later one. Without it, fp16(a * s) is
// compiled to v_fma_mixlo_f16(a, s, +0), which rounds the exact product once
// to fp16 instead of to fp32 first, and turns -0 * s into +0.
__device__ __forceinline__ float materialize(float v) {
  asm volatile("" : "+v"(v));
  return v;
}

// Exact decode of one weight from its codewords' halves: float32 sum in
// ascending codebook order starting from the first codeword, float32 scale,
// one round to float16.
__device__ __forceinline__ uint32_t decode1(uint32_t c0, float s) {
  return f2h(materialize(materialize(h2f(c0)) * s));
}
__device__ __forceinline__ uint32_t decode2(uint32_t c0, uint32_t c1, float s) {
  const float sum = materialize(materialize(h2f(c0)) + materialize(h2f(c1)));
  return f2h(materialize(sum * s));
}

// Decode a packed pair of halves (one 32-bit word of each codeword).
__device__ __forceinline__ uint32_t decode_word2(uint32_t a, uint32_t b, float s) {
  return decode2(a & 0xFFFFu, b & 0xFFFFu, s) | (decode2(a >> 16, b >> 16, s) << 16);
}
__device__ __forceinline__ uint32_t decode_word1(uint32_t a, float s) {
  return decode1(a & 0xFFFFu, s) | (decode1(a >> 16, s) << 16);
}

// DPP row/bank controls (gfx9 family).
constexpr int kDppQuadXor1 = 0xB1;     // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;     // quad_perm [2,3,0,1]
constexpr int kDppQuadBcast0 = 0x00;   // quad_perm [0,0,0,0]
constexpr int kDppQuadBcast1 = 0x55;   // quad_perm [1,1,1,1]
constexpr int kDppQuadBcast2 = 0xAA;   // quad_perm [2,2,2,2]
constexpr int kDppQuadBcast3 = 0xFF;   // quad_perm [3,3,3,3]
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;
constexpr int kDppRowBcast15 = 0x142;
constexpr int kDppRowBcast31 = 0x143;

template <int CTRL, int ROW_MASK = 0xF, int BANK_MASK = 0xF, bool BOUND_CTRL = false>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROW_MASK, BANK_MASK,
                                         BOUND_CTRL));
}

// Sum over aligned groups of LPR lanes (16, 32 or 64) in a fixed order; the
// group's total is valid in its last lane.
template <int LPR>
__device__ __forceinline__ float row_sum(float v) {
  v += dpp<kDppQuadXor1>(v);
  v += dpp<kDppQuadXor2>(v);
  v += dpp<kDppRowHalfMirror>(v);
  v += dpp<kDppRowMirror>(v);
  if constexpr (LPR >= 32) v += dpp<kDppRowBcast15, 0xA>(v);
  if constexpr (LPR >= 64) v += dpp<kDppRowBcast31, 0xC>(v);
  return v;
}

// Sum over the 64 lanes of a wavefront in a fixed order; the total is valid in
// lane 63 (other lanes hold partial sums).
__device__ __forceinline__ float wave_sum_to_lane63(float v) {
  v += dpp<kDppQuadXor1>(v);
  v += dpp<kDppQuadXor2>(v);
  v += dpp<kDppRowHalfMirror>(v);
  v += dpp<kDppRowMirror>(v);
  v += dpp<kDppRowBcast15, 0xA>(v);
  v += dpp<kDppRowBcast31, 0xC>(v);
  return v;
}

// Sum over the 16 quads of a wavefront when every lane of a quad holds its
// quad's value, in a fixed order; the total is valid in lane 63.
__device__ __forceinline__ float quads_sum_to_lane63(float v) {
  v += dpp<kDppRowHalfMirror>(v);
  v += dpp<kDppRowMirror>(v);
  v += dpp<kDppRowBcast15, 0xA>(v);
  v += dpp<kDppRowBcast31, 0xC>(v);
  return v;
}

}  // namespace aqlm
