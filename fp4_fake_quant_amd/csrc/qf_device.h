// Device-side number formats and cross-lane reductions for gfx950 (CDNA4).
//
// Format rules follow the QATFactory project page ("Supported formats" table):
// E2M1 elements, E4M3 and E8M0 block scales, FP16 super-block scales, BF16
// values.  The bit-level rules (RNE everywhere, saturation, signed zeros) are
// the library's stated choices, documented in include/qf.h.
//
// Four gfx950 conversion instructions are used directly; each agrees bit for
// bit with the software definition next to it over its whole input domain
// (checked on the device by qf_selftest_conversions):
//   v_cvt_pk_bf16_f32            two f32 -> two bf16, RNE, subnormals kept
//   v_cvt_scalef32_pk_fp4_f32    two f32 -> two E2M1 codes, RNE, saturating at 6,
//                                divided by 2^(e-127) where e is the exponent field
//                                of the scale operand (1.0f: no scaling); NaN -> 7
//   v_cvt_scalef32_pk_fp4_bf16   the same from two bf16
//   v_cvt_scalef32_pk_{f32,bf16}_fp4  E2M1 code * 2^(e-127), exact
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qf {

// Largest MXFP4 shared exponent of the noclip rule: 6 * 2^(252-127) = 1.5 * 2^127 is the
// top of the last E2M1 grid that bf16 can hold (6 * 2^126 is beyond its range).
constexpr int MX_NOCLIP_E_MAX = 252;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));

// ------------------------------------------------------- buffer access ----
// Raw buffer loads and stores with the hardware range check: an access whose byte
// offset is at or past the resource's size reads 0 and writes nothing.  Offsets of
// BUF_OOR or more are always out of range (sizes stay below 2^31 bytes).
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
constexpr uint32_t BUF_OOR = 0x80000000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_buf(const void* p, int64_t bytes) {
  // word 3: 32-bit data format, as plain dword loads and stores need
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}
// The same load with the non-temporal cache policy (the "nt" bit, auxiliary operand 2), for
// data read exactly once.
__device__ __forceinline__ uint4 buf_load16_nt(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 2));
}
__device__ __forceinline__ void buf_store16(__amdgpu_buffer_rsrc_t r, uint32_t off, uint4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), r, (int)off, 0, 0);
}
__device__ __forceinline__ void buf_store4(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t v) {
  __builtin_amdgcn_raw_buffer_store_b32(v, r, (int)off, 0, 0);
}
__device__ __forceinline__ void buf_store1(__amdgpu_buffer_rsrc_t r, uint32_t off, uint8_t v) {
  __builtin_amdgcn_raw_buffer_store_b8(v, r, (int)off, 0, 0);
}

// ----------------------------------------------------------------- bf16 ----
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Two f32 -> packed bf16 pair (lo in bits 0..15), RNE (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// Software reference of the same rounding (finite inputs): RNE on the 16 dropped bits.
__device__ __forceinline__ uint32_t bf16_rne_sw(float f) {
  uint32_t b = __float_as_uint(f);
  return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
}

// Largest |x| of 8 bf16 values (one 16-byte chunk) as the bits of a non-negative bf16.
// Non-negative bf16 patterns order like their values, so an unsigned max suffices.
__device__ __forceinline__ uint32_t amax_bits8(uint4 w) {
  const uint32_t M = 0x7FFF7FFFu;
  u16x2_t a = __builtin_bit_cast(u16x2_t, w.x & M);
  u16x2_t b = __builtin_bit_cast(u16x2_t, w.y & M);
  u16x2_t c = __builtin_bit_cast(u16x2_t, w.z & M);
  u16x2_t d = __builtin_bit_cast(u16x2_t, w.w & M);
  u16x2_t m = __builtin_elementwise_max(__builtin_elementwise_max(a, b), __builtin_elementwise_max(c, d));
  return m.x > m.y ? m.x : m.y;
}

// Largest bf16 exponent field of 8 bf16 values, in bits 7..14 of the result: the
// exponent of max|x| (mantissas and signs masked off before the unsigned max).
__device__ __forceinline__ uint32_t maxexp_bits8(uint4 w) {
  const uint32_t M = 0x7F807F80u;
  u16x2_t a = __builtin_bit_cast(u16x2_t, w.x & M);
  u16x2_t b = __builtin_bit_cast(u16x2_t, w.y & M);
  u16x2_t c = __builtin_bit_cast(u16x2_t, w.z & M);
  u16x2_t d = __builtin_bit_cast(u16x2_t, w.w & M);
  u16x2_t m = __builtin_elementwise_max(__builtin_elementwise_max(a, b), __builtin_elementwise_max(c, d));
  return m.x > m.y ? m.x : m.y;
}

// ----------------------------------------------------------------- E4M3 ----
// E4M3 ("FN": bias 7, max 448, no Inf) code of u >= 0: round to nearest even,
// anything at or above 448 gives 448 (0x7E).  Below 2^-6 the step is 2^-9.
// Both cases are computed with plain arithmetic and one is selected, so the code has no
// branch: below 2^-6, u * 512 (exact) + 2^23 rounds to the integer code (ties to even) in
// the low mantissa bits.
__device__ __forceinline__ uint32_t e4m3_encode(float u) {
  const uint32_t sub = __float_as_uint(u * 512.0f + 8388608.0f) - 0x4B000000u;   // 0..8; 8 is 2^-6
  uint32_t b = __float_as_uint(u);
  b += 0x7FFFFu + ((b >> 20) & 1u);                                   // RNE to 3 mantissa bits
  const uint32_t nrm = (((b >> 23) - 120u) << 3) | ((b >> 20) & 7u);
  return !(u < 448.0f) ? 0x7Eu : (u < 0.015625f ? sub : nrm);
}

__device__ __forceinline__ float e4m3_value(uint32_t c) {
  const uint32_t e = c >> 3, m = c & 7u;
  const float sub = (__uint_as_float(0x4B000000u | m) - 8388608.0f) * 0.001953125f;   // m * 2^-9, exact
  return e == 0 ? sub : __uint_as_float(((e + 120u) << 23) | (m << 20));
}

// ----------------------------------------------------------------- fp16 ----
// f32 -> IEEE binary16 bits for 0 <= f (finite): RNE with subnormals, saturating at 65504.
__device__ __forceinline__ uint32_t f16_bits_sat(float f) {
  if (!(f < 65504.0f)) return 0x7BFFu;
  uint32_t b = __float_as_uint(f);
  int e = (int)(b >> 23) - 127;
  if (e >= -14) {                                                     // normal fp16
    uint32_t r = b + 0xFFFu + ((b >> 13) & 1u);                       // RNE to 10 mantissa bits
    return ((((r >> 23) - 112u) << 10) | ((r >> 13) & 0x3FFu));
  }
  // subnormal fp16: value = k * 2^-24, k = rint(f * 2^24) (exact scaling)
  return (uint32_t)__builtin_rintf(f * 16777216.0f);                 // 0..1024; 1024 = 2^-14
}

// The same conversion through v_cvt_f16_f32 (RNE, fp16 subnormals kept): clamping
// to 65504 first makes the result saturate instead of overflowing.  Agrees with
// f16_bits_sat for every non-negative finite fp32 (device self-test).
__device__ __forceinline__ uint32_t f16_bits_sat_hw(float f) {
  return (uint32_t)__builtin_bit_cast(unsigned short, (_Float16)fminf(f, 65504.0f));
}

__device__ __forceinline__ float f16_value(uint32_t h) {
  uint32_t e = (h >> 10) & 0x1Fu, m = h & 0x3FFu;
  if (e == 0) return (float)m * 5.9604644775390625e-8f;               // m * 2^-24, exact
  return __uint_as_float(((e + 112u) << 23) | (m << 13));
}

// fp16 bits -> f32 through v_cvt_f32_f16 (exact, subnormals included; self-test).
__device__ __forceinline__ float f16_value_hw(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (unsigned short)h);
}
// Bits of a value already on the fp16 grid.
__device__ __forceinline__ uint32_t f16_bits_of(float v) {
  return (uint32_t)__builtin_bit_cast(unsigned short, (_Float16)v);
}

// ------------------------------------------------- division by constants ----
// fl(x / y) for a constant y with inv_y = fl(1 / y): the product x * inv_y is
// corrected once with the exact remainder r = x - q y (one FMA), then
// q + r * inv_y is rounded once.  For y = 15 and y = 63 this equals the IEEE
// quotient for every non-negative finite x (device self-test, exhaustive).
__device__ __forceinline__ float div_const(float x, float y, float inv_y) {
  const float q = x * inv_y;
  const float r = __builtin_fmaf(-q, y, x);
  return __builtin_fmaf(r, inv_y, q);
}
__device__ __forceinline__ float div15(float x) { return div_const(x, 15.0f, 1.0f / 15.0f); }
__device__ __forceinline__ float div63(float x) { return div_const(x, 63.0f, 1.0f / 63.0f); }

// ------------------------------------------------------- cross-lane ops ----
// DPP patterns: quad_perm [1,0,3,2] (lane ^ 1), quad_perm [2,3,0,1] (lane ^ 2),
// row_half_mirror (lane i <-> 7 - i inside 8), row_mirror (i <-> 15 - i inside 16),
// and ds_swizzle xor 16 inside 32.  For quad-uniform (resp. 8-, 16-uniform)
// values the mirrors pair each lane with the other half, which is all a
// max/min/or reduction needs.
__device__ __forceinline__ uint32_t dpp_xor1(uint32_t v) { return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, true); }
__device__ __forceinline__ uint32_t dpp_xor2(uint32_t v) { return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, true); }
__device__ __forceinline__ uint32_t dpp_hmirror(uint32_t v) { return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x141, 0xF, 0xF, true); }
__device__ __forceinline__ uint32_t dpp_mirror(uint32_t v) { return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x140, 0xF, 0xF, true); }
__device__ __forceinline__ uint32_t swz_xor16(uint32_t v) { return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x401F); }
// Broadcast lane 0 (resp. 1) of every quad to the whole quad.
__device__ __forceinline__ uint32_t quad_bcast0(uint32_t v) { return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x00, 0xF, 0xF, true); }
__device__ __forceinline__ uint32_t quad_bcast1(uint32_t v) { return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x55, 0xF, 0xF, true); }

__device__ __forceinline__ uint32_t umax(uint32_t a, uint32_t b) { return a > b ? a : b; }
__device__ __forceinline__ uint32_t umin(uint32_t a, uint32_t b) { return a < b ? a : b; }

// ------------------------------------------------------ NVFP4 QDQ chunk ----
// NVFP4 QDQ of one lane's 8 bf16 elements (QATFactory project page, "Supported
// formats" table: E2M1 elements, one E4M3 scale per 16-block, an FP32 tensor scale
// s_t).  Lanes 2i and 2i+1 hold one 16-block and both must execute this together.
// k = 6 s_t.  Block scale S = E4M3(amax / k) (RNE, saturating); with d = s S the
// element code is E2M1(x / d) (RNE, saturating) and the QDQ'd value is
// bf16((E2M1(code) s) s_t), each product rounded in fp32.
struct Nvfp4Chunk {
  uint32_t codes;   // nibble e holds element e's code
  uint32_t S;       // the block's E4M3 scale byte
  uint4 y;          // QDQ'd values, bf16
};

// NVFP4 element codes (4 bytes) and QDQ'd bf16 values of one 8-element chunk, given its
// block's scale value s, the tensor scale s_t and r = fl(1/fl(s s_t)) (0 when d == 0).
struct Nvfp4Enc {
  uint32_t codes;
  uint4 y;
};
__device__ __forceinline__ Nvfp4Enc nvfp4_encode_chunk(uint4 w, float s, float s_t, float r) {
  const uint32_t wv[4] = {w.x, w.y, w.z, w.w};
  float y[8];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    y[2 * e] = bf16_lo(wv[e]) * r;
    y[2 * e + 1] = bf16_hi(wv[e]) * r;
  }
  if (__builtin_expect(r > __FLT_MAX__, 0)) {
    // 1/d overflowed (the whole tied group lies below ~1e-35): 0 * inf must still
    // give magnitude 0 with the element's own sign.
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float lo = bf16_lo(wv[e]), hi = bf16_hi(wv[e]);
      if (lo == 0.0f) y[2 * e] = lo;
      if (hi == 0.0f) y[2 * e + 1] = hi;
    }
  }
  uint32_t codes = 0;
  codes = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(codes, y[0], y[1], 1.0f, 0);
  codes = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(codes, y[2], y[3], 1.0f, 1);
  codes = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(codes, y[4], y[5], 1.0f, 2);
  codes = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(codes, y[6], y[7], 1.0f, 3);
  Nvfp4Enc o;
  o.codes = codes;
  const f32x2_t v0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 0);
  const f32x2_t v1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 1);
  const f32x2_t v2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 2);
  const f32x2_t v3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 3);
  o.y.x = pack_bf16x2((v0.x * s) * s_t, (v0.y * s) * s_t);
  o.y.y = pack_bf16x2((v1.x * s) * s_t, (v1.y * s) * s_t);
  o.y.z = pack_bf16x2((v2.x * s) * s_t, (v2.y * s) * s_t);
  o.y.w = pack_bf16x2((v3.x * s) * s_t, (v3.y * s) * s_t);
  return o;
}

// The block scale of a 16-block with maximum |x| bits m (abs bf16 pattern): S = E4M3 of
// fl(amax / k), k = fl(6 s_t); s its value; r = fl(1 / fl(s s_t)), or 0 when that is 0.
struct Nvfp4Scale {
  uint32_t S;
  float s, r;
};
__device__ __forceinline__ Nvfp4Scale nvfp4_block_scale(uint32_t m, float s_t, float k) {
  const float amax = __uint_as_float(m << 16);
  Nvfp4Scale o;
  o.S = e4m3_encode(amax / k);
  o.s = e4m3_value(o.S);
  const float d = o.s * s_t;
  o.r = (d == 0.0f) ? 0.0f : 1.0f / d;
  return o;
}

__device__ __forceinline__ Nvfp4Chunk nvfp4_qdq_chunk(uint4 w, float s_t, float k) {
  uint32_t m = amax_bits8(w);
  m = umax(m, dpp_xor1(m));
  const Nvfp4Scale sc = nvfp4_block_scale(m, s_t, k);
  const Nvfp4Enc e = nvfp4_encode_chunk(w, sc.s, s_t, sc.r);
  Nvfp4Chunk o;
  o.S = sc.S;
  o.codes = e.codes;
  o.y = e.y;
  return o;
}

}  // namespace qf
