// Shared device helpers for the gfx950 MoE-FP4 kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_fp4.h"

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int32_t i32x8 __attribute__((ext_vector_type(8)));

namespace moe {

constexpr int kWave = 64;

// ---------------------------------------------------------------- host side
void set_error(const char* fmt, ...);
moe_status launch_status(const char* what);

// ------------------------------------------------------------- bf16 helpers
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// float -> bf16 bits, round to nearest even (finite inputs), in integer ops
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return f32_to_bf16_bits(a) | (f32_to_bf16_bits(b) << 16);
}
// the same rounding with the gfx950 packed convert: one instruction for the
// pair (the MFMA kernels' epilogues; the weight-streaming kernel keeps the
// integer form, with which the compiler schedules it better)
__device__ __forceinline__ uint32_t cvt_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}

// --------------------------------------------------------- scale decoders
// E8M0 byte -> float 2^(b-127); 0xFF -> NaN; 0x00 -> 2^-127 (a float subnormal).
__device__ __forceinline__ float e8m0_to_f32(uint32_t b) {
  uint32_t u = b << 23;
  u = (b == 0u) ? 0x00400000u : u;        // selects, no branches
  u = (b == 0xFFu) ? 0x7FC00000u : u;
  return __uint_as_float(u);
}

// E4M3 (FN) -> float (exact; 0x7F / 0xFF -> NaN) by the gfx950 FP8 convert,
// which decodes OCP E4M3 -- subnormals, signs and NaN included -- exactly like
// the definition (checked for every byte value and byte position).
// e4m3_to_f32: the low byte of b; e4m3_byte<SEL>: byte SEL of a word.
__device__ __forceinline__ float e4m3_to_f32(uint32_t b) { return __builtin_amdgcn_cvt_f32_fp8((int)b, 0); }
template <int SEL>
__device__ __forceinline__ float e4m3_byte(uint32_t w) { return __builtin_amdgcn_cvt_f32_fp8((int)w, SEL); }

__device__ __forceinline__ bool is_pow2_scale(float s) {
  uint32_t u = __float_as_uint(s);
  uint32_t e = (u >> 23) & 0xFFu;
  return (u & 0x007FFFFFu) == 0 && e != 0 && e != 0xFFu;
}

// ------------------------------------------------------- FP4 -> bf16 x 8
// 8 E2M1 codes (one dword, element 0 in the low nibble) times `scale` -> 8 bf16.
// The gfx950 convert instruction applies only the power-of-two part of its
// scale operand; the exact general path goes through float.
__device__ __forceinline__ bf16x8 fp4x8_to_bf16_pow2(uint32_t codes, float pow2_scale) {
  bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, pow2_scale, 0);
  bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, pow2_scale, 1);
  bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, pow2_scale, 2);
  bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, pow2_scale, 3);
  bf16x8 r = {p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
  return r;
}

__device__ __forceinline__ bf16x8 fp4x8_to_bf16_general(uint32_t codes, float scale) {
  bf16x8 r;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    f32x2 v;
    switch (b) {   // the selector must be a constant
      case 0: v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 0); break;
      case 1: v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 1); break;
      case 2: v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 2); break;
      default: v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 3); break;
    }
    // code (2 significant bits) x E4M3 scale (4 bits): exact in float and in bf16
    uint32_t w = pack_bf16x2(v[0] * scale, v[1] * scale);
    bf16x2 p = __builtin_bit_cast(bf16x2, w);
    r[2 * b] = p[0];
    r[2 * b + 1] = p[1];
  }
  return r;
}

__device__ __forceinline__ bf16x8 fp4x8_to_bf16(uint32_t codes, float scale) {
  if (is_pow2_scale(scale)) return fp4x8_to_bf16_pow2(codes, scale);
  return fp4x8_to_bf16_general(codes, scale);
}

// 4 NVFP4 codes (16 bits, element 0 in the low nibble) times s * g -> 4 bf16
// (two dwords).  code (2 significant bits) x E4M3 scale (4) x power of two is
// exact in float and in bfloat16, so keeping the high half is exact.
__device__ __forceinline__ u32x2 nvfp4_dequant4(uint32_t bits, float sg) {
  const f32x2 a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(bits, 1.0f, 0);
  const f32x2 b = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(bits, 1.0f, 1);
  const uint32_t w0 = (__float_as_uint(a[0] * sg) >> 16) | (__float_as_uint(a[1] * sg) & 0xFFFF0000u);
  const uint32_t w1 = (__float_as_uint(b[0] * sg) >> 16) | (__float_as_uint(b[1] * sg) & 0xFFFF0000u);
  return u32x2{w0, w1};
}

// ---------------------------------------------------------- buffer loads
// Raw buffer descriptor over [base, base + bytes): loads whose offset falls
// outside the range return zero and touch no memory (hardware range check).
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr uint32_t kOutOfRange = 0x80000000u;

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 bload128(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0));
}
__device__ __forceinline__ u32x2 bload64(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, (int)voff, (int)soff, 0));
}
// Streaming reads: the non-temporal cache policy (the NT bit of the buffer
// instruction's cache-policy operand, value 2 on gfx950), for data read once
// per launch -- the weight stream of the weight-streaming GEMM.  Results are
// the same; only the caches' retention of the lines changes.
constexpr int kCPolNT = 2;
__device__ __forceinline__ u32x4 bload128_nt(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, kCPolNT));
}
__device__ __forceinline__ u32x2 bload64_nt(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, (int)voff, (int)soff, kCPolNT));
}
__device__ __forceinline__ uint32_t bload32(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, (int)soff, 0);
}
__device__ __forceinline__ uint32_t bload16(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b16(r, (int)voff, (int)soff, 0);
}
__device__ __forceinline__ uint32_t bload8(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b8(r, (int)voff, (int)soff, 0);
}

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// -------------------------------------------------- NVFP4 quantisation
// Round a non-negative float to E4M3 (nearest even, saturating at 448).  The
// input is an exactly-known float (the caller guarantees a single rounding).
__device__ __forceinline__ uint32_t f32_to_e4m3_sat(float v) {
  if (!(v > 0.0f)) return 0u;
  if (v >= 448.0f) return 0x7Eu;
  uint32_t u = __float_as_uint(v);
  int e = (int)((u >> 23) & 0xFF) - 127;             // v = 1.f * 2^e
  if (e < -6) {
    // subnormal range: value = M * 2^-9, M = rne(v * 2^9) in 0..8 (8 -> min normal 0x08)
    float t = v * 512.0f;                             // exact (power-of-two scaling)
    float r = __builtin_rintf(t);                     // round half to even
    return (uint32_t)r;                               // 0..8; 8 == 0x08 == 2^-6
  }
  // normal: keep 3 mantissa bits, round to nearest even on the float bits
  uint32_t mant = u & 0x7FFFFFu;
  uint32_t keep = mant >> 20, rest = mant & 0xFFFFFu;
  uint32_t half = 0x80000u;
  if (rest > half || (rest == half && (keep & 1u))) keep += 1;
  uint32_t ee = (uint32_t)(e + 7);
  if (keep == 8) { keep = 0; ee += 1; }
  uint32_t byte = (ee << 3) | keep;
  return byte > 0x7Eu ? 0x7Eu : byte;
}

// E2M1 magnitude code for |x| / s by exact comparison against the midpoints
// times s (every product has <= 7 significant bits, so it is exact in float).
// Ties go to the even code.
__device__ __forceinline__ uint32_t e2m1_code(float ax, float s) {
  // midpoints between codes k and k+1, and whether the tie rounds up (to k+1 even)
  const float m0 = 0.25f * s, m1 = 0.75f * s, m2 = 1.25f * s, m3 = 1.75f * s;
  const float m4 = 2.5f * s, m5 = 3.5f * s, m6 = 5.0f * s;
  uint32_t c = 0;
  c += (ax > m0);                  // tie at 0.25 -> 0 (even)
  c += (ax >= m1);                 // tie at 0.75 -> 2 (even)
  c += (ax > m2);                  // tie at 1.25 -> 2
  c += (ax >= m3);                 // tie at 1.75 -> 4
  c += (ax > m4);                  // tie at 2.5  -> 4
  c += (ax >= m5);                 // tie at 3.5  -> 6
  c += (ax > m6);                  // tie at 5    -> 6
  return c;
}

// ------------------------------------------------------------- MXFP8
// floor(log2 a) for a finite float a > 0, normal or subnormal
__device__ __forceinline__ int floor_log2_f32(float a) {
  const uint32_t u = __float_as_uint(a);
  const int e = (int)((u >> 23) & 0xFFu);
  if (e) return e - 127;
  return (31 - (int)__clz(u & 0x7FFFFFu)) - 149;
}

// Shared-scale exponent of an MXFP8 block (OCP Microscaling rule): floor(log2
// amax) minus 8 (the exponent of E4M3's largest power of two), kept in E8M0's
// range; an all-zero block gets 2^-127.
__device__ __forceinline__ int mxfp8_scale_exp(float amax) {
  if (!(amax > 0.0f)) return -127;
  const int e = floor_log2_f32(amax) - 8;
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// 2^e as a float, exactly, for e in [-127, 127]
__device__ __forceinline__ float exp2_int(int e) {
  return e >= -126 ? __uint_as_float((uint32_t)(e + 127) << 23) : __uint_as_float(0x00400000u);
}

// Signed E4M3 code of v: magnitude rounded to nearest-even, saturating at 448;
// the sign bit follows v (so -0 and small negatives give 0x80).
__device__ __forceinline__ uint32_t e4m3_code_signed(float v) {
  return f32_to_e4m3_sat(fabsf(v)) | ((__float_as_uint(v) >> 24) & 0x80u);
}

// --------------------------------------------- NVFP4 as two E4M3 planes
// An NVFP4 value c * s (E2M1 code c, E4M3 scale s = 2^k (lead + f1/2 +
// (2 f2 + f3)/8), k = max(exponent field, 1) - 7) is hi + lo times 2^(k-1) with
// hi = c (2 lead + f1) and lo = c (2 f2 + f3) / 4, both exact E4M3 values
// (every scale byte and code checked with exact rationals).  Four codes
// (16 bits, element 0 in the low nibble) -> four hi bytes and four lo bytes;
// the values are exact, so the hardware FP8 convert's rounding never acts.
__device__ __forceinline__ void nvfp4_planes4(uint32_t bits, uint32_t sb, uint32_t& hi, uint32_t& lo) {
  const uint32_t e = (sb >> 3) & 15u, m = sb & 7u;
  const float mh = (float)(2u * (e > 0u ? 1u : 0u) + ((m >> 2) & 1u));
  const float ml = (float)(2u * ((m >> 1) & 1u) + (m & 1u)) * 0.25f;
  const f32x2 c01 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(bits, 1.0f, 0);
  const f32x2 c23 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(bits, 1.0f, 1);
  int h = __builtin_amdgcn_cvt_pk_fp8_f32(c01[0] * mh, c01[1] * mh, 0, false);
  h = __builtin_amdgcn_cvt_pk_fp8_f32(c23[0] * mh, c23[1] * mh, h, true);
  int l = __builtin_amdgcn_cvt_pk_fp8_f32(c01[0] * ml, c01[1] * ml, 0, false);
  l = __builtin_amdgcn_cvt_pk_fp8_f32(c23[0] * ml, c23[1] * ml, l, true);
  hi = (uint32_t)h;
  lo = (uint32_t)l;
}

// E8M0 byte of the planes' shared scale 2^(k-1) * g, g = 2^g_log2
__device__ __forceinline__ uint32_t nvfp4_plane_scale(uint32_t sb, int g_log2) {
  const int e = (int)((sb >> 3) & 15u);
  const int k = (e > 1 ? e : 1) - 7;
  return (uint32_t)(k - 1 + g_log2 + 127);
}

}  // namespace moe
