// NVFP4 activation quantisation (E2M1 codes, one E4M3 scale per 16 values, a
// power-of-two global scale): "AxionML / MiMo-V2.6-Flash-MOPD-NVFP4", paragraph
// "About NVFP4 quantization" and "Quantization Details" (unit global scale).
// Each thread quantises 8 consecutive values (16 bytes of bf16, consecutive
// threads on consecutive 16-byte pieces, so every load and store of a wave is
// one contiguous range); the two threads of a 16-value block share its amax
// through one lane exchange.  Out: 4 bytes of codes per thread, the block's
// scale byte, and optionally the 8 NVFP4 values themselves (codes x scale x
// global, exact in bfloat16).
#include "common.h"

namespace moe {

// 8 values of x (flat index 8 t) as floats
__device__ __forceinline__ void load8(const uint16_t* __restrict__ x, int64_t t, float (&v)[8]) {
  const u32x4 w = *(const u32x4*)(x + 8 * t);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    v[2 * j] = bf16_lo(w[j]);
    v[2 * j + 1] = bf16_hi(w[j]);
  }
}

// the NVFP4 scale byte of the 16-value block whose other half the lane
// t ^ 1 holds: s = E4M3(amax / (6 g)), amax * inv_g exact, the division
// correctly rounded
__device__ __forceinline__ uint32_t nvfp4_pair_scale(const float (&v)[8], float inv_g) {
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
  amax = fmaxf(amax, __shfl_xor(amax, 1, kWave));
  return f32_to_e4m3_sat((amax * inv_g) / 6.0f);
}

// the 8 E2M1 codes (nibble i = value i) under scale byte sb
__device__ __forceinline__ uint32_t nvfp4_codes8(const float (&v)[8], float inv_g, uint32_t sb) {
  const float s = e4m3_to_f32(sb);
  uint32_t w = 0u;
  if (s > 0.0f) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float xs = v[i] * inv_g;                        // exact
      w |= (e2m1_code(fabsf(xs), s) | ((__float_as_uint(xs) >> 28) & 8u)) << (4 * i);   // sign of x
    }
  }
  return w;
}

__global__ __launch_bounds__(256) void quant_kernel(const uint16_t* __restrict__ x, int64_t n8, float inv_g,
                                                    uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
                                                    uint16_t* __restrict__ dq) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;   // 8-value piece; n8 is even
  if (t >= n8) return;
  float v[8];
  load8(x, t, v);
  const uint32_t sb = nvfp4_pair_scale(v, inv_g);
  const uint32_t w = nvfp4_codes8(v, inv_g, sb);
  *(uint32_t*)(codes + 4 * t) = w;                                   // codes [rows, k/2] flat
  if ((t & 1) == 0) scales[t >> 1] = (uint8_t)sb;                    // scales [rows, k/16] flat
  if (dq) {
    const float sg = e4m3_to_f32(sb) / inv_g;                        // s x g, exact (g a power of two)
    const u32x2 d0 = nvfp4_dequant4(w & 0xFFFFu, sg), d1 = nvfp4_dequant4(w >> 16, sg);
    *(u32x4*)(dq + 8 * t) = u32x4{d0[0], d0[1], d1[0], d1[1]};
  }
}

moe_status launch_quant(const void* x, int64_t rows, int k, float input_scale, uint8_t* codes, uint8_t* scales,
                        void* dq, hipStream_t stream) {
  if (rows == 0) return MOE_OK;
  const int64_t n8 = rows * (k / 8);      // 8-value pieces; k % 32 == 0 keeps each 16-block's pair together
  hipLaunchKernelGGL(quant_kernel, dim3((uint32_t)((n8 + 255) / 256)), dim3(256), 0, stream, (const uint16_t*)x, n8,
                     1.0f / input_scale, codes, scales, (uint16_t*)dq);
  return launch_status("moe_quantize_nvfp4");
}

// ------------------------------------------------------------------ MXFP8
// MXFP8 activations for the block-scaled MFMA GEMMs ("MiMo-V2.6-Flash-MOPD on
// one RTX PRO 6000", "Quantization, context and quality": E4M3 with a
// power-of-two scale per 32 values for the expert GEMMs).  Scale rule: the OCP
// Microscaling one, X = 2^(floor(log2 amax) - 8); codes = E4M3_rne(x / X),
// saturating at 448.  Each thread takes 8 consecutive values (16 bytes of bf16
// in, 8 code bytes out, consecutive threads on consecutive pieces); the four
// threads of a 32-value block share its amax through two lane exchanges, and
// the first writes the E8M0 byte.
__global__ __launch_bounds__(256) void quant_mxfp8_kernel(const uint16_t* __restrict__ x, int64_t n8,
                                                          uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // n8 is a multiple of 4
  if (t >= n8) return;
  float v[8];
  load8(x, t, v);
  float amax = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(v[j]));
  amax = fmaxf(amax, __shfl_xor(amax, 1, kWave));
  amax = fmaxf(amax, __shfl_xor(amax, 2, kWave));
  const int e = mxfp8_scale_exp(amax);
  const float inv = exp2_int(-e);                         // exact: x * inv is x / X
  u32x2 out;
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    uint32_t wd = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) wd |= e4m3_code_signed(v[q * 4 + j] * inv) << (8 * j);
    out[q] = wd;
  }
  *(u32x2*)(codes + 8 * t) = out;                         // codes [rows, k] flat
  if ((t & 3) == 0) scales[t >> 2] = (uint8_t)(e + 127);  // scales [rows, k/32] flat
}

moe_status launch_quant_mxfp8(const void* x, int64_t rows, int k, uint8_t* codes, uint8_t* scales,
                              hipStream_t stream) {
  if (rows == 0) return MOE_OK;
  const int64_t n8 = rows * (k / 8);
  hipLaunchKernelGGL(quant_mxfp8_kernel, dim3((uint32_t)((n8 + 255) / 256)), dim3(256), 0, stream,
                     (const uint16_t*)x, n8, codes, scales);
  return launch_status("moe_quantize_mxfp8");
}

// ------------------------------------------------- NVFP4 as two E4M3 planes
// The NVFP4 quantisation above, written for the block-scaled MFMA: each
// 16-value block becomes 32 E4M3 bytes (16 "hi" then 16 "lo" plane values) and
// one E8M0 scale 2^(k-1) g, with hi + lo times that scale equal to the NVFP4
// value code x s x g exactly (the identity in common.h).  Each thread takes 8
// consecutive values (the pair of threads of a 16-value block share its amax
// as in quant_kernel) and writes their 8 hi and 8 lo bytes into the block's
// 32-byte record.
__global__ __launch_bounds__(256) void quant_planes_kernel(const uint16_t* __restrict__ x, int64_t n8, float inv_g,
                                                           int g_log2, uint8_t* __restrict__ planes,
                                                           uint8_t* __restrict__ pscales) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;   // n8 is even
  if (t >= n8) return;
  float v[8];
  load8(x, t, v);
  const uint32_t sb = nvfp4_pair_scale(v, inv_g);
  const uint32_t w = nvfp4_codes8(v, inv_g, sb);
  uint32_t h0, h1, l0, l1;
  nvfp4_planes4(w & 0xFFFFu, sb, h0, l0);
  nvfp4_planes4(w >> 16, sb, h1, l1);
  uint8_t* dst = planes + 32 * (t >> 1) + 8 * (t & 1);              // planes [rows, 2k] flat: 32 B per block
  *(u32x2*)dst = u32x2{h0, h1};
  *(u32x2*)(dst + 16) = u32x2{l0, l1};
  if ((t & 1) == 0) pscales[t >> 1] = (uint8_t)nvfp4_plane_scale(sb, g_log2);
}

moe_status launch_quant_planes(const void* x, int64_t rows, int k, float input_scale, uint8_t* planes,
                               uint8_t* pscales, hipStream_t stream) {
  if (rows == 0) return MOE_OK;
  const int64_t n8 = rows * (k / 8);
  int g_log2;
  (void)frexpf(input_scale, &g_log2);
  g_log2 -= 1;                                            // input_scale = 2^g_log2 (checked on the host)
  hipLaunchKernelGGL(quant_planes_kernel, dim3((uint32_t)((n8 + 255) / 256)), dim3(256), 0, stream,
                     (const uint16_t*)x, n8, 1.0f / input_scale, g_log2, planes, pscales);
  return launch_status("moe_quantize_nvfp4_planes");
}

}  // namespace moe
