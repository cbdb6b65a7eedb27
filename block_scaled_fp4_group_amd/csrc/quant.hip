// NVFP4 activation quantisation (E2M1 codes, one E4M3 scale per 16 values, a
// power-of-two global scale): "AxionML / MiMo-V2.6-Flash-MOPD-NVFP4", paragraph
// "About NVFP4 quantization" and "Quantization Details" (unit global scale).
// Each thread quantises two 16-value blocks: 64 bytes of bf16 in, 16 bytes of
// codes and 2 scale bytes out, and optionally the 32 NVFP4 values themselves
// (codes x scale x global, exact in bfloat16).
#include "common.h"

namespace moe {

__global__ __launch_bounds__(256) void quant_kernel(const uint16_t* __restrict__ x, int64_t nblk2, int k,
                                                    float inv_g, uint8_t* __restrict__ codes,
                                                    uint8_t* __restrict__ scales, uint16_t* __restrict__ dq) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;   // pair of 16-blocks
  if (i >= nblk2) return;
  const int bpr = k / 16;                 // blocks per row
  int64_t b0 = 2 * i;                     // first block (flat over rows)
  float v[32];                            // k % 32 == 0: both blocks sit in one row
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    int64_t blk = b0 + (q >> 1);
    int64_t row = blk / bpr, col = (blk % bpr) * 16 + (q & 1) * 8;
    u32x4 w = *(const u32x4*)(x + row * k + col);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[q * 8 + 2 * j] = bf16_lo(w[j]);
      v[q * 8 + 2 * j + 1] = bf16_hi(w[j]);
    }
  }
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    int64_t blk = b0 + h;
    int64_t row = blk / bpr, cb = blk % bpr;
    uint32_t lo, hi;
    uint32_t sb = quant16(v + 16 * h, inv_g, lo, hi);
    u32x2 cw = {lo, hi};
    *(u32x2*)(codes + row * (k / 2) + cb * 8) = cw;
    scales[row * bpr + cb] = (uint8_t)sb;
    if (dq) {
      const float sg = e4m3_to_f32(sb) / inv_g;            // s x g, exact (g a power of two)
      const u32x2 d0 = nvfp4_dequant4(lo & 0xFFFFu, sg), d1 = nvfp4_dequant4(lo >> 16, sg);
      const u32x2 d2 = nvfp4_dequant4(hi & 0xFFFFu, sg), d3 = nvfp4_dequant4(hi >> 16, sg);
      u32x4* dst = (u32x4*)(dq + row * k + cb * 16);
      dst[0] = u32x4{d0[0], d0[1], d1[0], d1[1]};
      dst[1] = u32x4{d2[0], d2[1], d3[0], d3[1]};
    }
  }
}

moe_status launch_quant(const void* x, int64_t rows, int k, float input_scale, uint8_t* codes, uint8_t* scales,
                        void* dq, hipStream_t stream) {
  if (rows == 0) return MOE_OK;
  int64_t nblk = rows * (k / 16);         // total 16-blocks; k % 32 == 0 makes it even
  int64_t n2 = nblk / 2;
  int64_t grid = (n2 + 255) / 256;
  hipLaunchKernelGGL(quant_kernel, dim3((uint32_t)grid), dim3(256), 0, stream, (const uint16_t*)x, n2, k,
                     1.0f / input_scale, codes, scales, (uint16_t*)dq);
  return launch_status("moe_quantize_nvfp4");
}

// ------------------------------------------------------------------ MXFP8
// MXFP8 activations for the block-scaled MFMA GEMMs ("MiMo-V2.6-Flash-MOPD on
// one RTX PRO 6000", "Quantization, context and quality": E4M3 with a
// power-of-two scale per 32 values for the expert GEMMs).  Scale rule: the OCP
// Microscaling one, X = 2^(floor(log2 amax) - 8); codes = E4M3_rne(x / X),
// saturating at 448.  One thread per 32-value block: 64 bytes of bf16 in, 32
// code bytes and one E8M0 byte out.
__global__ __launch_bounds__(256) void quant_mxfp8_kernel(const uint16_t* __restrict__ x, int64_t nblk, int k,
                                                          uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= nblk) return;
  const int bpr = k / 32;
  const int64_t row = i / bpr, col = (i % bpr) * 32;
  float v[32];
  float amax = 0.0f;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const u32x4 w = *(const u32x4*)(x + row * k + col + q * 8);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[q * 8 + 2 * j] = bf16_lo(w[j]);
      v[q * 8 + 2 * j + 1] = bf16_hi(w[j]);
    }
  }
#pragma unroll
  for (int j = 0; j < 32; ++j) amax = fmaxf(amax, fabsf(v[j]));
  const int e = mxfp8_scale_exp(amax);
  const float inv = exp2_int(-e);                         // exact: x * inv is x / X
  u32x4 out[2];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    uint32_t wd = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) wd |= e4m3_code_signed(v[q * 4 + j] * inv) << (8 * j);
    out[q >> 2][q & 3] = wd;
  }
  *(u32x4*)(codes + row * k + col) = out[0];
  *(u32x4*)(codes + row * k + col + 16) = out[1];
  scales[i] = (uint8_t)(e + 127);
}

moe_status launch_quant_mxfp8(const void* x, int64_t rows, int k, uint8_t* codes, uint8_t* scales,
                              hipStream_t stream) {
  if (rows == 0) return MOE_OK;
  const int64_t nblk = rows * (k / 32);
  hipLaunchKernelGGL(quant_mxfp8_kernel, dim3((uint32_t)((nblk + 255) / 256)), dim3(256), 0, stream,
                     (const uint16_t*)x, nblk, k, codes, scales);
  return launch_status("moe_quantize_mxfp8");
}

// ------------------------------------------------- NVFP4 as two E4M3 planes
// The NVFP4 quantisation above, written for the block-scaled MFMA: each
// 16-value block becomes 32 E4M3 bytes (16 "hi" then 16 "lo" plane values) and
// one E8M0 scale 2^(k-1) g, with hi + lo times that scale equal to the NVFP4
// value code x s x g exactly (the identity in common.h).  One thread per
// 16-value block.
__global__ __launch_bounds__(256) void quant_planes_kernel(const uint16_t* __restrict__ x, int64_t nblk, int k,
                                                           float inv_g, int g_log2, uint8_t* __restrict__ planes,
                                                           uint8_t* __restrict__ pscales) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= nblk) return;
  const int bpr = k / 16;
  const int64_t row = i / bpr, col = (i % bpr) * 16;
  float v[16];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const u32x4 w = *(const u32x4*)(x + row * k + col + q * 8);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[q * 8 + 2 * j] = bf16_lo(w[j]);
      v[q * 8 + 2 * j + 1] = bf16_hi(w[j]);
    }
  }
  uint32_t lo, hi;
  const uint32_t sb = quant16(v, inv_g, lo, hi);
  uint32_t h0, h1, h2, h3, l0, l1, l2, l3;
  nvfp4_planes4(lo & 0xFFFFu, sb, h0, l0);
  nvfp4_planes4(lo >> 16, sb, h1, l1);
  nvfp4_planes4(hi & 0xFFFFu, sb, h2, l2);
  nvfp4_planes4(hi >> 16, sb, h3, l3);
  const u32x4 ph = {h0, h1, h2, h3}, pl = {l0, l1, l2, l3};
  uint8_t* dst = planes + row * (2 * (int64_t)k) + 2 * col;
  *(u32x4*)dst = ph;
  *(u32x4*)(dst + 16) = pl;
  pscales[i] = (uint8_t)nvfp4_plane_scale(sb, g_log2);
}

moe_status launch_quant_planes(const void* x, int64_t rows, int k, float input_scale, uint8_t* planes,
                               uint8_t* pscales, hipStream_t stream) {
  if (rows == 0) return MOE_OK;
  const int64_t nblk = rows * (k / 16);
  int g_log2;
  (void)frexpf(input_scale, &g_log2);
  g_log2 -= 1;                                            // input_scale = 2^g_log2 (checked on the host)
  hipLaunchKernelGGL(quant_planes_kernel, dim3((uint32_t)((nblk + 255) / 256)), dim3(256), 0, stream,
                     (const uint16_t*)x, nblk, k, 1.0f / input_scale, g_log2, planes, pscales);
  return launch_status("moe_quantize_nvfp4_planes");
}

}  // namespace moe
