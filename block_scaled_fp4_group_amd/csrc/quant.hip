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

}  // namespace moe
