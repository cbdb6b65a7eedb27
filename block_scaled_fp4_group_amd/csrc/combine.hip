// Weighted combine of the top_k expert outputs of each token (plus an optional
// residual), FP32 accumulation in slot order, one bf16 rounding at the end.
// The router's top-k weights scale each expert's output ("MiMo-V2.6-Flash --
// REAP-50" card, "Pruning Method": g_{t,j} times the expert output).
//
// One block per token; each thread owns 8 consecutive hidden elements (16-byte
// loads of bf16), so every gathered expert row is read once, coalesced.
#include "common.h"

namespace moe {

constexpr int kCombThreads = 256;

__global__ __launch_bounds__(kCombThreads) void combine_kernel(const uint16_t* __restrict__ eo,
                                                               const int32_t* __restrict__ slot_rows,
                                                               const float* __restrict__ w,
                                                               const uint16_t* __restrict__ resid, int top_k,
                                                               int h, uint16_t* __restrict__ y) {
  const int64_t t = blockIdx.x;
  __shared__ int32_t rows[32];
  __shared__ float wts[32];
  if (threadIdx.x < top_k) {
    rows[threadIdx.x] = slot_rows[t * top_k + threadIdx.x];
    wts[threadIdx.x] = w[t * top_k + threadIdx.x];
  }
  __syncthreads();
  for (int c = threadIdx.x * 8; c < h; c += kCombThreads * 8) {
    float acc[8];
    if (resid) {
      u32x4 v = *(const u32x4*)(resid + t * h + c);
#pragma unroll
      for (int i = 0; i < 4; ++i) { acc[2 * i] = bf16_lo(v[i]); acc[2 * i + 1] = bf16_hi(v[i]); }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
    }
    for (int j = 0; j < top_k; ++j) {
      int r = rows[j];
      if (r < 0) continue;
      float wj = wts[j];
      u32x4 v = *(const u32x4*)(eo + (int64_t)r * h + c);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[2 * i] = fmaf(wj, bf16_lo(v[i]), acc[2 * i]);
        acc[2 * i + 1] = fmaf(wj, bf16_hi(v[i]), acc[2 * i + 1]);
      }
    }
    u32x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = pack_bf16x2(acc[2 * i], acc[2 * i + 1]);
    *(u32x4*)(y + t * h + c) = o;
  }
}

moe_status launch_combine(const void* eo, const int32_t* slot_rows, const float* w, const void* resid, int64_t T,
                          int top_k, int h, void* y, hipStream_t stream) {
  if (T == 0) return MOE_OK;
  hipLaunchKernelGGL(combine_kernel, dim3((uint32_t)T), dim3(kCombThreads), 0, stream, (const uint16_t*)eo,
                     slot_rows, w, (const uint16_t*)resid, top_k, h, (uint16_t*)y);
  return launch_status("moe_combine");
}

}  // namespace moe
