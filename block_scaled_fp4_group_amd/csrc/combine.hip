// Weighted combine of the top_k expert outputs of each token (plus an optional
// residual), FP32 accumulation in slot order, one bf16 rounding at the end.
// The router's top-k weights scale each expert's output ("MiMo-V2.6-Flash --
// REAP-50" card, "Pruning Method": g_{t,j} times the expert output).
//
// A workgroup takes one token and 2048 hidden elements; each thread owns 8
// consecutive elements (16-byte loads of bf16), so every gathered expert row
// is read once, coalesced.  Expert rows and the residual are read with the
// non-temporal cache policy: nothing reads them again (prefill layer 0.7%
// faster).
#include "common.h"

namespace moe {

constexpr int kCombThreads = 256;

// TK > 0: top_k known at compile time -- every gathered row load is issued
// before the first multiply-add, so a thread waits for one memory latency, not
// top_k of them.  TK == 0: any top_k (rows loaded as the sum proceeds).
template <int TK>
__global__ __launch_bounds__(kCombThreads) void combine_kernel(const uint16_t* __restrict__ eo,
                                                               const int32_t* __restrict__ slot_rows,
                                                               const float* __restrict__ w,
                                                               const uint16_t* __restrict__ resid, int top_k,
                                                               int h, uint16_t* __restrict__ y) {
  const int64_t t = blockIdx.x;
  const int c = (blockIdx.y * kCombThreads + threadIdx.x) * 8;      // 8 hidden elements per thread
  if (c >= h) return;
  const int kk = TK > 0 ? TK : top_k;
  float acc[8];
  if (resid) {
    const u32x4 v = __builtin_nontemporal_load((const u32x4*)(resid + t * h + c));
#pragma unroll
    for (int i = 0; i < 4; ++i) { acc[2 * i] = bf16_lo(v[i]); acc[2 * i + 1] = bf16_hi(v[i]); }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
  }
  auto add = [&](const u32x4& v, float wj) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[2 * i] = fmaf(wj, bf16_lo(v[i]), acc[2 * i]);
      acc[2 * i + 1] = fmaf(wj, bf16_hi(v[i]), acc[2 * i + 1]);
    }
  };
  if constexpr (TK > 0) {
    u32x4 v[TK];
    int r[TK];
#pragma unroll
    for (int j = 0; j < TK; ++j) {
      r[j] = slot_rows[t * TK + j];                                  // uniform: scalar loads
      v[j] = __builtin_nontemporal_load((const u32x4*)(eo + (int64_t)max(r[j], 0) * h + c));
    }
#pragma unroll
    for (int j = 0; j < TK; ++j)
      if (r[j] >= 0) add(v[j], w[t * TK + j]);                       // slot order; -1 adds nothing
  } else {
    for (int j = 0; j < kk; ++j) {
      const int r = slot_rows[t * kk + j];
      if (r < 0) continue;
      add(*(const u32x4*)(eo + (int64_t)r * h + c), w[t * kk + j]);
    }
  }
  u32x4 o;
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = cvt_bf16x2(acc[2 * i], acc[2 * i + 1]);
  *(u32x4*)(y + t * h + c) = o;
}

moe_status launch_combine(const void* eo, const int32_t* slot_rows, const float* w, const void* resid, int64_t T,
                          int top_k, int h, void* y, hipStream_t stream) {
  if (T == 0) return MOE_OK;
  const dim3 grid((uint32_t)T, (uint32_t)((h + kCombThreads * 8 - 1) / (kCombThreads * 8)));
  if (top_k == 8)
    hipLaunchKernelGGL(combine_kernel<8>, grid, dim3(kCombThreads), 0, stream, (const uint16_t*)eo, slot_rows, w,
                       (const uint16_t*)resid, top_k, h, (uint16_t*)y);
  else
    hipLaunchKernelGGL(combine_kernel<0>, grid, dim3(kCombThreads), 0, stream, (const uint16_t*)eo, slot_rows, w,
                       (const uint16_t*)resid, top_k, h, (uint16_t*)y);
  return launch_status("moe_combine");
}

}  // namespace moe
