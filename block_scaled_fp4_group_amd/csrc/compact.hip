// Compact MXFP4 expert storage at 4.125 bits per weight ("MiMo-V2.6-Flash-MOPD
// on one RTX PRO 6000", "What makes it fast": the experts' lossless compact
// encoding, 4.125 instead of 4.5 bits, same values).  The layout is this
// library's (documented with moe_fp4_compact_mx): the E2M1 codes stay as they
// are; each 32-value block keeps a 4-bit exponent code c against one
// power-of-two base 2^b per matrix (b = largest block exponent - 15), its scale
// being 2^(b + c).
//
// Integer work, bound by HBM: pass 1 reduces the largest finite E8M0 byte of
// each matrix (one workgroup per matrix) and writes the base and the block
// count; pass 2 turns 32 E8M0 bytes into 16 code bytes per thread and counts
// the rare blocks below the window (all-zero: exact; otherwise re-rounded) and
// NaN scales with integer atomics.
#include "common.h"

namespace moe {

constexpr int kCpThreads = 256;
constexpr int kCpSpan = 15;

__global__ __launch_bounds__(kCpThreads) void compact_base_kernel(const uint8_t* __restrict__ mx, int64_t per_mat,
                                                                  float* __restrict__ base,
                                                                  int64_t* __restrict__ counters) {
  if (blockIdx.x == 0 && threadIdx.x < 4) counters[threadIdx.x] = threadIdx.x == 0 ? (int64_t)gridDim.x * per_mat : 0;
  if (per_mat == 0) return;                        // no matrices: the counters only
  const uint8_t* p = mx + (int64_t)blockIdx.x * per_mat;
  int best = -1;                                   // largest finite byte, -1 if none
  for (int64_t i = (int64_t)threadIdx.x * 16; i < per_mat; i += kCpThreads * 16) {
    const u32x4 v = *(const u32x4*)(p + i);
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int x = (v[j] >> (8 * b)) & 0xFF;
        best = (x != 0xFF && x > best) ? x : best;
      }
  }
  __shared__ int wbest[kCpThreads / kWave];
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) best = max(best, __shfl_xor(best, off, kWave));
  if ((threadIdx.x & 63) == 0) wbest[threadIdx.x >> 6] = best;
  __syncthreads();
  if (threadIdx.x == 0) {
    int b = wbest[0];
    for (int i = 1; i < kCpThreads / kWave; ++i) b = max(b, wbest[i]);
    const int e = b < 0 ? kCpSpan : (b - 127);     // a matrix with no finite block: b = 0
    base[blockIdx.x] = ldexpf(1.0f, e - kCpSpan);  // >= 2^-142: a float (subnormal below 2^-126)
  }
}

__device__ __forceinline__ int base_exp(float b) {
  // exact log2 of a power-of-two float, normal or subnormal
  const uint32_t u = __float_as_uint(b);
  const int e = (int)((u >> 23) & 0xFF);
  if (e != 0) return e - 127;
  return -149 + (31 - __clz(u & 0x7FFFFF));
}

// thread i: the 32 E8M0 bytes 32 i .. 32 i + 31 -> 16 code bytes (per_mat % 32 == 0,
// so the 32 blocks belong to one matrix)
__global__ __launch_bounds__(kCpThreads) void compact_map_kernel(const uint8_t* __restrict__ mx,
                                                                 const uint8_t* __restrict__ packed, int64_t total32,
                                                                 int64_t per_mat, const float* __restrict__ base,
                                                                 uint8_t* __restrict__ out,
                                                                 int64_t* __restrict__ counters) {
  const int64_t i = (int64_t)blockIdx.x * kCpThreads + threadIdx.x;
  if (i >= total32) return;
  const int64_t first = i * 32;                     // first block (flat)
  const int64_t m = first / per_mat;                // per_mat % 32 == 0: one matrix per thread
  const int b = base_exp(base[m]);
  const u32x4 v0 = *(const u32x4*)(mx + first), v1 = *(const u32x4*)(mx + first + 16);
  uint32_t words[4] = {0u, 0u, 0u, 0u};
  int zero_oor = 0, rerounded = 0, nan = 0;
#pragma unroll
  for (int q = 0; q < 32; ++q) {
    const uint32_t w = q < 16 ? v0[q >> 2] : v1[(q - 16) >> 2];
    const int x = (int)((w >> (8 * (q & 3))) & 0xFF);
    int c;
    if (x == 0xFF) {
      c = kCpSpan;
      ++nan;
    } else {
      c = (x - 127) - b;
      if (c < 0) {
        // below the window: exact only if every code of the block is +-0
        const u32x4 a = *(const u32x4*)(packed + (first + q) * 16);
        const uint32_t mag = (a[0] | a[1] | a[2] | a[3]) & 0x77777777u;
        if (mag == 0) ++zero_oor;
        else ++rerounded;
        c = 0;
      }
      c = c > kCpSpan ? kCpSpan : c;               // (never: b is the largest exponent - 15)
    }
    words[q >> 3] |= (uint32_t)c << (4 * (q & 7));
  }
  *(u32x4*)(out + i * 16) = u32x4{words[0], words[1], words[2], words[3]};
  if (zero_oor) atomicAdd((unsigned long long*)&counters[1], (unsigned long long)zero_oor);
  if (rerounded) atomicAdd((unsigned long long*)&counters[2], (unsigned long long)rerounded);
  if (nan) atomicAdd((unsigned long long*)&counters[3], (unsigned long long)nan);
}

moe_status launch_compact(const uint8_t* mx, const uint8_t* packed, int64_t M, int n, int k, uint8_t* out,
                          float* base, int64_t* counters, hipStream_t stream) {
  const int64_t per_mat = (int64_t)n * (k / 32);
  if (M == 0) {
    hipLaunchKernelGGL(compact_base_kernel, dim3(1), dim3(kCpThreads), 0, stream, mx, (int64_t)0, base, counters);
    return launch_status("moe_fp4_compact_mx");
  }
  hipLaunchKernelGGL(compact_base_kernel, dim3((uint32_t)M), dim3(kCpThreads), 0, stream, mx, per_mat, base,
                     counters);
  const int64_t total32 = M * per_mat / 32;
  hipLaunchKernelGGL(compact_map_kernel, dim3((uint32_t)((total32 + kCpThreads - 1) / kCpThreads)), dim3(kCpThreads),
                     0, stream, mx, packed, total32, per_mat, base, out, counters);
  return launch_status("moe_fp4_compact_mx");
}

}  // namespace moe
