// Exact MXFP4 -> NVFP4 scale transcode with its audit counters.
//
// "AxionML / MiMo-V2.6-Flash-MOPD-NVFP4", header and "Reproduce the
// checkpoint": codes stay byte for byte, each E8M0 block scale becomes two E4M3
// block scales, and the tool reports blocks / all-zero / re-rounded counts.
// "MiMo-V2.6-Flash-RL: exact NVFP4 weight conversion", "What changed": the two
// E4M3 scales combine with an exact power-of-two global scale.  The global
// exponent G = (largest finite block exponent of the matrix) - 8 is this
// library's reading (the pages do not print theirs).
//
// Pure integer work, bound by HBM: pass 1 reduces the largest exponent of each
// matrix (one block per matrix, 16-byte loads) and writes the block count;
// pass 2 maps 16 E8M0 bytes to 32 E4M3 bytes per thread and counts the rare
// all-zero / re-rounded / NaN blocks with integer atomics.
#include "common.h"

namespace moe {

constexpr int kTcThreads = 256;

__global__ __launch_bounds__(kTcThreads) void transcode_emax(const uint8_t* __restrict__ mx, int64_t per_mat,
                                                             float* __restrict__ gscale,
                                                             int64_t* __restrict__ counters) {
  // counters: the block count is known (one E8M0 byte per block); the others
  // start at zero before pass 2 adds to them
  if (blockIdx.x == 0 && threadIdx.x < 4) counters[threadIdx.x] = threadIdx.x == 0 ? (int64_t)gridDim.x * per_mat : 0;
  const uint8_t* p = mx + (int64_t)blockIdx.x * per_mat;
  int best = -1;                         // largest finite byte (0..254), -1 if none
  auto take = [&](const u32x4& v) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int x = (v[j] >> (8 * b)) & 0xFF;
        best = (x != 0xFF && x > best) ? x : best;
      }
    }
  };
  // whole sweeps with 8 independent 16-byte loads in flight per thread, then
  // the remainder with single loads (every offset < per_mat)
  constexpr int kU = 8;
  constexpr int64_t kSweep = (int64_t)kTcThreads * 16 * kU;
  const int64_t full = (per_mat / kSweep) * kSweep;
  for (int64_t s0 = 0; s0 < full; s0 += kSweep) {
    u32x4 v[kU];
#pragma unroll
    for (int q = 0; q < kU; ++q) v[q] = *(const u32x4*)(p + s0 + (int64_t)threadIdx.x * 16 + q * kTcThreads * 16);
#pragma unroll
    for (int q = 0; q < kU; ++q) take(v[q]);
  }
  for (int64_t i = full + (int64_t)threadIdx.x * 16; i < per_mat; i += kTcThreads * 16) take(*(const u32x4*)(p + i));
  __shared__ int wbest[kTcThreads / kWave];
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) best = max(best, __shfl_xor(best, off, kWave));
  if ((threadIdx.x & 63) == 0) wbest[threadIdx.x >> 6] = best;
  __syncthreads();
  if (threadIdx.x == 0) {
    int b = wbest[0];
    for (int i = 1; i < kTcThreads / kWave; ++i) b = max(b, wbest[i]);
    int G = b < 0 ? 0 : (b - 127) - 8;   // G in [-135, 119]: 2^G is a float (subnormal below -126)
    gscale[blockIdx.x] = ldexpf(1.0f, G);
  }
}

__global__ void transcode_zero_counters(int64_t* counters) {
  if (threadIdx.x < 4) counters[threadIdx.x] = 0;
}

__device__ __forceinline__ int float_exp2(float g) {
  // exact log2 of a power-of-two float, normal or subnormal
  uint32_t u = __float_as_uint(g);
  int e = (int)((u >> 23) & 0xFF);
  if (e != 0) return e - 127;
  return -149 + (31 - __clz(u & 0x7FFFFF));
}

__global__ __launch_bounds__(kTcThreads) void transcode_map(const uint8_t* __restrict__ mx,
                                                            const uint8_t* __restrict__ packed, int64_t total16,
                                                            int64_t per_mat, const float* __restrict__ gscale,
                                                            uint8_t* __restrict__ nv, int64_t* __restrict__ counters) {
  int64_t i = (int64_t)blockIdx.x * kTcThreads + threadIdx.x;   // 16 E8M0 bytes each
  uint32_t c_zero = 0, c_rr = 0, c_nan = 0;
  if (i < total16) {
    int64_t off = i * 16;
    int64_t mat = off / per_mat;
    int G = float_exp2(gscale[mat]);
    u32x4 v = *(const u32x4*)(mx + off);
    uint32_t outw[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t o0 = 0, o1 = 0;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        uint32_t x = (v[j] >> (8 * b)) & 0xFF;
        uint32_t byte;
        if (x == 0xFF) {
          byte = 0x7F;
          ++c_nan;
        } else {
          int k = ((int)x - 127) - G;
          if (k >= -6) byte = (uint32_t)(k + 7) << 3;
          else if (k >= -9) byte = 1u << (k + 9);
          else {
            // below E4M3's smallest power of two: zero if all 32 codes are +-0
            u32x4 cw = *(const u32x4*)(packed + (off + j * 4 + b) * 16);
            uint32_t any = (cw[0] | cw[1] | cw[2] | cw[3]) & 0x77777777u;
            if (any == 0) { byte = 0x00; ++c_zero; }
            else { byte = 0x01; ++c_rr; }
          }
        }
        uint32_t two = byte | (byte << 8);
        if (b < 2) o0 |= two << (16 * b);
        else o1 |= two << (16 * (b - 2));
      }
      outw[2 * j] = o0;
      outw[2 * j + 1] = o1;
    }
    u32x4 w0 = {outw[0], outw[1], outw[2], outw[3]};
    u32x4 w1 = {outw[4], outw[5], outw[6], outw[7]};
    *(u32x4*)(nv + off * 2) = w0;
    *(u32x4*)(nv + off * 2 + 16) = w1;
  }
  // the rare special blocks: one atomic per wave that has any (integer sums,
  // exact in any order); the common case issues none
  if (__ballot(c_zero | c_rr | c_nan) != 0) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      c_zero += __shfl_xor(c_zero, o, kWave);
      c_rr += __shfl_xor(c_rr, o, kWave);
      c_nan += __shfl_xor(c_nan, o, kWave);
    }
    if ((threadIdx.x & 63) == 0) {
      if (c_zero) atomicAdd((unsigned long long*)&counters[1], (unsigned long long)c_zero);
      if (c_rr) atomicAdd((unsigned long long*)&counters[2], (unsigned long long)c_rr);
      if (c_nan) atomicAdd((unsigned long long*)&counters[3], (unsigned long long)c_nan);
    }
  }
}

moe_status launch_transcode(const uint8_t* mx, const uint8_t* packed, int64_t M, int n, int k, uint8_t* nv,
                            float* gscale, int64_t* counters, hipStream_t stream) {
  int64_t per_mat = (int64_t)n * (k / 32);          // E8M0 bytes per matrix, a multiple of 16
  if (M == 0) {
    hipLaunchKernelGGL(transcode_zero_counters, dim3(1), dim3(64), 0, stream, counters);
    return launch_status("fp4_transcode_mx_to_nv");
  }
  hipLaunchKernelGGL(transcode_emax, dim3((uint32_t)M), dim3(kTcThreads), 0, stream, mx, per_mat, gscale, counters);
  int64_t total16 = M * per_mat / 16;
  int64_t grid = (total16 + kTcThreads - 1) / kTcThreads;
  hipLaunchKernelGGL(transcode_map, dim3((uint32_t)grid), dim3(kTcThreads), 0, stream, mx, packed, total16, per_mat,
                     gscale, nv, counters);
  return launch_status("fp4_transcode_mx_to_nv");
}

}  // namespace moe
