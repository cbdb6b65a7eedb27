// Arguments and shared pieces of the grouped FP4 expert GEMM kernels.
#pragma once
#include "common.h"

namespace moe {

struct GemmArgs {
  // activations A [rows_src, K]: bf16, or NVFP4 codes [rows_src, K/2] + E4M3 scales [rows_src, K/16]
  const uint8_t* a_data;
  const uint8_t* a_scales;
  float a_gscale;                 // NVFP4 global scale (power of two)
  const int32_t* gather;          // permuted row r reads source row gather[r] / gather_div
  int gather_div;
  int64_t a_bytes;                // bytes of a_data (bf16 rows or NVFP4 codes)
  // weights [E, N, K]: codes [E, N, K/2]; MX E8M0 [E, N, K/32] | NV E4M3 [E, N, K/16] + float [E]
  const uint8_t* w_packed[2];
  const uint8_t* w_scale[2];
  const float* w_global[2];
  int E, N, K;
  int64_t rows;                   // rows of the output (bound for every row index)
  const int32_t* offsets;         // [E+1]
  // outputs
  uint16_t* out_bf16;             // [rows, N] or null
  uint8_t* out_codes;             // [rows, N/2] or null
  uint8_t* out_scales;            // [rows, N/16]
  float out_inv_g;                // 1 / output global scale
  uint16_t* out_dq;               // [rows, N] bf16 NVFP4 values (codes x scale x global) or null
  float out_g;                    // output global scale
  int out_format;                 // MOE_OUT_NVFP4 / MOE_OUT_MXFP8 / MOE_OUT_NVFP4_PLANES (codes, scales)
  int out_g_log2;                 // log2(out_g) (NVFP4 planes: folded into their E8M0 scales)
  float* out_sumsq;               // [rows, N/64]: per-row sums of squares of the FP32 outputs, or null
  int tiled;                      // weights in the tiled layout (host-side dispatch)
};

// Offsets of one wavefront's weight operands.  Lane (li, lg) of a 16-row tile
// holds row li, code chunk lg of each 128-column step and row li's scales of
// each 4-step window; the tile's own base and the step / window count are
// added by the caller (a tile spans 16 * K/2 code bytes and 16 * sc_row scale
// bytes in either layout).  WB: scale bytes per row and 4-step (512-column)
// window -- MXFP4 16 (E8M0), NVFP4 32 (E4M3), compact MXFP4 8 (4-bit codes).
template <bool TL, int WB>
struct WeightLaneB {
  static constexpr uint32_t kStep = TL ? 1024u : 64u;                       // code bytes per step
  static constexpr uint32_t kWin = TL ? 16u * WB : (uint32_t)WB;             // scale bytes per window
  __host__ __device__ static uint32_t code(int li, int lg, int K) {
    return TL ? (uint32_t)(lg * 16 + li) * 16u : (uint32_t)li * (uint32_t)(K / 2) + (uint32_t)lg * 16u;
  }
  __host__ __device__ static uint32_t scale(int li, int K) {
    return TL ? (uint32_t)li * (uint32_t)WB : (uint32_t)li * (uint32_t)(K / (512 / WB));
  }
};
template <bool TL, bool W_NV>
using WeightLane = WeightLaneB<TL, W_NV ? 32 : 16>;

// Locate the j-th expert with at least one row (experts in index order).
// Returns false when fewer than j+1 experts are active.  All threads of the
// block must call it.  The thread that finds the expert also hands over its
// row range, so no second offsets load follows the search.
__device__ __forceinline__ bool find_active_expert(const int32_t* __restrict__ offsets, int E, int64_t rows, int j,
                                                   int& e_out, int& r0, int& r1) {
  __shared__ int s_found[3];                                  // expert, first row, end row
  __shared__ int s_wc[16];
  const int nthr = blockDim.x, lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = nthr >> 6;
  if (threadIdx.x == 0) s_found[0] = -1;
  int running = 0;
  for (int e0 = 0; e0 < E; e0 += nthr) {
    const int e = e0 + threadIdx.x;
    int o0 = 0, o1 = 0;
    if (e < E) {
      o0 = offsets[e];
      o1 = offsets[e + 1];
    }
    const bool act = o1 > o0;
    uint64_t b = __ballot(act);
    if (lane == 0) s_wc[w] = __popcll(b);
    __syncthreads();
    int before = running;
    for (int i = 0; i < w; ++i) before += s_wc[i];
    int rank = before + __popcll(b & ((1ull << lane) - 1ull));
    if (act && rank == j) {
      // rows outside [0, rows) are never touched, whatever the offsets hold
      const int c0 = (int)max((int64_t)0, min((int64_t)o0, rows));
      s_found[0] = e;
      s_found[1] = c0;
      s_found[2] = (int)max((int64_t)c0, min((int64_t)o1, rows));
    }
    int tot = 0;
    for (int i = 0; i < nw; ++i) tot += s_wc[i];
    running += tot;
    __syncthreads();
    if (running > j) break;
  }
  __syncthreads();
  const int e = s_found[0];
  if (e < 0) return false;
  e_out = e;
  r0 = s_found[1];
  r1 = s_found[2];
  return r1 > r0;
}

// g * sigmoid(g) with the hardware reciprocal (1 ulp) instead of a correctly
// rounded division: about half the instructions of the MFMA kernels' SwiGLU
// epilogues
__device__ __forceinline__ float silu_f(float g) { return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)); }
// the division form, kept by the weight-streaming kernel: with the shorter
// epilogue the compiler interleaved the next tile's work into it, which took
// more registers and measured 3.8% slower at 64 tokens
__device__ __forceinline__ float silu_div(float g) { return g / (1.0f + __expf(-g)); }

// compute units of the current device (persistent grids: one workgroup per CU)
inline int device_cus() {
  static int cus = 0;
  if (!cus) {
    int dev = 0;
    (void)hipGetDevice(&dev);
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
  }
  return cus;
}

}  // namespace moe
