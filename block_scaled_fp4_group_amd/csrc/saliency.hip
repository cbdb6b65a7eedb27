// REAP expert saliency, accumulated over batches ("MiMo-V2.6-Flash -- REAP-50"
// card, "Pruning Method": S_j is the mean over the tokens routed to expert j of
// g_{t,j} times the L2 norm of the expert's output for token t).
//
// The down projection's epilogue leaves, for each permuted row r, the sums of
// squares of its FP32 outputs in parts of 64 columns (row_sumsq [rows, parts]).
// One workgroup per expert then adds, for each of the expert's rows in row
// order, its parts in column order (float64), takes the square root and
// multiplies by the row's router weight g (the combine weight of its slot);
// the rows' terms meet in a fixed-shape tree, and the expert's sum and row
// count are added to the caller's running totals.  No floating-point atomics:
// every run gives the same bits.
#include "common.h"

namespace moe {

constexpr int kSalThreads = 256;

__global__ __launch_bounds__(kSalThreads) void saliency_kernel(const float* __restrict__ row_sumsq, int64_t rows,
                                                               int parts, const int32_t* __restrict__ offsets,
                                                               const int32_t* __restrict__ sorted_slots,
                                                               const float* __restrict__ topk_weights,
                                                               double* __restrict__ sums,
                                                               int64_t* __restrict__ counts) {
  __shared__ double red[kSalThreads];
  const int e = blockIdx.x;
  const int64_t r0 = max((int64_t)0, min((int64_t)offsets[e], rows));
  const int64_t r1 = max(r0, min((int64_t)offsets[e + 1], rows));
  double acc = 0.0;
  for (int64_t r = r0 + threadIdx.x; r < r1; r += kSalThreads) {
    const float* q = row_sumsq + r * parts;
    double n2 = 0.0;
    for (int c = 0; c < parts; ++c) n2 += (double)q[c];
    acc += (double)topk_weights[sorted_slots[r]] * sqrt(n2);
  }
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int w = kSalThreads / 2; w > 0; w >>= 1) {
    if (threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0 && r1 > r0) {
    sums[e] += red[0];
    counts[e] += r1 - r0;
  }
}

moe_status launch_saliency(const float* row_sumsq, int64_t rows, int parts, const int32_t* offsets, int E,
                           const int32_t* sorted_slots, const float* topk_weights, double* sums, int64_t* counts,
                           hipStream_t stream) {
  if (E == 0 || rows == 0) return MOE_OK;
  hipLaunchKernelGGL(saliency_kernel, dim3((uint32_t)E), dim3(kSalThreads), 0, stream, row_sumsq, rows, parts,
                     offsets, sorted_slots, topk_weights, sums, counts);
  return launch_status("moe_reap_saliency_accumulate");
}

}  // namespace moe
