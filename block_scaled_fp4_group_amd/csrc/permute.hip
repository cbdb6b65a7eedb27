// Deterministic token permutation: a stable counting sort of the (token, k)
// slots by expert over LDS-staged chunks of 2048 slots.
//
//   count:   each block histograms its chunk in LDS and writes one row of a
//            [blocks, E] count table (integer LDS atomics: exact, order-free);
//   scan:    one block turns the table into per-(block, expert) base rows and
//            the expert_offsets exclusive prefix sum;
//   scatter: each block ranks its slots stably inside the chunk -- wave-level
//            multisplit (the lanes holding the same expert are found with one
//            ballot per expert-id bit), then a prefix over the chunk's 64-slot
//            sub-chunks in LDS -- and writes sorted_slots and slot_rows.
// A single chunk (R <= 2048, every decode batch) runs all three steps in one
// block and one launch.  Nothing depends on the order in which atomics or
// blocks execute, so every run gives identical bytes.  The pages only imply
// this step: one grouped kernel runs over the routed experts ("MiMo-V2.6-Flash-
// MOPD on one RTX PRO 6000", "What makes it fast", speed v4).
#include "permute.h"

namespace moe {

size_t permute_ws_bytes(int64_t R, int E) {
  int64_t blocks = (R + kPermChunk - 1) / kPermChunk;
  if (blocks < 1) blocks = 1;
  return (size_t)blocks * (size_t)E * sizeof(int32_t);
}

// ---------------------------------------------------------- one chunk
__global__ __launch_bounds__(kPermThreads) void permute_single(const int32_t* __restrict__ ids, int64_t R, int E,
                                                               int nbits, int32_t* __restrict__ offsets,
                                                               int32_t* __restrict__ sorted_slots,
                                                               int32_t* __restrict__ slot_rows) {
  permute_one_chunk(ids, R, E, nbits, offsets, sorted_slots, slot_rows);
}

// ------------------------------------------------------ multi-chunk path
__global__ __launch_bounds__(kPermThreads) void permute_count(const int32_t* __restrict__ ids, int64_t R, int E,
                                                              int32_t* __restrict__ table) {
  __shared__ int32_t hist[kPermMaxE];
  for (int e = threadIdx.x; e < E; e += kPermThreads) hist[e] = 0;
  __syncthreads();
  int64_t base = (int64_t)blockIdx.x * kPermChunk;
  for (int i = threadIdx.x; i < kPermChunk; i += kPermThreads) {
    int64_t s = base + i;
    if (s < R) {
      int e = ids[s];
      if (e >= 0 && e < E) atomicAdd(&hist[e], 1);
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kPermThreads) table[(int64_t)blockIdx.x * E + e] = hist[e];
}

// The [nblk, E] count table is read twice, kScanBatch blocks at a time with
// every load of a batch in flight together: once to total each expert, once
// (after the scan over experts) to write each (block, expert) base row.
constexpr int kScanBatch = 16;

__global__ __launch_bounds__(kPermThreads) void permute_scan(int32_t* __restrict__ table, int nblk, int E,
                                                             int32_t* __restrict__ offsets) {
  __shared__ int32_t tot[kPermMaxE];
  __shared__ int32_t wsum[kPermThreads / kWave];
  __shared__ int32_t range_total;
  for (int e = threadIdx.x; e < E; e += kPermThreads) {
    int32_t run = 0;
    for (int b0 = 0; b0 < nblk; b0 += kScanBatch) {
      int32_t c[kScanBatch];
#pragma unroll
      for (int u = 0; u < kScanBatch; ++u) c[u] = table[(int64_t)min(b0 + u, nblk - 1) * E + e];
#pragma unroll
      for (int u = 0; u < kScanBatch; ++u) run += b0 + u < nblk ? c[u] : 0;
    }
    tot[e] = run;
  }
  __syncthreads();
  int32_t carry = 0;
  for (int e0 = 0; e0 < E; e0 += kPermThreads) {
    int e = e0 + threadIdx.x;
    int32_t v = e < E ? tot[e] : 0;
    int32_t ex = block_excl_scan(v, wsum, &range_total);
    if (e < E) {
      offsets[e] = carry + ex;
      tot[e] = carry + ex;
    }
    carry += range_total;
    __syncthreads();
  }
  if (threadIdx.x == 0) offsets[E] = carry;
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kPermThreads) {
    int32_t run = tot[e];
    for (int b0 = 0; b0 < nblk; b0 += kScanBatch) {
      int32_t c[kScanBatch];
#pragma unroll
      for (int u = 0; u < kScanBatch; ++u) c[u] = table[(int64_t)min(b0 + u, nblk - 1) * E + e];
#pragma unroll
      for (int u = 0; u < kScanBatch; ++u) {
        if (b0 + u < nblk) {
          table[(int64_t)(b0 + u) * E + e] = run;
          run += c[u];
        }
      }
    }
  }
}

__global__ __launch_bounds__(kPermThreads) void permute_scatter(const int32_t* __restrict__ ids, int64_t R, int E,
                                                                int nbits, const int32_t* __restrict__ table,
                                                                int32_t* __restrict__ sorted_slots,
                                                                int32_t* __restrict__ slot_rows) {
  __shared__ uint16_t cnt[kPermSub][kERange];
  __shared__ int32_t tot[kERange];
  const int64_t base = (int64_t)blockIdx.x * kPermChunk;
  SubRanks r;
  rank_subchunks(ids, R, E, nbits, base, r);
  const int32_t* brow = table + (int64_t)blockIdx.x * E;
  const int nsub = (int)min((int64_t)kPermSub, (R - base + kWave - 1) / kWave);
  for (int e0 = 0; e0 < E; e0 += kERange) {
    subchunk_prefix(r, e0, cnt, tot, nsub);
    write_rows(r, e0, cnt, brow + e0, R, base, sorted_slots, slot_rows);
    __syncthreads();
  }
}

moe_status launch_permute(const int32_t* ids, int64_t T, int top_k, int E, int32_t* offsets,
                          int32_t* sorted_slots, int32_t* slot_rows, void* ws, hipStream_t stream) {
  int64_t R = T * top_k;
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  int64_t nblk = (R + kPermChunk - 1) / kPermChunk;
  if (nblk <= 1) {
    hipLaunchKernelGGL(permute_single, dim3(1), dim3(kPermThreads), 0, stream, ids, R, E, nbits, offsets,
                       sorted_slots, slot_rows);
    return launch_status("moe_permute");
  }
  int32_t* table = (int32_t*)ws;
  hipLaunchKernelGGL(permute_count, dim3((uint32_t)nblk), dim3(kPermThreads), 0, stream, ids, R, E, table);
  hipLaunchKernelGGL(permute_scan, dim3(1), dim3(kPermThreads), 0, stream, table, (int)nblk, E, offsets);
  hipLaunchKernelGGL(permute_scatter, dim3((uint32_t)nblk), dim3(kPermThreads), 0, stream, ids, R, E, nbits,
                     table, sorted_slots, slot_rows);
  return launch_status("moe_permute");
}

}  // namespace moe
