// Device code of the token permutation shared by its kernels and by the
// router's fused variant: wave-level stable ranking of the slots of a chunk
// and the single-chunk counting sort.  The algorithm is described in
// permute.hip.
#pragma once
#include "common.h"

namespace moe {


constexpr int kPermThreads = 256;
constexpr int kPermChunk = 2048;                                  // slots per block
constexpr int kPermSub = kPermChunk / kWave;                      // 32 sub-chunks of 64 slots
constexpr int kSubPerWave = kPermSub / (kPermThreads / kWave);    // 8 per wave
constexpr int kPermMaxE = 1024;
constexpr int kERange = 256;                                      // experts per LDS pass


// Sub-chunk q of wave w: interleaved over the waves, so a short chunk (a
// decode batch) still spreads its slots over every wave.
__device__ __forceinline__ int sub_of(int w, int q) { return q * (kPermThreads / kWave) + w; }

// Ranks of this wave's 8 sub-chunks: expert id (-1 when absent/invalid), rank
// among equal ids inside the 64-slot sub-chunk, and the group size.
struct SubRanks {
  int e[kSubPerWave];
  int rank[kSubPerWave];
  int size[kSubPerWave];
};

__device__ __forceinline__ void rank_subchunks(const int32_t* __restrict__ ids, int64_t R, int E, int nbits,
                                               int64_t base, SubRanks& r) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  // all of the wave's loads in flight before the first is used (slots past R
  // read slot base instead; an empty chunk, R = 0, reads nothing)
  int v[kSubPerWave];
  if (R > base) {
#pragma unroll
    for (int q = 0; q < kSubPerWave; ++q) {
      const int64_t s = base + (int64_t)sub_of(w, q) * kWave + lane;
      v[q] = ids[s < R ? s : base];
    }
  } else {
#pragma unroll
    for (int q = 0; q < kSubPerWave; ++q) v[q] = -1;
  }
#pragma unroll
  for (int q = 0; q < kSubPerWave; ++q) {
    const int64_t s = base + (int64_t)sub_of(w, q) * kWave + lane;
    const int e = (s < R && v[q] >= 0 && v[q] < E) ? v[q] : -1;
    // lanes of an absent slot (e = -1, every bit set) stay out of every valid
    // lane's peers through the first ballot; their own ranks are never used.
    // A sub-chunk with no slot (past R) skips the bit ballots.
    uint64_t peers = __ballot(e >= 0);
    for (int b = 0; b < nbits && peers != 0; ++b) {
      const bool bit = (e >> b) & 1;
      const uint64_t m = __ballot(bit);
      peers &= bit ? m : ~m;
    }
    r.e[q] = e;
    r.rank[q] = __popcll(peers & ((1ull << lane) - 1ull));
    r.size[q] = __popcll(peers);
  }
}

// cnt[sub][e - e0] <- group sizes of the sub-chunks, then exclusive prefix over
// the sub-chunks.  Returns (in tot, for threads e-e0 < 256) the chunk total.
// Only the first nsub sub-chunks hold slots (a short last chunk uses fewer).
__device__ __forceinline__ void subchunk_prefix(const SubRanks& r, int e0, uint16_t (*cnt)[kERange],
                                                int32_t* tot, int nsub) {
  const int w = threadIdx.x >> 6;
  for (int i = threadIdx.x; i < nsub * kERange; i += kPermThreads) (&cnt[0][0])[i] = 0;
  __syncthreads();
#pragma unroll
  for (int q = 0; q < kSubPerWave; ++q) {
    int e = r.e[q];
    if (e >= e0 && e < e0 + kERange && r.rank[q] == 0) cnt[sub_of(w, q)][e - e0] = (uint16_t)r.size[q];
    // (a sub-chunk past nsub holds no slot, so e < 0 there and nothing is written)
  }
  __syncthreads();
  {
    int j = threadIdx.x;    // one expert of the range per thread
    int32_t run = 0;
    for (int sub = 0; sub < nsub; ++sub) {
      int32_t c = cnt[sub][j];
      cnt[sub][j] = (uint16_t)run;
      run += c;
    }
    tot[j] = run;
  }
  __syncthreads();
}

__device__ __forceinline__ void write_rows(const SubRanks& r, int e0, const uint16_t (*cnt)[kERange],
                                           const int32_t* ebase /* LDS or global, indexed e - e0 */,
                                           int64_t R, int64_t base, int32_t* __restrict__ sorted_slots,
                                           int32_t* __restrict__ slot_rows) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int q = 0; q < kSubPerWave; ++q) {
    const int sub = sub_of(w, q);
    const int64_t s = base + (int64_t)sub * kWave + lane;
    int e = r.e[q];
    if (e >= e0 && e < e0 + kERange) {
      int32_t pos = ebase[e - e0] + (int32_t)cnt[sub][e - e0] + r.rank[q];
      sorted_slots[pos] = (int32_t)s;
      slot_rows[s] = pos;
    } else if (e < 0 && e0 == 0 && s < R) {
      slot_rows[s] = -1;
    }
  }
}

// Exclusive scan of v over threads (block of 256); returns the exclusive value,
// total in *total (LDS).
__device__ __forceinline__ int32_t block_excl_scan(int32_t v, int32_t* wsum, int32_t* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int32_t x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    int32_t y = __shfl_up(x, off, kWave);
    if (lane >= off) x += y;
  }
  if (lane == 63) wsum[w] = x;
  __syncthreads();
  int32_t before = 0;
  for (int i = 0; i < w; ++i) before += wsum[i];
  if (threadIdx.x == kPermThreads - 1) *total = before + x;
  __syncthreads();
  return before + x - v;
}

// ---------------------------------------------------------- one chunk
// The whole permutation of R <= kPermChunk slots by one block of kPermThreads
// threads (the single-chunk kernel, and the router's last block).
__device__ __forceinline__ void permute_one_chunk(const int32_t* __restrict__ ids, int64_t R, int E, int nbits,
                                                  int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_slots,
                                                  int32_t* __restrict__ slot_rows) {
  __shared__ uint16_t cnt[kPermSub][kERange];
  __shared__ int32_t tot[kERange];
  __shared__ int32_t wsum[kPermThreads / kWave];
  __shared__ int32_t range_total;
  SubRanks r;
  rank_subchunks(ids, R, E, nbits, 0, r);
  const int nsub = (int)min((int64_t)kPermSub, (R + kWave - 1) / kWave);
  int32_t carry = 0;
  for (int e0 = 0; e0 < E; e0 += kERange) {
    subchunk_prefix(r, e0, cnt, tot, nsub);
    int j = threadIdx.x;
    int32_t v = (e0 + j < E) ? tot[j] : 0;
    int32_t ex = block_excl_scan(v, wsum, &range_total);
    __syncthreads();
    tot[j] = carry + ex;
    if (e0 + j < E) offsets[e0 + j] = carry + ex;
    carry += range_total;
    __syncthreads();
    write_rows(r, e0, cnt, tot, R, 0, sorted_slots, slot_rows);
    __syncthreads();
  }
  if (threadIdx.x == 0) offsets[E] = carry;
}

}  // namespace moe
