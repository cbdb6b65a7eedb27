// Group-limited sigmoid top-k router: one wavefront per token, float64 scores.
//
// "MiMo-V2.6-Flash -- REAP-50" card, "Pruning Method": grouped sigmoid top-k
// routing, experts reshaped to [n_group, E / n_group], topk_group groups kept,
// num_experts_per_tok experts taken, weights scaled by routed_scaling_factor;
// "Evaluation Status Note": e_score_correction_bias.  The selection rules
// where the card is silent (top-2 group score, bias for selection only,
// lower-index tie-breaks, normalisation) are documented in moe_fp4.h.
//
// Lane l of the wave owns experts l, l+64, l+128, l+192 (E <= 256), so every
// load of the logits row is coalesced.  The reductions run in registers:
// within a row of 16 lanes with DPP moves (quad permutes, half-row and row
// mirrors), across rows with the gfx950 16- and 32-lane swaps, so a wave-wide
// maximum costs a few dozen cycles per level instead of an LDS round trip.
//   * group score (sum of the two largest biased scores): a segmented top-2
//     merge over the group's lanes when the group size is a power of two, an
//     LDS scan otherwise;
//   * kept groups: every lane ranks the group scores (ties to the lower index);
//   * experts: top_k rounds of a wave-wide maximum over order-preserving
//     64-bit keys of the biased scores, then the lowest expert index holding
//     that key (ties to the lower index) from one ballot per register.
// All loads of a row are issued before any of them is used.
#include "permute.h"

namespace moe {

constexpr int kRouteMaxPer = 4;        // experts per lane, E <= 256
constexpr int kRouteWaves = 4;         // tokens per 256-thread block

// ---- cross-lane moves of 32- and 64-bit values
template <int CTRL>
__device__ __forceinline__ int dpp_i32(int x) {
  return __builtin_amdgcn_update_dpp(x, x, CTRL, 0xF, 0xF, false);
}
// partner across the 16-lane row pair (l ^ 16) and across the wave halves (l ^ 32)
__device__ __forceinline__ int swap16_i32(int x) {
  auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  return (threadIdx.x & 16) ? r[0] : r[1];
}
__device__ __forceinline__ int swap32_i32(int x) {
  auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return (threadIdx.x & 32) ? r[0] : r[1];
}
// level L of a butterfly over aligned groups of 2^(L+1) lanes: the partner is
// always in the other half of the group (quad permutes, then the half-row and
// row mirrors, then the swaps)
template <int L>
__device__ __forceinline__ int partner_i32(int x) {
  if constexpr (L == 0) return dpp_i32<0xB1>(x);        // quad_perm [1,0,3,2]
  else if constexpr (L == 1) return dpp_i32<0x4E>(x);   // quad_perm [2,3,0,1]
  else if constexpr (L == 2) return dpp_i32<0x141>(x);  // row_half_mirror
  else if constexpr (L == 3) return dpp_i32<0x140>(x);  // row_mirror
  else if constexpr (L == 4) return swap16_i32(x);
  else return swap32_i32(x);
}
template <int L>
__device__ __forceinline__ double partner_f64(double x) {
  const uint64_t u = (uint64_t)__double_as_longlong(x);
  const uint32_t lo = (uint32_t)partner_i32<L>((int)(uint32_t)u);
  const uint32_t hi = (uint32_t)partner_i32<L>((int)(uint32_t)(u >> 32));
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// ---- order-preserving keys: for doubles that are not NaN, x > y exactly when
// key(x) > key(y), and equal values get equal keys (a biased score is never
// -0, since a sigmoid is >= +0).  Key 0 is below every real key: "no candidate".
__device__ __forceinline__ uint64_t order_key(double x) {
  const uint64_t b = (uint64_t)__double_as_longlong(x);
  return (b >> 63) ? ~b : (b | 0x8000000000000000ull);
}
template <int L>
__device__ __forceinline__ uint64_t partner_u64(uint64_t x) {
  const uint32_t lo = (uint32_t)partner_i32<L>((int)(uint32_t)x);
  const uint32_t hi = (uint32_t)partner_i32<L>((int)(uint32_t)(x >> 32));
  return ((uint64_t)hi << 32) | lo;
}
template <int L>
__device__ __forceinline__ void max_level(uint64_t& k) {
  const uint64_t o = partner_u64<L>(k);
  k = o > k ? o : k;
}
// every lane gets the wave's largest key
__device__ __forceinline__ uint64_t wave_max_key(uint64_t k) {
  max_level<0>(k);
  max_level<1>(k);
  max_level<2>(k);
  max_level<3>(k);
  max_level<4>(k);
  max_level<5>(k);
  return k;
}

// ---- top-2 of a multiset as (b1 >= b2); merging two disjoint halves
__device__ __forceinline__ void top2_merge(double& b1, double& b2, double o1, double o2) {
  const double n2 = (b1 >= o1) ? fmax(b2, o1) : fmax(b1, o2);
  b1 = fmax(b1, o1);
  b2 = n2;
}
template <int L>
__device__ __forceinline__ void top2_level(double& b1, double& b2) {
  top2_merge(b1, b2, partner_f64<L>(b1), partner_f64<L>(b2));
}
// segmented over aligned groups of 2^levels lanes
__device__ __forceinline__ void top2_segment(double& b1, double& b2, int levels) {
  if (levels > 0) top2_level<0>(b1, b2);
  if (levels > 1) top2_level<1>(b1, b2);
  if (levels > 2) top2_level<2>(b1, b2);
  if (levels > 3) top2_level<3>(b1, b2);
  if (levels > 4) top2_level<4>(b1, b2);
  if (levels > 5) top2_level<5>(b1, b2);
}

// The kRouteWaves tokens of this block, one per wave.  All threads of the
// block must call it (it synchronises the block).
static_assert(kPermThreads == 256, "the router block runs the permutation");

// Wave wv routes token tb + wv; the logits are FP32 (the router output as
// stored) or float64 (the fused router matmul's own sums).
// s_ids (optional, LDS): the block's picks also go there, at [wv * top_k + r]
template <typename LT, int NW = kRouteWaves>
__device__ __forceinline__ void route_tokens(const LT* __restrict__ logits, const float* __restrict__ bias,
                                             int64_t tb, int64_t T, int E, int n_group, int topk_group, int top_k,
                                             float scale, int norm, int32_t* __restrict__ ids,
                                             float* __restrict__ weights, int* s_ids = nullptr) {
  __shared__ double gscore[NW][64];
  __shared__ double cval[NW][256];
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int64_t t0 = tb + wv;
  const bool valid = t0 < T;           // no early exit: the block synchronises below
  const int64_t t = valid ? t0 : T - 1;
  const int gs = E / n_group;
  const bool pow2 = (gs & (gs - 1)) == 0;
  const LT* lrow = logits + t * E;

  // every load in flight at once (lanes past E read expert E - 1 and drop it)
  LT lv[kRouteMaxPer];
  float bv[kRouteMaxPer];
#pragma unroll
  for (int j = 0; j < kRouteMaxPer; ++j) lv[j] = lrow[min(lane + 64 * j, E - 1)];
  if (bias) {
#pragma unroll
    for (int j = 0; j < kRouteMaxPer; ++j) bv[j] = bias[min(lane + 64 * j, E - 1)];
  } else {
#pragma unroll
    for (int j = 0; j < kRouteMaxPer; ++j) bv[j] = 0.0f;
  }
  double s[kRouteMaxPer], c[kRouteMaxPer];
#pragma unroll
  for (int j = 0; j < kRouteMaxPer; ++j) {
    const bool in = lane + 64 * j < E;
    const double sg = 1.0 / (1.0 + exp(-(double)lv[j]));
    s[j] = in ? sg : 0.0;
    c[j] = in ? sg + (double)bv[j] : -INFINITY;
  }

  // ---- group scores -> gscore[wv][g]
  if (pow2) {
    const int levels = 31 - __clz(min(gs, 64));
    double p1[kRouteMaxPer], p2[kRouteMaxPer];
#pragma unroll
    for (int j = 0; j < kRouteMaxPer; ++j) {
      p1[j] = c[j];
      p2[j] = -INFINITY;
      top2_segment(p1[j], p2[j], levels);
    }
    if (gs <= 64) {
      // lane l heads the group of experts l + 64j .. l + 64j + gs - 1
      if ((lane & (gs - 1)) == 0) {
#pragma unroll
        for (int j = 0; j < kRouteMaxPer; ++j)
          if (lane + 64 * j < E) gscore[wv][(lane + 64 * j) / gs] = p1[j] + p2[j];
      }
    } else if (lane == 0) {
      // a group spans gs / 64 rows of the wave: merge them in order
      for (int g = 0; g < n_group; ++g) {
        double b1 = -INFINITY, b2 = -INFINITY;
#pragma unroll
        for (int j = 0; j < kRouteMaxPer; ++j)
          if ((64 * j) / gs == g && 64 * j < E) top2_merge(b1, b2, p1[j], p2[j]);
        gscore[wv][g] = b1 + b2;
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < kRouteMaxPer; ++j)
      if (lane + 64 * j < E) cval[wv][lane + 64 * j] = c[j];
    __syncthreads();
    if (lane < n_group) {
      double b1 = -INFINITY, b2 = -INFINITY;
      for (int e = lane * gs; e < (lane + 1) * gs; ++e) {
        const double v = cval[wv][e];
        if (v > b1) { b2 = b1; b1 = v; }
        else if (v > b2) { b2 = v; }
      }
      gscore[wv][lane] = b1 + b2;
    }
  }
  __syncthreads();

  // ---- keep the topk_group best groups: lane g ranks group g
  bool keep = false;
  if (lane < n_group) {
    const double mine = gscore[wv][lane];
    int rank = 0;
    for (int g = 0; g < n_group; ++g) {
      const double o = gscore[wv][g];
      rank += (o > mine || (o == mine && g < lane)) ? 1 : 0;
    }
    keep = rank < topk_group;
  }
  const uint64_t kept = __ballot(keep);

  // ---- top_k experts among the kept groups
  uint64_t key[kRouteMaxPer];
#pragma unroll
  for (int j = 0; j < kRouteMaxPer; ++j) {
    const int e = lane + 64 * j;
    const bool elig = (e < E) && ((kept >> (e / gs)) & 1ull);
    key[j] = elig ? order_key(c[j]) : 0ull;
  }
  double sel_s = 0.0, tot = 0.0;     // lane r < top_k keeps the r-th pick
  int sel_e = 0;
  for (int r = 0; r < top_k; ++r) {
    uint64_t m = key[0];
#pragma unroll
    for (int j = 1; j < kRouteMaxPer; ++j) m = key[j] > m ? key[j] : m;
    m = wave_max_key(m);
    // the lowest expert index whose key is the maximum (a uniform value)
    int pick = 0;
#pragma unroll
    for (int j = kRouteMaxPer - 1; j >= 0; --j) {
      const uint64_t hit = __ballot((key[j] == m) & (lane + 64 * j < E));
      pick = hit ? 64 * j + __ffsll((long long)hit) - 1 : pick;
    }
    const int pl = pick & 63, pj = pick >> 6;
    // its owner lane supplies the unbiased score; the pick leaves the candidates
    double sj = s[0];
#pragma unroll
    for (int j = 1; j < kRouteMaxPer; ++j) sj = pj == j ? s[j] : sj;
#pragma unroll
    for (int j = 0; j < kRouteMaxPer; ++j) key[j] = ((pj == j) & (lane == pl)) ? 0ull : key[j];
    const uint64_t su = (uint64_t)__double_as_longlong(sj);
    const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)su, pl);
    const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(su >> 32), pl);
    const double sv = __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
    tot += sv;                                     // sum in pick order
    if (lane == r) { sel_s = sv; sel_e = pick; }
  }
  if (valid && lane < top_k) {
    const double w = norm ? sel_s / tot * (double)scale : sel_s * (double)scale;
    ids[t * top_k + lane] = sel_e;
    weights[t * top_k + lane] = (float)w;
    if (s_ids) s_ids[wv * top_k + lane] = sel_e;
  }
}

__global__ __launch_bounds__(256) void route_kernel(const float* __restrict__ logits,
                                                    const float* __restrict__ bias, int64_t T, int E,
                                                    int n_group, int topk_group, int top_k, float scale,
                                                    int norm, int32_t* __restrict__ ids,
                                                    float* __restrict__ weights) {
  route_tokens(logits, bias, (int64_t)blockIdx.x * kRouteWaves, T, E, n_group, topk_group, top_k, scale, norm, ids,
               weights);
}

// Router and permutation in one launch (R = T * top_k <= kPermChunk).  A
// single block (T <= 4) routes and permutes with no hand-off.  Otherwise each
// block routes its tokens, then adds one to *counter; the block that brings
// it to gridDim.x has every block's ids behind it and runs the permutation,
// then sets the counter back to zero for the next launch.  The fences are
// device-scope: a release by every wave after its own stores (before the block
// counts itself in) and an acquire by the last block before its loads; the
// other blocks skip the acquire and its cache invalidation.  The blocks sit on
// different XCDs, whose L2 caches are not coherent with each other.
__global__ __launch_bounds__(256) void route_permute_kernel(const float* __restrict__ logits,
                                                            const float* __restrict__ bias, int64_t T, int E,
                                                            int n_group, int topk_group, int top_k, float scale,
                                                            int norm, int32_t* __restrict__ ids,
                                                            float* __restrict__ weights, int nbits,
                                                            int32_t* __restrict__ offsets,
                                                            int32_t* __restrict__ sorted_slots,
                                                            int32_t* __restrict__ slot_rows,
                                                            uint32_t* __restrict__ counter) {
  __shared__ int s_last;
  __shared__ int s_ids[kRouteWaves * 16];                      // top_k <= 16
  route_tokens(logits, bias, (int64_t)blockIdx.x * kRouteWaves, T, E, n_group, topk_group, top_k, scale, norm, ids,
               weights, gridDim.x == 1 ? s_ids : nullptr);
  if (gridDim.x == 1) {
    // one block routes every token (R = T * top_k <= 64 slots) and keeps its
    // picks in LDS: no global round trip, no device-scope cache write-back or
    // invalidation, no counter; the stable counting sort is a direct count
    // per slot and per expert
    __syncthreads();
    const int R = (int)T * top_k;
    if (threadIdx.x < R) {
      // row of slot j: slots of lower experts, then lower slots of the same expert
      const int j = threadIdx.x, e = s_ids[j];
      int row = 0;
      for (int i = 0; i < R; ++i) row += (s_ids[i] < e || (s_ids[i] == e && i < j)) ? 1 : 0;
      sorted_slots[row] = j;
      slot_rows[j] = row;
    }
    for (int e = threadIdx.x; e <= E; e += blockDim.x) {
      int c = 0;
      for (int i = 0; i < R; ++i) c += s_ids[i] < e ? 1 : 0;
      offsets[e] = c;
    }
    return;
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");   // each wave, after its own stores
  __syncthreads();
  if (threadIdx.x == 0) s_last = atomicAdd(counter, 1u) == gridDim.x - 1;
  __syncthreads();
  if (!s_last) return;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  permute_one_chunk(ids, T * top_k, E, nbits, offsets, sorted_slots, slot_rows);
  if (threadIdx.x == 0) atomicExch(counter, 0u);
}

moe_status launch_route(const float* logits, const float* bias, int64_t T, const moe_route_params* p,
                        int32_t* ids, float* weights, hipStream_t stream) {
  if (T == 0) return MOE_OK;
  int64_t blocks = (T + kRouteWaves - 1) / kRouteWaves;
  hipLaunchKernelGGL(route_kernel, dim3((uint32_t)blocks), dim3(256), 0, stream, logits, bias, T,
                     p->num_experts, p->n_group, p->topk_group, p->top_k, p->routed_scaling_factor,
                     p->norm_topk_prob, ids, weights);
  return launch_status("moe_route");
}

bool route_permute_fits(int64_t T, int top_k) { return T >= 1 && T * top_k <= kPermChunk; }

// ------------------------------------------------- router matmul + top-k
// The router's matmul, then the group top-k on its float64 logits ("MiMo-
// V2.6-Flash-MOPD on one RTX PRO 6000", "What makes it fast": one router
// matmul and a fused top-k per layer; "MiMo-V2.6-Flash-RL Mixed-Quant GGUF",
// "Quantization targets": routers stay F32).  logits[t, e] = sum_k x[t, k]
// W[e, k] for bf16 x and the FP32 weight W: each product is exact in float64
// and the sum is float64, in a fixed order, so the selection sees the
// oracle's float64 logits up to the order of one float64 summation.  Two
// launches on the caller's stream: a hand-off inside one launch (a device-
// scope release by every workgroup and an acquire by the last, i.e. an L2
// write-back per workgroup and an L2 invalidation) measured slower than the
// kernel boundary.
//   * T > 16 or hidden != 4096: workgroup (b, q) of 16 waves computes a
//     16-token x 16-expert tile (tokens 16q.., experts 16b..); wave w takes the
//     w-th sixteenth of the hidden dimension and runs float64 16x16x4 MFMAs
//     over it, each lane group g of the wave supplying a contiguous quarter of
//     that range (the k of one MFMA is one value from each lane group), so
//     every lane reads contiguous 16-byte pieces of its token row and expert
//     row; the 16 partial tiles meet in LDS and are added in wave order.
constexpr int kGemvWaves = 16;
constexpr int kGemvTile = 16;

typedef double f64x4 __attribute__((ext_vector_type(4)));

// KG: values per lane group known at compile time (64 for hidden 4096, so the
// whole loop unrolls and every load is in flight before the first MFMA), or 0.
template <int KG>
__global__ __launch_bounds__(kGemvWaves * 64) void route_gemv_kernel(
    const uint16_t* __restrict__ x, const float* __restrict__ W, int64_t T, int H, int E,
    double* __restrict__ logits) {
  __shared__ double part[kGemvWaves][kGemvTile * kGemvTile];
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int64_t t0 = (int64_t)blockIdx.y * kGemvTile;
  const int e0 = blockIdx.x * kGemvTile;
  const int64_t t = min(t0 + r, T - 1);                       // rows past the end reread the last one
  const int e = min(e0 + r, E - 1);
  const int kg = KG > 0 ? KG : H / (kGemvWaves * 4);          // values per lane group (a multiple of 8)
  const uint16_t* xr = x + t * H + (int64_t)(wv * 4 + g) * kg;
  const float* wr = W + (int64_t)e * H + (int64_t)(wv * 4 + g) * kg;
  f64x4 acc = {0.0, 0.0, 0.0, 0.0};
  auto chunk = [&](int m) {
    const u32x4 xv = *(const u32x4*)(xr + m);
    const f32x4 w0 = *(const f32x4*)(wr + m);
    const f32x4 w1 = *(const f32x4*)(wr + m + 4);
    // D[token][expert] += x[token][k] W[expert][k]: A = token rows, B = expert columns
    acc = __builtin_amdgcn_mfma_f64_16x16x4f64((double)bf16_lo(xv[0]), (double)w0[0], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f64_16x16x4f64((double)bf16_hi(xv[0]), (double)w0[1], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f64_16x16x4f64((double)bf16_lo(xv[1]), (double)w0[2], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f64_16x16x4f64((double)bf16_hi(xv[1]), (double)w0[3], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f64_16x16x4f64((double)bf16_lo(xv[2]), (double)w1[0], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f64_16x16x4f64((double)bf16_hi(xv[2]), (double)w1[1], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f64_16x16x4f64((double)bf16_lo(xv[3]), (double)w1[2], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f64_16x16x4f64((double)bf16_hi(xv[3]), (double)w1[3], acc, 0, 0, 0);
  };
  if constexpr (KG > 0) {
#pragma unroll
    for (int m = 0; m < KG; m += 8) chunk(m);
  } else {
    for (int m = 0; m < kg; m += 8) chunk(m);
  }
  // the float64 16x16x4 MFMA leaves D[token g + 4 i][expert r] in lane (r, g), element i (measured)
#pragma unroll
  for (int i = 0; i < 4; ++i) part[wv][(g + 4 * i) * kGemvTile + r] = acc[i];
  __syncthreads();
  if (threadIdx.x < kGemvTile * kGemvTile) {
    double sum = 0.0;
#pragma unroll
    for (int w = 0; w < kGemvWaves; ++w) sum += part[w][threadIdx.x];
    const int64_t tt = t0 + threadIdx.x / kGemvTile;
    const int ee = e0 + threadIdx.x % kGemvTile;
    if (tt < T && ee < E) logits[tt * E + ee] = sum;
  }
}

// Small batches (T <= 16, hidden 4096): workgroups of 16 waves over 8 experts
// each.  Wave w takes the w-th sixteenth of the hidden dimension; lane l takes
// expert l / 8 of the workgroup and the (l % 8)-th eighth of the wave's range,
// so it reads 32 contiguous weights and the same range of each token row (four
// tokens at a time), the loads issued before the first product.  Each lane sums its products in
// order in float64, the eight lanes of an expert are added by a butterfly
// (the same result in each), and the 16 wave sums are added in wave order in
// LDS.
constexpr int kGemvSmallE = 8;        // experts per workgroup

constexpr int kGemvSmallH = 4096;

template <int TT>
__global__ __launch_bounds__(1024) void route_gemv_small_kernel(
    const uint16_t* __restrict__ x, const float* __restrict__ W, int T, int H, int E, double* __restrict__ logits) {
  __shared__ double part[kGemvWaves][kGemvSmallE][TT];
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int el = lane >> 3, q = lane & 7;
  const int e = min((int)blockIdx.x * kGemvSmallE + el, E - 1);
  constexpr int kq = kGemvSmallH / (kGemvWaves * kGemvSmallE);   // 32 values per lane
  const int64_t k0 = (int64_t)wv * (H / kGemvWaves) + (int64_t)q * kq;
  const float* wr = W + (int64_t)e * H + k0;
  // tokens in groups of 4 (the loads of one group in flight at once)
  for (int tg = 0; tg < TT; tg += 4) {
    double acc[4] = {0.0, 0.0, 0.0, 0.0};
    {
      f32x4 w[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) w[i] = *(const f32x4*)(wr + 4 * i);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (TT == 1 && j > 0) break;
        const uint16_t* xr = x + (int64_t)min(tg + j, T - 1) * H + k0;
        u32x4 xv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) xv[i] = *(const u32x4*)(xr + 8 * i);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const uint32_t lo = xv[i >> 1][2 * (i & 1)], hi = xv[i >> 1][2 * (i & 1) + 1];
          acc[j] = fma((double)bf16_lo(lo), (double)w[i][0], acc[j]);
          acc[j] = fma((double)bf16_hi(lo), (double)w[i][1], acc[j]);
          acc[j] = fma((double)bf16_lo(hi), (double)w[i][2], acc[j]);
          acc[j] = fma((double)bf16_hi(hi), (double)w[i][3], acc[j]);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      acc[j] += __shfl_xor(acc[j], 1, kWave);
      acc[j] += __shfl_xor(acc[j], 2, kWave);
      acc[j] += __shfl_xor(acc[j], 4, kWave);
      if (q == 0 && tg + j < TT) part[wv][el][tg + j] = acc[j];
    }
  }
  __syncthreads();
  if (threadIdx.x < kGemvSmallE * T) {
    const int t = threadIdx.x / kGemvSmallE, ee = threadIdx.x % kGemvSmallE;
    double sum = 0.0;
#pragma unroll
    for (int w = 0; w < kGemvWaves; ++w) sum += part[w][ee][t];
    const int eo = blockIdx.x * kGemvSmallE + ee;
    if (eo < E) logits[(int64_t)t * E + eo] = sum;
  }
}

// the group top-k of moe_route on the float64 logits, one wave per token
__global__ __launch_bounds__(256) void route_f64_kernel(const double* __restrict__ logits,
                                                        const float* __restrict__ bias, int64_t T, int E,
                                                        int n_group, int topk_group, int top_k, float scale,
                                                        int norm, int32_t* __restrict__ ids,
                                                        float* __restrict__ weights) {
  route_tokens(logits, bias, (int64_t)blockIdx.x * kRouteWaves, T, E, n_group, topk_group, top_k, scale, norm, ids,
               weights);
}

size_t route_gemv_ws_bytes(int64_t T, int E) {
  return ((size_t)T * (size_t)E * sizeof(double) + 255) & ~(size_t)255;   // the float64 logits
}

moe_status launch_route_gemv(const void* x, const float* W, const float* bias, int64_t T, int H,
                             const moe_route_params* p, int32_t* ids, float* weights, void* ws, hipStream_t stream) {
  if (T == 0) return MOE_OK;
  const int E = p->num_experts;
  double* logits = (double*)ws;
  if (T <= kGemvTile && H == kGemvSmallH) {
    auto small = T == 1   ? route_gemv_small_kernel<1>
                 : T <= 4 ? route_gemv_small_kernel<4>
                 : T <= 8 ? route_gemv_small_kernel<8>
                          : route_gemv_small_kernel<16>;
    hipLaunchKernelGGL(small, dim3((uint32_t)((E + kGemvSmallE - 1) / kGemvSmallE)), dim3(1024), 0, stream,
                       (const uint16_t*)x, W, (int)T, H, E, logits);
  } else {
    const dim3 grid((uint32_t)((E + kGemvTile - 1) / kGemvTile), (uint32_t)((T + kGemvTile - 1) / kGemvTile));
    hipLaunchKernelGGL(H == 4096 ? route_gemv_kernel<64> : route_gemv_kernel<0>, grid, dim3(kGemvWaves * 64), 0,
                       stream, (const uint16_t*)x, W, T, H, E, logits);
  }
  const moe_status st = launch_status("moe_route_gemv");
  if (st != MOE_OK) return st;
  hipLaunchKernelGGL(route_f64_kernel, dim3((uint32_t)((T + kRouteWaves - 1) / kRouteWaves)), dim3(256), 0, stream,
                     logits, bias, T, E, p->n_group, p->topk_group, p->top_k, p->routed_scaling_factor,
                     p->norm_topk_prob, ids, weights);
  return launch_status("moe_route_gemv");
}

moe_status launch_route_permute(const float* logits, const float* bias, int64_t T, const moe_route_params* p,
                                int32_t* ids, float* weights, int32_t* offsets, int32_t* sorted_slots,
                                int32_t* slot_rows, uint32_t* counter, hipStream_t stream) {
  int nbits = 0;
  while ((1 << nbits) < p->num_experts) ++nbits;
  const int64_t blocks = (T + kRouteWaves - 1) / kRouteWaves;
  hipLaunchKernelGGL(route_permute_kernel, dim3((uint32_t)blocks), dim3(256), 0, stream, logits, bias, T,
                     p->num_experts, p->n_group, p->topk_group, p->top_k, p->routed_scaling_factor,
                     p->norm_topk_prob, ids, weights, nbits, offsets, sorted_slots, slot_rows, counter);
  return launch_status("moe_route_permute");
}

}  // namespace moe
