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
// load of the logits row is coalesced.  Group scores live in LDS; each
// selection round is a wave-wide argmax by shuffles over (value, index) pairs.
#include "common.h"

namespace moe {

constexpr int kRouteMaxPer = 4;        // experts per lane, E <= 256
constexpr int kRouteWaves = 4;         // tokens per 256-thread block

__device__ __forceinline__ void wave_argmax(double& v, int& i) {
  // maximise v; on equal v keep the lower index; index -1 means "empty"
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    double ov = __shfl_xor(v, off, kWave);
    int oi = __shfl_xor(i, off, kWave);
    bool take = (oi >= 0) && (i < 0 || ov > v || (ov == v && oi < i));
    if (take) { v = ov; i = oi; }
  }
}

__global__ __launch_bounds__(256) void route_kernel(const float* __restrict__ logits,
                                                    const float* __restrict__ bias, int64_t T, int E,
                                                    int n_group, int topk_group, int top_k, float scale,
                                                    int norm, int32_t* __restrict__ ids,
                                                    float* __restrict__ weights) {
  __shared__ double gscore[kRouteWaves][64];
  __shared__ double cval[kRouteWaves][256];
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int64_t t0 = (int64_t)blockIdx.x * kRouteWaves + wv;
  const bool valid = t0 < T;           // no early exit: the block synchronises below
  const int64_t t = valid ? t0 : T - 1;
  const int gs = E / n_group;
  const float* lrow = logits + t * E;

  double s[kRouteMaxPer], c[kRouteMaxPer];
#pragma unroll
  for (int j = 0; j < kRouteMaxPer; ++j) {
    int e = lane + 64 * j;
    if (e < E) {
      double l = (double)lrow[e];
      s[j] = 1.0 / (1.0 + exp(-l));
      c[j] = s[j] + (bias ? (double)bias[e] : 0.0);
      cval[wv][e] = c[j];
    } else {
      s[j] = 0.0;
      c[j] = 0.0;
    }
  }
  __syncthreads();

  // group score: sum of the two largest c in the group (lane g scans group g)
  if (lane < n_group) {
    double b1 = -INFINITY, b2 = -INFINITY;
    for (int e = lane * gs; e < (lane + 1) * gs; ++e) {
      double v = cval[wv][e];
      if (v > b1) { b2 = b1; b1 = v; }
      else if (v > b2) { b2 = v; }
    }
    gscore[wv][lane] = b1 + b2;
  }
  __syncthreads();

  // keep topk_group groups: repeated wave argmax over the group scores
  uint64_t kept = 0;   // bit g set when group g is kept
  for (int r = 0; r < topk_group; ++r) {
    double v = -INFINITY;
    int i = -1;
    if (lane < n_group && !((kept >> lane) & 1ull)) { v = gscore[wv][lane]; i = lane; }
    wave_argmax(v, i);
    kept |= 1ull << i;
  }

  // top_k experts among kept groups
  bool taken[kRouteMaxPer];
  bool elig[kRouteMaxPer];
#pragma unroll
  for (int j = 0; j < kRouteMaxPer; ++j) {
    int e = lane + 64 * j;
    taken[j] = false;
    elig[j] = (e < E) && ((kept >> (e / gs)) & 1ull);
  }
  double sel_s = 0.0;    // lane r < top_k keeps the r-th pick's score
  int sel_e = 0;
  for (int r = 0; r < top_k; ++r) {
    double v = -INFINITY;
    int i = -1;
#pragma unroll
    for (int j = 0; j < kRouteMaxPer; ++j) {
      int e = lane + 64 * j;
      if (elig[j] && !taken[j] && (i < 0 || c[j] > v)) { v = c[j]; i = e; }
    }
    wave_argmax(v, i);
#pragma unroll
    for (int j = 0; j < kRouteMaxPer; ++j)
      if (lane + 64 * j == i) taken[j] = true;
    // the owner broadcasts the unbiased score of the pick
    double sv = 0.0;
#pragma unroll
    for (int j = 0; j < kRouteMaxPer; ++j)
      if (lane + 64 * j == i) sv = s[j];
    int owner = i & 63;
    sv = __shfl(sv, owner, kWave);
    if (lane == r) { sel_s = sv; sel_e = i; }
  }
  // weights: normalise over the picks (sum in pick order), scale
  double tot = 0.0;
  for (int r = 0; r < top_k; ++r) tot += __shfl(sel_s, r, kWave);
  if (valid && lane < top_k) {
    double w = norm ? sel_s / tot * (double)scale : sel_s * (double)scale;
    ids[t * top_k + lane] = sel_e;
    weights[t * top_k + lane] = (float)w;
  }
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

}  // namespace moe
