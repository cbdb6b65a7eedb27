// Grouped FP4 expert GEMM, MFMA-bound ("prefill") form: many token rows per
// expert, so the kernel is bound by bf16 MFMA throughput.
//
// Same contraction as the weight-streaming kernel (the SwiGLU expert FFN of
// "MiMo-V2.6-Flash -- REAP-50", "Pruning Method"; MXFP4 / NVFP4 weights with
// FP32 accumulation, "AxionML / MiMo-V2.6-Flash-MOPD-NVFP4", "About NVFP4
// quantization"), tiled for reuse:
//   * a workgroup of 8 waves owns a tile of BM token rows x BN weight rows
//     (SwiGLU: BN/2 gate + BN/2 up rows of the same outputs) and walks K in
//     steps of BK = 128; bf16 tokens use 64 x 512 tiles (one wave along
//     tokens, eight along weight rows) where N allows, else 128 x 256 (2 x 4);
//   * each wave dequantises its 64 weight rows from LDS with the gfx950
//     convert instruction and runs 4 x 4 bf16 16x16x32 MFMA tiles (64 tokens
//     x 64 weight rows); the token operands of the next k-slot are read while
//     the current slot's MFMAs run;
//   * LDS layouts are swizzled so the MFMA operand reads are conflict
//     free: token chunk c (16 B) of row r at a linear map of (c, r) in a 256-B row,
//     weight chunk c of row n at c ^ ((n / 2 ^ n / 8) % 4) in a 64-B row;
//   * persistent workgroups: the tile list, ordered (expert, n-tile, m-tile),
//     is cut into one contiguous slice per XCD (workgroup b runs on XCD b % 8),
//     so the workgroups sharing an L2 work on the same experts' token rows and
//     weight slices at the same time.
// Two operand pipelines:
//   * bf16 tokens: every step's operands go from HBM straight into one of
//     three LDS stages (direct-to-LDS loads, no registers), two steps ahead;
//     one barrier per step;
//   * NVFP4 tokens (W4A4): the token rows must be dequantised on the way in,
//     so operands are fetched two steps ahead into registers and written to
//     one of two LDS stages one step ahead.
#pragma once
#include <algorithm>
#include <type_traits>

#include "gemm_common.h"

namespace moe {

constexpr int kPfBK = 128;
constexpr int kPfThreads = 512;                          // 8 waves of 64 tokens x 64 weight rows each
constexpr int kPfMaxE = 1000;                            // tile prefix table in LDS beside three stages
constexpr int kPfXcds = 8;

// Tile shapes: BM token rows x BN weight rows (SwiGLU: BN/2 gate + BN/2 up rows
// of the same outputs), BM/64 waves along tokens x WN along weight rows.
template <int BM_, int BN_>
struct PfShape {
  static constexpr int BM = BM_, BN = BN_;
  static constexpr int WN = 8 / (BM / 64);
  static constexpr int AStage = BM * kPfBK * 2;            // bf16 tokens
  static constexpr int WStage = BN * kPfBK / 2;            // FP4 codes
  static constexpr int SStage = BN * 8;                    // scales (MX uses half), a stage of their own
  static constexpr int Stage = AStage + WStage;
};
// 128 x 256: the NVFP4-token kernel, and N not a multiple of 512 (256 SwiGLU)
using PfTall = PfShape<128, 256>;
// 64 x 512: bf16 tokens; pads experts in 64-row units, reads each token row
// for half as many n-tiles, and dequantises each weight row in one wave only
using PfWide = PfShape<64, 512>;
constexpr int kPfStageMax = PfWide::Stage > PfTall::Stage ? PfWide::Stage : PfTall::Stage;

constexpr int kPfSStageMax = PfWide::SStage > PfTall::SStage ? PfWide::SStage : PfTall::SStage;

// the three stages of the direct-to-LDS pipeline: separate objects, so the
// compiler can tell a stage being read from the stages being filled.  The
// weight scales have stages of their own: inside the token / weight stages,
// the first scale read of each step made the compiler wait for every load in
// flight (the register weight path then drained the pipeline once per step).
__shared__ __attribute__((aligned(16))) uint8_t pf_stage0[kPfStageMax];
__shared__ __attribute__((aligned(16))) uint8_t pf_stage1[kPfStageMax];
__shared__ __attribute__((aligned(16))) uint8_t pf_stage2[kPfStageMax];
__shared__ __attribute__((aligned(16))) uint8_t pf_sstage0[kPfSStageMax];
__shared__ __attribute__((aligned(16))) uint8_t pf_sstage1[kPfSStageMax];
__shared__ __attribute__((aligned(16))) uint8_t pf_sstage2[kPfSStageMax];

typedef __attribute__((address_space(3))) void lds_void_t;

// Token stage: 16-byte chunk c of row r sits at slot P(c) ^ f(r) of the row's
// 256 bytes, P swapping bits 2 and 3 of c, f(r) = r % 4 + 4 * (r / 8 % 2).
// gfx950 serves a ds_read_b128 in lane groups for which the plain c ^ (r % 16)
// puts two lanes on the same banks (measured: half the LDS cycles were
// conflicts); this linear map keeps the 16 lanes of every group on distinct
// banks for each k-slot of the MFMA operand read.
__device__ __forceinline__ int swz_a_slot(int row, int chunk) {
  const int p = (chunk & 3) | ((chunk >> 3) & 1) << 2 | ((chunk >> 2) & 1) << 3;
  return p ^ ((row & 3) | ((row >> 3) & 1) << 2);
}
// the chunk stored at slot `slot` of row `row` (the inverse map: P is its own inverse)
__device__ __forceinline__ int swz_a_chunk(int row, int slot) {
  const int q = slot ^ ((row & 3) | ((row >> 3) & 1) << 2);
  return (q & 3) | ((q >> 3) & 1) << 2 | ((q >> 2) & 1) << 3;
}
__device__ __forceinline__ uint32_t swz_a(int row, int chunk) { return (uint32_t)(row * 256 + (swz_a_slot(row, chunk) << 4)); }
// (n / 2 ^ n / 8) % 4 keeps any 8 consecutive rows (one 128-B bank sweep) and
// any 16 consecutive rows (one 256-B sweep) on distinct 16-B slots
__device__ __forceinline__ int swz_w_key(int row) { return ((row >> 1) ^ (row >> 3)) & 3; }
__device__ __forceinline__ uint32_t swz_w(int row, int chunk) { return (uint32_t)(row * 64 + ((chunk ^ swz_w_key(row)) << 4)); }

__device__ __forceinline__ uint32_t quant4_lanes(const float* v, float inv_g, uint32_t& sb_out) {
  float amax = fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3])));
  amax = fmaxf(amax, __shfl_xor(amax, 16, kWave));
  amax = fmaxf(amax, __shfl_xor(amax, 32, kWave));
  float target = (amax * inv_g) / 6.0f;
  uint32_t sb = f32_to_e4m3_sat(target);
  float s = e4m3_to_f32(sb);
  uint32_t bits = 0;
  if (s > 0.0f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float xs = v[i] * inv_g;
      bits |= (e2m1_code(fabsf(xs), s) | ((__float_as_uint(xs) >> 28) & 8u)) << (4 * i);
    }
  }
  sb_out = sb;
  return bits;
}

// ---------------------------------------------------------------- tiles
// s_pref[e] = tiles before expert e (expert e owns ceil(rows_e / BM) * ntn tiles);
// s_rng[e] (if given) = expert e's rows [r0, r1), clamped to [0, rows)
template <int NTHR, int BM>
__device__ __forceinline__ int build_tile_table(const GemmArgs& p, int ntn, int* s_pref, int* s_wc,
                                                int2* s_rng = nullptr) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  int running = 0;
  for (int e0 = 0; e0 < p.E; e0 += NTHR) {
    const int e = e0 + tid;
    int cnt = 0;
    if (e < p.E) {
      int r0 = (int)max((int64_t)0, min((int64_t)p.offsets[e], p.rows));
      int r1 = (int)max((int64_t)r0, min((int64_t)p.offsets[e + 1], p.rows));
      cnt = ((r1 - r0 + BM - 1) / BM) * ntn;
      if (s_rng) s_rng[e] = make_int2(r0, r1);
    }
    int x = cnt;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      int y = __shfl_up(x, off, kWave);
      if (lane >= off) x += y;
    }
    if (lane == 63) s_wc[wv] = x;
    __syncthreads();
    int before = running;
    for (int i = 0; i < wv; ++i) before += s_wc[i];
    if (e < p.E) s_pref[e] = before + x - cnt;
    int tot = 0;
    for (int i = 0; i < NTHR / kWave; ++i) tot += s_wc[i];
    running += tot;
    __syncthreads();
  }
  if (tid == 0) s_pref[p.E] = running;
  __syncthreads();
  return s_pref[p.E];
}

struct PfTile {
  int e, rbase, mrows, nbase;
};

// (expert, n-tile, m-tile) of a tile index; the m-tiles of one n-tile are consecutive
template <int NMAT, typename SH>
__device__ __forceinline__ PfTile locate_tile(const GemmArgs& p, const int* s_pref, int tile) {
  int lo = 0, hi = p.E - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (s_pref[mid] <= tile) lo = mid;
    else hi = mid - 1;
  }
  PfTile t;
  t.e = lo;
  const int r0 = (int)max((int64_t)0, min((int64_t)p.offsets[lo], p.rows));
  const int r1 = (int)max((int64_t)r0, min((int64_t)p.offsets[lo + 1], p.rows));
  const int mt_cnt = (r1 - r0 + SH::BM - 1) / SH::BM;
  const int local = tile - s_pref[lo];
  const int nt = local / mt_cnt, mt = local % mt_cnt;
  t.rbase = r0 + mt * SH::BM;
  t.mrows = min(SH::BM, r1 - t.rbase);
  t.nbase = nt * (SH::BN / NMAT);                                   // first row of each matrix's slab
  return t;
}

// this workgroup's share of the tile list: a contiguous slice per XCD
__device__ __forceinline__ void xcd_slice(int total, int& begin, int& end, int& stride) {
  const int nx = (gridDim.x % kPfXcds == 0) ? kPfXcds : 1;
  const int xcd = blockIdx.x % nx, slot = blockIdx.x / nx;
  stride = gridDim.x / nx;
  begin = (int)((int64_t)total * xcd / nx) + slot;
  end = (int)((int64_t)total * (xcd + 1) / nx);
}

// block-local weight row n (0..BN-1): matrix n / (BN/2) (SwiGLU), row within the slab
template <int NMAT, int BN>
__device__ __forceinline__ int pf_wrow(int n) { return NMAT == 2 ? (n & (BN / 2 - 1)) : n; }
// wave (wm, wn)'s weight group g (16 rows): block-local row base
template <int NMAT, int BN>
__device__ __forceinline__ int pf_lrow(int wn, int g) {
  return NMAT == 2 ? (g >> 1) * (BN / 2) + wn * 32 + (g & 1) * 16 : wn * 64 + g * 16;
}

// Scale bytes of global weight row R for one step: a per-lane part and a
// per-step part (uniform).  Row-major: R * sc_row + 4 kb (MX) | 8 kb + 4 half
// (NV).  Tiled: row R's 16 B (MX) or 32 B (NV) window slice in its tile's
// block of window kb / 4, step kb % 4 within it.
template <bool TL, bool W_NV>
__device__ __forceinline__ uint32_t pf_scale_lane(int R, int half, int K) {
  if (TL) {
    const uint32_t blk = W_NV ? 512u : 256u;
    return (uint32_t)(R >> 4) * (uint32_t)(K / 512) * blk + (uint32_t)(R & 15) * (W_NV ? 32u : 16u) +
           (W_NV ? (uint32_t)half * 4u : 0u);
  }
  return (uint32_t)R * (uint32_t)(W_NV ? K / 16 : K / 32) + (W_NV ? (uint32_t)half * 4u : 0u);
}
template <bool TL, bool W_NV>
__device__ __forceinline__ uint32_t pf_scale_step(int kb) {
  if (TL) return (uint32_t)(kb >> 2) * (W_NV ? 512u : 256u) + (uint32_t)(kb & 3) * (W_NV ? 8u : 4u);
  return (uint32_t)kb * (W_NV ? 8u : 4u);
}

// One step from an LDS stage into acc[weight group][token group].  WF: weight
// scale format -- 0 MXFP4, 1 NVFP4 with power-of-two scales (the exact MXFP4
// transcode), 2 NVFP4 with any E4M3 scales (converted through float).
struct PfNoHook {
  __device__ __forceinline__ void operator()(int) const {}
};

// hook(s) runs at the start of k-slot s (the direct-to-LDS kernel issues part
// of the next stage's loads there, between MFMAs).
// TL: the weight stage holds each 16-row group as one 1 KB tiled block (lane
// (li, lg) at 16 * (16 lg + li)) instead of swizzled rows.
// WREG: the weight codes come in registers (wreg[g]) instead of the LDS stage.
// RB: the 16-row token blocks that hold rows of the tile (the rest are padding:
// no LDS reads, no MFMAs)
template <int NMAT, int WF, bool TL, typename SH, bool WREG = false, int RB = 4, typename Hook = PfNoHook>
__device__ __forceinline__ void pf_compute(const uint8_t* st, const uint8_t* ss, f32x4 (&acc)[4][4], int wm, int wn,
                                           int li, int lg, Hook&& hook = Hook(), const u32x4* wreg = nullptr) {
  constexpr bool W_NV = WF != 0;
  const uint8_t* sa = st;
  const uint8_t* sw = st + SH::AStage;
  u32x4 wq[4];
  float s_lo[4], s_hi[4];
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int n = pf_lrow<NMAT, SH::BN>(wn, g) + li;
    if (WREG) wq[g] = wreg[g];
    else wq[g] = *(const u32x4*)(sw + (TL ? (uint32_t)(n >> 4) * 1024u + (uint32_t)(lg * 16 + li) * 16u : swz_w(n, lg)));
    if (W_NV) {
      const uint32_t b2 = *(const uint16_t*)(ss + n * 8 + lg * 2);
      s_lo[g] = e4m3_byte<0>(b2);
      s_hi[g] = e4m3_byte<1>(b2);
    } else {
      s_lo[g] = s_hi[g] = e8m0_to_f32(ss[n * 4 + lg]);
    }
  }
  bf16x8 bt[2][4];
  auto read_bt = [&](bf16x8 (&b)[4], int s) {
#pragma unroll
    for (int t = 0; t < RB; ++t)
      b[t] = __builtin_bit_cast(bf16x8, *(const u32x4*)(sa + swz_a(wm * 64 + t * 16 + li, lg * 4 + s)));
  };
  // weight group g of k-slot s, dequantised to bf16
  auto cvt = [&](int s, int g) {
    const float sc = s < 2 ? s_lo[g] : s_hi[g];
    return WF == 2 ? fp4x8_to_bf16_general(wq[g][s], sc) : fp4x8_to_bf16_pow2(wq[g][s], sc);
  };
  read_bt(bt[0], 0);
  // the converts run one weight group ahead of the MFMAs that use them, in a
  // register set of their own, so they issue while the matrix core works
  bf16x8 af[2];
  af[0] = cvt(0, 0);
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    if (s < 3) {
      read_bt(bt[(s + 1) & 1], s + 1);
      // keep the next slot's reads above this slot's MFMAs (the scheduler
      // would otherwise sink them and reuse one register set)
      __builtin_amdgcn_sched_barrier(0);
    }
    hook(s);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int i = s * 4 + g;
      if (i + 1 < 16) af[(i + 1) & 1] = cvt((i + 1) >> 2, (i + 1) & 3);
#pragma unroll
      for (int t = 0; t < RB; ++t) acc[g][t] = mfma16(af[i & 1], bt[s & 1][t], acc[g][t]);
    }
  }
}

// Epilogue: lane holds D[weight row 4*lg + i of group g][token row li of group t].
// (One matrix: with p.out_sumsq, the sum of squares of the row's FP32 outputs
// over the wave's 64 columns goes to out_sumsq[row, column / 64] -- the REAP
// saliency's per-row norm, in parts that a later pass adds in order.)
template <int NMAT>
__device__ __forceinline__ void pf_epilogue(const GemmArgs& p, const PfTile& T, const f32x4 (&acc)[4][4],
                                            const float (&wglob)[NMAT], int wm, int wn, int li, int lg) {
  const int N = p.N;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int mrow = wm * 64 + t * 16 + li;
    const bool ok = mrow < T.mrows;
    const int64_t ro = T.rbase + mrow;
    float sq = 0.0f;
#pragma unroll
    for (int gp = 0; gp < (NMAT == 2 ? 2 : 4); ++gp) {
      float v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float g = acc[gp][t][i] * wglob[0];
        v[i] = NMAT == 2 ? silu_f(g) * (acc[gp + 2][t][i] * wglob[NMAT - 1]) : g;
        if (NMAT == 1) sq = fmaf(v[i], v[i], sq);
      }
      const int col = T.nbase + (NMAT == 2 ? wn * 32 + gp * 16 : wn * 64 + gp * 16) + 4 * lg;
      const uint32_t b01 = cvt_bf16x2(v[0], v[1]), b23 = cvt_bf16x2(v[2], v[3]);
      if (p.out_bf16 && ok) *(u32x2*)(p.out_bf16 + ro * N + col) = u32x2{b01, b23};
      if (p.out_codes || p.out_dq) {
        float q[4] = {bf16_lo(b01), bf16_hi(b01), bf16_lo(b23), bf16_hi(b23)};
        uint32_t sb;
        const uint32_t bits = quant4_lanes(q, p.out_inv_g, sb);
        if (ok) {
          if (p.out_codes) {
            *(uint16_t*)(p.out_codes + ro * (N / 2) + col / 2) = (uint16_t)bits;
            if (lg == 0) p.out_scales[ro * (N / 16) + (col - 4 * lg) / 16] = (uint8_t)sb;
          }
          if (p.out_dq) *(u32x2*)(p.out_dq + ro * N + col) = nvfp4_dequant4(bits, e4m3_to_f32(sb) * p.out_g);
        }
      }
    }
    if (NMAT == 1 && p.out_sumsq) {
      // lanes li + 16 lg hold the 4 x 4 columns of each group: add the four lane groups in a fixed order
      const float s1 = sq + __shfl_xor(sq, 16, kWave);
      const float s2 = s1 + __shfl_xor(s1, 32, kWave);
      if (ok && lg == 0) p.out_sumsq[ro * (N / 64) + (T.nbase + wn * 64) / 64] = s2;
    }
  }
}

// bf16 output through LDS: each wave's outputs (64 token rows x 64 columns,
// SwiGLU 32) go to LDS in the MFMA layout (8 bytes per lane and 16-row group)
// and come back as whole rows, so each global store writes 8 (16) rows of 128
// (64) contiguous bytes instead of 16 rows of 32.  (The down projection's 64
// KB of output per tile, stored in 32-byte pieces, took 11% of its time,
// partly by slowing the next steps' loads.)  The staging area is a token
// stage that no load is filling (the last step's, after a barrier): 2 KB per
// wave, one 16-row group at a time.  16-byte
// chunk c of row r sits at chunk c ^ (r / R256 mod chunks-per-row), R256 the
// rows per 256 bytes: the 16 rows of an 8-byte write and the rows of a 16-byte
// read then cover distinct banks.  The rows are stored with the
// non-temporal cache policy (prefill layer 0.6% faster: the stream of
// outputs no longer displaces the tiles' weight slices and token rows).
template <int NMAT>
__device__ __forceinline__ void pf_epilogue_staged(const GemmArgs& p, const PfTile& T, const f32x4 (&acc)[4][4],
                                                 const float (&wglob)[NMAT], int wn, int li, int lg, uint8_t* ob) {
  constexpr int RBY = NMAT == 2 ? 64 : 128;                  // bytes per output row of the wave
  constexpr int CPR = RBY / 16;                              // 16-byte chunks per row
  constexpr int RPI = 64 / CPR;                              // rows per read-back instruction
  constexpr int R256 = 256 / RBY;                            // rows per 256 bytes (one bank sweep)
  auto slot = [](int row, int c) { return ((c ^ ((row / R256) & (CPR - 1))) << 4); };
  const int N = p.N;
  const int lane = threadIdx.x & 63;
  const int col0 = T.nbase + (NMAT == 2 ? wn * 32 : wn * 64);
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    float sq = 0.0f;
#pragma unroll
    for (int gp = 0; gp < (NMAT == 2 ? 2 : 4); ++gp) {
      float v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float g = acc[gp][t][i] * wglob[0];
        v[i] = NMAT == 2 ? silu_f(g) * (acc[gp + 2][t][i] * wglob[NMAT - 1]) : g;
        if (NMAT == 1) sq = fmaf(v[i], v[i], sq);
      }
      const int cb = gp * 32 + lg * 8;                       // byte of the row: columns gp * 16 + 4 lg ..
      *(u32x2*)(ob + li * RBY + slot(li, cb >> 4) + (cb & 15)) = u32x2{cvt_bf16x2(v[0], v[1]), cvt_bf16x2(v[2], v[3])};
    }
    if (NMAT == 1 && p.out_sumsq) {
      // lanes li + 16 lg hold the 4 x 4 columns of each group: add the four lane groups in a fixed order
      const float s1 = sq + __shfl_xor(sq, 16, kWave);
      const float s2 = s1 + __shfl_xor(s1, 32, kWave);
      if (t * 16 + li < T.mrows && lg == 0) p.out_sumsq[(T.rbase + t * 16 + li) * (N / 64) + col0 / 64] = s2;
    }
    // (the LDS operations of one wave complete in order: the reads see the writes, the next group's writes
    // follow the reads)
#pragma unroll
    for (int r0 = 0; r0 < 16; r0 += RPI) {
      const int row = r0 + lane / CPR, c = lane % CPR;
      const u32x4 d = *(const u32x4*)(ob + row * RBY + slot(row, c));
      if (t * 16 + row < T.mrows) __builtin_nontemporal_store(d, (u32x4*)(p.out_bf16 + (T.rbase + t * 16 + row) * N + col0 + c * 8));
    }
  }
}

// ------------------------------------------------ bf16 tokens: direct to LDS
// 64 x 512 tiles: weight codes in registers, not LDS (3-4% faster, although the
// compiler then drains the loads in flight once per step before the first LDS read)
constexpr bool kPfWeightRegs = true;
template <int S>
__device__ __forceinline__ uint8_t* pf_stage() {
  return S == 0 ? pf_stage0 : (S == 1 ? pf_stage1 : pf_stage2);
}
template <int S>
__device__ __forceinline__ uint8_t* pf_sstage() {
  return S == 0 ? pf_sstage0 : (S == 1 ? pf_sstage1 : pf_sstage2);
}

template <int NMAT, int WF, bool TL, typename SH>
__global__ __launch_bounds__(kPfThreads) void gemm_prefill_dma_kernel(GemmArgs p) {
  constexpr bool W_NV = WF != 0;
  static_assert(3 * (kPfStageMax + kPfSStageMax) + (kPfMaxE + 1) * 4 + kPfThreads / kWave * 4 <= 160 * 1024, "LDS");
  __shared__ int s_pref[kPfMaxE + 1];
  __shared__ int s_wc[kPfThreads / kWave];
  // direct-to-LDS loads per wave and step: tokens (1 KB = 4 rows each), weight
  // codes (1 KB = 16 rows), scales (256 B: 64 MX rows or 32 NV rows)
  // 64 x 512: every weight row belongs to one wave, so its codes go straight
  // into that wave's registers (4 loads of 16 B per lane and step, three steps
  // deep) instead of through LDS
  constexpr bool WREG = kPfWeightRegs && SH::BM == 64;
  using WL = WeightLane<TL, W_NV>;
  constexpr int kA = SH::BM / 32, kW = WREG ? 4 : SH::BN / 128;
  constexpr int kSRows = W_NV ? 32 : 64;                              // weight rows per scale load
  constexpr int kSLoads = SH::BN / kSRows;                            // scale loads per step (all waves)
  constexpr int kS = kSLoads > 8 ? kSLoads / 8 : 1;                   // per wave (MX 128 x 256: waves 4..7 repeat 0..3)
  constexpr int kDmaPerStep = kA + kW + kS;
  static_assert(kDmaPerStep <= 8, "two loads per k-slot");

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wv / SH::WN, wn = wv % SH::WN;                      // (128 x 256: SIMD s holds waves s and s + 4)
  const int li = lane & 15, lg = lane >> 4;
  const int K = p.K, N = p.N;
  const int ntn = N / (SH::BN / NMAT);
  const int nk = K / kPfBK;
  const int total = build_tile_table<kPfThreads, SH::BM>(p, ntn, s_pref, s_wc);
  int t_begin, t_end, t_stride;
  xcd_slice(total, t_begin, t_end, t_stride);

  const uint32_t sc_row = (uint32_t)(W_NV ? K / 16 : K / 32);
  const int64_t mat_codes = (int64_t)N * (K / 2);
  const int64_t mat_scales = (int64_t)N * sc_row;

  for (int tile = t_begin; tile < t_end; tile += t_stride) {
    const PfTile T = locate_tile<NMAT, SH>(p, s_pref, tile);
    float wglob[NMAT];
#pragma unroll
    for (int m = 0; m < NMAT; ++m) wglob[m] = W_NV ? p.w_global[m][T.e] : 1.0f;

    // per-lane sources of this wave's loads as 32-bit offsets from uniform
    // bases (scalar registers); LDS slot = wave base + lane * size
    // tokens: load i fills rows 4 * (kA wv + i) .. +3, lane -> (row, slot lane % 16)
    uint32_t a_off[kA];
#pragma unroll
    for (int i = 0; i < kA; ++i) {
      const int row = (wv * kA + i) * 4 + (lane >> 4);
      const int chunk = swz_a_chunk(row, lane & 15);
      const int64_t r = T.rbase + min(row, T.mrows - 1);            // rows past the tile's end reread a valid row
      const int64_t src = p.gather ? (int64_t)(p.gather[r] / p.gather_div) : r;
      a_off[i] = (uint32_t)(src * (int64_t)K * 2) + (uint32_t)chunk * 16u;   // < 2 GiB (checked on the host)
    }
    // weight codes: load j fills rows 16 * (kW wv + j) .. +15 (matrix wv / 4 for SwiGLU);
    // tiled: that group's 1 KB block of the step, in lane order.  WREG: load j
    // is this wave's weight group j (rows lrow(wn, j) ..), row li, piece lg
    const int wmat = NMAT == 2 ? (wv >> 2) : 0;
    const uint8_t* w_base = p.w_packed[wmat] + T.e * mat_codes;
    uint32_t w_off[kW];
    rsrc_t wrs[NMAT];
    if (WREG) {
#pragma unroll
      for (int m = 0; m < NMAT; ++m) wrs[m] = make_rsrc(p.w_packed[m] + T.e * mat_codes, (uint32_t)mat_codes);
    }
#pragma unroll
    for (int j = 0; j < kW; ++j) {
      if (WREG) {
        const int R = T.nbase + pf_wrow<NMAT, SH::BN>(pf_lrow<NMAT, SH::BN>(wn, j));
        w_off[j] = (uint32_t)R * (uint32_t)(K / 2) + WL::code(li, lg, K);
      } else if (TL) {
        const int tile = (T.nbase + pf_wrow<NMAT, SH::BN>((wv * kW + j) * 16)) >> 4;
        w_off[j] = (uint32_t)tile * (uint32_t)(K / 128) * 1024u + (uint32_t)lane * 16u;
      } else {
        const int n = (wv * kW + j) * 16 + (lane >> 2);
        const int chunk = (lane & 3) ^ swz_w_key(n);
        w_off[j] = (uint32_t)(T.nbase + pf_wrow<NMAT, SH::BN>(n)) * (uint32_t)(K / 2) + (uint32_t)chunk * 16u;
      }
    }
    // scales: load h covers rows kSRows * ((kS wv + h) % kSLoads) ..; MX one row per
    // lane, NV row lane / 2 with half lane % 2; LDS slot 256 * (kS wv + h)
    const uint8_t* s_base[kS];
    uint32_t s_off[kS];
#pragma unroll
    for (int h = 0; h < kS; ++h) {
      const int ld = (wv * kS + h) % kSLoads;
      const int s_n = ld * kSRows + (W_NV ? (lane >> 1) : lane);
      const int smat = NMAT == 2 ? (ld * kSRows) / (SH::BN / 2) : 0;
      s_base[h] = p.w_scale[smat] + T.e * mat_scales;
      s_off[h] = pf_scale_lane<TL, W_NV>(T.nbase + pf_wrow<NMAT, SH::BN>(s_n), lane & 1, K);
    }

    u32x4 wring[3][4];                                               // WREG: codes of steps k .. k + 2
    // load q of step kb into stage S: kA token loads, kW weight-code loads, kS scale loads
    auto issue_one = [&](auto S_tag, int kb, int q) {
      constexpr int S = decltype(S_tag)::value;
      uint8_t* st = pf_stage<S>();
      // (WREG: the register loads go first, then the direct-to-LDS ones)
      constexpr int qa = WREG ? kW : 0, qw = WREG ? 0 : kA;
      if (q >= qa && q < qa + kA) {
        __builtin_amdgcn_global_load_lds((const void*)(p.a_data + kb * 256 + a_off[q - qa]),
                                         (lds_void_t*)(st + (wv * kA + q - qa) * 1024), 16, 0, 0);
      } else if (q >= qw && q < qw + kW) {
        const int j = q - qw;
        if (WREG) {
          wring[S][j] = bload128(wrs[NMAT == 2 ? (j >> 1) : 0], w_off[j] + (uint32_t)kb * WL::kStep, 0);
        } else {
          __builtin_amdgcn_global_load_lds((const void*)(w_base + kb * (TL ? 1024 : 64) + w_off[j]),
                                           (lds_void_t*)(st + SH::AStage + (wv * kW + j) * 1024), 16, 0, 0);
        }
      } else {
        const int h = q - kA - kW;
        __builtin_amdgcn_global_load_lds((const void*)(s_base[h] + pf_scale_step<TL, W_NV>(kb) + s_off[h]),
                                         (lds_void_t*)(pf_sstage<S>() + (wv * kS + h) * 256), 4, 0, 0);
      }
    };
    auto issue = [&](auto S_tag, int kb) {
#pragma unroll
      for (int q = 0; q < kDmaPerStep; ++q) issue_one(S_tag, kb, q);
    };

    // the tile's K loop, for RB token blocks of 16 rows that hold rows of the
    // tile (a 64-row tile of an expert's last rows often holds fewer than 64)
    auto run = [&](auto RB_tag) {
      constexpr int RB = decltype(RB_tag)::value;
      f32x4 acc[4][4];
  #pragma unroll
      for (int g = 0; g < 4; ++g)
  #pragma unroll
        for (int t = 0; t < 4; ++t) acc[g][t] = f32x4{0.f, 0.f, 0.f, 0.f};

      // step k from stage S: wait for this wave's loads of step k (those of step
      // k + 1 may stay in flight), barrier (every wave's loads landed, every wave
      // done with step k - 1), refill the stage of step k - 1 with step k + 2
      // (past the end: step nk - 1 again, unread), compute
      auto step = [&](auto S_tag, int k) {
        constexpr int S = decltype(S_tag)::value;
        __builtin_amdgcn_s_waitcnt((kDmaPerStep & 15) | (7 << 4) | (15 << 8));      // vmcnt(kDmaPerStep)
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        const int kn = min(k + 2, nk - 1);
        constexpr auto SN = std::integral_constant<int, (S + 2) % 3>();
        // the next stage's loads go out between this step's MFMA slots (two per
        // slot), so the load unit drains them while the matrix cores work
        auto hook = [&](int s) {
          if (2 * s < kDmaPerStep) issue_one(SN, kn, 2 * s);
          if (2 * s + 1 < kDmaPerStep) issue_one(SN, kn, 2 * s + 1);
        };
        // every wave computes, also on rows past the tile's end (their outputs
        // are not stored): a branch here made the compiler drain every load in
        // flight before each step's first LDS read, losing the two-step lead
        pf_compute<NMAT, WF, TL, SH, WREG, RB>(pf_stage<S>(), pf_sstage<S>(), acc, wm, wn, li, lg, hook, wring[S]);
      };

      __syncthreads();                                                 // previous tile done with the stages
      issue(std::integral_constant<int, 0>(), 0);
      issue(std::integral_constant<int, 1>(), min(1, nk - 1));
      int kb = 0;
      for (; kb + 3 <= nk; kb += 3) {
        step(std::integral_constant<int, 0>(), kb);
        step(std::integral_constant<int, 1>(), kb + 1);
        step(std::integral_constant<int, 2>(), kb + 2);
      }
      if (kb < nk) step(std::integral_constant<int, 0>(), kb);
      if (kb + 1 < nk) step(std::integral_constant<int, 1>(), kb + 1);
      if (NMAT == 1 && WF != 2 && SH::BM == 64 && p.out_bf16 && !p.out_codes && !p.out_dq) {
        // the down projection's bf16 out through LDS (pf_epilogue_staged), staged in the last step's
        // stage: the loads in flight (its repeats) fill the other two
        __builtin_amdgcn_s_barrier();
        uint8_t* ob = ((nk - 1) % 3 == 0 ? pf_stage<0>() : ((nk - 1) % 3 == 1 ? pf_stage<1>() : pf_stage<2>())) + wv * 2048;
        pf_epilogue_staged<NMAT>(p, T, acc, wglob, wn, li, lg, ob);
      } else {
        pf_epilogue<NMAT>(p, T, acc, wglob, wm, wn, li, lg);
      }
    };
    if constexpr (SH::BM == 64) {
      const int rb = (T.mrows + 15) >> 4;                            // workgroup-uniform
      if (rb >= 4) run(std::integral_constant<int, 4>());
      else if (rb == 3) run(std::integral_constant<int, 3>());
      else if (rb == 2) run(std::integral_constant<int, 2>());
      else run(std::integral_constant<int, 1>());
    } else {
      run(std::integral_constant<int, 4>());
    }
  }
  // the last tile leaves its unread repeat loads in flight: let them land
  // before the workgroup's LDS is released
  __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8));             // vmcnt(0)
}

// ------------------------------- bf16 tokens: the pipeline carried across tiles
// The kernel above stops its pipeline at every tile: the tile lookup, the
// gather-index loads and the first two steps' loads run one after another
// before the tile's first MFMA.  Here the pipeline runs on from one tile into
// the workgroup's next (64 x 512 tiles, K a multiple of 512):
//   * four LDS stages and four register sets of weight codes, loads issued three
//     steps ahead; a tile's step count is a multiple of four, so step k of every
//     tile uses stage k % 4, and the last three steps of a tile issue the first
//     three steps of the next tile;
//   * the tile after next is looked up (two ballots over the tile table and the
//     experts' row ranges in LDS) and its gather indices are loaded while the
//     last MFMAs of a tile drain, before its epilogue.
// Each step waits until at most two steps' loads of this wave are in flight.
// Loads complete in order, so that leaves exactly the step's own loads done;
// the epilogue's stores, counted by the same counter, can only lengthen a wait.
__shared__ __attribute__((aligned(16))) uint8_t px_stage0[PfWide::AStage];
__shared__ __attribute__((aligned(16))) uint8_t px_stage1[PfWide::AStage];
__shared__ __attribute__((aligned(16))) uint8_t px_stage2[PfWide::AStage];
__shared__ __attribute__((aligned(16))) uint8_t px_stage3[PfWide::AStage];
__shared__ __attribute__((aligned(16))) uint8_t px_sstage0[PfWide::SStage];
__shared__ __attribute__((aligned(16))) uint8_t px_sstage1[PfWide::SStage];
__shared__ __attribute__((aligned(16))) uint8_t px_sstage2[PfWide::SStage];
__shared__ __attribute__((aligned(16))) uint8_t px_sstage3[PfWide::SStage];
template <int S>
__device__ __forceinline__ uint8_t* px_stage() {
  return S == 0 ? px_stage0 : (S == 1 ? px_stage1 : (S == 2 ? px_stage2 : px_stage3));
}
template <int S>
__device__ __forceinline__ uint8_t* px_sstage() {
  return S == 0 ? px_sstage0 : (S == 1 ? px_sstage1 : (S == 2 ? px_sstage2 : px_sstage3));
}

// s_waitcnt immediate for "vmcnt <= n" alone (vmcnt in bits 3:0 and 15:14)
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// a value at a workgroup-uniform address, through the scalar data cache (the
// kernel never writes it)
__device__ __forceinline__ float load_uniform_f32(const float* ptr) {
  return *(const __attribute__((address_space(4))) float*)ptr;
}
__device__ __forceinline__ int load_uniform_i32(const int32_t* ptr) {
  return *(const __attribute__((address_space(4))) int32_t*)ptr;
}

// The tile at index `tile` (< the tile count) from the tables in LDS.  Its
// expert is the last e with s_pref[e] <= tile (an expert without tiles has the
// prefix of the next one); lane l first tests expert l * stride, then lane l
// tests expert seg * stride + l of the segment found (E <= 64 * 64).  The
// result is workgroup-uniform.
template <int NMAT, typename SH>
__device__ __forceinline__ PfTile locate_tile_lds(const int* s_pref, const int2* s_rng, int E, int tile) {
  const int lane = threadIdx.x & 63;
  const int stride = (E + 63) >> 6;
  const int e1 = lane * stride;
  const int v1 = e1 < E ? s_pref[e1] : 0x7fffffff;
  const uint64_t b1 = __ballot(v1 <= tile);                        // lane 0: prefix 0
  const int seg = 63 - __clzll((long long)b1);
  const int e2 = seg * stride + lane;
  const int v2 = (lane < stride && e2 < E) ? s_pref[e2] : 0x7fffffff;
  const uint64_t b2 = __ballot(v2 <= tile);                        // lane 0: lane seg's expert above
  const int e = __builtin_amdgcn_readfirstlane(seg * stride + 63 - __clzll((long long)b2));
  const int2 rg = s_rng[e];
  const int r0 = __builtin_amdgcn_readfirstlane(rg.x);
  const int r1 = __builtin_amdgcn_readfirstlane(rg.y);
  const int local = tile - __builtin_amdgcn_readfirstlane(s_pref[e]);
  const int mt_cnt = (r1 - r0 + SH::BM - 1) / SH::BM;
  const int nt = local / mt_cnt, mt = local - nt * mt_cnt;
  PfTile t;
  t.e = e;
  t.rbase = r0 + mt * SH::BM;
  t.mrows = min(SH::BM, r1 - t.rbase);
  t.nbase = nt * (SH::BN / NMAT);
  return t;
}

template <int NMAT, int WF, bool TL>
__global__ __launch_bounds__(kPfThreads) void gemm_prefill_xt_kernel(GemmArgs p) {
  using SH = PfWide;
  constexpr bool W_NV = WF != 0;
  constexpr int kStages = 4;
  static_assert(kStages * (SH::AStage + SH::SStage) + (kPfMaxE + 1) * 12 + kPfThreads / kWave * 4 <= 160 * 1024,
                "LDS");
  static_assert(kPfThreads / kWave * 2048 <= SH::AStage, "epilogue staging: 2 KB per wave in one token stage");
  __shared__ int s_pref[kPfMaxE + 1];
  __shared__ int2 s_rng[kPfMaxE + 1];
  __shared__ int s_wc[kPfThreads / kWave];
  using WL = WeightLane<TL, W_NV>;
  // loads per wave and step: 4 weight-code loads into registers (16 rows each),
  // 2 token loads (1 KB = 4 rows each, direct to LDS), kS scale loads (64 MX
  // rows or 32 NV rows each, direct to LDS)
  constexpr int kA = SH::BM / 32, kW = 4;
  constexpr int kSRows = W_NV ? 32 : 64;
  constexpr int kSLoads = SH::BN / kSRows;
  constexpr int kS = kSLoads / 8;
  constexpr int kDma = kW + kA + kS;
  static_assert(kDma <= 8 && kS >= 1, "two loads per k-slot");

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn = wv;                                                 // 1 x 8 waves along weight rows
  const int li = lane & 15, lg = lane >> 4;
  const int K = p.K, N = p.N;
  const int ntn = N / (SH::BN / NMAT);
  const int nk = K / kPfBK;                                          // a multiple of 4 (checked on the host)
  const int total = build_tile_table<kPfThreads, SH::BM>(p, ntn, s_pref, s_wc, s_rng);
  int t_begin, t_end, t_stride;
  xcd_slice(total, t_begin, t_end, t_stride);
  if (t_begin >= t_end) return;                                      // uniform; nothing issued
  const int n_tiles = (t_end - t_begin + t_stride - 1) / t_stride;
  const int t_last = t_begin + (n_tiles - 1) * t_stride;
  // the i-th tile of this workgroup; past the end the last one again (its
  // loads then go out unread, so every wait counts the same loads)
  auto tile_at = [&](int i) { return min(t_begin + i * t_stride, t_last); };

  const int64_t mat_codes = (int64_t)N * (K / 2);
  const uint32_t sc_row = (uint32_t)(W_NV ? K / 16 : K / 32);
  const int64_t mat_scales = (int64_t)N * sc_row;
  const uint32_t code_tile = 16u * (uint32_t)(K / 2);                // 16 weight rows of codes
  // scale load h covers rows kSRows * (kS wv + h) of the tile's weight rows: both loads of a wave lie in one matrix
  const int smat = NMAT == 2 ? (wv * kS * kSRows) / (SH::BN / 2) : 0;
  const uint32_t s_delta = TL ? (uint32_t)(kSRows / 16) * (uint32_t)(K / 512) * (W_NV ? 512u : 256u)
                              : (uint32_t)kSRows * sc_row;

  // what a tile's loads need: token source offsets (gathered rows), the offset
  // of weight load 0 (load j adds a uniform multiple of 16 rows) and of scale
  // load 0 (load h adds h * s_delta)
  struct Ctx {
    PfTile T;
    uint32_t a_off[kA];
    uint32_t w_off;
    uint32_t s_off;
  };
  // a tile's token source rows (rows past the tile's end reread its last row).
  // The wave's loads cover tile rows 8 wv .. 8 wv + 7; their gather indices
  // come through the scalar data cache (uniform addresses, not counted with
  // the vector loads), and each lane picks its row's.
  auto src_rows = [&](const PfTile& T, int (&src)[kA]) {
    const int base = min(wv * 8, T.mrows - 1);
    const int a = T.rbase + base;
    int g[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int r = (int)min((int64_t)(a + j), p.rows - 1);                 // rows past the tile's end are not used
      g[j] = p.gather ? load_uniform_i32(p.gather + r) : r;
    }
#pragma unroll
    for (int i = 0; i < kA; ++i) {
      const int row = (wv * kA + i) * 4 + (lane >> 4);
      const int idx = min(row, T.mrows - 1) - base;                         // 0 .. 7
      int v = g[0];
#pragma unroll
      for (int j = 1; j < 8; ++j) v = idx == j ? g[j] : v;
      src[i] = v;
    }
  };
  auto make_ctx = [&](const PfTile& T, const int (&src)[kA]) {
    Ctx c;
    // (the tile is workgroup-uniform: scalar registers, so the buffer descriptors built from it are too)
    c.T.e = __builtin_amdgcn_readfirstlane(T.e);
    c.T.rbase = __builtin_amdgcn_readfirstlane(T.rbase);
    c.T.mrows = __builtin_amdgcn_readfirstlane(T.mrows);
    c.T.nbase = __builtin_amdgcn_readfirstlane(T.nbase);
#pragma unroll
    for (int i = 0; i < kA; ++i) {
      const int row = (wv * kA + i) * 4 + (lane >> 4);
      const int chunk = swz_a_chunk(row, lane & 15);
      const int64_t s = p.gather ? (int64_t)(src[i] / p.gather_div) : (int64_t)src[i];
      c.a_off[i] = (uint32_t)(s * (int64_t)K * 2) + (uint32_t)chunk * 16u;    // < 2 GiB (checked on the host)
    }
    const int R0 = T.nbase + pf_wrow<NMAT, SH::BN>(pf_lrow<NMAT, SH::BN>(wn, 0));
    c.w_off = (uint32_t)R0 * (uint32_t)(K / 2) + WL::code(li, lg, K);
    const int s_n = wv * kS * kSRows + (W_NV ? (lane >> 1) : lane);
    c.s_off = pf_scale_lane<TL, W_NV>(T.nbase + pf_wrow<NMAT, SH::BN>(s_n), lane & 1, K);
    return c;
  };

  u32x4 wring[kStages][4];                                           // weight codes of steps k .. k + 3
  // every load is a buffer load: 32-bit lane offsets, the step's part uniform.
  // (The compiler does not count the direct-to-LDS ones with the vector loads
  // when it places its own waits for loaded registers, so its waits can only
  // be stricter than needed; as global loads with 64-bit addresses they cost
  // 16 more registers and made it wait for every load in flight once per four steps.)
  const rsrc_t a_rsrc = make_rsrc(p.a_data, (uint32_t)min(p.a_bytes, (int64_t)0xffffffff));
  // load q of step kb of the tile of c into stage S: weight codes, tokens, scales
  auto issue_one = [&](auto S_tag, const Ctx& c, int kb, int q) {
    constexpr int S = decltype(S_tag)::value;
    if (q < kW) {
      const int m = NMAT == 2 ? (q >> 1) : 0;
      const uint32_t rows16 = (uint32_t)(NMAT == 2 ? (q & 1) : q) * code_tile;
      wring[S][q] = bload128(make_rsrc(p.w_packed[m] + c.T.e * mat_codes, (uint32_t)mat_codes), c.w_off,
                             rows16 + (uint32_t)kb * WL::kStep);
    } else if (q < kW + kA) {
      const int i = q - kW;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(a_rsrc, (lds_void_t*)(px_stage<S>() + (wv * kA + i) * 1024), 16,
                                               (int)c.a_off[i], kb * 256, 0, 0);
    } else {
      const int h = q - kW - kA;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          make_rsrc(p.w_scale[smat] + c.T.e * mat_scales, (uint32_t)mat_scales),
          (lds_void_t*)(px_sstage<S>() + (wv * kS + h) * 256), 4, (int)c.s_off,
          (int)(pf_scale_step<TL, W_NV>(kb) + (uint32_t)h * s_delta), 0, 0);
    }
  };
  auto issue = [&](auto S_tag, const Ctx& c, int kb) {
#pragma unroll
    for (int q = 0; q < kDma; ++q) issue_one(S_tag, c, kb, q);
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;

  // the first tile, and the tile after it (looked up, its gather indices read)
  PfTile pT = locate_tile_lds<NMAT, SH>(s_pref, s_rng, p.E, tile_at(0));
  int psrc[kA];
  src_rows(pT, psrc);
  Ctx cur = make_ctx(pT, psrc);
  pT = locate_tile_lds<NMAT, SH>(s_pref, s_rng, p.E, tile_at(1));
  src_rows(pT, psrc);
  issue(I0(), cur, 0);
  issue(I1(), cur, 1);
  issue(I2(), cur, 2);

  for (int i = 0; i < n_tiles; ++i) {
    // the next tile's loads go out in this tile's last three steps
    const Ctx nx = make_ctx(pT, psrc);
    float wglob[NMAT];
#pragma unroll
    for (int m = 0; m < NMAT; ++m) wglob[m] = W_NV ? load_uniform_f32(p.w_global[m] + cur.T.e) : 1.0f;

    // the tile's K loop.  Every 16-row token block is computed, also those past
    // the tile's end (their outputs are not stored).  Skipping the empty blocks
    // measured slower here: branches around whole steps or tiles made the
    // compiler copy the weight registers in flight at its joins and wait for
    // their loads, and branches around the MFMAs alone kept the converts from
    // overlapping them.  (The host picks this kernel when experts average
    // several tiles, so that the padding is a small part of the work.)
    f32x4 acc[4][4];
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int t = 0; t < 4; ++t) acc[g][t] = f32x4{0.f, 0.f, 0.f, 0.f};
    // step k from stage S: wait for this wave's loads of step k (those of steps
    // k + 1, k + 2 may stay in flight), barrier (every wave's loads landed, every
    // wave done with step k - 1, whose stage the step refills), then compute
    // while issuing step kn of tile lc (two loads per k-slot)
    auto step = [&](auto S_tag, const Ctx& lc, int kn) {
      constexpr int S = decltype(S_tag)::value;
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(2 * kDma));
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
      constexpr auto SN = std::integral_constant<int, (S + 3) % 4>();
      auto hook = [&](int s) {
        if (2 * s < kDma) issue_one(SN, lc, kn, 2 * s);
        if (2 * s + 1 < kDma) issue_one(SN, lc, kn, 2 * s + 1);
      };
      pf_compute<NMAT, WF, TL, SH, true, 4>(px_stage<S>(), px_sstage<S>(), acc, 0, wn, li, lg, hook, wring[S]);
    };
    int kb = 0;
    for (; kb + 4 < nk; kb += 4) {
      step(I0(), cur, kb + 3);
      step(I1(), cur, kb + 4);
      step(I2(), cur, kb + 5);
      step(I3(), cur, kb + 6);
    }
    step(I0(), cur, nk - 1);
    step(I1(), nx, 0);
    step(I2(), nx, 1);
    step(I3(), nx, 2);
    // the tile after next: looked up while the last MFMAs drain; its gather
    // indices load during the epilogue
    pT = locate_tile_lds<NMAT, SH>(s_pref, s_rng, p.E, tile_at(i + 2));
    src_rows(pT, psrc);
    if (p.out_bf16 && !p.out_codes && !p.out_dq) {                // bf16 out (+ row sums of squares)
      // every wave done reading stage 3 (the last step's operands) before any overwrites it
      __builtin_amdgcn_s_barrier();
      pf_epilogue_staged<NMAT>(p, cur.T, acc, wglob, wn, li, lg, px_stage<3>() + wv * 2048);
    } else {
      pf_epilogue<NMAT>(p, cur.T, acc, wglob, 0, wn, li, lg);
    }
    cur = nx;
  }
  // the last tile leaves its unread repeat loads in flight: let them land
  // before the workgroup's LDS is released
  __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8));             // vmcnt(0)
}

// --------------------------------------- NVFP4 tokens: through registers
// registers of one step in flight (per thread)
struct PfRegs {
  u32x4 a;                 // 32 token codes
  uint32_t asc;            // their two E4M3 scales
  u32x4 w[2];              // 2 weight-code chunks
  uint32_t s;              // one dword of weight scales
};

// one register-fed stage: token and weight codes, then the weight scales
constexpr int kPfNvStage = PfTall::Stage + PfTall::SStage;

template <int NMAT, int WF, bool TL>
__global__ __launch_bounds__(kPfThreads) void gemm_prefill_nv_kernel(GemmArgs p) {
  constexpr bool W_NV = WF != 0;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];      // 2 stages
  __shared__ int s_pref[kPfMaxE + 1];
  __shared__ int s_wc[kPfThreads / kWave];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  const int wm = wv >> 2, wn = wv & 3;                               // SIMD s holds waves s (wm 0) and s + 4 (wm 1)
  const int li = lane & 15, lg = lane >> 4;
  const int K = p.K, N = p.N;
  const int ntn = N / (PfTall::BN / NMAT);
  const int nk = K / kPfBK;                                          // even (checked on the host)
  const int total = build_tile_table<kPfThreads, PfTall::BM>(p, ntn, s_pref, s_wc);
  int t_begin, t_end, t_stride;
  xcd_slice(total, t_begin, t_end, t_stride);

  const uint32_t sc_row = (uint32_t)(W_NV ? K / 16 : K / 32);
  const uint32_t mat_codes = (uint32_t)N * (uint32_t)(K / 2);
  const uint32_t mat_scales = (uint32_t)N * sc_row;
  const rsrc_t ar = make_rsrc(p.a_data, (uint32_t)p.a_bytes);
  const rsrc_t asr = make_rsrc(p.a_scales, (uint32_t)(p.a_bytes / 8));
  // the matrix of a load is uniform per wave: code chunk j of any thread is in
  // matrix j (SwiGLU), a scale dword of wave w in matrix w / 4 (NV) or (w / 2) % 2 (MX)
  const int wvu = __builtin_amdgcn_readfirstlane(wv);
  const int smat = NMAT == 2 ? (W_NV ? (wvu >> 2) : ((wvu >> 1) & 1)) : 0;

  for (int tile = t_begin; tile < t_end; tile += t_stride) {
    const PfTile T = locate_tile<NMAT, PfTall>(p, s_pref, tile);
    // a wave whose 64 token rows all lie past the tile's end skips its MFMAs;
    // it still fetches, stores and syncs (the barriers here wait for every load anyway)
    const bool active = wm * 64 < T.mrows;
    rsrc_t wr[NMAT], sr[NMAT];
#pragma unroll
    for (int m = 0; m < NMAT; ++m) {
      wr[m] = make_rsrc(p.w_packed[m] + (int64_t)T.e * mat_codes, mat_codes);
      sr[m] = make_rsrc(p.w_scale[m] + (int64_t)T.e * mat_scales, mat_scales);
    }
    const rsrc_t s_rsrc = smat == 0 ? sr[0] : sr[NMAT - 1];
    float wglob[NMAT];
#pragma unroll
    for (int m = 0; m < NMAT; ++m) wglob[m] = W_NV ? p.w_global[m][T.e] : 1.0f;

    // tokens: row tid / 4, 32 codes (tid % 4) and their two scales
    uint32_t a_off, as_off;
    {
      const int row = tid >> 2;
      const int64_t r = T.rbase + min(row, T.mrows - 1);            // rows past the tile's end reread a valid row
      const int64_t src = p.gather ? (int64_t)(p.gather[r] / p.gather_div) : r;
      a_off = (uint32_t)(src * (K / 2)) + (uint32_t)(tid & 3) * 16u;
      as_off = (uint32_t)(src * (K / 16)) + (uint32_t)(tid & 3) * 2u;
    }
    // weight codes: chunks q = tid + 512 j (row q / 4, chunk q % 4); scales: MX row tid % 256, NV row tid / 2, half tid % 2
    // (tiled: chunk q is lane q % 64 of 16-row group q / 64's block)
    uint32_t w_off[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int q = tid + kPfThreads * j;
      if (TL) {
        const int tile = (T.nbase + pf_wrow<NMAT, PfTall::BN>((q >> 6) * 16)) >> 4;
        w_off[j] = (uint32_t)tile * (uint32_t)(K / 128) * 1024u + (uint32_t)(q & 63) * 16u;
      } else {
        w_off[j] = (uint32_t)(T.nbase + pf_wrow<NMAT, PfTall::BN>(q >> 2)) * (uint32_t)(K / 2) + (uint32_t)(q & 3) * 16u;
      }
    }
    const int s_n = W_NV ? (tid >> 1) : (tid & 255);
    const uint32_t s_off = pf_scale_lane<TL, W_NV>(T.nbase + pf_wrow<NMAT, PfTall::BN>(s_n), tid & 1, K);

    auto fetch = [&](PfRegs& R, int kb) {
      R.a = bload128(ar, a_off + (uint32_t)kb * 64u, 0);
      R.asc = bload16(asr, as_off + (uint32_t)kb * 8u, 0);
#pragma unroll
      for (int j = 0; j < 2; ++j) R.w[j] = bload128(wr[NMAT == 2 ? j : 0], w_off[j] + (uint32_t)kb * (TL ? 1024u : 64u), 0);
      R.s = bload32(s_rsrc, s_off + pf_scale_step<TL, W_NV>(kb), 0);
    };
    auto store = [&](const PfRegs& R, uint8_t* st) {
      uint8_t* sa = st;
      uint8_t* sw = st + PfTall::AStage;
      uint8_t* ss = st + PfTall::Stage;
      const int row = tid >> 2, c = tid & 3;
      const float s_lo = e4m3_byte<0>(R.asc) * p.a_gscale, s_hi = e4m3_byte<1>(R.asc) * p.a_gscale;
#pragma unroll
      for (int s = 0; s < 4; ++s)
        *(u32x4*)(sa + swz_a(row, c * 4 + s)) = __builtin_bit_cast(u32x4, fp4x8_to_bf16(R.a[s], s < 2 ? s_lo : s_hi));
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int q = tid + kPfThreads * j;
        *(u32x4*)(sw + (TL ? (uint32_t)q * 16u : swz_w(q >> 2, q & 3))) = R.w[j];
      }
      // NV: row tid / 2, half tid % 2; MX: row tid (threads >= 256 write an unread copy)
      *(uint32_t*)(ss + tid * 4) = R.s;
    };

    f32x4 acc[4][4];
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int t = 0; t < 4; ++t) acc[g][t] = f32x4{0.f, 0.f, 0.f, 0.f};

    uint8_t* st0 = lds;
    uint8_t* st1 = lds + kPfNvStage;
    PfRegs R0, R1;
    __syncthreads();                                                 // previous tile done with LDS
    fetch(R0, 0);
    fetch(R1, 1);
    store(R0, st0);
    __syncthreads();
    // Loads and stores are unconditional (past the last step they repeat it, from
    // L2) so the compiler can count every wait exactly; scheduling fences keep
    // each fetch at the top of its half-iteration.
    for (int kb = 0; kb < nk; kb += 2) {
      fetch(R0, min(kb + 2, nk - 1));
      __builtin_amdgcn_sched_barrier(0);
      if (active) pf_compute<NMAT, WF, TL, PfTall>(st0, st0 + PfTall::Stage, acc, wm, wn, li, lg);
      __builtin_amdgcn_sched_barrier(0);
      store(R1, st1);                                                // step kb + 1
      __syncthreads();
      fetch(R1, min(kb + 3, nk - 1));
      __builtin_amdgcn_sched_barrier(0);
      if (active) pf_compute<NMAT, WF, TL, PfTall>(st1, st1 + PfTall::Stage, acc, wm, wn, li, lg);
      __builtin_amdgcn_sched_barrier(0);
      store(R0, st0);                                                // step kb + 2
      __syncthreads();
    }

    pf_epilogue<NMAT>(p, T, acc, wglob, wm, wn, li, lg);
  }
}

// ------------------------------------------------------------------- host
// the cross-tile kernel: 64 x 512 tiles, K a multiple of 512, power-of-two weight scales
// and at least 160 rows per expert on average: below that the last, partly
// filled tile of each expert is a large share of the work, and the per-tile
// kernel, which skips a tile's empty 16-row blocks, is as fast or faster
// (measured at 128 rows per expert: 2-3% faster)
template <int WF>
static bool xt_fits(int N, int K, int NMAT, int64_t rows, int E) {
  return WF != 2 && N % (PfWide::BN / NMAT) == 0 && K % 512 == 0 && rows >= 160LL * E;
}

template <int NMAT, int WF, bool A_NV, bool TL>
static void launch_prefill_one(const GemmArgs& a, hipStream_t stream) {
  // persistent: one workgroup per CU (8 waves); tiles are distributed on the device
  if (A_NV) {
    auto kern = gemm_prefill_nv_kernel<NMAT, WF, TL>;
    static bool attr_set = false;
    if (!attr_set) {
      (void)hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, 2 * kPfNvStage);
      attr_set = true;
    }
    hipLaunchKernelGGL(kern, dim3(device_cus()), dim3(kPfThreads), 2 * kPfNvStage, stream, a);
  } else if (xt_fits<WF>(a.N, a.K, NMAT, a.rows, a.E)) {
    // bf16 tokens, 64 x 512 tiles, the pipeline carried across tiles
    if constexpr (WF != 2)
      hipLaunchKernelGGL((gemm_prefill_xt_kernel<NMAT, WF, TL>), dim3(device_cus()), dim3(kPfThreads), 0, stream, a);
  } else if (a.N % (PfWide::BN / NMAT) == 0) {      // bf16 tokens: 64 x 512 tiles where N allows
    hipLaunchKernelGGL((gemm_prefill_dma_kernel<NMAT, WF, TL, PfWide>), dim3(device_cus()), dim3(kPfThreads), 0, stream, a);
  } else {
    hipLaunchKernelGGL((gemm_prefill_dma_kernel<NMAT, WF, TL, PfTall>), dim3(device_cus()), dim3(kPfThreads), 0, stream, a);
  }
}

template <bool TL, int NMAT>
static void launch_prefill_f(const GemmArgs& a, int wf, bool a_nv, hipStream_t stream) {
  switch (wf) {
    case 0: a_nv ? launch_prefill_one<NMAT, 0, true, TL>(a, stream) : launch_prefill_one<NMAT, 0, false, TL>(a, stream); break;
    case 1: a_nv ? launch_prefill_one<NMAT, 1, true, TL>(a, stream) : launch_prefill_one<NMAT, 1, false, TL>(a, stream); break;
    default: a_nv ? launch_prefill_one<NMAT, 2, true, TL>(a, stream) : launch_prefill_one<NMAT, 2, false, TL>(a, stream); break;
  }
}

// the kernels of one weight layout (TL: tiled), instantiated in their own
// translation unit so they compile in parallel
template <bool TL>
void prefill_run(const GemmArgs& a, bool swiglu, int wf, bool a_nv, hipStream_t stream) {
  if (swiglu) launch_prefill_f<TL, 2>(a, wf, a_nv, stream);
  else launch_prefill_f<TL, 1>(a, wf, a_nv, stream);
}

extern template void prefill_run<false>(const GemmArgs&, bool, int, bool, hipStream_t);
extern template void prefill_run<true>(const GemmArgs&, bool, int, bool, hipStream_t);

}  // namespace moe
