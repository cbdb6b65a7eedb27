// Grouped FP4 expert GEMM, weight-streaming ("decode") form: few rows per
// expert, so the kernel is bound by reading the FP4 weights from HBM once.
//
// The expert FFN is W_down(SiLU(W_gate h) * (W_up h)) ("MiMo-V2.6-Flash --
// REAP-50", "Pruning Method", saliency equation); weights are MXFP4 or their
// exact NVFP4 transcode; accumulation is FP32 ("AxionML / MiMo-V2.6-Flash-
// MOPD-NVFP4", "About NVFP4 quantization").
//
// Work split: a workgroup takes the j-th expert that has rows and a tile of
// 16*NWN*NT weight rows (output features), laid out so that one expert's
// workgroups run on one XCD.  Each wave owns 16 weight rows and
// walks its K range in steps of 128: in one step, lane group g (lanes
// 16g..16g+15) reads one whole 32-value block (16 code bytes) of each of the 16
// rows, dequantises it in registers (E2M1 x power-of-two scale -> bf16 with the
// gfx950 convert instruction) and feeds four bf16 16x16x32 MFMAs whose other
// operand holds the pass's token rows (up to MR = 8 of its 16).  Scales
// arrive as one 16-byte window per four steps (MX) or two (NV).  For the
// model's K (4096, 2048) the step loop is
// unrolled at compile time, so weight loads run PF steps ahead and token loads
// PA steps ahead with every wait counted exactly; other K take a runtime loop.
// Weight codes and scale windows are read with the non-temporal cache policy:
// each is read once per pass, and streaming them past the caches measured 6%
// faster per 64-token layer (gate/up at 77% instead of 73% of HBM peak).
// For tiny batches KS waves split one tile's K range into contiguous pieces;
// their partial sums meet in LDS in a fixed order (deterministic).  The
// epilogue (SwiGLU, global scales, bf16 and/or NVFP4 output) runs on the
// accumulator registers.  An expert with more than MR token rows takes
// further passes over the same weights (rare where this kernel is chosen: it
// runs below 4 rows per expert on average).  Token rows past the
// pass's end read a valid row; their output columns are never stored.
#pragma once
#include <algorithm>

#include "gemm_common.h"

namespace moe {

template <int NMAT>
struct WStage {
  u32x4 w[NMAT];          // 32 codes of this lane's block, per matrix
};

struct AStage {
  u32x4 a[4];             // 32 bf16 activations of this lane's token row and block
};

// 4 values of one 16-wide NVFP4 block held by this lane; the other 12 are in
// lanes +-16, +-32 (same token row).  Returns 16 bits of codes for the 4 values
// and the block's scale byte.
__device__ __forceinline__ uint32_t quant4_across_lanes(const float* v, float inv_g, uint32_t& sb_out) {
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
      uint32_t c = e2m1_code(fabsf(xs), s) | ((__float_as_uint(xs) >> 28) & 8u);
      bits |= c << (4 * i);
    }
  }
  sb_out = sb;
  return bits;
}

// WF: weight scale format -- 0 MXFP4 (E8M0 per 32), 1 NVFP4 whose E4M3 scales
// are all powers of two (the exact MXFP4 transcode), 2 NVFP4 with any scales,
// 3 compact MXFP4 (4-bit exponent code c per 32: scale 2^c here, the matrix's
// base 2^b applied with the global scales in the epilogue -- a power-of-two
// factor on every product, so the sums are those of the MXFP4 path times 2^-b).
template <int NMAT, int WF, bool TL = false>
struct DecodeWave {
  static constexpr bool W_NV = WF == 1 || WF == 2;
  static constexpr bool W_CP = WF == 3;
  static constexpr int WB = W_CP ? 8 : (W_NV ? 32 : 16);
  using WL = WeightLaneB<TL, WB>;
  static constexpr bool W_GEN = WF == 2;     // general E4M3 scales: convert through float
  static constexpr int SWN = W_NV ? 2 : 1;   // dwordx4 per scale window (compact: its low half)
  rsrc_t wr_[NMAT];          // this expert's codes [N, K/2]
  rsrc_t sr_[NMAT];          // this expert's scales [N, K/32] | [N, K/16] | [N, K/64]
  uint32_t wo;               // code offset of (row n0+li, block 4*st0+lg), first tile
  uint32_t so;               // scale offset of (row n0+li, block 4*st0), first tile
  uint32_t wtile, stile;     // offset from one 16-row tile to the next (codes, scales)
  const uint8_t* al;         // LDS: this lane's token row at block 4*st0+lg (bf16)
  int lg;
  f32x4 acc[NMAT];

  __device__ __forceinline__ void wload(WStage<NMAT>& S, int t, int i) const {
#pragma unroll
    for (int m = 0; m < NMAT; ++m) S.w[m] = bload128_nt(wr_[m], wo + t * wtile + i * WL::kStep, 0);
  }
  __device__ __forceinline__ void aload(AStage& S, int i) const {
    const u32x4* a4 = (const u32x4*)(al + i * 256);
#pragma unroll
    for (int s = 0; s < 4; ++s) S.a[s] = a4[s];
  }
  // scale window of super-step c of tile t (4 steps x 4 lane groups): MX 16 B, NV 32 B, compact 8 B
  __device__ __forceinline__ void sload(u32x4 (&W)[NMAT][SWN], int t, int c) const {
#pragma unroll
    for (int m = 0; m < NMAT; ++m) {
      if (W_CP) {
        const u32x2 v = bload64_nt(sr_[m], so + t * stile + c * WL::kWin, 0);
        W[m][0] = u32x4{v[0], v[1], 0u, 0u};
      } else {
#pragma unroll
        for (int h = 0; h < SWN; ++h) W[m][h] = bload128_nt(sr_[m], so + t * stile + c * WL::kWin + 16 * h, 0);
      }
    }
  }
  // this lane's scale bits (E8M0 byte, two E4M3 bytes, or a 4-bit code) for step j of a window
  __device__ __forceinline__ uint32_t sbits(const u32x4 (&W)[SWN], int j) const {
    if (W_CP) return (W[0][j >> 1] >> (4 * (4 * (j & 1) + lg))) & 0xFu;   // block 4j + lg: nibble of dword j/2
    if (W_NV) {                 // dword 2j + lg / 2 of the window, chosen by a select (no indexed registers)
      const uint32_t d0 = W[(2 * j) >> 2][(2 * j) & 3], d1 = W[(2 * j + 1) >> 2][(2 * j + 1) & 3];
      return (((lg >> 1) ? d1 : d0) >> (16 * (lg & 1))) & 0xFFFFu;
    }
    return (W[0][j] >> (8 * lg)) & 0xFFu;
  }
  // this lane's scale bits for own step i of tile t, loaded on their own (remainder steps)
  __device__ __forceinline__ uint32_t sbits_direct(int m, int t, int i) const {
    if (W_NV) return bload16(sr_[m], so + t * stile + (4 * i + lg) * 2, 0);
    if (W_CP) return (bload8(sr_[m], so + t * stile + ((4 * i + lg) >> 1), 0) >> (4 * (lg & 1))) & 0xFu;
    return bload8(sr_[m], so + t * stile + 4 * i + lg, 0);
  }
  __device__ __forceinline__ void consume(const WStage<NMAT>& W, const AStage& A, const uint32_t (&sb)[NMAT]) {
    bf16x8 af[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) af[s] = __builtin_bit_cast(bf16x8, A.a[s]);
#pragma unroll
    for (int m = 0; m < NMAT; ++m) {
      float s_lo, s_hi;
      if (W_NV) {
        s_lo = e4m3_byte<0>(sb[m]);
        s_hi = e4m3_byte<1>(sb[m]);
      } else if (W_CP) {
        s_lo = s_hi = __uint_as_float((sb[m] + 127u) << 23);   // 2^c, c in [0, 15]
      } else {
        s_lo = s_hi = e8m0_to_f32(sb[m]);
      }
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const float sc = s < 2 ? s_lo : s_hi;
        const bf16x8 wf = W_GEN ? fp4x8_to_bf16_general(W.w[m][s], sc) : fp4x8_to_bf16_pow2(W.w[m][s], sc);
        acc[m] = mfma16(wf, af[s], acc[m]);
      }
    }
  }
  __device__ __forceinline__ void clear() {
#pragma unroll
    for (int m = 0; m < NMAT; ++m) acc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // The first PF weight steps are issued before the token rows are staged.
  template <int PF, int NT, int NS>
  __device__ __forceinline__ void prefetch(WStage<NMAT> (&wr)[PF], u32x4 (&sw)[NMAT][SWN]) const {
    sload(sw, 0, 0);
#pragma unroll
    for (int q = 0; q < PF; ++q)
      if (q < NT * NS) wload(wr[q], q / NS, q % NS);
  }

  // NT tiles x NS own steps known at compile time: one fully unrolled pipeline
  // that runs across tile boundaries; epi(t) finishes tile t.
  template <int NT, int NS, int PF, int PA, typename Epi>
  __device__ __forceinline__ void run_static(WStage<NMAT> (&wr)[PF], u32x4 (&sw0)[NMAT][SWN], Epi&& epi) {
    static_assert(NS % 4 == 0, "super-steps of 4");
    constexpr int TOT = NT * NS;
    AStage ar[PA];
    u32x4 sw1[NMAT][SWN];
#pragma unroll
    for (int q = 0; q < PA; ++q)
      if (q < NS) aload(ar[q], q);
    clear();
#pragma unroll
    for (int i = 0; i < TOT; ++i) {
      const int t = i / NS, il = i % NS;
      const int cg = i / 4, j = i % 4;                        // global super-step, step in it
      if (j == 0 && (cg + 1) * 4 < TOT) {
        const int tn = ((cg + 1) * 4) / NS, cn = (((cg + 1) * 4) % NS) / 4;
        if (cg & 1) sload(sw0, tn, cn);
        else sload(sw1, tn, cn);
      }
      uint32_t sb[NMAT];
#pragma unroll
      for (int m = 0; m < NMAT; ++m) sb[m] = sbits((cg & 1) ? sw1[m] : sw0[m], j);
      consume(wr[i % PF], ar[i % PA], sb);
      if (i + PA < TOT) aload(ar[i % PA], (i + PA) % NS);
      if (i + PF < TOT) wload(wr[i % PF], (i + PF) / NS, (i + PF) % NS);
      if (il == NS - 1) {
        epi(t);
        clear();
      }
    }
  }

  // Any step count (K other than the model's): windows for whole super-steps,
  // single-step scale loads for the remainder (never past the row's end).
  template <typename Epi>
  __device__ __forceinline__ void run_dynamic(int nt, int ns, Epi&& epi) {
    for (int t = 0; t < nt; ++t) {
      clear();
      int c = 0;
      for (; 4 * c + 4 <= ns; ++c) {
        u32x4 sw[NMAT][SWN];
        sload(sw, t, c);
        WStage<NMAT> wr[4];
        AStage ar[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          wload(wr[j], t, 4 * c + j);
          aload(ar[j], 4 * c + j);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          uint32_t sb[NMAT];
#pragma unroll
          for (int m = 0; m < NMAT; ++m) sb[m] = sbits(sw[m], j);
          consume(wr[j], ar[j], sb);
        }
      }
      for (int i = 4 * c; i < (TL ? 4 * c : ns); ++i) {       // (tiled: k % 512 == 0, no remainder)
        WStage<NMAT> w;
        AStage a;
        wload(w, t, i);
        aload(a, i);
        uint32_t sb[NMAT];
#pragma unroll
        for (int m = 0; m < NMAT; ++m) sb[m] = sbits_direct(m, t, i);
        consume(w, a, sb);
      }
      epi(t);
    }
  }
};

// Finish one 16-row tile: lane holds D[nt0 + 4*lg + i][token row ro] (i < 4);
// SwiGLU and global weight scales, then bf16 and/or NVFP4 output.
template <int NMAT>
__device__ __forceinline__ void decode_finish(const GemmArgs& p, const f32x4 (&acc)[NMAT], const float (&wglob)[NMAT],
                                              int64_t ro, bool ok, int nt0, int lg) {
  const int N = p.N;
  float v[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float g = acc[0][i] * wglob[0];
    v[i] = NMAT == 2 ? silu_div(g) * (acc[NMAT - 1][i] * wglob[NMAT - 1]) : g;
  }
  const uint32_t b01 = pack_bf16x2(v[0], v[1]), b23 = pack_bf16x2(v[2], v[3]);
  const int col = nt0 + 4 * lg;
  if (p.out_bf16 && ok) *(u32x2*)(p.out_bf16 + ro * N + col) = u32x2{b01, b23};
  if (p.out_codes || p.out_dq) {
    float q[4] = {bf16_lo(b01), bf16_hi(b01), bf16_lo(b23), bf16_hi(b23)};
    uint32_t sb;
    const uint32_t bits = quant4_across_lanes(q, p.out_inv_g, sb);
    if (ok) {
      if (p.out_codes) {
        *(uint16_t*)(p.out_codes + ro * (N / 2) + col / 2) = (uint16_t)bits;
        if (lg == 0) p.out_scales[ro * (N / 16) + nt0 / 16] = (uint8_t)sb;
      }
      if (p.out_dq) *(u32x2*)(p.out_dq + ro * N + col) = nvfp4_dequant4(bits, e4m3_to_f32(sb) * p.out_g);
    }
  }
}

// Stage the token rows [rbase, rbase + mrows) of this expert into LDS as bf16
// (row pitch K*2 + 16 bytes so the 16 rows of one MFMA read hit distinct
// banks).  NVFP4 activations are dequantised here, once per block.
template <bool A_NV>
__device__ __forceinline__ void stage_rows(const GemmArgs& p, uint8_t* lds, int rbase, int mrows, int pitch) {
  const int K = p.K;
  if (A_NV) {
    const int nblk = K / 32;                                  // 32-value blocks per row
    for (int t = threadIdx.x; t < mrows * nblk; t += blockDim.x) {
      const int row = t / nblk, b = t % nblk;
      const int64_t r = rbase + row;
      const int64_t src = p.gather ? (int64_t)(p.gather[r] / p.gather_div) : r;
      u32x4 cw = *(const u32x4*)(p.a_data + src * (K / 2) + b * 16);
      uint32_t sw = *(const uint16_t*)(p.a_scales + src * (K / 16) + b * 2);
      float s_lo = e4m3_byte<0>(sw) * p.a_gscale;
      float s_hi = e4m3_byte<1>(sw) * p.a_gscale;
      u32x4* dst = (u32x4*)(lds + row * pitch + b * 64);
#pragma unroll
      for (int s = 0; s < 4; ++s) dst[s] = __builtin_bit_cast(u32x4, fp4x8_to_bf16(cw[s], s < 2 ? s_lo : s_hi));
    }
  } else {
    const int nch = K / 8;                                    // 16-byte chunks per row
    for (int t = threadIdx.x; t < mrows * nch; t += blockDim.x) {
      const int row = t / nch, c = t % nch;
      const int64_t r = rbase + row;
      const int64_t src = p.gather ? (int64_t)(p.gather[r] / p.gather_div) : r;
      *(u32x4*)(lds + row * pitch + c * 16) = *(const u32x4*)(p.a_data + src * (int64_t)K * 2 + c * 16);
    }
  }
}

// Token rows per pass (LDS holds kDecRows rows of K bf16), weight steps in
// flight per wave (the LDS stage caps occupancy, so deep register rings are
// free), 16-row tiles per gate/up wave, and waves per workgroup when many waves
// stream (measured best of 4, 8 and 16 waves; 4 / 8 / 16 rows per pass; 1 or 2
// tiles per wave).
constexpr int kDecRows = 8;
constexpr int kDecRing2 = 8;           // gate/up (two matrices)
constexpr int kDecRing1 = 4;           // down
constexpr int kDecTiles2 = 2;
constexpr int kDecWaves1 = 8;          // down
constexpr int kDecWaves2 = 4;          // gate/up
__host__ __device__ constexpr int decode_rows_per_pass(int) { return kDecRows; }
__host__ __device__ constexpr int decode_pitch(int K) { return K * 2 + 16; }

template <int NMAT, int NWN, int KS, int NT, int NS, int WF, bool A_NV, bool TL>
__global__ __launch_bounds__(NWN * KS * 64) void gemm_decode_kernel(GemmArgs p) {
  // the general NVFP4 conversion needs more registers: a shorter weight ring
  constexpr int PF = NMAT == 2 ? (WF == 2 ? 4 : kDecRing2) : kDecRing1, PA = 2;
  static_assert(KS == 1 || NT == 1, "the K split runs one tile per wave");
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int wn = wv % NWN, ks = wv / NWN;
  const int li = lane & 15, lg = lane >> 4;
  extern __shared__ __attribute__((aligned(16))) uint8_t a_lds[];

  // 1-D grid, XCD-aware: workgroup b runs on XCD b % 8; the n-blocks of the
  // j-th active expert all get the same b % 8 (= j % 8), so they share that
  // XCD's L2 for the expert's token rows
  const int K = p.K, N = p.N;
  const int nxb = N / (16 * NWN * NT);                        // n-blocks per expert
  const int xcd = blockIdx.x & 7, rank = blockIdx.x >> 3;
  const int xb = rank % nxb, jexp = (rank / nxb) * 8 + xcd;
  int e, r0, r1;
  if (!find_active_expert(p.offsets, p.E, p.rows, jexp, e, r0, r1)) return;
  const int MR = decode_rows_per_pass(K), pitch = decode_pitch(K);
  // this wave's NT tiles of 16 weight rows: n0 + 16 * NWN * t
  const int n0 = xb * (16 * NWN * NT) + wn * 16;
  const int ns = NS > 0 ? NS : (K / 128) / KS;                // own steps per tile (contiguous range)
  const int st0 = ks * ns;                                    // first global step

  using DW = DecodeWave<NMAT, WF, TL>;
  DW dw;
  using WL = typename DW::WL;
  dw.lg = lg;
  const uint32_t mat_codes = (uint32_t)N * (uint32_t)(K / 2);
  const uint32_t sc_row = (uint32_t)(K / (512 / DW::WB));
  const uint32_t mat_scales = (uint32_t)N * sc_row;
#pragma unroll
  for (int m = 0; m < NMAT; ++m) {
    dw.wr_[m] = make_rsrc(p.w_packed[m] + (int64_t)e * mat_codes, mat_codes);
    dw.sr_[m] = make_rsrc(p.w_scale[m] + (int64_t)e * mat_scales, mat_scales);
  }
  // tile base + lane part + the first own step (st0 is a multiple of 4: whole windows)
  dw.wo = (uint32_t)n0 * (uint32_t)(K / 2) + WL::code(li, lg, K) + (uint32_t)st0 * WL::kStep;
  dw.so = (uint32_t)n0 * sc_row + WL::scale(li, K) + (uint32_t)(st0 / 4) * WL::kWin;
  dw.wtile = (uint32_t)(16 * NWN) * (uint32_t)(K / 2);
  dw.stile = (uint32_t)(16 * NWN) * sc_row;

  float wglob[NMAT];
#pragma unroll
  for (int m = 0; m < NMAT; ++m) wglob[m] = WF != 0 ? p.w_global[m][e] : 1.0f;   // NV global | compact base

  __shared__ f32x4 red[KS > 1 ? (KS - 1) * NWN * NMAT * 64 : 1];

  for (int rbase = r0; rbase < r1; rbase += MR) {
    const int mrows = min(MR, r1 - rbase);
    const bool arow_ok = li < mrows;
    // rows >= mrows read row 0 of the stage; their output columns are dropped
    dw.al = a_lds + (arow_ok ? li : 0) * pitch + (4 * st0 + lg) * 64;

    // finish tile t: K-split reduction, SwiGLU / global scales, bf16 and/or NVFP4 out
    auto epi = [&](int t) {
      if (KS > 1) {
        if (ks > 0) {
#pragma unroll
          for (int m = 0; m < NMAT; ++m) red[(((ks - 1) * NWN + wn) * NMAT + m) * 64 + lane] = dw.acc[m];
        }
        __syncthreads();
        if (ks == 0) {
          for (int k2 = 1; k2 < KS; ++k2)
#pragma unroll
            for (int m = 0; m < NMAT; ++m) dw.acc[m] += red[(((k2 - 1) * NWN + wn) * NMAT + m) * 64 + lane];
        }
        __syncthreads();
      }
      if (ks != 0) return;
      decode_finish<NMAT>(p, dw.acc, wglob, rbase + li, arow_ok, n0 + t * 16 * NWN, lg);
    };

    if constexpr (NS > 0) {
      WStage<NMAT> wr[PF];
      u32x4 sw0[NMAT][DecodeWave<NMAT, WF, TL>::SWN];
      dw.template prefetch<PF, NT, NS>(wr, sw0);          // weights in flight while the rows stage
      if (rbase != r0) __syncthreads();                  // previous pass done with the stage
      stage_rows<A_NV>(p, a_lds, rbase, mrows, pitch);
      __syncthreads();
      dw.template run_static<NT, NS, PF, PA>(wr, sw0, epi);
    } else {
      if (rbase != r0) __syncthreads();
      stage_rows<A_NV>(p, a_lds, rbase, mrows, pitch);
      __syncthreads();
      dw.run_dynamic(NT, ns, epi);
    }
  }
}

template <int NMAT, int NWN, int KS, int NT, int NS, int WF, bool A_NV, bool TL>
static void launch_decode_one(const GemmArgs& a, int nact, hipStream_t stream) {
  auto kern = gemm_decode_kernel<NMAT, NWN, KS, NT, NS, WF, A_NV, TL>;
  const size_t lds = (size_t)decode_rows_per_pass(a.K) * decode_pitch(a.K);
  static bool attr_set = false;               // one-time opt-in to > 64 KB of LDS
  if (!attr_set) {
    (void)hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, 96 * 1024);
    attr_set = true;
  }
  const int nxb = a.N / (16 * NWN * NT);
  const int64_t blocks = (int64_t)nxb * ((nact + 7) / 8) * 8;   // whole groups of 8 experts (see the kernel)
  hipLaunchKernelGGL(kern, dim3((uint32_t)blocks), dim3(NWN * KS * 64), lds, stream, a);
}

template <bool TL, int NMAT, int NWN, int KS, int NT, int NS>
static void launch_decode_t(const GemmArgs& a, int wf, bool a_nv, int nact, hipStream_t stream) {
  switch (wf) {
    case 0: a_nv ? launch_decode_one<NMAT, NWN, KS, NT, NS, 0, true, TL>(a, nact, stream)
                 : launch_decode_one<NMAT, NWN, KS, NT, NS, 0, false, TL>(a, nact, stream); break;
    case 1: a_nv ? launch_decode_one<NMAT, NWN, KS, NT, NS, 1, true, TL>(a, nact, stream)
                 : launch_decode_one<NMAT, NWN, KS, NT, NS, 1, false, TL>(a, nact, stream); break;
    case 2: a_nv ? launch_decode_one<NMAT, NWN, KS, NT, NS, 2, true, TL>(a, nact, stream)
                 : launch_decode_one<NMAT, NWN, KS, NT, NS, 2, false, TL>(a, nact, stream); break;
    default: a_nv ? launch_decode_one<NMAT, NWN, KS, NT, NS, 3, true, TL>(a, nact, stream)
                  : launch_decode_one<NMAT, NWN, KS, NT, NS, 3, false, TL>(a, nact, stream); break;
  }
}

// K split into KS contiguous pieces of NS own steps (compile time for the model's K);
// NT tiles of 16 rows per wave when K is not split.
template <bool TL, int NMAT, int NWN, int KS>
static void launch_decode_k(const GemmArgs& a, int wf, bool a_nv, int nact, hipStream_t stream) {
  const int nsteps = a.K / 128;
  constexpr int NT = (KS > 1 || NMAT == 1) ? 1 : kDecTiles2;
  if (KS == 1 && a.N % (16 * NWN * NT) == 0) {
    if (nsteps == 32) return launch_decode_t<TL, NMAT, NWN, KS, NT, 32>(a, wf, a_nv, nact, stream);
    if (nsteps == 16) return launch_decode_t<TL, NMAT, NWN, KS, NT, 16>(a, wf, a_nv, nact, stream);
  }
  if (nsteps == 32) launch_decode_t<TL, NMAT, NWN, KS, 1, 32 / KS>(a, wf, a_nv, nact, stream);
  else if (nsteps == 16) launch_decode_t<TL, NMAT, NWN, KS, 1, 16 / KS>(a, wf, a_nv, nact, stream);
  else launch_decode_t<TL, NMAT, NWN, KS, 1, 0>(a, wf, a_nv, nact, stream);
}

template <bool TL, int NMAT>
static void launch_decode_ks(const GemmArgs& a, int wf, bool a_nv, int nact, hipStream_t stream) {
  // split K when too few waves would stream weights (aim for >= 8 waves per
  // CU); each piece keeps a multiple of 4 steps (one scale window per 4).
  const int64_t waves = (int64_t)nact * (a.N / 16);
  const int nsteps = a.K / 128;
  if (a.N % 64 != 0) {
    launch_decode_k<TL, NMAT, 1, 1>(a, wf, a_nv, nact, stream);
  } else if (waves >= 2048 || nsteps % 8 != 0) {
    constexpr int NWN = NMAT == 1 ? kDecWaves1 : kDecWaves2;
    if (a.N % (16 * NWN) == 0) launch_decode_k<TL, NMAT, NWN, 1>(a, wf, a_nv, nact, stream);
    else launch_decode_k<TL, NMAT, 4, 1>(a, wf, a_nv, nact, stream);
  } else if (waves >= 1024 || nsteps % 16 != 0) {
    launch_decode_k<TL, NMAT, 2, 2>(a, wf, a_nv, nact, stream);
  } else {
    launch_decode_k<TL, NMAT, 1, 4>(a, wf, a_nv, nact, stream);
  }
}

// Launchers of one weight layout (TL: tiled), each instantiated in its own
// translation unit so the kernel variants compile in parallel.
template <bool TL>
void decode_wg(const GemmArgs& a, bool swiglu, int wf, bool a_nv, int nact, hipStream_t stream) {
  if (swiglu) launch_decode_ks<TL, 2>(a, wf, a_nv, nact, stream);
  else launch_decode_ks<TL, 1>(a, wf, a_nv, nact, stream);
}

extern template void decode_wg<false>(const GemmArgs&, bool, int, bool, int, hipStream_t);
extern template void decode_wg<true>(const GemmArgs&, bool, int, bool, int, hipStream_t);

}  // namespace moe
