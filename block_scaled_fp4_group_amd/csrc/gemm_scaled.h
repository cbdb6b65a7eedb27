// Grouped FP4 expert GEMM on gfx950's block-scaled MFMA
// (V_MFMA_SCALE_F32_16X16X128_F8F6F4): the FP4 expert weights are the native
// E2M1 operand with their own E8M0 scale per 32 values, the tokens an FP8
// (E4M3) operand with an E8M0 scale per 32 values, FP32 accumulation.  No
// weight is dequantised.
//
// Token operand modes:
//   * MXFP8 (W4A8): E4M3 activations with a power-of-two scale per 32 values,
//     as the expert GEMMs of the "MiMo-V2.6-Flash-MOPD on one RTX PRO 6000"
//     recipe run prompt batches ("Quantization, context and quality",
//     Activations; "What makes it fast", speed v5.2: FP8 x FP4 block-scaled
//     GEMMs).  One MFMA K-chunk of 128 per 128 values of K.
//   * NVFP4 planes (W4A4, "AxionML / MiMo-V2.6-Flash-MOPD-NVFP4", header): an
//     NVFP4 activation's arbitrary E4M3 scale per 16 values has no E8M0 form,
//     so each 16-value block arrives as two exact E4M3 planes (hi, lo) under
//     one power-of-two scale (common.h, nvfp4_planes4).  A 32-value MFMA scale
//     block holds one 16-block's [hi | lo] pair; the weight operand feeds that
//     16-block's FP4 codes twice, under the weight block's own E8M0 scale.  Two
//     MFMA K-chunks per 128 values of K: the exact W4A4 product at the FP8
//     rate, i.e. the same MFMA time as bf16 after dequantisation, but with the
//     weights native and no convert instructions.
//
// Operand layout of the 16x16x128 instruction (measured on the chip):
//   FP4 operand: lane l holds row l % 16, K values 32 (l/16) .. +31 in 4 dwords;
//   FP8 operand: lane l holds row l % 16, K values 16 (l/16) .. +15 in dwords
//                0-3 and 64 + 16 (l/16) .. +15 in dwords 4-7;
//   scales: lane l's E8M0 byte scales row l % 16 over K block (l/16) of 32.
// Output: lane l holds D[weight row 4 (l/16) + i][token l % 16], i < 4, as
// the bf16 kernels' 16x16x32 MFMA, so the epilogues are shared.
//
// Structure as the bf16-token prefill kernel (gemm_prefill.h): persistent
// workgroups of 8 waves walk the XCD-sliced tile list; a tile is 64 tokens x
// 512 weight rows (SwiGLU: 256 gate + 256 up); the token codes and scales and
// the weight scales of each K step go straight from HBM into one of three LDS
// stages two steps ahead (direct-to-LDS loads), the weight codes straight into
// each wave's registers (three steps deep).
#pragma once
#include "gemm_prefill.h"

namespace moe {

template <bool PL>
struct SxShape {
  static constexpr int BM = 64, BN = 512, WN = 8;
  static constexpr int ARow = PL ? 256 : 128;          // token operand bytes per row and step
  static constexpr int AStage = BM * ARow;
  static constexpr int TSRow = PL ? 8 : 4;             // token scale bytes per row and step
  static constexpr int TSStage = BM * TSRow;
  static constexpr int WSStage = BN * 8;               // weight scale bytes (MX uses half)
  static constexpr int Stage = AStage + TSStage;         // token stage (weight scales: sw_stage)
  static constexpr int NH = PL ? 2 : 1;                // MFMA K-chunks per step of 128 values
};
constexpr int kSxStageMax = SxShape<true>::Stage;

__shared__ __attribute__((aligned(16))) uint8_t sx_stage0[kSxStageMax];
__shared__ __attribute__((aligned(16))) uint8_t sx_stage1[kSxStageMax];
__shared__ __attribute__((aligned(16))) uint8_t sx_stage2[kSxStageMax];

template <int S>
__device__ __forceinline__ uint8_t* sx_stage() {
  return S == 0 ? sx_stage0 : (S == 1 ? sx_stage1 : sx_stage2);
}
// Weight scales have stages of their own: objects separate from the token
// stages let the compiler see that a weight-scale read of one stage does not
// depend on the direct-to-LDS loads in flight into the others (with the scales
// inside the token stages it waited for every load in flight before the first
// scale read of each step).
__shared__ __attribute__((aligned(16))) uint8_t sw_stage0[SxShape<true>::WSStage];
__shared__ __attribute__((aligned(16))) uint8_t sw_stage1[SxShape<true>::WSStage];
__shared__ __attribute__((aligned(16))) uint8_t sw_stage2[SxShape<true>::WSStage];
template <int S>
__device__ __forceinline__ uint8_t* sw_stage() {
  return S == 0 ? sw_stage0 : (S == 1 ? sw_stage1 : sw_stage2);
}

// Token stage: 16-byte chunk c of row r sits at slot sx_swz(r, c) of the row
// (an involution in c).  The operand read takes chunk c of 16 consecutive rows
// at once; both maps put those 16 rows on 16 distinct 16-byte slots of each
// 256-byte bank sweep (MXFP8 rows are 128 bytes: two rows per sweep).
template <bool PL>
__device__ __forceinline__ int sx_swz(int r, int c) {
  return PL ? (c ^ (r & 15)) : (c ^ ((r >> 1) & 7));
}

__device__ __forceinline__ f32x4 mfma_fp4w_fp8t(i32x8 w, i32x8 t, f32x4 acc, int wsc, int tsc) {
  // A = FP4 weights (format 4), B = FP8 E4M3 tokens (format 0); scale bytes in bits 0-7
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(w, t, acc, 4, 0, 0, wsc, 0, tsc);
}

// E8M0 byte of an NVFP4 weight block that is an exact MXFP4 transcode: a
// power-of-two E4M3 scale (both 16-halves equal) times the matrix's
// power-of-two global.  2^-127 (E8M0 byte 0) is a float subnormal whose
// exponent field is 0, as is a zero scale (an all-zero block).
__device__ __forceinline__ int nv_pow2_e8m0(uint32_t byte, float gmul) {
  return (int)((__float_as_uint(e4m3_to_f32(byte) * gmul) >> 23) & 0xFFu);
}

// One K step (128 values) from an LDS stage: 4 weight groups x RB token groups
// of 16 x 16, NH MFMA K-chunks each (RB: the 16-row token groups that hold
// rows of the tile; the rest are padding, with no LDS reads and no MFMAs).
// hook(s), s < 4 NH, issues loads between the MFMAs, spread evenly.
// The token operand of the next (chunk, token group) is read while the
// current one's MFMAs run (two register sets), so the LDS latency overlaps
// the matrix core.  Each token row's swizzle depends only on its row within
// the 16-row group (sx_swz), so a lane's reads for all groups share one base
// and differ by constant offsets.
template <int NMAT, bool PL, bool W_NV, int RB, typename Hook>
__device__ __forceinline__ void sx_compute(const uint8_t* st, const uint8_t* sws, f32x4 (&acc)[4][4], int wn, int li, int lg,
                                           const u32x4* wreg, const float* gmul, Hook&& hook) {
  using SH = SxShape<PL>;
  constexpr int NI = RB * SH::NH;                           // (chunk h, token group t < RB) in order
  constexpr int NS = 4 * SH::NH;                            // hook slots, spread over the NI groups
  const uint8_t* sa = st + li * SH::ARow;                   // this lane's row of token group 0
  const uint8_t* sts = st + SH::AStage + li * 4 + lg;       // its token scale byte of group 0, chunk 0
  uint32_t aoff[SH::NH][2];
#pragma unroll
  for (int h = 0; h < SH::NH; ++h)
#pragma unroll
    for (int u = 0; u < 2; ++u) aoff[h][u] = 16u * (uint32_t)sx_swz<PL>(li, (PL ? 8 * h : 0) + lg + 4 * u);
  i32x8 tb[2];
  int tsc[2];
  auto read_t = [&](int i) {
    const int h = i / RB, t = i % RB;
    const u32x4 b0 = *(const u32x4*)(sa + t * 16 * SH::ARow + aoff[h][0]);
    const u32x4 b1 = *(const u32x4*)(sa + t * 16 * SH::ARow + aoff[h][1]);
    tb[i & 1] = __builtin_bit_cast(i32x8, __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7));
    tsc[i & 1] = sts[(PL ? h * 256 : 0) + t * 64];
  };
  int wsc[4];
  i32x8 wop[4];
  read_t(0);
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int h = i / RB, t = i % RB;
    if (t == 0) {
      const int blk = PL ? 2 * h + (lg >> 1) : lg;          // weight 32-block of this lane's K block
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int n = pf_lrow<NMAT, SH::BN>(wn, g) + li;    // block-local weight row
        if (W_NV) wsc[g] = nv_pow2_e8m0(sws[n * 8 + 2 * blk], gmul[NMAT == 2 ? (g >> 1) : 0]);
        else wsc[g] = sws[n * 4 + blk];
        const u32x4 w = wreg[g];
        // MXFP8: the lane's 32 codes; planes: its 16-block's 16 codes, twice
        const u32x4 wv = PL ? (h == 0 ? u32x4{w[0], w[1], w[0], w[1]} : u32x4{w[2], w[3], w[2], w[3]}) : w;
        // the FP4 operand occupies the low 4 dwords; the instruction does not read the others
        wop[g] = __builtin_bit_cast(i32x8, __builtin_shufflevector(wv, wv, 0, 1, 2, 3, -1, -1, -1, -1));
      }
    }
    if (i + 1 < NI) {
      read_t(i + 1);
      // keep the next group's reads above this group's MFMAs
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int s = i * NS / NI; s < (i + 1) * NS / NI; ++s) hook(s);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int g = 0; g < 4; ++g) acc[g][t] = mfma_fp4w_fp8t(wop[g], tb[i & 1], acc[g][t], wsc[g], tsc[i & 1]);
  }
}

// MXFP8 and NVFP4-plane outputs of the epilogue: the lane holds D[weight row
// 4 lg + i of group gp][token li of group t]; output columns are weight rows.
// The stored value is first rounded to bf16 (the intermediate the method
// stores), then quantised.
template <int NMAT>
__device__ __forceinline__ void sx_epilogue(const GemmArgs& p, const PfTile& T, const f32x4 (&acc)[4][4], int wn,
                                            int li, int lg) {
  const int N = p.N;
  constexpr int NG = NMAT == 2 ? 2 : 4;                    // 16-column groups per wave
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int mrow = t * 16 + li;
    const bool ok = mrow < T.mrows;
    const int64_t ro = T.rbase + mrow;
    float r[NG][4];
#pragma unroll
    for (int gp = 0; gp < NG; ++gp) {
      float v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float g = acc[gp][t][i];
        v[i] = NMAT == 2 ? silu_f(g) * acc[gp + 2][t][i] : g;
      }
      const uint32_t b01 = cvt_bf16x2(v[0], v[1]), b23 = cvt_bf16x2(v[2], v[3]);
      const int col = T.nbase + (NMAT == 2 ? wn * 32 : wn * 64) + gp * 16 + 4 * lg;
      if (p.out_bf16 && ok) *(u32x2*)(p.out_bf16 + ro * N + col) = u32x2{b01, b23};
      r[gp][0] = bf16_lo(b01);
      r[gp][1] = bf16_hi(b01);
      r[gp][2] = bf16_lo(b23);
      r[gp][3] = bf16_hi(b23);
    }
    if (!p.out_codes) continue;
    if (p.out_format == MOE_OUT_MXFP8) {
#pragma unroll
      for (int pb = 0; pb < NG / 2; ++pb) {                // 32-column blocks: groups 2 pb, 2 pb + 1
        float amax = 0.0f;
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
          for (int i = 0; i < 4; ++i) amax = fmaxf(amax, fabsf(r[2 * pb + q][i]));
        amax = fmaxf(amax, __shfl_xor(amax, 16, kWave));
        amax = fmaxf(amax, __shfl_xor(amax, 32, kWave));
        const int e = mxfp8_scale_exp(amax);
        const float inv = exp2_int(-e);
        const int col0 = T.nbase + (NMAT == 2 ? wn * 32 : wn * 64 + pb * 32);
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          uint32_t wd = 0;
#pragma unroll
          for (int i = 0; i < 4; ++i) wd |= e4m3_code_signed(r[2 * pb + q][i] * inv) << (8 * i);
          if (ok) *(uint32_t*)(p.out_codes + ro * N + col0 + q * 16 + 4 * lg) = wd;
        }
        if (ok && lg == 0) p.out_scales[ro * (N / 32) + col0 / 32] = (uint8_t)(e + 127);
      }
    } else if (p.out_format == MOE_OUT_NVFP4_PLANES) {
#pragma unroll
      for (int gp = 0; gp < NG; ++gp) {
        uint32_t sb;
        const uint32_t bits = quant4_lanes(r[gp], p.out_inv_g, sb);
        uint32_t hi, lo;
        nvfp4_planes4(bits, sb, hi, lo);
        const int col16 = T.nbase + (NMAT == 2 ? wn * 32 : wn * 64) + gp * 16;     // first column of the 16-block
        if (ok) {
          uint8_t* dst = p.out_codes + ro * (2 * (int64_t)N) + 2 * col16;
          *(uint32_t*)(dst + 4 * lg) = hi;
          *(uint32_t*)(dst + 16 + 4 * lg) = lo;
          if (lg == 0) p.out_scales[ro * (N / 16) + col16 / 16] = (uint8_t)nvfp4_plane_scale(sb, p.out_g_log2);
        }
      }
    }
  }
}

template <int NMAT, bool PL, bool TL, bool W_NV>
__global__ __launch_bounds__(kPfThreads) void gemm_scaled_kernel(GemmArgs p) {
  using SH = SxShape<PL>;
  using WL = WeightLane<TL, W_NV>;
  static_assert(3 * (kSxStageMax + SH::WSStage) + (kPfMaxE + 1) * 4 + kPfThreads / kWave * 4 <= 160 * 1024, "LDS");
  __shared__ int s_pref[kPfMaxE + 1];
  __shared__ int s_wc[kPfThreads / kWave];
  // loads per wave and step: token codes (1 KB each), weight codes into
  // registers (MXFP8: one 16-byte piece per 16-row group; planes: two 8-byte
  // pieces, one per 16-block the lane's K blocks need), weight scales (256 B
  // each: 64 MX rows or 32 NV rows), token scales (256 B: every wave issues
  // one; waves past the needed count repeat a load, writing the same bytes)
  constexpr int kA = SH::AStage / 1024 / 8;
  constexpr int kW = PL ? 8 : 4;
  constexpr int kSRows = W_NV ? 32 : 64;
  constexpr int kSLoads = SH::BN / kSRows;
  constexpr int kS = kSLoads / 8;
  constexpr int kT = 1;
  constexpr int kDma = kA + kW + kS + kT;
  constexpr int kSlots = 4 * SH::NH;
  static_assert(kDma <= 2 * kSlots && kDma < 16, "two loads per compute slot; vmcnt in 4 bits");

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn = wv;                                              // one wave along tokens, eight along weight rows
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
  const int a_row = PL ? 2 * K : K;                               // token operand bytes per row
  const int ts_row = PL ? K / 16 : K / 32;                        // token scale bytes per row
  // every direct-to-LDS load is a buffer load: 32-bit lane offsets, the step's
  // part uniform (64-bit global addresses cost two registers per load).  The
  // token scales are a_bytes / 32 bytes in both modes (K/16 per 2K-byte plane
  // row, K/32 per K-byte MXFP8 row).
  const rsrc_t a_rsrc = make_rsrc(p.a_data, (uint32_t)min(p.a_bytes, (int64_t)0xffffffff));
  const rsrc_t ts_rsrc = make_rsrc(p.a_scales, (uint32_t)min(p.a_bytes / 32, (int64_t)0xffffffff));

  for (int tile = t_begin; tile < t_end; tile += t_stride) {
    const PfTile T = locate_tile<NMAT, SH>(p, s_pref, tile);
    float gmul[NMAT];
#pragma unroll
    for (int m = 0; m < NMAT; ++m) gmul[m] = W_NV ? p.w_global[m][T.e] : 1.0f;

    // token codes: load i fills LDS bytes [(kA wv + i) KB, +1 KB) = 1024 / ARow
    // rows, lane -> (row, slot); the chunk that belongs at that slot
    uint32_t a_off[kA];
#pragma unroll
    for (int i = 0; i < kA; ++i) {
      constexpr int CPR = SH::ARow / 16;
      const int row = (wv * kA + i) * (1024 / SH::ARow) + lane / CPR;
      const int chunk = sx_swz<PL>(row, lane % CPR);
      const int64_t r = T.rbase + min(row, T.mrows - 1);          // rows past the tile's end reread a valid row
      const int64_t src = p.gather ? (int64_t)(p.gather[r] / p.gather_div) : r;
      a_off[i] = (uint32_t)(src * (int64_t)a_row) + (uint32_t)chunk * 16u;   // < 2 GiB (checked on the host)
    }
    // token scales: lane -> row; planes: waves of odd index load the second 4 bytes
    const int ts_half = PL ? (wv & 1) : 0;
    uint32_t ts_off;
    {
      const int64_t r = T.rbase + min(lane, T.mrows - 1);
      const int64_t src = p.gather ? (int64_t)(p.gather[r] / p.gather_div) : r;
      ts_off = (uint32_t)(src * (int64_t)ts_row) + (uint32_t)ts_half * 4u;
    }
    // weight codes into registers: group j = rows pf_lrow(wn, j) .. +15 (matrix j / 2 for SwiGLU)
    rsrc_t wrs[NMAT];
#pragma unroll
    for (int m = 0; m < NMAT; ++m) wrs[m] = make_rsrc(p.w_packed[m] + T.e * mat_codes, (uint32_t)mat_codes);
    uint32_t w_off[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int R = T.nbase + pf_wrow<NMAT, SH::BN>(pf_lrow<NMAT, SH::BN>(wn, j));   // first row of the group
      w_off[j] = (uint32_t)R * (uint32_t)(K / 2);                 // the group's tile block in either layout
      w_off[j] += PL ? (TL ? (uint32_t)(16 * li) : (uint32_t)li * (uint32_t)(K / 2)) : WL::code(li, lg, K);
    }
    // planes: 8-byte piece of 16-block q (q = lg, then 4 + lg) of the lane's row, within a step
    auto plane_piece = [&](int q) -> uint32_t {
      return TL ? (uint32_t)(256 * (q >> 1) + 8 * (q & 1)) : (uint32_t)(8 * q);
    };
    // weight scales, as the bf16-token kernel: load h covers rows kSRows * (kS wv + h) ..
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

    u32x4 wring[3][4];                                           // weight codes of steps k .. k + 2
    // load q of step kb into stage S: kW register loads first, then kA token,
    // kS weight-scale and kT token-scale loads straight into LDS
    auto issue_one = [&](auto S_tag, int kb, int q) {
      constexpr int S = decltype(S_tag)::value;
      uint8_t* st = sx_stage<S>();
      if (q < kW) {
        if (PL) {
          const int j = q >> 1, half = q & 1;
          const uint32_t step = (uint32_t)kb * WL::kStep + plane_piece(half * 4 + lg);
          const u32x2 d = __builtin_bit_cast(
              u32x2, __builtin_amdgcn_raw_buffer_load_b64(wrs[NMAT == 2 ? (j >> 1) : 0], (int)(w_off[j] + step), 0, 0));
          wring[S][j][2 * half] = d[0];
          wring[S][j][2 * half + 1] = d[1];
        } else {
          wring[S][q] = bload128(wrs[NMAT == 2 ? (q >> 1) : 0], w_off[q] + (uint32_t)kb * WL::kStep, 0);
        }
      } else if (q < kW + kA) {
        const int i = q - kW;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(a_rsrc, (lds_void_t*)(st + (wv * kA + i) * 1024), 16, (int)a_off[i],
                                                 (int)(kb * SH::ARow), 0, 0);
      } else if (q < kW + kA + kS) {
        const int h = q - kW - kA;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(make_rsrc(s_base[h], (uint32_t)mat_scales),
                                                 (lds_void_t*)(sw_stage<S>() + (wv * kS + h) * 256), 4, (int)s_off[h],
                                                 (int)pf_scale_step<TL, W_NV>(kb), 0, 0);
      } else {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ts_rsrc, (lds_void_t*)(st + SH::AStage + ts_half * 256), 4, (int)ts_off,
                                                 (int)(kb * SH::TSRow), 0, 0);
      }
    };
    auto issue = [&](auto S_tag, int kb) {
#pragma unroll
      for (int q = 0; q < kDma; ++q) issue_one(S_tag, kb, q);
    };

    // the tile's K loop and epilogue for RB token groups of 16 rows that hold
    // rows of the tile (an expert's last tile often holds fewer than 64)
    auto run = [&](auto RB_tag) {
      constexpr int RB = decltype(RB_tag)::value;
      f32x4 acc[4][4];
  #pragma unroll
      for (int g = 0; g < 4; ++g)
  #pragma unroll
        for (int t = 0; t < 4; ++t) acc[g][t] = f32x4{0.f, 0.f, 0.f, 0.f};

      // step k from stage S: this wave's loads of step k done (step k + 1's may
      // be in flight), barrier (every wave's landed; every wave done with step
      // k - 1), refill the stage of step k - 1 with step k + 2 between the MFMA
      // slots (past the end: step nk - 1 again, unread), compute
      auto step = [&](auto S_tag, int k) {
        constexpr int S = decltype(S_tag)::value;
        __builtin_amdgcn_s_waitcnt((kDma & 15) | (7 << 4) | (15 << 8));      // vmcnt(kDma)
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        const int kn = min(k + 2, nk - 1);
        constexpr auto SN = std::integral_constant<int, (S + 2) % 3>();
        auto hook = [&](int s) {
          if (2 * s < kDma) issue_one(SN, kn, 2 * s);
          if (2 * s + 1 < kDma) issue_one(SN, kn, 2 * s + 1);
        };
        sx_compute<NMAT, PL, W_NV, RB>(sx_stage<S>(), sw_stage<S>(), acc, wn, li, lg, wring[S], gmul, hook);
      };

      __syncthreads();                                             // previous tile done with the stages
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

      if (p.out_format == MOE_OUT_NVFP4) {
        // bf16 (and NVFP4) outputs: the shared epilogues; the global scales are
        // already inside the E8M0 scales
        float wglob[NMAT];
  #pragma unroll
        for (int m = 0; m < NMAT; ++m) wglob[m] = 1.0f;
        if (NMAT == 1 && !PL && p.out_bf16 && !p.out_codes && !p.out_dq) {
          // the down projection's bf16 out through LDS (pf_epilogue_staged), staged in the last
          // step's token stage: the loads in flight (its repeats) fill the other two.  (Not in the
          // planes kernel: there the staging code pushed the registers into spills, measured 2.5%
          // slower.)
          static_assert(kPfThreads / kWave * 2048 <= kSxStageMax, "epilogue staging: 2 KB per wave");
          __builtin_amdgcn_s_barrier();
          uint8_t* ob = ((nk - 1) % 3 == 0 ? sx_stage<0>() : ((nk - 1) % 3 == 1 ? sx_stage<1>() : sx_stage<2>())) + wv * 2048;
          pf_epilogue_staged<NMAT>(p, T, acc, wglob, wn, li, lg, ob);
        } else {
          pf_epilogue<NMAT>(p, T, acc, wglob, 0, wn, li, lg);
        }
      } else {
        sx_epilogue<NMAT>(p, T, acc, wn, li, lg);
      }
    };
    const int rb = (T.mrows + 15) >> 4;                              // workgroup-uniform
    if (rb >= 4) run(std::integral_constant<int, 4>());
    else if (rb == 3) run(std::integral_constant<int, 3>());
    else if (rb == 2) run(std::integral_constant<int, 2>());
    else run(std::integral_constant<int, 1>());
  }
  // the last tile leaves its unread repeat loads in flight: let them land
  // before the workgroup's LDS is released
  __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8));          // vmcnt(0)
}

template <int NMAT, bool PL, bool TL, bool W_NV>
static void launch_scaled_one(const GemmArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL((gemm_scaled_kernel<NMAT, PL, TL, W_NV>), dim3(device_cus()), dim3(kPfThreads), 0, stream, a);
}

// the kernels of one weight layout (TL: tiled), instantiated in their own
// translation unit so they compile in parallel
template <bool TL>
void scaled_run(const GemmArgs& a, bool swiglu, bool planes, bool w_nv, hipStream_t stream) {
  if (swiglu) {
    if (planes) w_nv ? launch_scaled_one<2, true, TL, true>(a, stream) : launch_scaled_one<2, true, TL, false>(a, stream);
    else w_nv ? launch_scaled_one<2, false, TL, true>(a, stream) : launch_scaled_one<2, false, TL, false>(a, stream);
  } else {
    if (planes) w_nv ? launch_scaled_one<1, true, TL, true>(a, stream) : launch_scaled_one<1, true, TL, false>(a, stream);
    else w_nv ? launch_scaled_one<1, false, TL, true>(a, stream) : launch_scaled_one<1, false, TL, false>(a, stream);
  }
}

extern template void scaled_run<false>(const GemmArgs&, bool, bool, bool, hipStream_t);
extern template void scaled_run<true>(const GemmArgs&, bool, bool, bool, hipStream_t);

}  // namespace moe
