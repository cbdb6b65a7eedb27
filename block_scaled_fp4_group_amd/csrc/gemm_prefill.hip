// Grouped FP4 expert GEMM, MFMA-bound ("prefill") form: many token rows per
// expert, so the kernel is bound by bf16 MFMA throughput.
//
// Same contraction as the weight-streaming kernel (the SwiGLU expert FFN of
// "MiMo-V2.6-Flash -- REAP-50", "Pruning Method"; MXFP4 / NVFP4 weights with
// FP32 accumulation, "AxionML / MiMo-V2.6-Flash-MOPD-NVFP4", "About NVFP4
// quantization"), tiled for reuse:
//   * a workgroup of 8 waves owns a tile of BM = 128 token rows x BN = 256
//     weight rows (SwiGLU: 128 gate + 128 up rows of the same outputs) and
//     walks K in steps of BK = 128;
//   * the token tile is gathered from HBM/L2 into registers one step ahead and
//     written to a double-buffered LDS stage with an XOR swizzle (16-byte
//     chunk c of row r sits at c ^ (r % 16)), so the 16 rows of one MFMA
//     operand read hit 16 distinct bank groups; NVFP4 token rows are
//     dequantised to bf16 on the way in;
//   * each wave keeps its 64 weight rows' FP4 codes in registers (one step
//     ahead), dequantises them with the gfx950 convert instruction and runs
//     4 x 4 bf16 16x16x32 MFMA tiles (64 tokens x 64 weight rows);
//   * persistent workgroups walk the tiles expert by expert, the m-tiles of one
//     (expert, n-tile) back to back so their weights are shared in cache.
#include <algorithm>

#include "gemm_common.h"

namespace moe {

constexpr int kPfBM = 128, kPfBN = 256, kPfBK = 128;
constexpr int kPfThreads = 512;                    // 8 waves: 2 along tokens x 4 along weight rows
constexpr int kPfStage = kPfBM * kPfBK * 2;        // 32 KB of bf16 per LDS stage
constexpr int kPfMaxE = 1024;

__device__ __forceinline__ uint32_t swz(int row, int chunk) { return (uint32_t)(row * 256 + ((chunk ^ (row & 15)) << 4)); }

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

template <int NMAT, bool W_NV, bool A_NV>
__global__ __launch_bounds__(kPfThreads) void gemm_prefill_kernel(GemmArgs p) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];      // 2 stages
  __shared__ int s_pref[kPfMaxE + 1];                                // tiles before expert e
  __shared__ int s_wc[kPfThreads / kWave];

  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int wm = wv & 1, wn = wv >> 1;                               // 2 x 4 waves
  const int li = lane & 15, lg = lane >> 4;
  const int E = p.E, K = p.K, N = p.N;
  const int ntn = N / (kPfBN / NMAT);                                // n-tiles per expert
  const int nk = K / kPfBK;

  // ---- tile table: expert e owns ceil(rows_e / BM) * ntn tiles
  {
    int running = 0;
    for (int e0 = 0; e0 < E; e0 += kPfThreads) {
      const int e = e0 + threadIdx.x;
      int cnt = 0;
      if (e < E) {
        int r0 = (int)max((int64_t)0, min((int64_t)p.offsets[e], p.rows));
        int r1 = (int)max((int64_t)r0, min((int64_t)p.offsets[e + 1], p.rows));
        cnt = ((r1 - r0 + kPfBM - 1) / kPfBM) * ntn;
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
      if (e < E) s_pref[e] = before + x - cnt;
      int tot = 0;
      for (int i = 0; i < kPfThreads / kWave; ++i) tot += s_wc[i];
      running += tot;
      __syncthreads();
    }
    if (threadIdx.x == 0) s_pref[E] = running;
    __syncthreads();
  }
  const int total = s_pref[E];

  const uint32_t sc_row = (uint32_t)(W_NV ? K / 16 : K / 32);
  const uint32_t mat_codes = (uint32_t)N * (uint32_t)(K / 2);
  const uint32_t mat_scales = (uint32_t)N * sc_row;

  for (int tile = blockIdx.x; tile < total; tile += gridDim.x) {
    // ---- locate (expert, n-tile, m-tile); m-tiles of one n-tile are consecutive
    int lo = 0, hi = E - 1;
    while (lo < hi) {
      int mid = (lo + hi + 1) >> 1;
      if (s_pref[mid] <= tile) lo = mid;
      else hi = mid - 1;
    }
    const int e = lo;
    const int r0 = (int)max((int64_t)0, min((int64_t)p.offsets[e], p.rows));
    const int r1 = (int)max((int64_t)r0, min((int64_t)p.offsets[e + 1], p.rows));
    const int mt_cnt = (r1 - r0 + kPfBM - 1) / kPfBM;
    const int local = tile - s_pref[e];
    const int nt = local / mt_cnt, mt = local % mt_cnt;
    const int rbase = r0 + mt * kPfBM;
    const int mrows = min(kPfBM, r1 - rbase);

    // ---- weight rows of this wave (4 groups of 16)
    rsrc_t wr[NMAT], sr[NMAT];
#pragma unroll
    for (int m = 0; m < NMAT; ++m) {
      wr[m] = make_rsrc(p.w_packed[m] + (int64_t)e * mat_codes, mat_codes);
      sr[m] = make_rsrc(p.w_scale[m] + (int64_t)e * mat_scales, mat_scales);
    }
    // row group g: matrix mat(g), row wrow(g) + li
    auto gmat = [&](int g) { return NMAT == 2 ? (g >> 1) : 0; };
    auto grow = [&](int g) {
      return NMAT == 2 ? nt * 128 + wn * 32 + (g & 1) * 16 : nt * 256 + wn * 64 + g * 16;
    };
    uint32_t wo[4], so[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      wo[g] = (uint32_t)(grow(g) + li) * (uint32_t)(K / 2) + (uint32_t)lg * 16u;
      so[g] = (uint32_t)(grow(g) + li) * sc_row + (uint32_t)(W_NV ? lg * 2 : lg);
    }
    float wglob[NMAT];
#pragma unroll
    for (int m = 0; m < NMAT; ++m) wglob[m] = W_NV ? p.w_global[m][e] : 1.0f;

    // ---- token tile loader: thread -> (row, 16-byte chunk) slots
    // bf16: 4 chunks per thread; NVFP4: one 32-value block per thread
    int64_t tsrc[4];
    int trow[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int q = A_NV ? (int)threadIdx.x : (int)threadIdx.x + kPfThreads * j;
      const int row = A_NV ? q / 4 : q / 16;
      trow[j] = row;
      tsrc[j] = -1;
      if (row < mrows && (!A_NV || j == 0)) {
        const int64_t r = rbase + row;
        tsrc[j] = p.gather ? (int64_t)(p.gather[r] / p.gather_div) : r;
      }
    }
    u32x4 treg[4];
    uint32_t tsc = 0;
    auto tload = [&](int kb) {
      if (A_NV) {
        const int b = threadIdx.x & 3;                               // block within BK
        if (tsrc[0] >= 0) {
          treg[0] = *(const u32x4*)(p.a_data + tsrc[0] * (K / 2) + (int64_t)(kb * 4 + b) * 16);
          tsc = *(const uint16_t*)(p.a_scales + tsrc[0] * (K / 16) + (int64_t)(kb * 4 + b) * 2);
        }
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int c = (threadIdx.x + kPfThreads * j) & 15;
          if (tsrc[j] >= 0) treg[j] = *(const u32x4*)(p.a_data + tsrc[j] * (int64_t)K * 2 + (int64_t)kb * 256 + c * 16);
        }
      }
    };
    auto tstore = [&](uint8_t* stage) {
      if (A_NV) {
        if (tsrc[0] >= 0) {
          const int b = threadIdx.x & 3;
          const float s_lo = e4m3_to_f32(tsc & 0xFF) * p.a_gscale, s_hi = e4m3_to_f32(tsc >> 8) * p.a_gscale;
#pragma unroll
          for (int s = 0; s < 4; ++s)
            *(u32x4*)(stage + swz(trow[0], b * 4 + s)) =
                __builtin_bit_cast(u32x4, fp4x8_to_bf16(treg[0][s], s < 2 ? s_lo : s_hi));
        }
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int c = (threadIdx.x + kPfThreads * j) & 15;
          if (tsrc[j] >= 0) *(u32x4*)(stage + swz(trow[j], c)) = treg[j];
        }
      }
    };
    // ---- weights one step ahead
    u32x4 wreg[2][4];
    uint32_t sreg[2][4];
    auto wload = [&](int buf, int kb) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        wreg[buf][g] = bload128(wr[gmat(g)], wo[g] + kb * 64, 0);
        sreg[buf][g] = W_NV ? bload16(sr[gmat(g)], so[g] + kb * 8, 0) : bload8(sr[gmat(g)], so[g] + kb * 4, 0);
      }
    };

    f32x4 acc[4][4];                                                 // [weight group][token group]
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int t = 0; t < 4; ++t) acc[g][t] = f32x4{0.f, 0.f, 0.f, 0.f};

    __syncthreads();                                                 // previous tile done with LDS
    tload(0);
    wload(0, 0);
    tstore(lds);
    __syncthreads();

    for (int kb = 0; kb < nk; ++kb) {
      const int cur = kb & 1;
      uint8_t* stage = lds + cur * kPfStage;
      if (kb + 1 < nk) {
        tload(kb + 1);
        wload(cur ^ 1, kb + 1);
      }
      // ---- 4 k-slots of 8 values inside this lane group's block
      float s_lo[4], s_hi[4];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        if (W_NV) {
          s_lo[g] = e4m3_to_f32(sreg[cur][g] & 0xFF);
          s_hi[g] = e4m3_to_f32((sreg[cur][g] >> 8) & 0xFF);
        } else {
          s_lo[g] = s_hi[g] = e8m0_to_f32(sreg[cur][g]);
        }
      }
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        bf16x8 bt[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int row = wm * 64 + t * 16 + li;
          bt[t] = __builtin_bit_cast(bf16x8, *(const u32x4*)(stage + swz(row, lg * 4 + s)));
        }
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const bf16x8 af = W_NV ? fp4x8_to_bf16(wreg[cur][g][s], s < 2 ? s_lo[g] : s_hi[g])
                                 : fp4x8_to_bf16_pow2(wreg[cur][g][s], s_lo[g]);
#pragma unroll
          for (int t = 0; t < 4; ++t) acc[g][t] = mfma16(af, bt[t], acc[g][t]);
        }
      }
      if (kb + 1 < nk) tstore(lds + (cur ^ 1) * kPfStage);
      __syncthreads();
    }

    // ---- epilogue: lane holds D[weight row 4*lg + i of group g][token row li of group t]
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int mrow = wm * 64 + t * 16 + li;
      const bool ok = mrow < mrows;
      const int64_t ro = rbase + mrow;
#pragma unroll
      for (int gp = 0; gp < (NMAT == 2 ? 2 : 4); ++gp) {
        float v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float g = acc[gp][t][i] * wglob[0];
          v[i] = NMAT == 2 ? silu_f(g) * (acc[gp + 2][t][i] * wglob[NMAT - 1]) : g;
        }
        const int col = (NMAT == 2 ? nt * 128 + wn * 32 + gp * 16 : nt * 256 + wn * 64 + gp * 16) + 4 * lg;
        const uint32_t b01 = pack_bf16x2(v[0], v[1]), b23 = pack_bf16x2(v[2], v[3]);
        if (p.out_bf16 && ok) *(u32x2*)(p.out_bf16 + ro * N + col) = u32x2{b01, b23};
        if (p.out_codes) {
          float q[4] = {bf16_lo(b01), bf16_hi(b01), bf16_lo(b23), bf16_hi(b23)};
          uint32_t sb;
          const uint32_t bits = quant4_lanes(q, p.out_inv_g, sb);
          if (ok) {
            *(uint16_t*)(p.out_codes + ro * (N / 2) + col / 2) = (uint16_t)bits;
            if (lg == 0) p.out_scales[ro * (N / 16) + (col - 4 * lg) / 16] = (uint8_t)sb;
          }
        }
      }
    }
  }
}

static int device_cus() {
  static int cus = 0;
  if (!cus) {
    int dev = 0;
    hipGetDevice(&dev);
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
  }
  return cus;
}

template <int NMAT, bool W_NV, bool A_NV>
static void launch_prefill_one(const GemmArgs& a, hipStream_t stream) {
  auto kern = gemm_prefill_kernel<NMAT, W_NV, A_NV>;
  static bool attr_set = false;
  if (!attr_set) {
    hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, 2 * kPfStage);
    attr_set = true;
  }
  // persistent: one workgroup per CU (8 waves); tiles are distributed on the device
  hipLaunchKernelGGL(kern, dim3(device_cus()), dim3(kPfThreads), 2 * kPfStage, stream, a);
}

moe_status launch_gemm_decode(const GemmArgs&, bool swiglu, bool w_nv, bool a_nv, int64_t rows, hipStream_t);

moe_status launch_gemm_prefill(const GemmArgs& a, bool swiglu, bool w_nv, bool a_nv, int64_t rows, hipStream_t stream) {
  const int bn = swiglu ? kPfBN / 2 : kPfBN;
  if (a.N % bn != 0 || a.K % kPfBK != 0 || a.E > kPfMaxE) {
    // shapes the tiled kernel does not cover run on the weight-streaming kernel
    return launch_gemm_decode(a, swiglu, w_nv, a_nv, rows, stream);
  }
  if (swiglu) {
    if (w_nv) a_nv ? launch_prefill_one<2, true, true>(a, stream) : launch_prefill_one<2, true, false>(a, stream);
    else a_nv ? launch_prefill_one<2, false, true>(a, stream) : launch_prefill_one<2, false, false>(a, stream);
  } else {
    if (w_nv) a_nv ? launch_prefill_one<1, true, true>(a, stream) : launch_prefill_one<1, true, false>(a, stream);
    else a_nv ? launch_prefill_one<1, false, true>(a, stream) : launch_prefill_one<1, false, false>(a, stream);
  }
  return launch_status("moe_fp4_grouped_gemm(prefill)");
}

}  // namespace moe
