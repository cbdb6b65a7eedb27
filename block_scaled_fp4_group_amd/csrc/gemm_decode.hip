// Grouped FP4 expert GEMM, weight-streaming ("decode") form: few rows per
// expert, so the kernel is bound by reading the FP4 weights from HBM once.
//
// The expert FFN is W_down(SiLU(W_gate h) * (W_up h)) ("MiMo-V2.6-Flash --
// REAP-50", "Pruning Method", saliency equation); weights are MXFP4 or their
// exact NVFP4 transcode; accumulation is FP32 ("AxionML / MiMo-V2.6-Flash-
// MOPD-NVFP4", "About NVFP4 quantization").
//
// Work split: blockIdx.y picks the j-th expert that has rows, blockIdx.x a tile
// of 16*NT output features.  The K dimension is cut into steps of 128: in one
// step, lane group g (lanes 16g..16g+15) of a wave reads one whole 32-value
// block (16 code bytes + its scale) for each of 16 weight rows, dequantises it
// in registers (E2M1 x power-of-two scale -> bf16 by the gfx950 convert
// instruction) and feeds four bf16 16x16x32 MFMAs whose other operand holds 16
// token rows.  Steps are dealt round-robin to the WAVES waves of the block;
// the per-wave partial sums meet in LDS in a fixed order (deterministic), and
// the epilogue applies SwiGLU / global scales and writes bf16 and/or NVFP4.
// Rows beyond 16*MC are handled by further passes over the same weights
// (served from L2).
#include <algorithm>

#include "gemm_common.h"

namespace moe {

template <int NMAT, int NT, int MC, int WAVES, int PF, bool W_NV, bool A_NV>
__global__ __launch_bounds__(WAVES * 64) void gemm_decode_kernel(GemmArgs p) {
  constexpr int BN = 16 * NT;            // output features per block
  constexpr int BM = 16 * MC;            // token rows per pass
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int li = lane & 15, lg = lane >> 4;

  int e, r0, r1;
  if (!find_active_expert(p.offsets, p.E, p.rows, blockIdx.y, e, r0, r1)) return;
  const int n0 = blockIdx.x * BN;
  const int K = p.K, N = p.N;
  const int nsteps = K / 128;
  const int64_t wrow_bytes = K / 2;
  const int sc_per_row = W_NV ? K / 16 : K / 32;

  extern __shared__ float red[];         // [WAVES][NMAT][BM][BN]

  float wglob[NMAT];
#pragma unroll
  for (int m = 0; m < NMAT; ++m) wglob[m] = W_NV ? p.w_global[m][e] : 1.0f;

  for (int rbase = r0; rbase < r1; rbase += BM) {
    const int mrows = min(BM, r1 - rbase);
    // activation source row of each of this lane's MC token rows
    const uint8_t* arow[MC];
    const uint8_t* asrow[MC];
#pragma unroll
    for (int c = 0; c < MC; ++c) {
      int m = c * 16 + li;
      arow[c] = nullptr;
      asrow[c] = nullptr;
      if (m < mrows) {
        int64_t r = rbase + m;
        int64_t src = p.gather ? (int64_t)(p.gather[r] / p.gather_div) : r;
        if (A_NV) {
          arow[c] = p.a_data + src * (K / 2);
          asrow[c] = p.a_scales + src * (K / 16);
        } else {
          arow[c] = p.a_data + src * (int64_t)K * 2;
        }
      }
    }

    f32x4 acc[NMAT][NT][MC];
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int c = 0; c < MC; ++c) acc[m][t][c] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int s0 = wv; s0 < nsteps; s0 += WAVES * PF) {
      // ---- issue the weight loads of up to PF steps
      u32x4 wc[PF][NMAT][NT];
      uint32_t wsc[PF][NMAT][NT];
#pragma unroll
      for (int q = 0; q < PF; ++q) {
        int st = s0 + q * WAVES;
        if (st < nsteps) {
          int blk = st * 4 + lg;
#pragma unroll
          for (int m = 0; m < NMAT; ++m)
#pragma unroll
            for (int t = 0; t < NT; ++t) {
              int64_t row = (int64_t)e * N + n0 + t * 16 + li;
              wc[q][m][t] = *(const u32x4*)(p.w_packed[m] + row * wrow_bytes + blk * 16);
              if (W_NV) wsc[q][m][t] = *(const uint16_t*)(p.w_scale[m] + row * sc_per_row + blk * 2);
              else wsc[q][m][t] = p.w_scale[m][row * sc_per_row + blk];
            }
        }
      }
      // ---- consume
#pragma unroll
      for (int q = 0; q < PF; ++q) {
        int st = s0 + q * WAVES;
        if (st < nsteps) {
          int blk = st * 4 + lg;
          // activation operands for the MC row chunks (4 k-slots of 8 values each)
          bf16x8 af[MC][4];
#pragma unroll
          for (int c = 0; c < MC; ++c) {
            if (arow[c]) {
              if (A_NV) {
                u32x4 cw = *(const u32x4*)(arow[c] + blk * 16);
                uint32_t sw = *(const uint16_t*)(asrow[c] + blk * 2);
                float s_lo = e4m3_to_f32(sw & 0xFF) * p.a_gscale;
                float s_hi = e4m3_to_f32(sw >> 8) * p.a_gscale;
#pragma unroll
                for (int s = 0; s < 4; ++s) af[c][s] = fp4x8_to_bf16(cw[s], s < 2 ? s_lo : s_hi);
              } else {
                const u32x4* src = (const u32x4*)(arow[c] + blk * 64);
#pragma unroll
                for (int s = 0; s < 4; ++s) af[c][s] = __builtin_bit_cast(bf16x8, src[s]);
              }
            } else {
#pragma unroll
              for (int s = 0; s < 4; ++s) af[c][s] = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
            }
          }
#pragma unroll
          for (int m = 0; m < NMAT; ++m)
#pragma unroll
            for (int t = 0; t < NT; ++t) {
              float s_lo, s_hi;
              if (W_NV) {
                s_lo = e4m3_to_f32(wsc[q][m][t] & 0xFF);
                s_hi = e4m3_to_f32(wsc[q][m][t] >> 8);
              } else {
                s_lo = s_hi = e8m0_to_f32(wsc[q][m][t]);
              }
#pragma unroll
              for (int s = 0; s < 4; ++s) {
                bf16x8 wf = W_NV ? fp4x8_to_bf16(wc[q][m][t][s], s < 2 ? s_lo : s_hi)
                                 : fp4x8_to_bf16_pow2(wc[q][m][t][s], s_lo);
#pragma unroll
                for (int c = 0; c < MC; ++c) acc[m][t][c] = mfma16(wf, af[c][s], acc[m][t][c]);
              }
            }
        }
      }
    }

    // ---- cross-wave reduction in LDS: D[n][m], lane holds n = 4*lg + i, m = li
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int c = 0; c < MC; ++c)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            int mm = c * 16 + li, nn = t * 16 + 4 * lg + i;
            red[((wv * NMAT + m) * BM + mm) * BN + nn] = acc[m][t][c][i];
          }
    __syncthreads();

    // ---- epilogue: one thread per (row, 16 features)
    for (int it = threadIdx.x; it < BM * (BN / 16); it += WAVES * 64) {
      int mm = it / (BN / 16), nb = it % (BN / 16);
      if (mm < mrows) {
        float v[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float g = 0.f, u = 0.f;
          for (int w = 0; w < WAVES; ++w) {
            g += red[((w * NMAT + 0) * BM + mm) * BN + nb * 16 + i];
            if (NMAT == 2) u += red[((w * NMAT + 1) * BM + mm) * BN + nb * 16 + i];
          }
          g *= wglob[0];
          if (NMAT == 2) {
            u *= wglob[NMAT - 1];
            v[i] = silu_f(g) * u;
          } else {
            v[i] = g;
          }
        }
        int64_t r = rbase + mm;
        int col = n0 + nb * 16;
        uint32_t bw[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) bw[i] = pack_bf16x2(v[2 * i], v[2 * i + 1]);
        if (p.out_bf16) {
          u32x4* o = (u32x4*)(p.out_bf16 + r * N + col);
          o[0] = u32x4{bw[0], bw[1], bw[2], bw[3]};
          o[1] = u32x4{bw[4], bw[5], bw[6], bw[7]};
        }
        if (p.out_codes) {
          float q[16];
#pragma unroll
          for (int i = 0; i < 8; ++i) { q[2 * i] = bf16_lo(bw[i]); q[2 * i + 1] = bf16_hi(bw[i]); }
          uint32_t lo, hi;
          uint32_t sb = quant16(q, p.out_inv_g, lo, hi);
          *(u32x2*)(p.out_codes + r * (N / 2) + col / 2) = u32x2{lo, hi};
          p.out_scales[r * (N / 16) + col / 16] = (uint8_t)sb;
        }
      }
    }
    __syncthreads();
  }
}

template <int NMAT, int NT, int MC, int WAVES, int PF>
static void launch_decode_t(const GemmArgs& a, bool w_nv, bool a_nv, int nact, hipStream_t stream) {
  dim3 grid(a.N / (16 * NT), nact);
  size_t lds = (size_t)WAVES * NMAT * (16 * MC) * (16 * NT) * sizeof(float);
  if (w_nv) {
    if (a_nv) hipLaunchKernelGGL((gemm_decode_kernel<NMAT, NT, MC, WAVES, PF, true, true>), grid, dim3(WAVES * 64), lds, stream, a);
    else hipLaunchKernelGGL((gemm_decode_kernel<NMAT, NT, MC, WAVES, PF, true, false>), grid, dim3(WAVES * 64), lds, stream, a);
  } else {
    if (a_nv) hipLaunchKernelGGL((gemm_decode_kernel<NMAT, NT, MC, WAVES, PF, false, true>), grid, dim3(WAVES * 64), lds, stream, a);
    else hipLaunchKernelGGL((gemm_decode_kernel<NMAT, NT, MC, WAVES, PF, false, false>), grid, dim3(WAVES * 64), lds, stream, a);
  }
}

moe_status launch_gemm_decode(const GemmArgs& a, bool swiglu, bool w_nv, bool a_nv, int64_t rows, hipStream_t stream) {
  int nact = (int)std::min<int64_t>(a.E, rows);
  if (nact <= 0) return MOE_OK;
  if (swiglu) {
    if (a.N % 16) return MOE_ERR_UNSUPPORTED;
    launch_decode_t<2, 1, 2, 8, 4>(a, w_nv, a_nv, nact, stream);
  } else {
    if (a.N % 32 == 0) launch_decode_t<1, 2, 2, 8, 4>(a, w_nv, a_nv, nact, stream);
    else launch_decode_t<1, 1, 2, 8, 4>(a, w_nv, a_nv, nact, stream);
  }
  return launch_status("moe_fp4_grouped_gemm(decode)");
}

}  // namespace moe
