// Tiled weight layout: a permutation of each expert matrix's FP4 codes and
// scales so that one wavefront load of the GEMM kernels (16 rows x 64 code
// bytes, or 16 rows x one 4-step scale window) is one contiguous block.  The
// layout itself is specified with moe_fp4_tile_weights in the C header; the
// values are the model's MXFP4 / NVFP4 (or compact MXFP4) weights unchanged.
#include "common.h"

namespace moe {

constexpr int kTileThreads = 256;

// one thread per 16-byte chunk of the tiled codes (writes coalesced)
__global__ __launch_bounds__(kTileThreads) void tile_codes_kernel(const uint8_t* __restrict__ in,
                                                                 uint8_t* __restrict__ out, int64_t chunks,
                                                                 int64_t per_mat, int row_bytes, int nsteps) {
  const int64_t q = (int64_t)blockIdx.x * kTileThreads + threadIdx.x;
  if (q >= chunks) return;
  const int64_t e = q / per_mat;
  const int64_t w = q - e * per_mat;                 // chunk within the matrix
  const int64_t blk = w >> 6;                        // 1 KB block = t * nsteps + s
  const int within = (int)(w & 63);                  // 16 * c + r
  const int64_t t = blk / nsteps;
  const int s = (int)(blk - t * nsteps);
  const int c = within >> 4, r = within & 15;
  const int64_t src = e * per_mat * 16 + (t * 16 + r) * row_bytes + s * 64 + c * 16;
  *(u32x4*)(out + q * 16) = *(const u32x4*)(in + src);
}

// one thread per P-byte piece of the tiled scales (P = 16, or 8 for the compact
// format's 8 bytes per row and window); G scale bytes per row and window
template <typename Piece>
__global__ __launch_bounds__(kTileThreads) void tile_scales_kernel(const uint8_t* __restrict__ in,
                                                                  uint8_t* __restrict__ out, int64_t pieces,
                                                                  int64_t per_mat, int row_bytes, int nwin, int G) {
  constexpr int P = (int)sizeof(Piece);
  const int64_t q = (int64_t)blockIdx.x * kTileThreads + threadIdx.x;
  if (q >= pieces) return;
  const int64_t e = q / per_mat;
  const int64_t w = q - e * per_mat;
  const int per_blk = 16 * G / P;                    // 16 rows x G bytes
  const int64_t blk = w / per_blk;                   // t * nwin + window
  const int within = (int)(w - blk * per_blk);
  const int64_t t = blk / nwin;
  const int win = (int)(blk - t * nwin);
  const int r = within / (G / P), h = within % (G / P);
  const int64_t src = e * per_mat * P + (t * 16 + r) * row_bytes + (int64_t)win * G + h * P;
  *(Piece*)(out + q * P) = *(const Piece*)(in + src);
}

// fmt: 0 MXFP4 (16 E8M0 bytes per row and window), 1 NVFP4 (32), 2 compact (8)
moe_status launch_tile(int fmt, int64_t E, int n, int k, const uint8_t* packed, const uint8_t* scale,
                       uint8_t* packed_t, uint8_t* scale_t, hipStream_t stream) {
  if (E == 0) return MOE_OK;
  const int64_t code_per_mat = (int64_t)n * (k / 2) / 16;
  const int64_t code_chunks = E * code_per_mat;
  hipLaunchKernelGGL(tile_codes_kernel, dim3((uint32_t)((code_chunks + kTileThreads - 1) / kTileThreads)),
                     dim3(kTileThreads), 0, stream, packed, packed_t, code_chunks, code_per_mat, k / 2, k / 128);
  const int G = fmt == 1 ? 32 : (fmt == 2 ? 8 : 16);
  const int srow = (k / 512) * G;
  if (G == 8) {
    const int64_t per_mat = (int64_t)n * srow / 8, pieces = E * per_mat;
    hipLaunchKernelGGL(tile_scales_kernel<u32x2>, dim3((uint32_t)((pieces + kTileThreads - 1) / kTileThreads)),
                       dim3(kTileThreads), 0, stream, scale, scale_t, pieces, per_mat, srow, k / 512, G);
  } else {
    const int64_t per_mat = (int64_t)n * srow / 16, pieces = E * per_mat;
    hipLaunchKernelGGL(tile_scales_kernel<u32x4>, dim3((uint32_t)((pieces + kTileThreads - 1) / kTileThreads)),
                       dim3(kTileThreads), 0, stream, scale, scale_t, pieces, per_mat, srow, k / 512, G);
  }
  return launch_status("moe_fp4_tile_weights");
}

}  // namespace moe
