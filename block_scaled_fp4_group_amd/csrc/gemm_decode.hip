// Grouped FP4 expert GEMM, weight-streaming ("decode") form: entry point, and
// the per-(expert, n-block) kernels on row-major weights.  The kernels are in
// gemm_decode.h; the tiled-layout variants are instantiated in
// gemm_decode_tiled.hip.
#include "gemm_decode.h"

namespace moe {

template void decode_wg<false>(const GemmArgs&, bool, int, bool, int, hipStream_t);

moe_status launch_gemm_decode(const GemmArgs& a, bool swiglu, int wf, bool a_nv, int64_t rows, hipStream_t stream) {
  int nact = (int)std::min<int64_t>(a.E, rows);
  if (nact <= 0) return MOE_OK;
  if ((size_t)decode_rows_per_pass(a.K) * decode_pitch(a.K) > 96 * 1024) {
    set_error("moe_fp4_grouped_gemm: decode kernel supports k <= 4096 (k=%d)", a.K);
    return MOE_ERR_UNSUPPORTED;
  }
  a.tiled ? decode_wg<true>(a, swiglu, wf, a_nv, nact, stream) : decode_wg<false>(a, swiglu, wf, a_nv, nact, stream);
  return launch_status("moe_fp4_grouped_gemm(decode)");
}

}  // namespace moe
