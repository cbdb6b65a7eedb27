// Grouped FP4 expert GEMM, MFMA-bound ("prefill") form -- placeholder that
// routes to the weight-streaming kernel until the LDS-tiled kernel lands.
#include "gemm_common.h"

namespace moe {

moe_status launch_gemm_decode(const GemmArgs&, bool swiglu, bool w_nv, bool a_nv, int64_t rows, hipStream_t);

moe_status launch_gemm_prefill(const GemmArgs& a, bool swiglu, bool w_nv, bool a_nv, int64_t rows, hipStream_t stream) {
  return launch_gemm_decode(a, swiglu, w_nv, a_nv, rows, stream);
}

}  // namespace moe
