// Grouped FP4 expert GEMM on the block-scaled MFMA (MXFP8 or NVFP4-plane
// tokens): the kernels on row-major weights (kernels in gemm_scaled.h; the
// tiled-layout variants are instantiated in gemm_scaled_tiled.hip).
#include "gemm_scaled.h"

namespace moe {

template void scaled_run<false>(const GemmArgs&, bool, bool, bool, hipStream_t);

moe_status launch_gemm_scaled(const GemmArgs& a, bool swiglu, bool planes, bool w_nv, hipStream_t stream) {
  a.tiled ? scaled_run<true>(a, swiglu, planes, w_nv, stream) : scaled_run<false>(a, swiglu, planes, w_nv, stream);
  return launch_status("moe_fp4_grouped_gemm(block-scaled)");
}

}  // namespace moe
