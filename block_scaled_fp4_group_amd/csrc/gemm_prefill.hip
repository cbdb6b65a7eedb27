// Grouped FP4 expert GEMM, MFMA-bound ("prefill") form: entry point and the
// kernels on row-major weights (kernels in gemm_prefill.h; the tiled-layout
// variants are instantiated in gemm_prefill_tiled.hip).
#include "gemm_prefill.h"

namespace moe {

template void prefill_run<false>(const GemmArgs&, bool, int, bool, hipStream_t);

moe_status launch_gemm_decode(const GemmArgs&, bool swiglu, int wf, bool a_nv, int64_t rows, hipStream_t);

moe_status launch_gemm_prefill(const GemmArgs& a, bool swiglu, int wf, bool a_nv, int64_t rows, hipStream_t stream) {
  const int bn = swiglu ? PfTall::BN / 2 : PfTall::BN;
  if (a.N % bn != 0 || a.K % (2 * kPfBK) != 0 || a.E > kPfMaxE) {
    // shapes the tiled kernels do not cover run on the weight-streaming kernel
    return launch_gemm_decode(a, swiglu, wf, a_nv, rows, stream);
  }
  a.tiled ? prefill_run<true>(a, swiglu, wf, a_nv, stream) : prefill_run<false>(a, swiglu, wf, a_nv, stream);
  return launch_status("moe_fp4_grouped_gemm(prefill)");
}

}  // namespace moe
