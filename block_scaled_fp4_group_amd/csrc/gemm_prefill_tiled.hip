// MFMA-bound expert GEMM kernels on the tiled weight layout (kernels in
// gemm_prefill.h; this unit only instantiates them).
#include "gemm_prefill.h"

namespace moe {

template void prefill_run<true>(const GemmArgs&, bool, int, bool, hipStream_t);

}  // namespace moe
