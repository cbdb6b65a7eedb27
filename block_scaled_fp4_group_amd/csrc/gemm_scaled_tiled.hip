// Block-scaled MFMA expert GEMM kernels on the tiled weight layout (kernels in
// gemm_scaled.h; this unit only instantiates them).
#include "gemm_scaled.h"

namespace moe {

template void scaled_run<true>(const GemmArgs&, bool, bool, bool, hipStream_t);

}  // namespace moe
