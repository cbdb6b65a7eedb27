// Weight-streaming expert GEMM kernels on the tiled weight layout (kernels in
// gemm_decode.h; this unit only instantiates them, so they compile in parallel
// with the row-major ones).
#include "gemm_decode.h"

namespace moe {

template void decode_wg<true>(const GemmArgs&, bool, int, bool, int, hipStream_t);

}  // namespace moe
