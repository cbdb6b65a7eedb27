// Persistent weight-streaming expert GEMM kernels, both weight layouts
// (kernels in gemm_decode.h; instantiated here to compile in parallel).
#include "gemm_decode.h"

namespace moe {

template void decode_persist<false>(const GemmArgs&, bool, int, bool, hipStream_t);
template void decode_persist<true>(const GemmArgs&, bool, int, bool, hipStream_t);

}  // namespace moe
