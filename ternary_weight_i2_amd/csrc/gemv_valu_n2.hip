// gemv_valu_n2.hip -- decode GEMV kernels for 2 tokens per pass, every token mode
// (every lane count), compiled on their own so the units build in parallel.
#include "gemv_valu.h"

namespace bitnet {
template hipError_t launch_gemv_nt<2, 0>(const GemvKernelArgs &, int, int, bool, unsigned, hipStream_t);
template hipError_t launch_gemv_nt<2, 1>(const GemvKernelArgs &, int, int, bool, unsigned, hipStream_t);
template hipError_t launch_gemv_nt<2, 2>(const GemvKernelArgs &, int, int, bool, unsigned, hipStream_t);
}  // namespace bitnet
