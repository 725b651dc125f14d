// gemv_valu_n1.hip -- decode GEMV kernels for 1 token per pass, every token mode
// (every lane count), compiled on their own so the units build in parallel.
#include "gemv_valu.h"

namespace bitnet {
template hipError_t launch_gemv_nt<1, 0>(const GemvKernelArgs &, int, int, bool, unsigned, hipStream_t);
template hipError_t launch_gemv_nt<1, 1>(const GemvKernelArgs &, int, int, bool, unsigned, hipStream_t);
template hipError_t launch_gemv_nt<1, 2>(const GemvKernelArgs &, int, int, bool, unsigned, hipStream_t);
}  // namespace bitnet
