// gemv_valu_n4.hip -- decode GEMV kernels for 3-4 tokens per pass, fp32 and bf16 tokens
// (every lane count), compiled on their own so the units build in parallel.
#include "gemv_valu.h"

namespace bitnet {
template hipError_t launch_gemv_nt<4, 1>(const GemvArgs &, int, bool, unsigned, hipStream_t);
template hipError_t launch_gemv_nt<4, 2>(const GemvArgs &, int, bool, unsigned, hipStream_t);
}  // namespace bitnet
