// gemv_valu_n8_bf16.hip -- decode GEMV kernels for 5-8 bf16 tokens per pass
// (every lane count), compiled on their own so the units build in parallel.
#include "gemv_valu.h"

namespace bitnet {
template hipError_t launch_gemv_nt<8, 2>(const GemvArgs &, int, bool, unsigned, hipStream_t);
}  // namespace bitnet
