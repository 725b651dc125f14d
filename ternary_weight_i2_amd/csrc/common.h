// common.h -- device helpers and launcher declarations shared by the HIP
// translation units of libbitnet_i2s.so (library-internal; not installed).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bitnet {

// I2_S block: 128 weights in 32 bytes; byte j of a block holds the 2-bit codes
// of block positions j, j+32, j+64, j+96 in bits 7-6, 5-4, 3-2, 1-0.
constexpr int kBlock = 128;
constexpr int kBlockBytes = 32;

typedef int v4i __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int dot4(int a, int b, int c) {
    // v_dot4_i32_i8: c + sum of the four signed byte products
    return __builtin_amdgcn_sdot4(a, b, c, false);
}

// Wave-wide (64 lanes) sums and maxima through cross-lane shuffles.
__device__ __forceinline__ int wave_sum_i32(int v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}
__device__ __forceinline__ float wave_max_f32(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}

// ---- launchers (each returns the hipError_t of its launch) ---------------
hipError_t launch_pack(const int8_t *w, int64_t M, int64_t K, uint8_t *packed,
                       unsigned *bad, hipStream_t st);
hipError_t launch_quant(const void *x, int bf16, int64_t N, int64_t K,
                        int8_t *xq, float *xs, int32_t *xsum, hipStream_t st);
hipError_t launch_gemv_valu(const uint8_t *packed, float alpha, int64_t M,
                            int64_t K, const int8_t *xq, const float *xs,
                            const int32_t *xsum, int64_t N, int32_t *dot,
                            float *y, hipStream_t st);
hipError_t launch_gemm_mfma(const uint8_t *packed, float alpha, int64_t M,
                            int64_t K, const int8_t *xq, const float *xs,
                            const int32_t *xsum, int64_t N, int32_t *dot,
                            float *y, hipStream_t st);

}  // namespace bitnet
