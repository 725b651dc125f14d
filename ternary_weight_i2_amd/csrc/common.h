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

// Per-token quantisation arithmetic, shared by the stand-alone quantiser and
// the fused decode prologue so both produce identical bits:
//   s = 127 / max(amax, 1e-5), the correctly rounded fp32 quotient (computed
//   in binary64 and rounded once: 53 >= 2*24 + 2 makes that exact), and
//   q = clamp(round_half_even(x * s), -128, 127) with x * s one fp32 product.
__device__ __forceinline__ float quant_scale(float amax) {
    const float denom = amax > 1e-5f ? amax : 1e-5f;
    return (float)(127.0 / (double)denom);
}
__device__ __forceinline__ int quant_one(float v, float s) {
    float r = __builtin_rintf(v * s);
    r = fminf(fmaxf(r, -128.0f), 127.0f);
    return (int)r;
}

// Grouped decode launch: up to kMaxMats matrices that share K and the same
// tokens; workgroups [wg_begin, next wg_begin) serve matrix i.
constexpr int kMaxMats = 8;
struct GemvMat {
    const uint8_t *packed;
    int32_t *dot;
    float *y;
    float alpha;
    int M;
    int wg_begin;
};
struct GemvArgs {
    GemvMat mat[kMaxMats];
    int nmats;
    int K;
    int ntok;
    int rows_per_wg;
    const void *x;          // int8 xq (mode 0), fp32 (mode 1) or bf16 (mode 2) tokens
    const float *xs_in;     // mode 0: per-token scale
    const int32_t *xsum_in; // mode 0: per-token sum of xq
    int8_t *xq_out;         // modes 1/2, optional: quantised tokens
    float *xs_out;          // modes 1/2, optional
    int32_t *xsum_out;      // modes 1/2, optional
};

// ---- launchers (each returns the hipError_t of its launch) ---------------
hipError_t launch_pack(const int8_t *w, int64_t M, int64_t K, uint8_t *packed,
                       unsigned *bad, hipStream_t st);
hipError_t launch_quant(const void *x, int bf16, int64_t N, int64_t K,
                        int8_t *xq, float *xs, int32_t *xsum, hipStream_t st);
// Decode GEMV on the vector ALUs for any N (tokens are processed in passes of
// at most 8).  mode 0: x is int8 xq with xs/xsum given; mode 1/2: x is fp32 /
// bf16 and is quantised inside the kernel (xq_out/xs_out/xsum_out optional).
hipError_t launch_gemv_valu(const GemvMat *mats, int nmats, int64_t K, int64_t N,
                            int mode, const void *x, const float *xs,
                            const int32_t *xsum, int8_t *xq_out, float *xs_out,
                            int32_t *xsum_out, hipStream_t st);
// Batched decode (1..64 tokens) on MFMA, weights streamed once.
hipError_t launch_gemv_mfma(const uint8_t *packed, float alpha, int64_t M, int64_t K,
                            const int8_t *xq, const float *xs, const int32_t *xsum, int64_t N,
                            int32_t *dot, float *y, hipStream_t st);
hipError_t launch_gemm_mfma(const uint8_t *packed, float alpha, int64_t M,
                            int64_t K, const int8_t *xq, const float *xs,
                            const int32_t *xsum, int64_t N, int32_t *dot,
                            float *y, hipStream_t st);

}  // namespace bitnet
