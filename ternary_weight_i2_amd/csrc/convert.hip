// convert.hip -- one-time weight conversion to I2_S: the AbsMean ternariser
// and the sign/threshold float packer.
//
// Pages: [P1] "BitNet 딥다이브" §6-2 (AbsMean: scale = max(mean|w|, 1e-5),
// q = round(w / scale) limited to -1..1, the scale stored for dequantisation),
// §4-2 (the float packer: near-zero weights, |v| < 1e-6, take code 1,
// positive ones code 2, negative ones code 0), §1-1 (code table); [P4]
// "bitnet.rs", "Mathematical Foundation" (AbsMean formula).
//
// AbsMean: the sum of |w| is taken exactly (exact_sum.h: every fp32
// magnitude added into 32-bit digits that span the whole fp32 range), then
// rounded once to binary64, divided by n in binary64 and rounded to fp32, so
// alpha does not depend on how the sum is split.  A grid of workgroups each
// adds a strided share and writes its digits (partial[]); one workgroup adds
// the partials and forms alpha.  The pack pass then reads alpha from device
// memory, so the three launches need no host round trip.
#include "common.h"
#include "exact_sum.h"

namespace bitnet {

constexpr int kConvThreads = 256;
static_assert(kConvDigits == kMagNorm, "digits of one AbsMean partial sum");

// 4 consecutive weights, widened to fp32 (16 bytes of fp32 or 8 of bf16)
template <int BF16>
__device__ __forceinline__ void load4(const void *w, int64_t g, float *v) {
    if constexpr (BF16) {
        const uint2 u = reinterpret_cast<const uint2 *>(w)[g];
        v[0] = __uint_as_float(u.x << 16);
        v[1] = __uint_as_float(u.x & 0xFFFF0000u);
        v[2] = __uint_as_float(u.y << 16);
        v[3] = __uint_as_float(u.y & 0xFFFF0000u);
    } else {
        const float4 f = reinterpret_cast<const float4 *>(w)[g];
        v[0] = f.x; v[1] = f.y; v[2] = f.z; v[3] = f.w;
    }
}

// Pass 1: the digits of sum |w| over groups of 4 weights g = b*256 + t,
// g += gridDim*256, normalised into partial[b][0..kMagNorm).
//
// Per weight, |w| = m * 2^(P-149) (m < 2^24, P in [0, 253]) goes into one of
// 16 binary64 buckets, bucket q = P >> 4 holding multiples of 2^(16q-149)
// below 2^39 of that unit each.  A bucket takes at most 4 * kAbsChunk
// = 2^13 terms before it is folded, so its sum stays below 2^52 units and
// every addition is exact in binary64: the bucket sums are exact whatever
// the order.  Each thread owns its buckets (a column of bk[][] in LDS, added
// to with LDS float atomics, so no weight waits on the one before); after
// each chunk it folds them, as integers, into the carry-save digits d of
// exact_sum.h (each add below 2^37, each digit of a workgroup below 2^64).
constexpr int kAbsBuckets = 16;
constexpr int kAbsChunk = 2048;   // groups of 4 weights per thread between folds

__device__ __forceinline__ void abs_bucket_add(double (*bk)[kConvThreads], int tid, float w) {
    const uint32_t bits = __float_as_uint(w) & 0x7fffffffu;
    const uint32_t E = bits >> 23;
    if (E == 0xffu) return;   // non-finite: the pack pass reports it
    const uint32_t m = E ? ((bits & 0x7fffffu) | 0x800000u) : bits;
    const int P = E ? (int)E - 1 : 0;
    __hip_atomic_fetch_add(&bk[P >> 4][tid], ldexp((double)m, P - 149), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_WORKGROUP);
}

__device__ __forceinline__ void abs_fold(double (*bk)[kConvThreads], int tid, uint64_t *d) {
#pragma unroll
    for (int q = 0; q < kAbsBuckets; ++q) {
        const double t = ldexp(bk[q][tid], 149 - 16 * q);   // an integer below 2^52
        bk[q][tid] = 0.0;
        const uint32_t hi = (uint32_t)(t * 0x1p-32);
        const uint32_t lo = (uint32_t)(t - (double)hi * 0x1p32);
        const int i = q >> 1;   // bucket unit 2^(16q) = digit i, shifted by 16 (q odd)
        if (q & 1) {
            d[i] += (uint64_t)(lo & 0xffffu) << 16;
            d[i + 1] += (uint64_t)(lo >> 16) + ((uint64_t)hi << 16);
        } else {
            d[i] += lo;
            d[i + 1] += hi;
        }
    }
}

template <int BF16>
__global__ __launch_bounds__(kConvThreads) void absmean_partial_kernel(
    const void *__restrict__ w, int64_t n4, uint32_t *__restrict__ partial) {
    __shared__ double bk[kAbsBuckets][kConvThreads];
    __shared__ uint64_t red[kConvThreads / 64][kMagDigits];
    const int tid = threadIdx.x;
#pragma unroll
    for (int q = 0; q < kAbsBuckets; ++q) bk[q][tid] = 0.0;
    uint64_t d[kMagDigits];
#pragma unroll
    for (int i = 0; i < kMagDigits; ++i) d[i] = 0;
    const int64_t stride = (int64_t)gridDim.x * kConvThreads;
    int64_t g = (int64_t)blockIdx.x * kConvThreads + tid;
    while (g < n4) {
        const int64_t gend = min(n4, g + (int64_t)kAbsChunk * stride);
        for (; g < gend; g += 4 * stride) {
            // four groups in flight (clamped addresses; only those below gend count)
            float v[4][4];
#pragma unroll
            for (int u = 0; u < 4; ++u) load4<BF16>(w, min(g + u * stride, n4 - 1), v[u]);
#pragma unroll
            for (int u = 0; u < 4; ++u)
                if (g + u * stride < gend) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) abs_bucket_add(bk, tid, v[u][e]);
                }
        }
        abs_fold(bk, tid, d);
    }
#pragma unroll
    for (int i = 0; i < kMagDigits; ++i) d[i] = wave_sum_u64(d[i]);
    if ((tid & 63) == 0) {
#pragma unroll
        for (int i = 0; i < kMagDigits; ++i) red[tid >> 6][i] = d[i];
    }
    __syncthreads();
    if (tid == 0) {
        uint64_t t[kMagDigits];
        for (int i = 0; i < kMagDigits; ++i) {
            t[i] = 0;
            for (int wv = 0; wv < kConvThreads / 64; ++wv) t[i] += red[wv][i];
        }
        mag_normalise(t, kMagDigits, partial + (int64_t)blockIdx.x * kMagNorm);
    }
}

// Pass 2 (one workgroup, a thread per partial): the exact total, rounded once
// to binary64; alpha = max(fp32(sum / n), 1e-5).  The partials' digits are
// transposed through LDS so that wave i adds digit i of every partial (16
// reads per lane and one wave reduction per digit, in parallel).
__global__ __launch_bounds__(1024) void absmean_final_kernel(
    const uint32_t *__restrict__ partial, int nparts, int64_t n, float *__restrict__ alpha) {
    static_assert(kMagNorm <= 1024 / 64, "a wave per digit");
    __shared__ uint32_t col[kMagNorm][1024];
    __shared__ uint64_t tot[kMagNorm];
    const int t = threadIdx.x, wv = t >> 6, lane = t & 63;
#pragma unroll
    for (int i = 0; i < kMagNorm; ++i)
        col[i][t] = t < nparts ? partial[(int64_t)t * kMagNorm + i] : 0u;
    __syncthreads();
    if (wv < kMagNorm) {
        uint64_t sum = 0;
#pragma unroll
        for (int j = 0; j < 1024 / 64; ++j) sum += col[wv][lane + 64 * j];
        sum = wave_sum_u64(sum);
        if (lane == 0) tot[wv] = sum;
    }
    __syncthreads();
    if (t == 0) {
        uint64_t d[kMagNorm];
#pragma unroll
        for (int i = 0; i < kMagNorm; ++i) d[i] = tot[i];
        uint32_t nd[kMagNorm];
        mag_normalise(d, kMagNorm, nd);
        const double s = mag_round(nd);
        const float a = (float)(s / (double)n);
        *alpha = a > 1e-5f ? a : 1e-5f;
    }
}

// Pass 3: one thread per packed dword (bytes g0..g0+3 of a 32-byte block =
// block positions g0+e+32*i), as the int8 packer.  MODE 0: AbsMean,
// q = clip(rint(w / alpha), -1, 1) with one fp32 division.  MODE 1: sign with
// the |v| < 1e-6 zero threshold (compared in binary64, as the constant is
// written), and each workgroup's max|v| into part[] (the grid is then at
// most kConvPartials workgroups; max_final_kernel reduces them).
// Non-finite weights are counted in *bad (code 1).
template <int BF16, int MODE>
__global__ __launch_bounds__(kConvThreads) void ternary_pack_kernel(
    const void *__restrict__ w, int64_t M, int64_t K, const float *__restrict__ alpha,
    uint8_t *__restrict__ packed, unsigned *__restrict__ bad, double *__restrict__ part) {
    const int64_t dw_per_row = K / 16;
    const int64_t total = M * dw_per_row;
    const float a = MODE == 0 ? *alpha : 1.0f;
    unsigned nbad = 0;
    float vmax = 0.0f;
    for (int64_t d = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; d < total;
         d += (int64_t)gridDim.x * blockDim.x) {
        const int64_t m = d / dw_per_row;
        const int64_t r = d - m * dw_per_row;
        const int64_t blk = r >> 3;          // 8 dwords per block
        const int g0 = (int)(r & 7) * 4;     // first block byte of this dword
        const int64_t base = m * K + blk * kBlock + g0;   // element index, multiple of 4
        uint32_t out = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float v[4];
            load4<BF16>(w, (base + 32 * i) >> 2, v);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                int code = 1;
                if (!__builtin_isfinite(v[e])) {
                    ++nbad;
                } else if constexpr (MODE == 0) {
                    const float q = fminf(fmaxf(__builtin_rintf(v[e] / a), -1.0f), 1.0f);
                    code = (int)q + 1;
                } else {
                    if (fabs((double)v[e]) >= 1e-6) code = v[e] > 0.0f ? 2 : 0;
                    vmax = fmaxf(vmax, fabsf(v[e]));
                }
                out |= (uint32_t)code << (8 * e + 6 - 2 * i);
            }
        }
        *reinterpret_cast<uint32_t *>(packed + m * (K / 4) + blk * kBlockBytes + g0) = out;
    }
    if (nbad) atomicAdd(bad, nbad);
    if constexpr (MODE == 1) {
        __shared__ float red[kConvThreads / 64];
        vmax = wave_max_f32(vmax);
        if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = vmax;
        __syncthreads();
        if (threadIdx.x == 0) {
            float m = red[0];
#pragma unroll
            for (int i = 1; i < kConvThreads / 64; ++i) m = fmaxf(m, red[i]);
            part[blockIdx.x] = (double)m;
        }
    }
}

// max over nparts workgroup maxima (one workgroup) -> *wmax
__global__ __launch_bounds__(1024) void max_final_kernel(const double *__restrict__ part,
                                                         int nparts, float *__restrict__ wmax) {
    __shared__ float red[16];
    float v = (int)threadIdx.x < nparts ? (float)part[threadIdx.x] : 0.0f;
    v = wave_max_f32(v);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    if (threadIdx.x == 0) {
        float m = red[0];
#pragma unroll
        for (int i = 1; i < 16; ++i) m = fmaxf(m, red[i]);
        *wmax = m;
    }
}

hipError_t launch_absmean_alpha(const void *w, int bf16, int64_t n, uint32_t *partial,
                                float *alpha, hipStream_t st) {
    const int64_t n4 = n / 4;
    int64_t parts = (n4 + kConvThreads * 8 - 1) / (kConvThreads * 8);   // >= 8 groups per thread
    if (parts > kConvPartials) parts = kConvPartials;
    if (parts < 1) parts = 1;
    if (bf16)
        hipLaunchKernelGGL(absmean_partial_kernel<1>, dim3((unsigned)parts), dim3(kConvThreads), 0, st,
                           w, n4, partial);
    else
        hipLaunchKernelGGL(absmean_partial_kernel<0>, dim3((unsigned)parts), dim3(kConvThreads), 0, st,
                           w, n4, partial);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(absmean_final_kernel, dim3(1), dim3(1024), 0, st, partial, (int)parts, n,
                       alpha);
    return hipGetLastError();
}

hipError_t launch_ternary_pack(const void *w, int bf16, int mode, int64_t M, int64_t K,
                               const float *alpha, uint8_t *packed, unsigned *bad,
                               double *part, float *wmax, hipStream_t st) {
    const int64_t total = M * (K / 16);
    int64_t blocks = (total + kConvThreads - 1) / kConvThreads;
    const int64_t cap = mode == 0 ? 65536 : kConvPartials;
    if (blocks > cap) blocks = cap;
    const dim3 g((unsigned)blocks), b(kConvThreads);
    if (mode == 0) {
        if (bf16) hipLaunchKernelGGL((ternary_pack_kernel<1, 0>), g, b, 0, st, w, M, K, alpha, packed, bad, part);
        else hipLaunchKernelGGL((ternary_pack_kernel<0, 0>), g, b, 0, st, w, M, K, alpha, packed, bad, part);
        return hipGetLastError();
    }
    if (bf16) hipLaunchKernelGGL((ternary_pack_kernel<1, 1>), g, b, 0, st, w, M, K, alpha, packed, bad, part);
    else hipLaunchKernelGGL((ternary_pack_kernel<0, 1>), g, b, 0, st, w, M, K, alpha, packed, bad, part);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(max_final_kernel, dim3(1), dim3(1024), 0, st, part, (int)blocks, wmax);
    return hipGetLastError();
}

}  // namespace bitnet
