// lut.hip -- decode matmul by table lookup, an alternative to the in-register
// unpack of the GEMV kernels (same integers, same epilogue).
//
// Method [P1 §4-3, §4-4 (the LUT route: tables built from the activations
// first, a barrier, then the lookups); P1 §11-2 (T-MAC, the lookup-based
// low-bit method)]: a weight group is the pair of 2-bit fields in one nibble
// of an I2_S byte -- for byte t of a row, the high nibble pairs the
// activations at (block start + t mod 32) and 32 places after, the low nibble
// those 64 and 96 places after.  A group's table holds the 16 raw-code sums
// c_hi * x_first + c_lo * x_second (codes 0..3, so any nibble is a valid
// index); the lookups over a row add up to the raw-code sum R, and
// D = R - sum(x) exactly as in the unpack route.
//
// GPU mapping: one workgroup per 64 output rows and token, up to 16 waves.
//   Phase 1: the waves write all K/2 tables of the token to LDS as int16
//   (|entry| <= 3 * 128 * 2), 32 bytes per group, while their first weight
//   loads are in flight.  The workgroup barrier separates the phases.
//   Phase 2: lane = output row, wave = a strided set of 128-weight blocks.
//   All lanes of a wave look up the same group at the same time, so one LDS
//   read touches one 32-byte table (8 banks; equal words are broadcast) and
//   never conflicts.  The waves' partial sums meet in LDS and wave 0 writes
//   D and y = D * alpha / s with the fp32 operations of the GEMV kernels.
#include "common.h"

namespace bitnet {

constexpr int kLutRows = 64;       // output rows per workgroup (one per lane)
constexpr int kLutMaxWaves = 16;   // waves per workgroup (K split across them)

__global__ __launch_bounds__(kLutMaxWaves * 64) void gemv_lut_kernel(
    const uint8_t *__restrict__ packed, float alpha, int M, int K,
    const int8_t *__restrict__ xq, const float *__restrict__ xs,
    const int32_t *__restrict__ xsum, int32_t *__restrict__ dot, float *__restrict__ y) {
    // [K/2 groups][16 int16 entries], then int32 partial[waves][64]
    extern __shared__ __attribute__((aligned(16))) uint32_t lut_lds[];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int nthreads = (int)blockDim.x, nw = nthreads >> 6;
    const int n = (int)blockIdx.y;
    const int row0 = (int)blockIdx.x * kLutRows;
    const int row = min(row0 + lane, M - 1);   // rows past M reload the last row, never stored
    const int nb = K / kBlock;
    const uint4 *src = reinterpret_cast<const uint4 *>(packed + (int64_t)row * (K >> 2));
    const int8_t *x = xq + (int64_t)n * K;

    // This wave's first block (32 bytes of the lane's row) goes out before the
    // table build so its latency overlaps phase 1.
    int b = wave;
    uint4 c0 = {}, c1 = {};
    if (b < nb) {
        c0 = src[2 * b];
        c1 = src[2 * b + 1];
    }

    // Phase 1: tables.  Entry e = 4*c_hi + c_lo sits at int16 offset e of the
    // group's 32 bytes; dword i holds entries 2i (low half) and 2i+1.
    const int groups = K >> 1;
    for (int g = tid; g < groups; g += nthreads) {
        const int t = g >> 1;
        const int first = (t >> 5) * kBlock + (t & 31) + 64 * (g & 1);
        const int xa = x[first], xb = x[first + 32];
        uint32_t w[8];
#pragma unroll
        for (int ch = 0; ch < 4; ++ch) {
            const int base = ch * xa;
            w[2 * ch] = (uint32_t)(uint16_t)base | ((uint32_t)(uint16_t)(base + xb) << 16);
            w[2 * ch + 1] =
                (uint32_t)(uint16_t)(base + 2 * xb) | ((uint32_t)(uint16_t)(base + 3 * xb) << 16);
        }
        uint4 *dst = reinterpret_cast<uint4 *>(lut_lds + g * 8);
        dst[0] = uint4{w[0], w[1], w[2], w[3]};
        dst[1] = uint4{w[4], w[5], w[6], w[7]};
    }
    __syncthreads();

    // Phase 2: lookups.  Block b's groups start at int16 offset 1024*b; byte j
    // of the block owns groups 2j (high nibble) and 2j+1 (low nibble).
    const int16_t *t16 = reinterpret_cast<const int16_t *>(lut_lds);
    int acc = 0;
    for (; b < nb; b += nw) {
        const int bn = b + nw;
        uint4 n0 = c0, n1 = c1;
        if (bn < nb) {   // next block of this wave, loaded while this one is looked up
            n0 = src[2 * bn];
            n1 = src[2 * bn + 1];
        }
        const int16_t *blk = t16 + b * 1024;
        const uint32_t d[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
#pragma unroll
        for (int j = 0; j < 32; ++j) {
            const uint32_t byte = (d[j >> 2] >> (8 * (j & 3))) & 0xFFu;
            acc += blk[32 * j + (byte >> 4)];
            acc += blk[32 * j + 16 + (byte & 15u)];
        }
        c0 = n0;
        c1 = n1;
    }

    int *part = reinterpret_cast<int *>(lut_lds + groups * 8);
    part[wave * 64 + lane] = acc;
    __syncthreads();
    if (wave == 0 && row0 + lane < M) {
        int r = 0;
        for (int w = 0; w < nw; ++w) r += part[w * 64 + lane];
        const int d = r - xsum[n];
        const int64_t o = (int64_t)n * M + row0 + lane;
        if (dot) dot[o] = d;
        if (y) y[o] = ((float)d * alpha) / xs[n];
    }
}

hipError_t launch_gemv_lut(const uint8_t *packed, float alpha, int64_t M, int64_t K,
                           const int8_t *xq, const float *xs, const int32_t *xsum, int64_t N,
                           int32_t *dot, float *y, hipStream_t st) {
    const int nb = (int)(K / kBlock);
    const int nw = nb < kLutMaxWaves ? nb : kLutMaxWaves;
    const size_t lds = (size_t)K * 16 + (size_t)nw * 64 * sizeof(int);
    const dim3 grid((unsigned)((M + kLutRows - 1) / kLutRows), (unsigned)N);
    hipLaunchKernelGGL(gemv_lut_kernel, grid, dim3((unsigned)(nw * 64)), lds, st, packed, alpha,
                       (int)M, (int)K, xq, xs, xsum, dot, y);
    return hipGetLastError();
}

}  // namespace bitnet
