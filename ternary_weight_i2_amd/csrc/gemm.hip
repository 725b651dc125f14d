// gemm.hip -- multi-token matmul on int8 MFMA (v_mfma_i32_16x16x64_i8).
//
// Pages: [P1] "BitNet 딥다이브" §4-2 (I2_S block interleave), §4-5 (separate
// prefill path); [P2] "[분석/검증-3]" §3 and [P3] "[기술 분석 보고서]"
// §3.2 (raw codes multiply the activations; the exact result subtracts
// sum(x)).
//
// The contraction over k is order-free, so the MFMA k-slots are assigned to
// match the I2_S byte layout instead of shuffling the weights:
//   one 16x16x64 step covers one half-block h (16 packed bytes per row);
//   lane group kq (lanes 16kq..16kq+15) takes packed dword kq of that half,
//   i.e. block bytes 16h+4kq..16h+4kq+3, whose four 2-bit fields i hold the
//   positions 32i + 16h + 4kq + e (e = 0..3).
// The A operand (weights, 16 bytes per lane) is that dword unpacked in
// registers: byte 4i+e = field i of byte e = code of position 32i+16h+4kq+e.
// The B operand (activations) must hold the same positions in the same byte
// order; the activation tile is therefore staged in LDS with its 32 dwords per
// block permuted so that those four dwords are contiguous and one 16-byte LDS
// read fetches a lane's B operand.  MFMA accumulates the raw-code sum R in
// int32; the epilogue writes D = R - sum(x) and y = D * alpha / s.
#include "common.h"

namespace bitnet {

constexpr int kPkStride = 48;    // LDS bytes per packed-tile row (32 + pad)
constexpr int kXStride = 144;    // LDS bytes per activation-tile row (128 + pad)

// new dword slot of original block dword dd = 8i + 4h + kq
__device__ __forceinline__ int xperm(int dd) {
    const int i = dd >> 3, h = (dd >> 2) & 1, kq = dd & 3;
    return (h * 4 + kq) * 4 + i;
}

template <int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(256) void gemm_mfma_kernel(
    const uint8_t *__restrict__ packed, float alpha, int M, int K,
    const int8_t *__restrict__ xq, const float *__restrict__ xs,
    const int32_t *__restrict__ xsum, int N, int32_t *__restrict__ dot,
    float *__restrict__ y) {
    static_assert(WM * WN == 4, "four waves per workgroup");
    constexpr int MI = BM / WM / 16;
    constexpr int NJ = BN / WN / 16;
    static_assert(MI >= 1 && NJ >= 1, "tile too small");
    __shared__ __attribute__((aligned(16))) uint8_t pk[BM * kPkStride];
    __shared__ __attribute__((aligned(16))) int8_t xt[BN * kXStride];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave % WM, wn = wave / WM;
    const int li = lane & 15, kq = lane >> 4;
    const int m0 = blockIdx.x * BM, n0 = blockIdx.y * BN;
    const int64_t prow_bytes = K >> 2;

    v4i acc[MI][NJ];
#pragma unroll
    for (int a = 0; a < MI; ++a)
#pragma unroll
        for (int b = 0; b < NJ; ++b) acc[a][b] = v4i{0, 0, 0, 0};

    const int nkb = K / kBlock;
    for (int kb = 0; kb < nkb; ++kb) {
        for (int c = tid; c < BM * 2; c += 256) {
            const int r = c >> 1, h = c & 1;
            int4 v = make_int4(0, 0, 0, 0);
            if (m0 + r < M)
                v = *reinterpret_cast<const int4 *>(packed + (int64_t)(m0 + r) * prow_bytes +
                                                    kb * kBlockBytes + h * 16);
            *reinterpret_cast<int4 *>(pk + r * kPkStride + h * 16) = v;
        }
        for (int c = tid; c < BN * 8; c += 256) {
            const int r = c >> 3, q = c & 7;
            int4 v = make_int4(0, 0, 0, 0);
            if (n0 + r < N)
                v = *reinterpret_cast<const int4 *>(xq + (int64_t)(n0 + r) * K +
                                                    kb * kBlock + q * 16);
            int *dst = reinterpret_cast<int *>(xt + r * kXStride);
            dst[xperm(4 * q + 0)] = v.x;
            dst[xperm(4 * q + 1)] = v.y;
            dst[xperm(4 * q + 2)] = v.z;
            dst[xperm(4 * q + 3)] = v.w;
        }
        __syncthreads();
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            v4i a[MI], b[NJ];
#pragma unroll
            for (int mi = 0; mi < MI; ++mi) {
                const uint32_t p = *reinterpret_cast<const uint32_t *>(
                    pk + ((wm * MI + mi) * 16 + li) * kPkStride + h * 16 + kq * 4);
                a[mi] = v4i{(int)((p >> 6) & 0x03030303u), (int)((p >> 4) & 0x03030303u),
                            (int)((p >> 2) & 0x03030303u), (int)(p & 0x03030303u)};
            }
#pragma unroll
            for (int nj = 0; nj < NJ; ++nj)
                b[nj] = *reinterpret_cast<const v4i *>(
                    xt + ((wn * NJ + nj) * 16 + li) * kXStride + (h * 4 + kq) * 16);
#pragma unroll
            for (int mi = 0; mi < MI; ++mi)
#pragma unroll
                for (int nj = 0; nj < NJ; ++nj)
                    acc[mi][nj] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[mi], b[nj],
                                                                        acc[mi][nj], 0, 0, 0);
        }
        __syncthreads();
    }

    // 16x16 result layout: lane l, register r holds row 4*(l/16)+r, column l%16
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
#pragma unroll
        for (int nj = 0; nj < NJ; ++nj) {
            const int n = n0 + (wn * NJ + nj) * 16 + li;
            if (n >= N) continue;
            const int sx = xsum[n];
            const float s = xs[n];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = m0 + (wm * MI + mi) * 16 + 4 * kq + r;
                if (m < M) {
                    const int d = acc[mi][nj][r] - sx;
                    if (dot) dot[(int64_t)n * M + m] = d;
                    if (y) y[(int64_t)n * M + m] = ((float)d * alpha) / s;
                }
            }
        }
    }
}

template <int BM, int BN, int WM, int WN>
static hipError_t run_gemm(const uint8_t *packed, float alpha, int64_t M, int64_t K,
                           const int8_t *xq, const float *xs, const int32_t *xsum,
                           int64_t N, int32_t *dot, float *y, hipStream_t st) {
    const dim3 grid((unsigned)((M + BM - 1) / BM), (unsigned)((N + BN - 1) / BN));
    hipLaunchKernelGGL((gemm_mfma_kernel<BM, BN, WM, WN>), grid, dim3(256), 0, st, packed,
                       alpha, (int)M, (int)K, xq, xs, xsum, (int)N, dot, y);
    return hipGetLastError();
}

hipError_t launch_gemm_mfma(const uint8_t *packed, float alpha, int64_t M,
                            int64_t K, const int8_t *xq, const float *xs,
                            const int32_t *xsum, int64_t N, int32_t *dot,
                            float *y, hipStream_t st) {
    if (N <= 16) return run_gemm<64, 16, 4, 1>(packed, alpha, M, K, xq, xs, xsum, N, dot, y, st);
    if (N <= 32) return run_gemm<64, 32, 4, 1>(packed, alpha, M, K, xq, xs, xsum, N, dot, y, st);
    if (N <= 64 || M * N < 256LL * 128 * 128)
        return run_gemm<64, 64, 2, 2>(packed, alpha, M, K, xq, xs, xsum, N, dot, y, st);
    return run_gemm<128, 128, 2, 2>(packed, alpha, M, K, xq, xs, xsum, N, dot, y, st);
}

}  // namespace bitnet
