// gemv.hip -- decode matmul for 1..8 tokens on the vector ALUs.
//
// Pages: [P2] "[분석/검증-3] BitNet.cpp ARM 커널 재작성" §3 and [P3] "[기술 분석
// 보고서] ARM64 ... 1.58-bit ..." §3.1-§4 (raw codes 0/1/2 multiply the
// activations at offsets k, k+32, k+64, k+96 of a block; the scale is applied
// by the caller); [P1] "BitNet 딥다이브" §4-3 (a weight block is loaded once
// and reused for several activation columns).
//
// Design (gfx950, wave64): one wave owns one output row at a time and walks
// the packed row with 16-byte loads, lane c taking chunk c, c+64, ...
// A 16-byte chunk is half an I2_S block: dword j holds block bytes
// g0+4j..g0+4j+3 and therefore the codes of positions g0+4j+e+32*i.  Masking
// a dword keeps one 2-bit field per byte, which v_dot4_i32_i8 multiplies
// straight against four contiguous int8 activations:
//   field i=3 (bits 1-0): w & 0x03030303       -> code * 1
//   field i=2 (bits 3-2): w & 0x0C0C0C0C       -> code * 4
//   field i=1 (bits 5-4): w & 0x30303030       -> code * 16
//   field i=0 (bits 7-6): (w >> 2) & 0x30303030 -> code * 16
// so three accumulators (x1, x4, x16) need no per-field shifts; their exact
// combination acc1 + acc4/4 + acc16/16 is the raw-code sum R, and the exact
// dot is D = R - sum(x).  Tokens are staged in LDS once per workgroup and
// every weight chunk is reused for all tokens of the call.
#include "common.h"

namespace bitnet {

constexpr int kGemvThreads = 256;
constexpr int kLdsBytes = 65536;   // activation staging budget per workgroup

template <int NT>
__global__ __launch_bounds__(kGemvThreads) void gemv_valu_kernel(
    const uint8_t *__restrict__ packed, float alpha, int M, int K,
    const int8_t *__restrict__ xq, const float *__restrict__ xs,
    const int32_t *__restrict__ xsum, int ntok, int32_t *__restrict__ dot,
    float *__restrict__ y, int rows_per_wg) {
    extern __shared__ int4 lds[];
    const int8_t *xl = reinterpret_cast<const int8_t *>(lds);
    {
        const int n16 = ntok * (K / 16);
        const int4 *src = reinterpret_cast<const int4 *>(xq);
        for (int i = threadIdx.x; i < n16; i += kGemvThreads) lds[i] = src[i];
    }
    __syncthreads();

    const int lane = threadIdx.x & 63;
    const int wv = threadIdx.x >> 6;
    const int C = K >> 6;   // 16-byte chunks per packed row
    const int row0 = blockIdx.x * rows_per_wg;
    const int row1 = min(M, row0 + rows_per_wg);
    for (int row = row0 + wv; row < row1; row += kGemvThreads / 64) {
        int a1[NT], a4[NT], a16[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) a1[t] = a4[t] = a16[t] = 0;
        const int4 *prow = reinterpret_cast<const int4 *>(packed + (int64_t)row * (K >> 2));
        for (int c = lane; c < C; c += 64) {
            const v4i pv = __builtin_nontemporal_load(reinterpret_cast<const v4i *>(prow) + c);
            const int4 p = make_int4(pv.x, pv.y, pv.z, pv.w);
            const int xoff = (c >> 1) * kBlock + (c & 1) * 16;
            const int pw[4] = {p.x, p.y, p.z, p.w};
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                if (t < ntok) {
                    const int8_t *xt = xl + t * K + xoff;
                    const int4 x0 = *reinterpret_cast<const int4 *>(xt);
                    const int4 x1 = *reinterpret_cast<const int4 *>(xt + 32);
                    const int4 x2 = *reinterpret_cast<const int4 *>(xt + 64);
                    const int4 x3 = *reinterpret_cast<const int4 *>(xt + 96);
                    const int xv0[4] = {x0.x, x0.y, x0.z, x0.w};
                    const int xv1[4] = {x1.x, x1.y, x1.z, x1.w};
                    const int xv2[4] = {x2.x, x2.y, x2.z, x2.w};
                    const int xv3[4] = {x3.x, x3.y, x3.z, x3.w};
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        a16[t] = dot4((pw[j] >> 2) & 0x30303030, xv0[j], a16[t]);
                        a16[t] = dot4(pw[j] & 0x30303030, xv1[j], a16[t]);
                        a4[t] = dot4(pw[j] & 0x0C0C0C0C, xv2[j], a4[t]);
                        a1[t] = dot4(pw[j] & 0x03030303, xv3[j], a1[t]);
                    }
                }
            }
        }
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            if (t < ntok) {
                // a4 and a16 are exact multiples of 4 and 16
                int r = a1[t] + (a4[t] >> 2) + (a16[t] >> 4);
                r = wave_sum_i32(r);
                if (lane == t) {
                    const int d = r - xsum[t];
                    if (dot) dot[(int64_t)t * M + row] = d;
                    if (y) y[(int64_t)t * M + row] = ((float)d * alpha) / xs[t];
                }
            }
        }
    }
}

template <int NT>
static hipError_t run_gemv(const uint8_t *packed, float alpha, int64_t M, int64_t K,
                           const int8_t *xq, const float *xs, const int32_t *xsum,
                           int ntok, int32_t *dot, float *y, hipStream_t st) {
    // rows per workgroup: aim for >= 4 workgroups per CU on a 256-CU part
    int rows_per_wg = 4;
    while (rows_per_wg < 64 && (M + rows_per_wg * 2 - 1) / (rows_per_wg * 2) >= 1024)
        rows_per_wg *= 2;
    const unsigned grid = (unsigned)((M + rows_per_wg - 1) / rows_per_wg);
    const size_t lds = (size_t)ntok * (size_t)K;
    hipLaunchKernelGGL(gemv_valu_kernel<NT>, dim3(grid), dim3(kGemvThreads), lds, st,
                       packed, alpha, (int)M, (int)K, xq, xs, xsum, ntok, dot, y,
                       rows_per_wg);
    return hipGetLastError();
}

hipError_t launch_gemv_valu(const uint8_t *packed, float alpha, int64_t M,
                            int64_t K, const int8_t *xq, const float *xs,
                            const int32_t *xsum, int64_t N, int32_t *dot,
                            float *y, hipStream_t st) {
    // tokens per pass: as many as fit in the LDS budget, at most 8
    int per = (int)(kLdsBytes / K);
    if (per > 8) per = 8;
    for (int64_t n0 = 0; n0 < N; n0 += per) {
        const int nt = (int)((N - n0) < per ? (N - n0) : per);
        const int8_t *xq_n = xq + n0 * K;
        int32_t *dot_n = dot ? dot + n0 * M : nullptr;
        float *y_n = y ? y + n0 * M : nullptr;
        hipError_t e;
        if (nt == 1)
            e = run_gemv<1>(packed, alpha, M, K, xq_n, xs + n0, xsum + n0, nt, dot_n, y_n, st);
        else if (nt == 2)
            e = run_gemv<2>(packed, alpha, M, K, xq_n, xs + n0, xsum + n0, nt, dot_n, y_n, st);
        else if (nt <= 4)
            e = run_gemv<4>(packed, alpha, M, K, xq_n, xs + n0, xsum + n0, nt, dot_n, y_n, st);
        else
            e = run_gemv<8>(packed, alpha, M, K, xq_n, xs + n0, xsum + n0, nt, dot_n, y_n, st);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace bitnet
