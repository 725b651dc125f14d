// gemv_mfma.hip -- batched decode matmul (up to 64 tokens) on int8 MFMA.
//
// Pages: [P1] "BitNet 딥다이브" §2-1 (decode is bound by reading the weights),
// §4-3 (a weight block is loaded once and reused for several activation
// columns); [P2] "[분석/검증-3]" §3 and [P3] "[기술 분석 보고서]" §3.2 (raw codes
// multiply the activations; the exact result subtracts sum(x)).
//
// At 3..16 tokens every packed byte feeds 24..128 int8 operations, more than
// the vector ALUs sustain at HBM speed, so the contraction runs on
// v_mfma_i32_16x16x64_i8 while the weights still stream from HBM once.
// Larger batches (to 64) go to the prefill GEMM with small tiles (below).
//
// Work split: a workgroup owns BM = 16*MI rows of one matrix and all N
// tokens (NJ 16-token tiles) over the full K, which its WAVES waves split
// into contiguous ranges of block pairs.  One launch serves up to kMaxMats matrices
// that share K and the tokens (q/k/v, gate/up): workgroups
// [tile_begin, next tile_begin) belong to matrix i.  Partial sums meet in LDS through exact integer adds (ds_add), so
// no second pass and no global scratch is needed; the epilogue then writes
// D = R - sum(x) and y = D * alpha / s.
//
// Operand layout: K advances a pair of 128-weight blocks at a time.  Lane
// (j, kq) loads the 16-byte half kq%2 of block kq/2 of the pair for weight
// row j, so the four lanes of a row read the pair's 64 contiguous packed
// bytes in one instruction, and MFMA step s (s = 0..3) takes the 2-bit field
// s of those bytes: positions 128*(kq/2) + 32s + 16*(kq%2) + 0..15 of the
// pair (the contraction is order-free).  The B operand (tokens) is built to
// match: the same 16 positions of token j, one 16-byte load straight from
// global memory (the int8 tokens are small and stay in L2).  One shift and
// one mask per dword extract a field.  Each wave double-buffers its pairs:
// the next pair's A and B loads are in flight while the current one is used.
#include "common.h"

namespace bitnet {

constexpr int kDecodeMaxN = 16;   // larger batches go to the small-tile GEMM
constexpr int64_t kDecodeGemmMinK = 8192;   // so do long reductions
constexpr int kCus = 256;         // MI355X compute units
constexpr int kWaveSlots = 32;    // waves resident per CU (8 per SIMD)

template <int MI, int NJ, int WAVES>
__global__ __launch_bounds__(WAVES * 64) void gemv_mfma_kernel(const GemmArgs a) {
    constexpr int BM = 16 * MI, BN = 16 * NJ;
    constexpr int LDA = BN + 4;   // padded LDS row (ints): conflict-free ds_add
    constexpr int NT = WAVES * 64;
    __shared__ int acc_lds[BM * LDA];

    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int li = lane & 15, kq = lane >> 4;
    int mat = 0;
#pragma unroll
    for (int i = 1; i < kMaxMats; ++i)
        if (i < a.nmats && (int)blockIdx.x >= a.mat[i].tile_begin) mat = i;
    const uint8_t *__restrict__ packed = a.mat[mat].packed;
    int32_t *__restrict__ dot = a.mat[mat].dot;
    float *__restrict__ y = a.mat[mat].y;
    const float alpha = a.mat[mat].alpha;
    const int M = a.mat[mat].M, K = a.K, N = a.N;
    const int8_t *__restrict__ xq = a.xq;
    const float *__restrict__ xs = a.xs;
    const int32_t *__restrict__ xsum = a.xsum;
    const int m0 = ((int)blockIdx.x - a.mat[mat].tile_begin) * BM;
    for (int i = tid; i < BM * LDA; i += NT) acc_lds[i] = 0;

    // The epilogue's per-token inputs (sum(x) and 1/s operands) for the E
    // outputs this thread writes, loaded before the K loop so their latency is
    // hidden instead of following the reduction.
    constexpr int E = (BM * BN + NT - 1) / NT;
    int sxe[E];
    float sse[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const int i = tid + e * NT;
        const int n = i / BM;
        const int nn = (i < BM * BN && n < N) ? n : 0;
        sxe[e] = xsum[nn];
        sse[e] = xs[nn];
    }

    // K advances two 128-weight blocks (a pair) at a time, the waves taking
    // contiguous ranges of pairs
    const int nblk = K >> 7;
    const int npair = (nblk + 1) >> 1;
    const int p0 = (int)((int64_t)npair * wv / WAVES);
    const int p1 = (int)((int64_t)npair * (wv + 1) / WAVES);
    const int64_t rowb = K >> 2;
    const int hb = kq >> 1;   // this lane's block of the pair

    const uint8_t *prow[MI];
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
        const int m = m0 + mi * 16 + li;
        prow[mi] = packed + (int64_t)(m < M ? m : 0) * rowb + (kq & 1) * 16;
    }
    const int8_t *xrow[NJ];
#pragma unroll
    for (int nj = 0; nj < NJ; ++nj) {
        const int n = nj * 16 + li;
        xrow[nj] = xq + (int64_t)(n < N ? n : 0) * K + (kq & 1) * 16;
    }

    v4i acc[MI][NJ];
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int nj = 0; nj < NJ; ++nj) acc[mi][nj] = v4i{0, 0, 0, 0};

    // Lane (j, kq) loads the 16-byte half kq%2 of block 2p + kq/2 of its row
    // -- the four lanes of a row read its pair's 64 contiguous bytes, one
    // request per two blocks instead of a 32-byte slice per block read twice
    // -- and its MFMA step s (64 k) takes field s of those bytes, i.e. the
    // 16 positions 128*(2p + kq/2) + 32s + 16*(kq%2) + 0..15; the token
    // operand is those 16 bytes of token j, read straight from L2.  Rows past
    // M and tokens past N load row 0 / token 0 (valid addresses) and are not
    // zeroed: a row or token only feeds its own output row or column, which is
    // never stored.  The second block of an odd tail pair is clamped to the
    // last block and its codes masked to 0.
    auto load = [&](int p, v4i *A, v4i (*B)[NJ]) {
        const int64_t b = min(2 * p + hb, nblk - 1);
#pragma unroll
        for (int mi = 0; mi < MI; ++mi)
            A[mi] = __builtin_nontemporal_load(reinterpret_cast<const v4i *>(prow[mi] + b * 32));
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int nj = 0; nj < NJ; ++nj)
                B[s][nj] = *reinterpret_cast<const v4i *>(xrow[nj] + b * 128 + s * 32);
    };
    auto compute = [&](int p, const v4i *A, v4i (*B)[NJ]) {
        const int msk = 2 * p + hb < nblk ? 0x03030303 : 0;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int sh = 6 - 2 * s;
#pragma unroll
            for (int mi = 0; mi < MI; ++mi) {
                const v4i a = v4i{(A[mi].x >> sh) & msk, (A[mi].y >> sh) & msk,
                                  (A[mi].z >> sh) & msk, (A[mi].w >> sh) & msk};
#pragma unroll
                for (int nj = 0; nj < NJ; ++nj)
                    acc[mi][nj] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, B[s][nj], acc[mi][nj],
                                                                        0, 0, 0);
            }
        }
    };

    v4i A0[MI], A1[MI];
    v4i B0[4][NJ], B1[4][NJ];
    if (p0 < p1) load(p0, A0, B0);
    for (int p = p0; p < p1; p += 2) {
        if (p + 1 < p1) load(p + 1, A1, B1);
        compute(p, A0, B0);
        if (p + 1 >= p1) break;
        if (p + 2 < p1) load(p + 2, A0, B0);
        compute(p + 1, A1, B1);
    }

    __syncthreads();   // acc_lds zeroed by every thread before any add
    // 16x16 result layout: lane l, register r holds row 4*(l/16)+r, column l%16
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int nj = 0; nj < NJ; ++nj)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                atomicAdd(&acc_lds[(mi * 16 + 4 * kq + r) * LDA + nj * 16 + li], acc[mi][nj][r]);
    __syncthreads();
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const int i = tid + e * NT;
        const int n = i / BM, ml = i - n * BM;
        const int m = m0 + ml;
        if (i < BM * BN && n < N && m < M) {
            const int d = acc_lds[ml * LDA + n] - sxe[e];
            if (dot) dot[(int64_t)n * M + m] = d;
            if (y) y[(int64_t)n * M + m] = ((float)d * alpha) / sse[e];
        }
    }
}

template <int MI, int NJ, int WAVES>
static hipError_t run(const GemmMat *mats, int nmats, int64_t K, const int8_t *xq,
                      const float *xs, const int32_t *xsum, int64_t N, hipStream_t st) {
    GemmArgs a{};
    int64_t tiles = 0;
    int n = 0;
    for (int i = 0; i < nmats; ++i) {
        if (mats[i].M <= 0) continue;
        a.mat[n] = mats[i];
        a.mat[n].tile_begin = (int)tiles;
        tiles += (mats[i].M + 16 * MI - 1) / (16 * MI);
        ++n;
    }
    if (n == 0) return hipSuccess;
    if (tiles > 0x7fffffffLL) return hipErrorInvalidValue;
    a.nmats = n;
    a.K = (int)K;
    a.N = (int)N;
    a.xq = xq;
    a.xs = xs;
    a.xsum = xsum;
    hipLaunchKernelGGL((gemv_mfma_kernel<MI, NJ, WAVES>), dim3((unsigned)tiles), dim3(WAVES * 64),
                       0, st, a);
    return hipGetLastError();
}

template <int MI, int NJ>
static hipError_t run_w(int waves, const GemmMat *mats, int nmats, int64_t K, const int8_t *xq,
                        const float *xs, const int32_t *xsum, int64_t N, hipStream_t st) {
    // 16 waves (1024 threads) cap a wave at 128 VGPRs: only for small tiles
    if constexpr (MI * NJ <= 2)
        if (waves >= 16) return run<MI, NJ, 16>(mats, nmats, K, xq, xs, xsum, N, st);
    if (waves == 10) return run<MI, NJ, 10>(mats, nmats, K, xq, xs, xsum, N, st);
    if (waves >= 8) return run<MI, NJ, 8>(mats, nmats, K, xq, xs, xsum, N, st);
    return run<MI, NJ, 4>(mats, nmats, K, xq, xs, xsum, N, st);
}

template <int NJ>
static hipError_t run_nj(const GemmMat *mats, int nmats, int64_t K, const int8_t *xq,
                         const float *xs, const int32_t *xsum, int64_t N, hipStream_t st) {
    // waves split K: about one or more pairs of 128-weight blocks per wave.
    // 17..20 blocks (K = 2560) take ten waves, at most one pair each, so no
    // wave needs a second round trip to memory while the others wait for it
    // at the reduction (measured with one block per step: 2-3% less time per
    // 2B-class step than eight waves).
    const int64_t nblk = K / 128;
    const int waves = nblk >= 32 ? 16 : (nblk > 16 && nblk <= 20) ? 10 : (nblk >= 16 ? 8 : 4);
    // rows per workgroup: 16 (most workgroups in flight at once), or 32 --
    // each token tile reused twice -- when the matrices are all large or when
    // 16-row workgroups would not all be resident at once (the grouped
    // gate/up launch of a 2B-class layer: 864 ten-wave workgroups against
    // 3 per CU; 32 rows: 3-6% less time per step)
    int64_t min_m = INT64_MAX, tiles16 = 0;
    for (int i = 0; i < nmats; ++i)
        if (mats[i].M > 0) {
            if (mats[i].M < min_m) min_m = mats[i].M;
            tiles16 += (mats[i].M + 15) / 16;
        }
    const int64_t resident = (int64_t)kCus * (kWaveSlots / waves);
    if constexpr (NJ <= 2)
        if ((min_m >= 8192 && min_m != INT64_MAX) || tiles16 > resident)
            return run_w<2, NJ>(waves, mats, nmats, K, xq, xs, xsum, N, st);
    return run_w<1, NJ>(waves, mats, nmats, K, xq, xs, xsum, N, st);
}

hipError_t launch_gemv_mfma(const GemmMat *mats, int nmats, int64_t K, const int8_t *xq,
                            const float *xs, const int32_t *xsum, int64_t N, hipStream_t st) {
    // Above kDecodeMaxN tokens this kernel's per-lane token loads (every
    // 16-row workgroup re-reads all tokens through L1) cost more than the
    // small-tile, K-split GEMM's LDS-staged token tiles: on a 2B-class layer
    // the GEMM takes 16% / 22% / 37% less time per step at N = 24 / 32 / 64,
    // while at N = 16 this kernel is 5% faster.
    //
    // At K >= kDecodeGemmMinK (the large-layer shapes, 8192 and 28672) the
    // GEMM is faster at every token count: each of this kernel's 32-row
    // workgroups re-reads all tokens (2 x the weight bytes at N = 16), the
    // GEMM's tiles stage them once; three large layers, N = 3 / 4 / 8 / 16:
    // 320 / 328 / 354 / 407 us -> 295 / 296 / 298 / 305 us.  At K = 6912
    // (the 2B-class down projection, 2560 rows) it is 10-15% slower.
    if (N > kDecodeMaxN || K >= kDecodeGemmMinK)
        return launch_gemm_mfma(mats, nmats, K, xq, xs, xsum, N, st);
    return run_nj<1>(mats, nmats, K, xq, xs, xsum, N, st);
}

}  // namespace bitnet
