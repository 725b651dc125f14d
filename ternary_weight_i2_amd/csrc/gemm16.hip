// gemm16.hip -- the prefill matmul's path for 1..16 tokens (batched decode
// on the large layer) on int8 MFMA v_mfma_i32_16x16x64_i8.
//
// Pages: [P1] "BitNet 딥다이브" §4-2 (I2_S block interleave); [P2]
// "[분석/검증-3]" §3 and [P3] "[기술 분석 보고서]" §3.2 (raw codes multiply the
// activations; the exact result subtracts sum(x)).
#include "gemm_tiles.h"

namespace bitnet {

// Up to 16 tokens (batched decode at K >= 8192): 16-token tiles on
// v_mfma_i32_16x16x64_i8, so no MFMA work is computed and thrown away.  The
// tokens are the A operand: for step s (64 k each, s = 0, 1) lane l supplies
// token l%16 at k = 64s + 16*(l/16) + 0..15, a plain 16-byte copy of the
// staged token row.  The weights are the B operand: lane l takes weight row
// l%16 of the tile, whose 16 bytes for those k are half (l/16)&1 of the row's
// 32-byte block slice, field 2s + (l/16)/2 -- one 16-byte LDS read per block
// serves both steps (shift and mask per dword).  The result register i of
// lane l holds token 4*(l/16) + i for weight row l%16.  Staging (LDS-DMA, one
// barrier per block), K groups and the epilogue follow gemm_mfma_kernel.
template <int BM, int WM, int kStages, int KS>
__global__ __launch_bounds__(WM * KS * 64) void gemm16_mfma_kernel(const GemmArgs a) {
    static_assert(kStages >= 2 && KS >= 1, "stages, K groups");
    constexpr int NW = WM;             // waves per K group
    constexpr int MI = BM / WM / 16;   // 16-row MFMA tiles per wave
    static_assert(MI >= 1 && BM % (16 * WM) == 0, "tile shape");
    constexpr int TA = BM / 32, TB = 2, T = TA + TB;   // 1 KB DMA instructions per block
    static_assert(BM % 32 == 0, "whole 1 KB DMA instructions");
    constexpr int CMAX = (T + NW - 1) / NW, CMIN = T / NW;
    static_assert(CMIN >= 1, "every wave issues at least one DMA per block");
    constexpr int A_BYTES = BM * kBlockBytes, B_BYTES = 16 * kBlock;
    constexpr int STAGE = A_BYTES + B_BYTES;
    constexpr int RED = KS > 1 ? (KS - 1) * NW * MI * 4 * 64 * 4 : 0;
    static_assert(RED <= KS * kStages * STAGE, "partial sums reuse the staging memory");
    __shared__ __attribute__((aligned(1024))) int8_t lds_all[KS * kStages * STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = (tid >> 6) % NW, grp = (tid >> 6) / NW;
    int8_t *const lds = lds_all + grp * (kStages * STAGE);
    const int c16 = lane & 15, g4 = lane >> 4;
    const int total = (int)gridDim.x;
    int id = (int)blockIdx.x;
#if BITNET_GEMM_XCD_REMAP
    if (total % kXcds == 0) id = (id % kXcds) * (total / kXcds) + id / kXcds;
#endif
    int mat = 0;
#pragma unroll
    for (int i = 1; i < kMaxMats; ++i)
        if (i < a.nmats && id >= a.mat[i].tile_begin) mat = i;
    const uint8_t *__restrict__ packed = a.mat[mat].packed;
    int32_t *__restrict__ dot = a.mat[mat].dot;
    float *__restrict__ y = a.mat[mat].y;
    const float alpha = a.mat[mat].alpha;
    const int M = a.mat[mat].M, K = a.K, N = a.N;
    const int8_t *__restrict__ xq = a.xq;
    const int local = id - a.mat[mat].tile_begin;
    const int mtiles = (M + BM - 1) / BM;
    const int m0 = (local % mtiles) * BM, n0 = (local / mtiles) * 16;
    const int64_t rowb = K >> 2;
    const int nkb = K / kBlock;
    const int nit = (nkb + KS - 1) / KS;

    // DMA sources, as gemm_mfma_kernel (rows and tokens past the end clamped)
    const bool full = wave < T - CMIN * NW;
    const int8_t *src[CMAX];
    int64_t step[CMAX];
#pragma unroll
    for (int c = 0; c < CMAX; ++c) {
        const int j = min(wave + NW * c, T - 1);
        if (j < TA) {
            const int row = 32 * j + (lane >> 1);
            src[c] = reinterpret_cast<const int8_t *>(packed) +
                     (int64_t)min(m0 + row, M - 1) * rowb + 16 * (lane & 1);
            step[c] = kBlockBytes;
        } else {
            const int row = 8 * (j - TA) + (lane >> 3);
            const int piece = (lane & 7) ^ tok_swz(row);
            src[c] = xq + (int64_t)min(n0 + row, N - 1) * K + 16 * piece;
            step[c] = kBlock;
        }
    }
    auto issue = [&](int kb, int st) {
        const int8_t *base = lds + st * STAGE;
#pragma unroll
        for (int c = 0; c < CMAX; ++c)
            if (c < CMIN || full)
                dma16(src[c] + (int64_t)kb * step[c], lds_addr_of(base + 1024 * (wave + NW * c)));
    };
    auto wait_block = [&]() {
        if (full) wait_vmcnt<CMAX * (kStages - 2)>();
        else wait_vmcnt<CMIN * (kStages - 2)>();
    };

    // this lane's four tokens: sum(x) and alpha / s, loaded before the loop
    int sx[4];
    float cf[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int nc = min(n0 + 4 * g4 + i, N - 1);
        sx[i] = a.xsum[nc];
        cf[i] = alpha / a.xs[nc];
    }
    v4i acc[MI];
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) acc[mi] = v4i{0, 0, 0, 0};
    const int tsw = tok_swz(c16);
    const int sh0 = 6 - 2 * (g4 >> 1);   // field 2s + g4/2 sits at bit 6 - 2*field

#pragma unroll
    for (int p = 0; p < kStages - 1; ++p) issue(min(p * KS + grp, nkb - 1), p);
    for (int it = 0; it < nit; ++it) {
        wait_block();
        __syncthreads();
        issue(min((it + kStages - 1) * KS + grp, nkb - 1), (it + kStages - 1) % kStages);
        if (KS > 1 && it * KS + grp >= nkb) continue;
        const int8_t *sa = lds + (it % kStages) * STAGE;
        const int8_t *sb = sa + A_BYTES;
        v4i wf[MI], tf[2];
#pragma unroll
        for (int mi = 0; mi < MI; ++mi)
            wf[mi] = *reinterpret_cast<const v4i *>(sa + ((wave * MI + mi) * 16 + c16) * kBlockBytes +
                                                    16 * (g4 & 1));
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2)
            tf[s2] = *reinterpret_cast<const v4i *>(sb + c16 * kBlock + 16 * ((4 * s2 + g4) ^ tsw));
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
            const int sh = sh0 - 4 * s2;
#pragma unroll
            for (int mi = 0; mi < MI; ++mi) {
                const v4i bf = v4i{(wf[mi].x >> sh) & 0x03030303, (wf[mi].y >> sh) & 0x03030303,
                                   (wf[mi].z >> sh) & 0x03030303, (wf[mi].w >> sh) & 0x03030303};
                acc[mi] = __builtin_amdgcn_mfma_i32_16x16x64_i8(tf[s2], bf, acc[mi], 0, 0, 0);
            }
        }
    }
    wait_vmcnt<0>();   // drain the trailing re-fetches before the workgroup ends
    if constexpr (KS > 1) {
        __syncthreads();
        int *red = reinterpret_cast<int *>(lds_all);
        if (grp > 0) {
            int *dst = red + (((grp - 1) * NW + wave) * MI * 4) * 64 + lane;
#pragma unroll
            for (int mi = 0; mi < MI; ++mi)
#pragma unroll
                for (int e = 0; e < 4; ++e) dst[(mi * 4 + e) * 64] = acc[mi][e];
        }
        __syncthreads();
        if (grp > 0) return;
        for (int gk = 1; gk < KS; ++gk) {
            const int *srcp = red + (((gk - 1) * NW + wave) * MI * 4) * 64 + lane;
#pragma unroll
            for (int mi = 0; mi < MI; ++mi)
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[mi][e] += srcp[(mi * 4 + e) * 64];
        }
    }
    // lane l: weight row m = tile row + l%16, tokens 4*(l/16) + i; consecutive
    // lanes write consecutive outputs of a token row
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
        const int m = m0 + (wave * MI + mi) * 16 + c16;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int n = n0 + 4 * g4 + i;
            if (m < M && n < N) {
                const int d = acc[mi][i] - sx[i];
                const int64_t o = (int64_t)n * M + m;
                if (dot) dot[o] = d;
                if (y) y[o] = (float)d * cf[i];
            }
        }
    }
}

template <int BM, int WM, int S, int KS>
static hipError_t run_gemm16(const GemmMat *mats, int nmats, int64_t K, const int8_t *xq,
                             const float *xs, const int32_t *xsum, int64_t N, hipStream_t st) {
    GemmArgs a{};
    int64_t tiles = 0;
    int n = 0;
    for (int i = 0; i < nmats; ++i) {
        if (mats[i].M <= 0) continue;
        a.mat[n] = mats[i];
        a.mat[n].tile_begin = (int)tiles;
        tiles += (mats[i].M + BM - 1) / BM;   // one 16-token tile (N <= 16)
        ++n;
    }
    if (n == 0) return hipSuccess;
    a.nmats = n;
    a.K = (int)K;
    a.N = (int)N;
    a.xq = xq;
    a.xs = xs;
    a.xsum = xsum;
    hipLaunchKernelGGL((gemm16_mfma_kernel<BM, WM, S, KS>), dim3((unsigned)tiles),
                       dim3(WM * KS * 64), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_gemm16(const GemmMat *mats, int nmats, int64_t K, const int8_t *xq,
                         const float *xs, const int32_t *xsum, int64_t N, hipStream_t st) {
    // 16-token tiles, so each block stages 2 KB of tokens instead of 4 KB for
    // a 32-token tile of which half is padding (large layer at N = 16: 987 us
    // per step on 32x32 tiles, 892 on 64x16 with the 32x32 MFMA's second half
    // discarded, 747 on the 16x16x64 MFMA).  The tallest row tile (128, 64,
    // else 32 rows) that still gives every CU a workgroup: 128-row tiles halve
    // the token staging per weight byte (gate/up at K = 8192: 896 workgroups
    // of 64 rows, 448 of 128; 747 -> 740 us per step).
    int64_t t32r = 0, t64r = 0, t128r = 0;
    for (int i = 0; i < nmats; ++i) {
        t32r += (mats[i].M + 31) / 32;
        t64r += (mats[i].M + 63) / 64;
        t128r += (mats[i].M + 127) / 128;
    }
    if (t128r >= 256) return run_gemm16<128, 2, 3, 4>(mats, nmats, K, xq, xs, xsum, N, st);
    if (t64r >= 256) return run_gemm16<64, 2, 3, 4>(mats, nmats, K, xq, xs, xsum, N, st);
    // long reductions (the large layer's down projection, K = 28672): K
    // split over eight wave groups instead of four (877 -> 854 us per step
    // on the earlier 32-token-wide tiles); so too at K >= 8192 where the
    // 32-row tiles give each CU at most one workgroup (the large layer's o
    // projection, 256 tiles: 9.2 -> 7.9 us), so twice the blocks are in flight
    // per CU.  Not with more tiles than CUs (q/k/v, 320 tiles: 10.2 us on
    // four groups, 10.4 on eight), and no further gain from more stages
    // (o: 8.1-8.6 us with five or six).
    if (K >= 16384 || (K >= 8192 && t32r <= 256))
        return run_gemm16<32, 1, 3, 8>(mats, nmats, K, xq, xs, xsum, N, st);
    return run_gemm16<32, 1, 3, 4>(mats, nmats, K, xq, xs, xsum, N, st);
}

}  // namespace bitnet
