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
// lane l holds token 4*(l/16) + i for weight row l%16.
//
// Staging: the workgroup's KS K groups share each pipeline stage, which holds
// KS consecutive blocks (group g computes block g of it): every weight row's
// KS x 32 bytes and every token's KS x 128 bytes sit contiguously, so each
// 1 KB LDS-DMA instruction moves 128- or 256-byte runs of a few rows instead
// of one 32-byte block slice of 32 rows -- a quarter of the requests per
// byte (large layer at N = 16: 71.6 -> 63.1 us per layer of four launches,
// N = 7: 64.6 -> 60.5 us).  The 16-byte chunks of a row are XOR-swizzled by
// row (token) index, so sixteen rows reading the same chunk hit distinct
// banks.  One barrier per stage; the K groups' sums and the epilogue follow
// gemm_mfma_kernel.
template <int BM, int WM, int kStages, int KS>
__global__ __launch_bounds__(WM * KS * 64) void gemm16_mfma_kernel(const GemmArgs a) {
    static_assert(kStages >= 2 && (KS == 4 || KS == 8), "stages, K groups");
    constexpr int NW = WM;                 // waves per K group
    constexpr int NWT = WM * KS;           // waves of the workgroup
    constexpr int MI = BM / WM / 16;       // 16-row MFMA tiles per wave
    static_assert(MI >= 1 && BM % (16 * WM) == 0, "tile shape");
    constexpr int RB = KS * kBlockBytes;   // weight bytes of one row in a stage
    constexpr int TBY = KS * kBlock;       // token bytes of one token in a stage
    constexpr int CPR_A = RB / 16, CPR_B = TBY / 16;   // 16-byte chunks per row
    constexpr int A_BYTES = BM * RB, B_BYTES = 16 * TBY;
    constexpr int STAGE = A_BYTES + B_BYTES;
    constexpr int TA = A_BYTES / 1024, TB = B_BYTES / 1024, T = TA + TB;
    static_assert(A_BYTES % 1024 == 0 && B_BYTES % 1024 == 0, "whole 1 KB DMA instructions");
    constexpr int RPI = 1024 / RB, TPI = 1024 / TBY;   // weight rows / tokens per instruction
    constexpr int CMAX = (T + NWT - 1) / NWT, CMIN = T / NWT;
    static_assert(CMIN >= 1, "every wave issues at least one DMA per stage");
    constexpr int RED = KS > 1 ? (KS - 1) * NW * MI * 4 * 64 * 4 : 0;
    static_assert(RED <= kStages * STAGE, "partial sums reuse the staging memory");
    __shared__ __attribute__((aligned(1024))) int8_t lds[kStages * STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wt = tid >> 6, wave = wt % NW, grp = wt / NW;
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
    const int nit = (nkb + KS - 1) / KS;   // stages of KS blocks (group g computes block g)

    // slot swizzles: sixteen consecutive weight rows (tokens) reading the same
    // chunk land on distinct banks
    auto swz_a = [](int r) { return KS == 4 ? (r >> 1) & 7 : r & 15; };
    auto swz_b = [](int t) { return t & 15; };

    // DMA instructions of a stage (weight rows first, then tokens) are dealt
    // to all waves round-robin; this lane's source of each: its row (token),
    // its chunk's block within the stage (clamped to the last block of K at
    // the tail) and the chunk's offset in that block.  Rows and tokens past
    // the matrix are clamped (their results are never stored).
    const bool full = wt < T - CMIN * NWT;
    const int8_t *src[CMAX];
    int cb[CMAX], bstep[CMAX];
#pragma unroll
    for (int c = 0; c < CMAX; ++c) {
        const int j = min(wt + NWT * c, T - 1);
        if (j < TA) {
            const int row = j * RPI + lane / CPR_A;
            const int chunk = (lane % CPR_A) ^ swz_a(row);
            cb[c] = chunk >> 1;
            bstep[c] = kBlockBytes;
            src[c] = reinterpret_cast<const int8_t *>(packed) +
                     (int64_t)min(m0 + row, M - 1) * rowb + 16 * (chunk & 1);
        } else {
            const int t = (j - TA) * TPI + lane / CPR_B;
            const int chunk = (lane % CPR_B) ^ swz_b(t);
            cb[c] = chunk >> 3;
            bstep[c] = kBlock;
            src[c] = xq + (int64_t)min(n0 + t, N - 1) * K + 16 * (chunk & 7);
        }
    }
    auto issue = [&](int it2, int st) {
        const int kb0 = min(it2, nit - 1) * KS;
        const int8_t *base = lds + st * STAGE;
#pragma unroll
        for (int c = 0; c < CMAX; ++c)
            if (c < CMIN || full)
                dma16(src[c] + (int64_t)min(kb0 + cb[c], nkb - 1) * bstep[c],
                      lds_addr_of(base + 1024 * (wt + NWT * c)));
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
    const int sh0 = 6 - 2 * (g4 >> 1);   // field 2s + g4/2 sits at bit 6 - 2*field

    // kStages-1 stages in flight (past the end the last stage is fetched
    // again into a stage that is never read), so the wait is a constant
#pragma unroll
    for (int p = 0; p < kStages - 1; ++p) issue(p, p);
    for (int it = 0; it < nit; ++it) {
        wait_block();
        __syncthreads();   // the stage is in LDS; stage (it-1) is free for the next DMA
        issue(it + kStages - 1, (it + kStages - 1) % kStages);
        if (it * KS + grp >= nkb) continue;   // past the end of K for this group
        const int8_t *sa = lds + (it % kStages) * STAGE;
        const int8_t *sb = sa + A_BYTES;
        v4i wf[MI], tf[2];
#pragma unroll
        for (int mi = 0; mi < MI; ++mi) {
            const int row = (wave * MI + mi) * 16 + c16;
            wf[mi] = *reinterpret_cast<const v4i *>(sa + row * RB +
                                                    16 * ((2 * grp + (g4 & 1)) ^ swz_a(row)));
        }
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2)
            tf[s2] = *reinterpret_cast<const v4i *>(sb + c16 * TBY +
                                                    16 * ((8 * grp + 4 * s2 + g4) ^ swz_b(c16)));
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
        int *red = reinterpret_cast<int *>(lds);
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
#pragma unroll
    // lane l: weight row m = tile row + l%16, tokens 4*(l/16) + i; consecutive
    // lanes write consecutive outputs of a token row
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
    // of 64 rows, 448 of 128; 747 -> 740 us per step).  With the shared
    // stages, 128-row tiles take two stages (48 KB, so a CU holds up to three
    // workgroups) and 32-row tiles four (large layer, four launches at N = 16:
    // 63.3 -> 61.4-62.5 us; N = 7: 60.5 -> 57.3-57.7 us).
    int64_t t32r = 0, t64r = 0, t128r = 0;
    for (int i = 0; i < nmats; ++i) {
        t32r += (mats[i].M + 31) / 32;
        t64r += (mats[i].M + 63) / 64;
        t128r += (mats[i].M + 127) / 128;
    }
    if (t128r >= 256) return run_gemm16<128, 2, 2, 4>(mats, nmats, K, xq, xs, xsum, N, st);
    if (t64r >= 256) return run_gemm16<64, 2, 3, 4>(mats, nmats, K, xq, xs, xsum, N, st);
    // long reductions (the large layer's down projection, K = 28672): K
    // split over eight wave groups instead of four (877 -> 854 us per step
    // on the earlier 32-token-wide tiles); so too at K >= 8192 where the
    // 32-row tiles give each CU at most one workgroup (the large layer's o
    // projection, 256 tiles: 9.2 -> 7.9 us), so twice the blocks are in flight
    // per CU.  Not with more tiles than CUs (q/k/v, 320 tiles: 10.2 us on
    // four groups, 10.4 on eight).
    if (K >= 16384 || (K >= 8192 && t32r <= 256))
        return run_gemm16<32, 1, 4, 8>(mats, nmats, K, xq, xs, xsum, N, st);
    return run_gemm16<32, 1, 4, 4>(mats, nmats, K, xq, xs, xsum, N, st);
}

}  // namespace bitnet
