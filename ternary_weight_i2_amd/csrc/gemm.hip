// gemm.hip -- multi-token (prefill) matmul on int8 MFMA (v_mfma_i32_32x32x32_i8).
//
// Pages: [P1] "BitNet 딥다이브" §4-2 (I2_S block interleave), §4-5 (a separate
// prefill path); [P2] "[분석/검증-3]" §3 and [P3] "[기술 분석 보고서]" §3.2 (raw
// codes multiply the activations; the exact result subtracts sum(x)).
//
// Tiling: a workgroup of WM x WN waves computes a BM x BN tile of the output
// (weight rows x tokens); wave (wm, wn) owns a (32*MI) x (32*NJ) sub-tile made
// of 32x32 MFMA tiles.  Up to 16 tokens take gemm16_mfma_kernel (gemm16.hip)
// on the 16x16x64 MFMA instead.
// K advances one 128-weight I2_S block at a time.  One launch may serve
// several matrices that share the tokens (tiles numbered matrix by matrix).
//
// Operand layout.  For MFMA step s of a block (32 k each, s = 0..3) lane
// (r, kg) -- r = lane%32, kg = lane/32 -- supplies 16 bytes for k = 32s + 16kg
// + 0..15 of row/token r (the A and B operands take the same lane layout).
// The token operand (A) is therefore a plain 16-byte copy of the token row;
// tokens are staged in LDS in their natural order, with an XOR swizzle of the
// 16-byte pieces inside a row so a wave's reads spread over the banks.  The
// contraction is order-free, so the weight operand (B) is built to match:
// those 16 positions are the 2-bit field s of the 16 packed bytes of half kg
// of the row's block.  One 16-byte read of the
// packed weight tile per lane per block serves all four steps (shift by 6-2s
// and mask per dword, no shuffle); the weights are never re-laid out.
//
// Pipelining: the packed weight tile (BM x 32 bytes) and the token tile
// (BN x 128 bytes) of a block move global -> LDS with the gfx950 LDS-DMA loads
// (global_load_lds_dwordx4: each lane's 16 bytes land at M0 + 16*lane; the
// 1 KB instructions are dealt to the waves round-robin), kStages-1 blocks in
// flight, so no registers carry staged data and the MFMAs of block kb overlap
// the loads of the next blocks; one barrier per block.  Accumulators hold the
// raw-code sum R; the epilogue writes D = R - sum(x) and y = D * (alpha / s),
// the factor computed once per token before the main loop (two fp32
// roundings, as D * alpha / s has; a division per output made the epilogue
// VALU-bound).
//
// K groups (KS > 1): for launches too small to fill the CUs (batched decode,
// prefill of a few hundred tokens) a workgroup holds KS groups of WM x WN
// waves that take alternate blocks of K through their own stages; the
// groups' int32 partial sums meet in LDS and group 0 writes the tile.
#include "gemm_tiles.h"

namespace bitnet {

typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));

template <int BM, int BN, int WM, int WN, int kStages, int KS>
__global__ __launch_bounds__(WM * WN * KS * 64) void gemm_mfma_kernel(const GemmArgs a) {
    static_assert(kStages >= 2, "at least double buffering");
    static_assert(KS >= 1, "K groups");
    constexpr int NW = WM * WN;        // waves per K group (one output tile)
    constexpr int MI = BM / WM / 32;   // 32-row MFMA tiles per wave
    constexpr int NJ = BN / WN / 32;   // 32-token MFMA tiles per wave
    static_assert(BN % (32 * WN) == 0, "whole 32-token MFMA tiles");
    static_assert(MI >= 1 && NJ >= 1, "tile too small");
    // LDS-DMA instructions per block (each moves 64 lanes x 16 bytes = 1 KB):
    // TA for the weight tile (BM rows x 32 bytes), TB for the token tile (BN
    // rows x 128 bytes), dealt to the waves round-robin: wave w issues
    // instructions w, w + NW, ...; CMAX or CMIN of them.
    constexpr int TA = BM / 32, TB = BN / 8, T = TA + TB;
    static_assert(BM % 32 == 0 && BN % 8 == 0, "tile shape: whole 1 KB DMA instructions");
    constexpr int CMAX = (T + NW - 1) / NW, CMIN = T / NW;
    static_assert(CMIN >= 1, "every wave issues at least one DMA per block");
    constexpr int A_BYTES = BM * kBlockBytes, B_BYTES = BN * kBlock;
    constexpr int STAGE = A_BYTES + B_BYTES;
    // KS > 1 (launches too small to fill the CUs): KS groups of NW waves
    // split K -- group g takes blocks g, g + KS, ... through its own stages --
    // and their int32 partial sums meet in LDS at the end (exact).
    constexpr int RED = KS > 1 ? (KS - 1) * NW * MI * NJ * 16 * 64 * 4 : 0;
    static_assert(RED <= KS * kStages * STAGE, "partial sums reuse the staging memory");
    __shared__ __attribute__((aligned(1024))) int8_t lds_all[KS * kStages * STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = (tid >> 6) % NW, grp = (tid >> 6) / NW;
    int8_t *const lds = lds_all + grp * (kStages * STAGE);
    const int wm = wave % WM, wn = wave / WM;
    const int r32 = lane & 31, kg = lane >> 5;
    // Tile of this workgroup.  Workgroups are dealt to the XCDs round-robin
    // (id % 8); renumbering so that each XCD gets a contiguous run of tiles,
    // M-tile fastest, makes the workgroups of one XCD share token tiles in its
    // L2 instead of every XCD fetching every token tile.
    // Tiles are numbered matrix by matrix, M-tile fastest.
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
    const float *__restrict__ xs = a.xs;
    const int32_t *__restrict__ xsum = a.xsum;
    const int local = id - a.mat[mat].tile_begin;
    const int mtiles = (M + BM - 1) / BM;
    const int m0 = (local % mtiles) * BM, n0 = (local / mtiles) * BN;
    const int64_t rowb = K >> 2;
    const int nkb = K / kBlock;
    const int nit = (nkb + KS - 1) / KS;   // iterations of every group (the last may idle)

    // Global source of this lane's 16 bytes in each of the wave's DMA
    // instructions (byte offset 1024*j of the stage; the weight tile first,
    // then the token tile).  Rows and tokens past the matrix are clamped to
    // the last valid one (their results are never stored).  Token rows are
    // swizzled by tok_swz.
    const bool full = wave < T - CMIN * NW;   // this wave issues CMAX, else CMIN
    const int8_t *src[CMAX];
    int64_t step[CMAX];                       // source advance per block
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
    // wait until this wave's DMAs of the oldest pending block have landed
    auto wait_block = [&]() {
        if (full) wait_vmcnt<CMAX * (kStages - 2)>();
        else wait_vmcnt<CMIN * (kStages - 2)>();
    };

    // Per-token epilogue inputs, loaded before the main loop so their latency
    // is hidden: sum(x) and the output factor alpha / s of each column.
    int sxv[NJ];
    float cfac[NJ];
#pragma unroll
    for (int nj = 0; nj < NJ; ++nj) {
        const int nc = min(n0 + (wn * NJ + nj) * 32 + r32, N - 1);
        sxv[nj] = xsum[nc];
        cfac[nj] = alpha / xs[nc];
    }

    v16i acc[MI][NJ];
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int nj = 0; nj < NJ; ++nj)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[mi][nj][e] = 0;

    // Always kStages-1 blocks in flight (past the end the last block is
    // re-fetched into a stage that is never read), so the wait below is a
    // constant: at most (kStages-2) newer blocks of DMA may still be pending.
#pragma unroll
    for (int p = 0; p < kStages - 1; ++p) issue(min(p * KS + grp, nkb - 1), p);
    for (int it = 0; it < nit; ++it) {
        wait_block();
        __syncthreads();   // every wave's share of this block is in LDS; stage (it-1) is free
        issue(min((it + kStages - 1) * KS + grp, nkb - 1), (it + kStages - 1) % kStages);
        if (KS > 1 && it * KS + grp >= nkb) continue;   // this group's share of K is done
        const int8_t *sa = lds + (it % kStages) * STAGE;
        const int8_t *sb = sa + A_BYTES;
        // All of the block's fragments are read from LDS up front (one LDS
        // round trip), then the 4*MI*NJ MFMAs run back to back while the next
        // step's codes are unpacked.
        v4i a[MI], bf[4][NJ];
#pragma unroll
        for (int mi = 0; mi < MI; ++mi)
            a[mi] = *reinterpret_cast<const v4i *>(sa + ((wm * MI + mi) * 32 + r32) * kBlockBytes +
                                                   16 * kg);
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int nj = 0; nj < NJ; ++nj) {
                const int row = (wn * NJ + nj) * 32 + r32;
                bf[s][nj] = *reinterpret_cast<const v4i *>(
                    sb + row * kBlock + 16 * ((2 * s + kg) ^ tok_swz(row)));
            }
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int sh = 6 - 2 * s;
            v4i af[MI];
#pragma unroll
            for (int mi = 0; mi < MI; ++mi)
                af[mi] = v4i{(a[mi].x >> sh) & 0x03030303, (a[mi].y >> sh) & 0x03030303,
                             (a[mi].z >> sh) & 0x03030303, (a[mi].w >> sh) & 0x03030303};
#pragma unroll
            for (int mi = 0; mi < MI; ++mi)
#pragma unroll
                for (int nj = 0; nj < NJ; ++nj)
                    acc[mi][nj] = __builtin_amdgcn_mfma_i32_32x32x32_i8(bf[s][nj], af[mi],
                                                                        acc[mi][nj], 0, 0, 0);
        }
    }
    wait_vmcnt<0>();   // drain the trailing re-fetches before the workgroup ends
    if constexpr (KS > 1) {
        // groups 1..KS-1 hand their sums to group 0 through LDS, register by
        // register (lane-contiguous, so no bank conflicts); group 0 adds them
        // in group order and alone runs the epilogue.
        __syncthreads();   // every group is done with its stages
        int *red = reinterpret_cast<int *>(lds_all);
        if (grp > 0) {
            int *dst = red + (((grp - 1) * NW + wave) * MI * NJ * 16) * 64 + lane;
#pragma unroll
            for (int mi = 0; mi < MI; ++mi)
#pragma unroll
                for (int nj = 0; nj < NJ; ++nj)
#pragma unroll
                    for (int e = 0; e < 16; ++e) dst[((mi * NJ + nj) * 16 + e) * 64] = acc[mi][nj][e];
        }
        __syncthreads();
        if (grp > 0) return;
        for (int g = 1; g < KS; ++g) {
            const int *srcp = red + (((g - 1) * NW + wave) * MI * NJ * 16) * 64 + lane;
#pragma unroll
            for (int mi = 0; mi < MI; ++mi)
#pragma unroll
                for (int nj = 0; nj < NJ; ++nj)
#pragma unroll
                    for (int e = 0; e < 16; ++e) acc[mi][nj][e] += srcp[((mi * NJ + nj) * 16 + e) * 64];
        }
    }

    // Result layout (tokens are the MFMA's A operand): lane l, register 4q + j
    // holds token 8q + 4*(l/32) + j of the fragment and weight row l%32.
    // Single-group tiles (the large prefill launches) turn each 32x32
    // fragment around in LDS (the stages are free once the K loop is done):
    // the wave writes its raw sums as [token][row] and reads them back as 16
    // bytes per lane, four rows of one token, so each store instruction
    // writes eight whole 128-byte token-row segments with a quarter of the
    // instructions of the per-dword stores below (0.6B-class layer at
    // N = 4096, y only: 104 -> 96 us).  Lane t (t < 32) holds token t's
    // sum(x) and factor; the others get them by lane shuffle.
    if constexpr (KS == 1) {
        __syncthreads();   // every wave is past its last fragment read of the stages
        constexpr int LROW = 36;   // ints per staged token row (padded)
        int *const stg = reinterpret_cast<int *>(lds_all) + wave * 32 * LROW;
        static_assert(NW * 32 * LROW * 4 <= kStages * STAGE, "epilogue staging fits the stages");
        const int tl = lane >> 3, rl = 4 * (lane & 7);   // read-back: tokens tl + 8p, rows rl..rl+3
        const bool vec = (M & 3) == 0;                   // 16-byte aligned output rows
#pragma unroll
        for (int nj = 0; nj < NJ; ++nj) {
            const int nb = n0 + (wn * NJ + nj) * 32;
            int sx[4];
            float c[4];
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                sx[p] = __shfl(sxv[nj], tl + 8 * p);
                c[p] = __shfl(cfac[nj], tl + 8 * p);
            }
#pragma unroll
            for (int mi = 0; mi < MI; ++mi) {
                const int m = m0 + (wm * MI + mi) * 32 + rl;
#pragma unroll
                for (int q = 0; q < 4; ++q)
#pragma unroll
                    for (int j = 0; j < 4; ++j) stg[(8 * q + 4 * kg + j) * LROW + r32] = acc[mi][nj][4 * q + j];
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    const int n = nb + tl + 8 * p;
                    const v4i r = *reinterpret_cast<const v4i *>(stg + (tl + 8 * p) * LROW + rl);
                    const v4i d = v4i{r.x - sx[p], r.y - sx[p], r.z - sx[p], r.w - sx[p]};
                    const int64_t o = (int64_t)n * M + m;
                    if (vec && n < N && m < M) {   // M % 4 == 0: all four rows exist
                        if (dot) *reinterpret_cast<v4i *>(dot + o) = d;
                        if (y) *reinterpret_cast<v4f *>(y + o) =
                            v4f{(float)d.x * c[p], (float)d.y * c[p], (float)d.z * c[p], (float)d.w * c[p]};
                    } else if (n < N) {
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            if (m + e < M) {
                                if (dot) dot[o + e] = d[e];
                                if (y) y[o + e] = (float)d[e] * c[p];
                            }
                        }
                    }
                }
            }
        }
        return;
    }
    // K groups: each dword store writes 32 consecutive outputs of two token
    // rows -- two whole 128-byte segments.  (Weights as the A operand put four
    // rows of one token in a lane: 16-byte stores, but each instruction
    // touching 32 token rows 32 bytes at a time; with y and D written that
    // took 188 against 154 us on the 0.6B-class layer at N = 4096.)
#pragma unroll
    for (int nj = 0; nj < NJ; ++nj) {
        const int nb = n0 + (wn * NJ + nj) * 32;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            int sx[4];
            float c[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                sx[j] = __shfl(sxv[nj], 8 * q + 4 * kg + j);
                c[j] = __shfl(cfac[nj], 8 * q + 4 * kg + j);
            }
#pragma unroll
            for (int mi = 0; mi < MI; ++mi) {
                const int m = m0 + (wm * MI + mi) * 32 + r32;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int n = nb + 8 * q + 4 * kg + j;
                    if (m < M && n < N) {
                        const int d = acc[mi][nj][4 * q + j] - sx[j];
                        const int64_t o = (int64_t)n * M + m;
                        if (dot) dot[o] = d;
                        if (y) y[o] = (float)d * c[j];
                    }
                }
            }
        }
    }
}

template <int BM, int BN, int WM, int WN, int S, int KS = 1>
static hipError_t run_gemm(const GemmMat *mats, int nmats, int64_t K, const int8_t *xq,
                           const float *xs, const int32_t *xsum, int64_t N, hipStream_t st) {
    GemmArgs a{};
    const int64_t ntiles = (N + BN - 1) / BN;
    int64_t tiles = 0;
    int n = 0;
    for (int i = 0; i < nmats; ++i) {
        if (mats[i].M <= 0) continue;
        a.mat[n] = mats[i];
        a.mat[n].tile_begin = (int)tiles;
        tiles += ((mats[i].M + BM - 1) / BM) * ntiles;
        ++n;
    }
    if (n == 0) return hipSuccess;
    if (tiles > 0x7fffffffLL) return hipErrorInvalidValue;   // tile ids are int
    a.nmats = n;
    a.K = (int)K;
    a.N = (int)N;
    a.xq = xq;
    a.xs = xs;
    a.xsum = xsum;
    hipLaunchKernelGGL((gemm_mfma_kernel<BM, BN, WM, WN, S, KS>), dim3((unsigned)tiles),
                       dim3(WM * WN * KS * 64), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_gemm_mfma(const GemmMat *mats, int nmats, int64_t K, const int8_t *xq,
                            const float *xs, const int32_t *xsum, int64_t N, hipStream_t st) {
    // Batched decode token counts (17..64): small row tiles, so that a launch
    // over a 2B-class layer's matrices spreads over the CUs, and K split over
    // 4 (32x32 tiles) or 2 (64x64) wave groups inside the workgroup.  Such
    // launches hold one workgroup per CU, whose waves otherwise spend each
    // block waiting on one barrier / LDS read / MFMA chain; more stages or a
    // second accumulator did not help.  Against 128-row tiles without the
    // split: 20-35% less time per 2B-class step at N = 32..64.
    // Above 32 tokens a launch with fewer than 128 tiles of 64x64 (at most
    // half the CUs busy) still takes the 32x32 tiles, four times the
    // workgroups (2B-class layer at N = 64: o 8.3 -> 7.2, down 14.8 -> 9.7 us;
    // 0.6B-class o and down at N = 128: 8.3 -> 7.5 and 9.3 -> 7.4 us); with a
    // threshold of 256 the gate/up launches (192-216 tiles) went 9.5 -> 14.0
    // and 8.2 -> 9.4 us.
    // Up to 16 tokens: 16-token tiles on the 16x16x64 MFMA (gemm16.hip).
    if (N <= 16) return launch_gemm16(mats, nmats, K, xq, xs, xsum, N, st);
    if (N <= 32) return run_gemm<32, 32, 1, 1, 3, 4>(mats, nmats, K, xq, xs, xsum, N, st);
    int64_t t64 = 0;
    for (int i = 0; i < nmats; ++i) t64 += (mats[i].M + 63) / 64;
    if (t64 * ((N + 63) / 64) < 128)
        return run_gemm<32, 32, 1, 1, 3, 4>(mats, nmats, K, xq, xs, xsum, N, st);
    if (N <= 64) return run_gemm<64, 64, 2, 2, 3, 2>(mats, nmats, K, xq, xs, xsum, N, st);
    // A launch with fewer 128x128 tiles than CUs (prefill of a few hundred
    // tokens) takes the batched-decode tiles: 64x64 with K split in two, four
    // times the workgroups and twice the waves per tile (the 0.6B-class layer
    // at N = 128: 51.9 -> 31.2 us; 128x128 tiles with the split: 50.4 us).
    int64_t t128 = 0;
    for (int i = 0; i < nmats; ++i) t128 += (mats[i].M + 127) / 128;
    if (t128 * ((N + 127) / 128) < 256)
        return run_gemm<64, 64, 2, 2, 3, 2>(mats, nmats, K, xq, xs, xsum, N, st);
    // 256x128 tiles of eight waves (64x64 each; 24 KB staged per block for
    // 128 MFMAs) when a launch has at least two per CU (the grouped q/k/v and
    // gate/up launches of a layer at N = 4096); 256x64, 128x128 and 256x256
    // measured slower there.  Otherwise 128x64 tiles of four waves: twice the
    // workgroups of 128x128, so a CU holds two and one's epilogue stores and
    // barrier waits overlap the other's K loop (0.6B-class o and down at
    // N = 4096: 19.0 -> 17.5 and 25.3 -> 23.0 us; q/k/v and gate/up at
    // N = 1024: 14.5 -> 12.3 and 17.5 -> 15.2 us).
    int64_t big = 0;
    for (int i = 0; i < nmats; ++i) big += (mats[i].M + 255) / 256;
    big *= (N + 127) / 128;
    if (big >= 512) return run_gemm<256, 128, 4, 2, 3>(mats, nmats, K, xq, xs, xsum, N, st);
    return run_gemm<128, 64, 2, 2, 4>(mats, nmats, K, xq, xs, xsum, N, st);
}

}  // namespace bitnet
