// ffn.hip -- the squared-ReLU gated FFN activation between the gate/up and
// down projections, quantised for the down projection.
//
// Pages: [P4] "bitnet.rs", "Forward Pass" (the FFN computes
// ffn_sub_norm(sqrelu(gate(x)) * up(x)) and feeds it to down); [P1]
// "BitNet 딥다이브" §4-5 (per-token absmax int8 activations).
//
// One workgroup per token, 512 threads on 16-byte pieces (four channels).
// Pass 1 forms h = (relu(g)^2) * u in fp32, keeps it in LDS and finds max|h|.
// The sub-norm's sum of squares is the exact sum rounded once to binary64
// (exact_sum.h): every thread splits the bits of its squares that lie in a
// 112-bit window below the largest square into three exact binary64 bin sums
// (straight-line FP64 code) and counts the squares with bits below the
// window; the waves' totals meet in LDS and wave 0 forms the 128-bit window
// integer and rounds -- or, when the count could carry into the round bit,
// the workgroup adds further windows into an exact integer first.  Each
// thread only ever touches its own pieces of h in LDS.
// c = fp32(1 / sqrt(sum / F + eps)).  Pass 2: v = (h * c) * gamma in place
// and its absmax; pass 3: the scale and the codes with the activation
// quantiser's arithmetic.
#include "common.h"
#include "exact_sum.h"

namespace bitnet {

constexpr int kFfnThreads = 512;
constexpr int kFfnWaves = kFfnThreads / 64;
constexpr int kFfnR = 4;   // 16-byte pieces per thread loaded together

struct FfnShared {
    uint64_t red[kFfnWaves][5];   // per-wave window sums (32-bit digits) + count
    double redb[kFfnWaves][3];    // per-wave level-1 bin sums (exact)
    uint32_t redc[kFfnWaves];     // per-wave count of squares below the window
    float redm[kFfnWaves];        // max|h| per wave
    float redf[kFfnWaves];        // max|v| per wave
    int redi[kFfnWaves];
    uint32_t big[kBigDigits];
    float c;                      // the sub-norm factor
    int more;                     // 1: another window level is needed
};

// Every wave's sum of (a, cnt) into sh.red (as 32-bit digits, each total
// below 2^42); the caller synchronises before reading them.
__device__ __forceinline__ void wave_window_sums(const U128 &a, uint32_t cnt, FfnShared &sh) {
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    uint64_t d[5] = {a.lo & 0xffffffffu, a.lo >> 32, a.hi & 0xffffffffu, a.hi >> 32, cnt};
#pragma unroll
    for (int i = 0; i < 5; ++i) d[i] = wave_sum_u64(d[i]);
    if (lane == 0) {
#pragma unroll
        for (int i = 0; i < 5; ++i) sh.red[wv][i] = d[i];
    }
}
// The workgroup totals from sh.red (the exact total is below 2^128).
__device__ __forceinline__ void window_totals(const FfnShared &sh, U128 *tot, uint64_t *tot_cnt) {
    uint64_t D[5] = {0, 0, 0, 0, 0};
#pragma unroll
    for (int w = 0; w < kFfnWaves; ++w)
#pragma unroll
        for (int i = 0; i < 5; ++i) D[i] += sh.red[w][i];
    U128 r{D[0], 0};
    add128(r, U128{D[1] << 32, D[1] >> 32});
    add128(r, U128{0, D[2]});
    add128(r, U128{0, D[3] << 32});
    *tot = r;
    *tot_cnt = D[4];
}

__device__ __forceinline__ double wave_sum_f64(double v) {   // exact here: integer multiples below 2^53
    uint64_t b;
    __builtin_memcpy(&b, &v, 8);
    auto add = [&](uint64_t o) {
        double x, y;
        __builtin_memcpy(&x, &b, 8);
        __builtin_memcpy(&y, &o, 8);
        x += y;
        __builtin_memcpy(&b, &x, 8);
    };
    add(dpp_u64<kDppXor1>(b));
    add(dpp_u64<kDppXor2>(b));
    add(dpp_u64<kDppHalfMirror>(b));
    add(dpp_u64<kDppMirror>(b));
    add(dpp_rows_u64<kDppRowBcast15, 0xA>(b));   // the rows a move skips add +0
    add(dpp_rows_u64<kDppRowBcast31, 0xC>(b));
    b = readlane63_u64(b);
    double r;
    __builtin_memcpy(&r, &b, 8);
    return r;
}

// Level 1 of the window on the FP64 units (exact_sum.h, window_add_f64):
// this thread's three bin sums and count.
__device__ __forceinline__ void window_pass_f64(const float4 *hl, int nq, int b, Bins3 *acc,
                                                uint32_t *cnt) {
    const double unit[3] = {pos_scale(b + 75), pos_scale(b + 37), pos_scale(b)};
    const double sigma[3] = {unit[0] * 0x1p52, unit[1] * 0x1p52, unit[2] * 0x1p52};
    Bins3 a{{0.0, 0.0, 0.0}};
    uint32_t c = 0;
    int q = threadIdx.x;
    for (; q + kFfnThreads < nq; q += 2 * kFfnThreads) {   // two pieces in flight
        const float4 h0 = hl[q], h1 = hl[q + kFfnThreads];
        window_add_f64(h0.x, unit, sigma, a, c);
        window_add_f64(h0.y, unit, sigma, a, c);
        window_add_f64(h0.z, unit, sigma, a, c);
        window_add_f64(h0.w, unit, sigma, a, c);
        window_add_f64(h1.x, unit, sigma, a, c);
        window_add_f64(h1.y, unit, sigma, a, c);
        window_add_f64(h1.z, unit, sigma, a, c);
        window_add_f64(h1.w, unit, sigma, a, c);
    }
    if (q < nq) {
        const float4 h0 = hl[q];
        window_add_f64(h0.x, unit, sigma, a, c);
        window_add_f64(h0.y, unit, sigma, a, c);
        window_add_f64(h0.z, unit, sigma, a, c);
        window_add_f64(h0.w, unit, sigma, a, c);
    }
    *acc = a;
    *cnt = c;
}

__device__ __forceinline__ float norm_factor(double ss, int F, float eps) {
    return (float)(1.0 / sqrt(ss / (double)F + (double)eps));
}

// This thread's part of window level b on the integer units: bits of its
// squares at positions >= b (below b + kWin when MASKED), and how many
// squares have bits below b (the rare further levels).
template <bool MASKED>
__device__ __forceinline__ void window_pass(const float4 *hl, int nq, int b, U128 *acc,
                                            uint32_t *cnt) {
    U128 a{0, 0};
    uint32_t c = 0;
    int q = threadIdx.x;
    for (; q + kFfnThreads < nq; q += 2 * kFfnThreads) {   // two pieces in flight
        const float4 h0 = hl[q], h1 = hl[q + kFfnThreads];
        window_add<MASKED>(h0.x, b, a, c);
        window_add<MASKED>(h0.y, b, a, c);
        window_add<MASKED>(h0.z, b, a, c);
        window_add<MASKED>(h0.w, b, a, c);
        window_add<MASKED>(h1.x, b, a, c);
        window_add<MASKED>(h1.y, b, a, c);
        window_add<MASKED>(h1.z, b, a, c);
        window_add<MASKED>(h1.w, b, a, c);
    }
    if (q < nq) {
        const float4 h0 = hl[q];
        window_add<MASKED>(h0.x, b, a, c);
        window_add<MASKED>(h0.y, b, a, c);
        window_add<MASKED>(h0.z, b, a, c);
        window_add<MASKED>(h0.w, b, a, c);
    }
    *acc = a;
    *cnt = c;
}

__global__ __launch_bounds__(kFfnThreads) void ffn_act_quant_kernel(
    const float *__restrict__ g, const float *__restrict__ u, const float *__restrict__ gamma,
    float eps, int F, int8_t *__restrict__ xq, float *__restrict__ xs,
    int32_t *__restrict__ xsum) {
    extern __shared__ float4 hl[];   // h (then v) of the token, F/4 pieces
    __shared__ FfnShared sh;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int nq = F >> 2;
    const int64_t row = (int64_t)blockIdx.x * F;
    const float4 *g4 = reinterpret_cast<const float4 *>(g + row);
    const float4 *u4 = reinterpret_cast<const float4 *>(u + row);
    const float4 *gm4 = reinterpret_cast<const float4 *>(gamma);

    // ---- pass 1: h and max|h|; the gain of the first batch loads alongside
    float4 gm0[kFfnR];
    float hmax = 0.0f;
    for (int base = 0; base < nq; base += kFfnR * kFfnThreads) {
        float4 gv[kFfnR], uv[kFfnR];
#pragma unroll
        for (int r = 0; r < kFfnR; ++r) {
            const int q = min(base + tid + r * kFfnThreads, nq - 1);
            gv[r] = g4[q];
            uv[r] = u4[q];
            if (base == 0) gm0[r] = gamma ? gm4[q] : make_float4(1.0f, 1.0f, 1.0f, 1.0f);
        }
#pragma unroll
        for (int r = 0; r < kFfnR; ++r) {
            const int q = base + tid + r * kFfnThreads;
            if (q < nq) {
                const float gg[4] = {gv[r].x, gv[r].y, gv[r].z, gv[r].w};
                const float uu[4] = {uv[r].x, uv[r].y, uv[r].z, uv[r].w};
                float h[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float rl = gg[e] > 0.0f ? gg[e] : 0.0f;
                    h[e] = (rl * rl) * uu[e];
                    hmax = fmaxf(hmax, fabsf(h[e]));
                }
                hl[q] = make_float4(h[0], h[1], h[2], h[3]);
            }
        }
    }
    hmax = wave_max_f32(hmax);
    if (lane == 0) sh.redm[wv] = hmax;
    __syncthreads();
    float hm = sh.redm[0];
#pragma unroll
    for (int w = 1; w < kFfnWaves; ++w) hm = fmaxf(hm, sh.redm[w]);

    // ---- the exactly rounded sum of h^2 -> the factor c (wave 0 rounds)
    // Both branches end on a barrier after sh.c is written (hm is the same
    // in every thread, so the branch is uniform).
    if (hm == 0.0f) {
        if (tid == 0) sh.c = norm_factor(0.0, F, eps);
        __syncthreads();
    } else {
        uint64_t vmax;
        int Pmax;
        square_parts(hm, vmax, Pmax);
        const int T = top_position(vmax, Pmax);
        U128 acc, A;
        uint32_t cnt;
        uint64_t C;
        {
            Bins3 bins;
            window_pass_f64(hl, nq, T - kWin, &bins, &cnt);
#pragma unroll
            for (int k = 0; k < 3; ++k) bins.s[k] = wave_sum_f64(bins.s[k]);
            cnt = (uint32_t)wave_sum_i32((int)cnt);
            if (lane == 0) {
#pragma unroll
                for (int k = 0; k < 3; ++k) sh.redb[wv][k] = bins.s[k];
                sh.redc[wv] = cnt;
            }
        }
        __syncthreads();
        if (wv == 0) {
            {
                double tot[3] = {0.0, 0.0, 0.0};
                C = 0;
#pragma unroll
                for (int w = 0; w < kFfnWaves; ++w) {
#pragma unroll
                    for (int k = 0; k < 3; ++k) tot[k] += sh.redb[w][k];
                    C += sh.redc[w];
                }
                A = bins_to_u128(tot, T - kWin);
            }
            double ss;
            const bool done = round_level1(A, C, T - kWin, &ss);
            if (lane == 0) {
                sh.more = done ? 0 : 1;
                if (done) {
                    sh.c = norm_factor(ss, F, eps);
                } else {
                    for (int i = 0; i < kBigDigits; ++i) sh.big[i] = 0;
                    big_shift_add(sh.big, A);
                }
            }
        }
        __syncthreads();
        // Rare: a carry into the round bit is possible.  Add the next windows
        // of every square into an exact integer until no square has bits left
        // below the window (at most five levels cover the whole range of
        // squares of fp32 values).
        for (int k = 2; k <= 8 && sh.more; ++k) {
            const int b = T - kWin * k;
            window_pass<true>(hl, nq, b, &acc, &cnt);
            wave_window_sums(acc, cnt, sh);
            __syncthreads();
            if (tid == 0) {
                window_totals(sh, &A, &C);
                big_shift_add(sh.big, A);
                if (C == 0) {
                    sh.c = norm_factor(big_round(sh.big, b), F, eps);
                    sh.more = 0;
                }
            }
            __syncthreads();
        }
    }
    const float c = sh.c;

    // ---- pass 2: v = (h * c) * gamma in place, and its absmax
    float amax = 0.0f;
    for (int q = tid, r = 0; q < nq; q += kFfnThreads, ++r) {
        const float4 gm = r < kFfnR ? gm0[r]
                        : gamma    ? gm4[q]
                                   : make_float4(1.0f, 1.0f, 1.0f, 1.0f);
        const float4 h = hl[q];
        const float4 v = make_float4((h.x * c) * gm.x, (h.y * c) * gm.y, (h.z * c) * gm.z,
                                     (h.w * c) * gm.w);
        hl[q] = v;
        amax = fmaxf(fmaxf(amax, fmaxf(fabsf(v.x), fabsf(v.y))), fmaxf(fabsf(v.z), fabsf(v.w)));
    }
    amax = wave_max_f32(amax);
    if (lane == 0) sh.redf[wv] = amax;
    __syncthreads();
    float a = sh.redf[0];
    for (int w = 1; w < kFfnWaves; ++w) a = fmaxf(a, sh.redf[w]);
    const float s = quant_scale(a);

    // ---- pass 3: codes, four per 4-byte store
    int sum = 0;
    uint32_t *q4 = reinterpret_cast<uint32_t *>(xq + row);
    for (int q = tid; q < nq; q += kFfnThreads) {
        const float4 v = hl[q];
        const uint32_t c = pack_low_bytes(quant_bits(v.x, s), quant_bits(v.y, s),
                                          quant_bits(v.z, s), quant_bits(v.w, s));
        sum = sum_codes4(c, sum);
        q4[q] = c;
    }
    sum = wave_sum_i32(sum);
    if (lane == 0) sh.redi[wv] = sum;
    __syncthreads();
    if (tid == 0) {
        int t = 0;
        for (int w = 0; w < kFfnWaves; ++w) t += sh.redi[w];
        xs[blockIdx.x] = s;
        xsum[blockIdx.x] = t;
    }
}

hipError_t launch_ffn_act_quant(const float *g, const float *u, const float *gamma, float eps,
                                int64_t N, int64_t F, int8_t *xq, float *xs, int32_t *xsum,
                                hipStream_t st) {
    const size_t lds = (size_t)F * sizeof(float);
    hipLaunchKernelGGL(ffn_act_quant_kernel, dim3((unsigned)N), dim3(kFfnThreads), lds, st, g, u,
                       gamma, eps, (int)F, xq, xs, xsum);
    return hipGetLastError();
}

}  // namespace bitnet
