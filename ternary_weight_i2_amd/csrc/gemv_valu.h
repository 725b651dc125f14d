// gemv_valu.h -- decode matmul (one or two tokens per pass) on the vector
// ALUs: the kernel template, instantiated per token count in gemv_valu_n1.hip
// and gemv_valu_n2.hip (so the two compile in parallel) and launched from
// gemv.hip.
//
// Pages: [P2] "[분석/검증-3] BitNet.cpp ARM 커널 재작성" §3 and [P3] "[기술 분석
// 보고서] ARM64 ... 1.58-bit ..." §3.1-§4 (raw codes 0/1/2 multiply the
// activations at offsets k, k+32, k+64, k+96 of a block; the scale is applied
// by the caller); [P1] "BitNet 딥다이브" §2-1 (decode is bound by reading the
// weights), §4-3 (a weight block is loaded once and reused for several
// activation columns), §4-5 (per-token activation scale).
//
// Work split (gfx950, wave64): a workgroup of 4 waves (16 for long rows, see
// gemv.hip) owns `rows_per_wg` consecutive rows of one matrix, walked in row
// groups (see the kernel).  A
// row is read as 16-byte chunks (coalesced dwordx4 loads, each packed byte
// fetched exactly once).  A 16-byte chunk c is
// half an I2_S block (b = c/2, half h = c%2): dword j holds block bytes
// 16h+4j..16h+4j+3 and so the codes of positions 32i + 16h + 4j + e.
// Masking a dword keeps one 2-bit field per byte and v_dot4_i32_i8 multiplies
// it with four contiguous int8 activations:
//   field i=3 (bits 1-0): w & 0x03030303        -> code * 1
//   field i=2 (bits 3-2): w & 0x0C0C0C0C        -> code * 4
//   field i=1 (bits 5-4): w & 0x30303030        -> code * 16
//   field i=0 (bits 7-6): (w >> 2) & 0x30303030 -> code * 16
// Three accumulators (x1, x4, x16) avoid per-field shifts; acc1 + acc4/4 +
// acc16/16 is the raw-code sum R exactly, and D = R - sum(x).
//
// Activations live in LDS in a group-major layout: token t, field i, chunk c
// at byte t*K + i*(K/4) + 16c holds x[128*(c/2) + 32i + 16*(c%2) + 0..15],
// so the four 16-byte reads a lane makes per chunk are contiguous across the
// wave (no bank conflicts).  Before the activations are staged, each wave has
// already issued the loads of its first row group, so the two memory
// latencies overlap.  A workgroup usually owns a single row group; where it
// owns several, each group is loaded and then consumed (a ping-pong register
// prefetch of the next group measured slower on gfx950).
//
// Modes: 0 = int8 xq (+ scale and sum) from global memory; 1/2 = fp32/bf16
// tokens quantised in the prologue with the same arithmetic as the
// stand-alone quantiser (every workgroup recomputes the identical values;
// workgroup 0 optionally stores them).  One launch may serve up to kMaxMats
// matrices that share the tokens (e.g. q/k/v, or gate/up).
#pragma once
#include "common.h"

namespace bitnet {

constexpr int kGemvWaves = 4;        // waves per workgroup (WAVES), short and mid rows
constexpr int kGemvWavesLong = 16;   // waves per workgroup for long rows (a row per wave per row group)
constexpr int kLdsBytes = 61440;   // activation staging budget per workgroup (60 KiB)
#ifndef BITNET_GEMV_TARGET_WGS
#define BITNET_GEMV_TARGET_WGS 1024   // workgroups per launch before slabs grow
#endif
#ifndef BITNET_GEMV_LPR
#define BITNET_GEMV_LPR 0             // 0: pick lanes per row from K
#endif

template <int MODE>
struct TokVec;   // 16 bytes of a token row, widened to fp32
template <>
struct TokVec<1> {
    static constexpr int kElems = 4;
    __device__ static void widen(const uint4 u, float *v) {
        v[0] = __uint_as_float(u.x); v[1] = __uint_as_float(u.y);
        v[2] = __uint_as_float(u.z); v[3] = __uint_as_float(u.w);
    }
    __device__ static void load(const char *row, int q, float *v) {
        widen(reinterpret_cast<const uint4 *>(row)[q], v);
    }
};
template <>
struct TokVec<2> {
    static constexpr int kElems = 8;
    __device__ static void widen(const uint4 u, float *v) {
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            v[2 * j] = __uint_as_float(w[j] << 16);            // low half = lower element
            v[2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
        }
    }
    __device__ static void load(const char *row, int q, float *v) {
        widen(reinterpret_cast<const uint4 *>(row)[q], v);
    }
};

// LDS byte offset of activation element k of token t (group-major layout)
__device__ __forceinline__ int lds_pos(int t, int K, int k) {
    const int b = k >> 7, i = (k >> 5) & 3, h = (k >> 4) & 1, e = k & 15;
    return t * K + i * (K >> 2) + 32 * b + 16 * h + e;
}

// Quantise ntok tokens of x (fp32 or bf16) into LDS; per-token s lands in
// s_tok and each wave's part of the per-token sum in redi (token_sums adds
// them after the barrier).  Workgroup 0 also writes the optional outputs.
// Short tokens (at most XR 16-byte pieces per thread) take the register path:
// load_tokens() issues every piece load up front -- before the caller issues
// its weight loads, so waiting for the tokens never waits for the weights --
// from clamped, always-valid addresses (a repeated last piece cannot change
// the absmax and is not emitted); finish() then reduces and quantises.
// Longer tokens are streamed through twice (absmax pass, quantise pass).
template <int NT, int MODE, int WAVES, int XRMAX = 4>
struct TokenPrologue {
    static constexpr int kThreads = WAVES * 64;
    using V = TokVec<MODE>;
    static constexpr int E = V::kElems;
    // register budget: at most XRMAX pieces (the most a short-row launch can
    // need), so no thread issues clamped loads of pieces no launch has
    static constexpr int XR0 = NT == 1 ? 4 : (NT == 2 ? 2 : 1);
    static constexpr int XR = XR0 < XRMAX ? XR0 : XRMAX;
    uint4 raw[NT][XR];      // token bits as loaded; widened only in finish()

    __device__ static bool fits(const GemvArgs &a) {
        return NT <= 2 && a.K / E <= XR * kThreads;
    }
    __device__ void load_tokens(const GemvArgs &a) {
        const int nq = a.K / E;
        const char *x = reinterpret_cast<const char *>(a.x);
        const int rowb = a.K * (MODE == 2 ? 2 : 4);
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const int tt = min(t, a.ntok - 1);
#pragma unroll
            for (int r = 0; r < XR; ++r)
                raw[t][r] = reinterpret_cast<const uint4 *>(x + tt * rowb)[min(
                    (int)threadIdx.x + r * kThreads, nq - 1)];
        }
    }
    __device__ void finish(const GemvArgs &a, bool in_regs, int8_t *xl, float *s_tok,
                           float (*redf)[NT], int (*redi)[NT]) {
        const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
        const int K = a.K, nq = K / E;
        const char *x = reinterpret_cast<const char *>(a.x);
        const int rowb = K * (MODE == 2 ? 2 : 4);
        float am[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            am[t] = 0.0f;
            if (t < a.ntok) {
                if (in_regs) {
#pragma unroll
                    for (int r = 0; r < XR; ++r) {
                        float v[E];
                        V::widen(raw[t][r], v);
#pragma unroll
                        for (int e = 0; e < E; ++e) am[t] = fmaxf(am[t], fabsf(v[e]));
                    }
                } else {
                    for (int q = tid; q < nq; q += kThreads) {
                        float v[E];
                        V::load(x + t * rowb, q, v);
#pragma unroll
                        for (int e = 0; e < E; ++e) am[t] = fmaxf(am[t], fabsf(v[e]));
                    }
                }
            }
            am[t] = wave_max_f32(am[t]);
        }
        if (lane == 0) {
#pragma unroll
            for (int t = 0; t < NT; ++t) redf[wv][t] = am[t];
        }
        __syncthreads();
        float s[NT];
        int sm[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            float amx = redf[0][t];
#pragma unroll
            for (int w = 1; w < WAVES; ++w) amx = fmaxf(amx, redf[w][t]);
            s[t] = quant_scale(amx);
            sm[t] = 0;
        }
        const bool store = blockIdx.x == 0 && a.xq_out != nullptr;
        auto emit = [&](int t, int q, const float *v) {
            uint32_t pq[E / 4];
#pragma unroll
            for (int j = 0; j < E / 4; ++j) {
                pq[j] = pack_low_bytes(quant_bits(v[4 * j], s[t]), quant_bits(v[4 * j + 1], s[t]),
                                       quant_bits(v[4 * j + 2], s[t]),
                                       quant_bits(v[4 * j + 3], s[t]));
                sm[t] = sum_codes4(pq[j], sm[t]);
            }
            const int pos = lds_pos(t, K, q * E);
            if constexpr (E == 8) {
                const uint2 u = make_uint2(pq[0], pq[E / 4 - 1]);
                *reinterpret_cast<uint2 *>(xl + pos) = u;
                if (store) reinterpret_cast<uint2 *>(a.xq_out + (int64_t)t * K)[q] = u;
            } else {
                *reinterpret_cast<uint32_t *>(xl + pos) = pq[0];
                if (store) reinterpret_cast<uint32_t *>(a.xq_out + (int64_t)t * K)[q] = pq[0];
            }
        };
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            if (t < a.ntok) {
                if (in_regs) {
#pragma unroll
                    for (int r = 0; r < XR; ++r) {
                        const int q = tid + r * kThreads;
                        float v[E];
                        V::widen(raw[t][r], v);
                        if (q < nq) emit(t, q, v);
                    }
                } else {
                    for (int q = tid; q < nq; q += kThreads) {
                        float v[E];
                        V::load(x + t * rowb, q, v);
                        emit(t, q, v);
                    }
                }
            }
            sm[t] = wave_sum_i32(sm[t]);
        }
        // The waves' partial sums are combined after the caller's barrier
        // (token_sums), so no barrier of its own stands before the dot products.
        if (lane == 0) {
#pragma unroll
            for (int t = 0; t < NT; ++t) redi[wv][t] = sm[t];
        }
        if (tid < NT && tid < a.ntok) {
            s_tok[tid] = s[tid];
            if (blockIdx.x == 0 && a.xs_out) a.xs_out[tid] = s[tid];
        }
    }
    // After the barrier that follows finish(): every thread's copy of the
    // per-token sums; workgroup 0 also writes the optional output.
    __device__ static void token_sums(const GemvArgs &a, const int (*redi)[NT], int *tsum) {
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            int v = 0;
#pragma unroll
            for (int w = 0; w < WAVES; ++w) v += redi[w][t];
            tsum[t] = v;
            if (blockIdx.x == 0 && threadIdx.x == t && t < a.ntok && a.xsum_out)
                a.xsum_out[t] = v;
        }
    }
};

// Work split: a wave handles row groups of 64/LPR rows, LPR lanes per row;
// lane u of a row takes the row's 16-byte chunks u, u+LPR, ..., at most JM of
// them (J = ceil(C/LPR) at run time).  The host picks LPR per launch (see
// pick_lpr): small launches spread a row over more lanes (2B-class q/k/v and o
// at K=2560: 16 lanes x 3 chunks; down at K=6912: 32 x 4), large ones keep
// J close to 8 (K=8192: 16 x 8; K=28672: 64 x 7).  All J loads of a row group
// are in flight together.
// JM: chunks per lane per row group (upper bound of J).  JM = 3 or 4 are the
// short-row variants for single-token launches with J <= 3 / J = 4: their
// chunk loop has no run-time guard (chunks past J carry zeroed weights), so
// the compiler can issue every chunk's LDS reads at once -- the tail after the
// weights arrive is a latency chain in these small launches.
// The instrumented build (-DBITNET_STAMPS, libbitnet_i2s_stamps.so) gives
// every launch a slot that receives the first wave's start and the last
// wave's end (s_memrealtime ticks, 100 MHz) by atomic min / max, so a launch's
// own duration can be read without a tracer.  The product build has no slot.
#ifdef BITNET_STAMPS
constexpr int kStampSubs = 64;   // sub-slots per launch (workgroup b takes b % 64)
struct GemvKernelArgs : GemvArgs {
    unsigned long long *stamp;   // this launch's slot (kStampSubs lines of 128 bytes), or null
};
unsigned long long *stamp_slot();   // gemv.hip: the slot of the next launch
#else
using GemvKernelArgs = GemvArgs;
#endif

template <int NT, int LPR, int MODE, int JM, int WAVES>
__global__ __launch_bounds__(WAVES * 64) void gemv_valu_kernel(const GemvKernelArgs a) {
    constexpr int kThreads = WAVES * 64;
    constexpr bool kAllChunks = JM <= 4;
    // token pieces per thread a single-token launch can need (its rows are
    // at most JM chunks per lane: K <= 64 * JM * LPR); passes of two tokens
    // keep the full register budget
    constexpr int kTokE = MODE == 1 ? 4 : 8;
    constexpr int kTokXR = NT == 1 ? (JM * LPR * 64 / kTokE + WAVES * 64 - 1) / (WAVES * 64) : 4;
    using Prologue = TokenPrologue<NT, MODE, WAVES, (kTokXR < 1 ? 1 : kTokXR)>;
    constexpr int RG = 64 / LPR;            // rows per wave per row group
    extern __shared__ int4 lds[];
    int8_t *xl = reinterpret_cast<int8_t *>(lds);
    __shared__ float s_tok[NT];
    __shared__ int sum_tok[NT];
    __shared__ float redf[WAVES][NT];
    __shared__ int redi[WAVES][NT];

    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
#ifdef BITNET_STAMPS
    // start: thread 0 of each workgroup; end: the workgroup's last wave to
    // finish (an LDS count), so a workgroup makes two global atomics
    unsigned long long *const stamp = a.stamp ? a.stamp + 16 * (blockIdx.x % kStampSubs) : nullptr;
    __shared__ int stamp_waves;
    if (tid == 0) {
        stamp_waves = 0;
        if (stamp) atomicMin(stamp, __builtin_amdgcn_s_memrealtime());
    }
#endif
    const int sub = lane / LPR, u = lane % LPR;
    int mi = 0;
#pragma unroll
    for (int i = 1; i < kMaxMats; ++i)
        if (i < a.nmats && (int)blockIdx.x >= a.mat[i].wg_begin) mi = i;
    const uint8_t *packed = a.mat[mi].packed;
    const int M = a.mat[mi].M;
    const int K = a.K;
    const int C = K >> 6;                       // 16-byte chunks per packed row
    const int J = (C + LPR - 1) / LPR;
    const int wg_local = (int)blockIdx.x - a.mat[mi].wg_begin;
    const int row0 = wg_local * a.rows_per_wg;
    const int row1 = min(M, row0 + a.rows_per_wg);
    // row groups of this wave: rows row0 + (g*WAVES + wv)*RG + sub
    const int ngroups = (row1 - row0 + RG * WAVES - 1) / (RG * WAVES);
    auto group_row = [&](int g) { return row0 + (g * WAVES + wv) * RG + sub; };
    // Every lane issues exactly JM loads per row group, from a clamped (always
    // valid) address; lanes or rows outside the matrix are zeroed after the
    // load.  A fixed, branch-free load count lets the compiler wait for just
    // the row group in use while the next one is still in flight.
    int4 cur[JM];
    auto load_group = [&](int g, int4 *r) {
        const int row = min(group_row(g), M - 1);
        const v4i *prow = reinterpret_cast<const v4i *>(packed + (int64_t)row * (K >> 2));
#pragma unroll
        for (int j = 0; j < JM; ++j) {
            const int c = min(u + LPR * j, C - 1);
            const v4i v = __builtin_nontemporal_load(prow + c);
            r[j] = make_int4(v.x, v.y, v.z, v.w);
        }
    };
    // ---- activations -> LDS (group-major), per-token scale and sum ----
    // Token loads are issued first, then the first row group's weight loads,
    // so the token work below overlaps the weight latency.
    if constexpr (MODE == 0) {
        const int n16 = a.ntok * (K >> 4);
        const int4 *src = reinterpret_cast<const int4 *>(a.x);
        // The per-token scale and sum are loaded before the weights: loads
        // complete in order, so storing a value loaded after them would wait
        // for every weight load (and, through the barrier, stall every wave).
        const int tsel = min(tid, a.ntok - 1);
        const float xs_r = a.xs_in[tsel];
        const int xsum_r = a.xsum_in[tsel];
        // Short tokens: two 16-byte pieces per thread, loaded ahead of the
        // weights and stored to LDS once the weight loads are issued.  Longer
        // tokens are staged first.  Either way the weight loads of the first
        // row group are issued by the same code after the branch, so the
        // compiler's wait counts stay exact for every chunk below.
        const bool in_regs = n16 <= 2 * kThreads;
        const int q0 = tid, q1 = tid + kThreads;
        int4 p0 = make_int4(0, 0, 0, 0), p1 = p0;
        if (in_regs) {
            p0 = src[min(q0, n16 - 1)];
            p1 = src[min(q1, n16 - 1)];
        } else {
            for (int q = tid; q < n16; q += kThreads) {
                const int t = q / (K >> 4), k = (q - t * (K >> 4)) << 4;
                *reinterpret_cast<int4 *>(xl + lds_pos(t, K, k)) = src[q];
            }
        }
        __builtin_amdgcn_sched_barrier(0);   // keep the token loads ahead of the weights
        load_group(0, cur);
        __builtin_amdgcn_sched_barrier(0);
        if (in_regs) {
            const int kp = K >> 4;
            if (q0 < n16) {
                const int t = q0 / kp;
                *reinterpret_cast<int4 *>(xl + lds_pos(t, K, (q0 - t * kp) << 4)) = p0;
            }
            if (q1 < n16) {
                const int t = q1 / kp;
                *reinterpret_cast<int4 *>(xl + lds_pos(t, K, (q1 - t * kp) << 4)) = p1;
            }
        }
        if (tid < NT && tid < a.ntok) {
            s_tok[tid] = xs_r;
            sum_tok[tid] = xsum_r;
        }
    } else {
        Prologue tp;
        const bool in_regs = Prologue::fits(a);
        if (in_regs) tp.load_tokens(a);
        __builtin_amdgcn_sched_barrier(0);       // keep the token loads ahead of the weights
        load_group(0, cur);
        __builtin_amdgcn_sched_barrier(0);
        tp.finish(a, in_regs, xl, s_tok, redf, redi);
    }
    __syncthreads();
    int tsum[NT];   // per-token sums of the quantised tokens
    if constexpr (MODE == 0) {
#pragma unroll
        for (int t = 0; t < NT; ++t) tsum[t] = sum_tok[t];
    } else {
        Prologue::token_sums(a, redi, tsum);
    }

    const int gstride = K >> 2;   // bytes between fields in LDS
    int32_t *dot = a.mat[mi].dot;
    float *y = a.mat[mi].y;
    const float alpha = a.mat[mi].alpha;
    auto compute = [&](int g, const int4 *w) {
        const bool row_ok = group_row(g) < row1;
        int a1[NT], a4[NT], a16[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) a1[t] = a4[t] = a16[t] = 0;
#pragma unroll
        for (int j = 0; j < JM; ++j) {
            const int c = u + LPR * j;
            if (kAllChunks || j < J) {
                const bool ok = c < C && row_ok;
                const int pw[4] = {ok ? w[j].x : 0, ok ? w[j].y : 0, ok ? w[j].z : 0,
                                   ok ? w[j].w : 0};
                const int cl = min(c, C - 1);
#pragma unroll
                for (int t = 0; t < NT; ++t) {
                    if (t < a.ntok) {
                        const int8_t *xt = xl + t * K + 16 * cl;
                        const int4 x0 = *reinterpret_cast<const int4 *>(xt);
                        const int4 x1 = *reinterpret_cast<const int4 *>(xt + gstride);
                        const int4 x2 = *reinterpret_cast<const int4 *>(xt + 2 * gstride);
                        const int4 x3 = *reinterpret_cast<const int4 *>(xt + 3 * gstride);
                        const int xv0[4] = {x0.x, x0.y, x0.z, x0.w};
                        const int xv1[4] = {x1.x, x1.y, x1.z, x1.w};
                        const int xv2[4] = {x2.x, x2.y, x2.z, x2.w};
                        const int xv3[4] = {x3.x, x3.y, x3.z, x3.w};
#pragma unroll
                        for (int d = 0; d < 4; ++d) {
                            a16[t] = dot4((pw[d] >> 2) & 0x30303030, xv0[d], a16[t]);
                            a16[t] = dot4(pw[d] & 0x30303030, xv1[d], a16[t]);
                            a4[t] = dot4(pw[d] & 0x0C0C0C0C, xv2[d], a4[t]);
                            a1[t] = dot4(pw[d] & 0x03030303, xv3[d], a1[t]);
                        }
                    }
                }
            }
        }
        const int row = group_row(g);
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            if (t < a.ntok) {
                // a4 and a16 are exact multiples of 4 and 16
                // the row's sum is complete in its last 16 lanes (group_sum_i32)
                const int r = group_sum_i32<LPR>(a1[t] + (a4[t] >> 2) + (a16[t] >> 4));
                if (u == LPR - 1 - t && row_ok) {
                    const int d = r - tsum[t];
                    if (dot) dot[(int64_t)t * M + row] = d;
                    if (y) y[(int64_t)t * M + row] = ((float)d * alpha) / s_tok[t];
                }
            }
        }
    };
    // Consume the first row group (its loads were issued before the
    // activations were staged), then load and consume the others.
    if constexpr (MODE == 0) {
        // int8 tokens: the first group stays outside the loop.  With it
        // inside, the compiler merged the loop entry (loads in flight) with
        // the back edge (none) and waited for every load before the first
        // dot product, so no chunk's arithmetic overlapped the later chunks'
        // memory latency (large stack at N = 1: 400 -> 381 us per step).
        compute(0, cur);
        for (int g = 1; g < ngroups; ++g) {
            load_group(g, cur);
            compute(g, cur);
        }
    } else {
        // Tokens quantised in the prologue: here the loop form is the faster
        // one (2B-class decode step of 120 launches 0.499 -> 0.487 ms, large
        // stack from bf16 tokens 412 -> 405 us, against the peeled form).
        for (int g = 0; g < ngroups; ++g) {
            if (g > 0) load_group(g, cur);
            compute(g, cur);
        }
    }
#ifdef BITNET_STAMPS
    if (stamp && lane == 0 && atomicAdd(&stamp_waves, 1) == WAVES - 1)
        atomicMax(stamp + 1, __builtin_amdgcn_s_memrealtime());
#endif
}

// One launch of the kernel for NT tokens per pass, token mode MODE and the
// lane count chosen by the host.
template <int NT, int MODE, int JM>
static hipError_t launch_gemv_ntj(const GemvKernelArgs &a, int lpr, unsigned grid, hipStream_t st) {
    const size_t lds = (size_t)a.ntok * (size_t)a.K;
    const dim3 b(kGemvWaves * 64);
    switch (lpr) {
        case 8: hipLaunchKernelGGL((gemv_valu_kernel<NT, 8, MODE, JM, kGemvWaves>), dim3(grid), b, lds, st, a); break;
        case 16: hipLaunchKernelGGL((gemv_valu_kernel<NT, 16, MODE, JM, kGemvWaves>), dim3(grid), b, lds, st, a); break;
        case 32: hipLaunchKernelGGL((gemv_valu_kernel<NT, 32, MODE, JM, kGemvWaves>), dim3(grid), b, lds, st, a); break;
        default: hipLaunchKernelGGL((gemv_valu_kernel<NT, 64, MODE, JM, kGemvWaves>), dim3(grid), b, lds, st, a); break;
    }
    return hipGetLastError();
}

// One launch of the kernel for NT tokens per pass, token mode MODE and the
// lane count chosen by the host (short: J <= 4, taken for NT == 1 only;
// long: 16 waves of 64 lanes per row).  Each (NT, MODE) pair is
// instantiated in one of the gemv_valu_n*.hip translation units.
template <int NT, int MODE>
hipError_t launch_gemv_nt(const GemvKernelArgs &a, int lpr, int short_j, bool long_rows,
                          unsigned grid, hipStream_t st) {
    if (long_rows) {
        const size_t lds = (size_t)a.ntok * (size_t)a.K;
        hipLaunchKernelGGL((gemv_valu_kernel<NT, 64, MODE, 8, kGemvWavesLong>), dim3(grid),
                           dim3(kGemvWavesLong * 64), lds, st, a);
        return hipGetLastError();
    }
    if constexpr (NT == 1) {
        if (short_j == 3) return launch_gemv_ntj<NT, MODE, 3>(a, lpr, grid, st);
        if (short_j == 4) return launch_gemv_ntj<NT, MODE, 4>(a, lpr, grid, st);
    }
    return launch_gemv_ntj<NT, MODE, 8>(a, lpr, grid, st);
}

#define BITNET_GEMV_EXTERN(NT, MODE) \
    extern template hipError_t launch_gemv_nt<NT, MODE>(const GemvKernelArgs &, int, int, bool, unsigned, \
                                                        hipStream_t)
// passes of one or two tokens (larger batches run on MFMA)
BITNET_GEMV_EXTERN(1, 0); BITNET_GEMV_EXTERN(1, 1); BITNET_GEMV_EXTERN(1, 2);
BITNET_GEMV_EXTERN(2, 0); BITNET_GEMV_EXTERN(2, 1); BITNET_GEMV_EXTERN(2, 2);
#undef BITNET_GEMV_EXTERN

}  // namespace bitnet
