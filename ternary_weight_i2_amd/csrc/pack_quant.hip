// pack_quant.hip -- I2_S packing and per-token absmax int8 quantisation.
//
// Pages: [P1] "BitNet 딥다이브" (fiv.co.kr), §1-1 code table, §4-2 block
// interleave, §4-5 per-token activation quantisation; [P4] "bitnet.rs",
// "Mathematical Foundation" (8-bit activation clip range).
#include "common.h"

namespace bitnet {

// ---------------------------------------------------------------------------
// Packing [P1 §1-1, §4-2].  Packed byte g of a 32-byte block holds block
// positions g, g+32, g+64, g+96; so bytes g0..g0+n-1 of a block come from n
// contiguous weights at each of the offsets 0, 32, 64, 96, and a thread that
// builds them issues four aligned loads and one store of n bytes (n = 16
// when w is 16-byte aligned, else 4).  A weight outside {-1,0,+1} is counted
// in *bad and stored as code 3.
// ---------------------------------------------------------------------------
// WIDE = 1 (w 16-byte aligned): one thread per 16-byte half of a packed
// block, four 16-byte loads and one 16-byte store.  WIDE = 0: one thread per
// packed dword, four 4-byte loads and one 4-byte store.
template <int WIDE>
__global__ __launch_bounds__(256) void pack_i2s_kernel(
    const int8_t *__restrict__ w, int64_t M, int64_t K,
    uint8_t *__restrict__ packed, unsigned *__restrict__ bad) {
    constexpr int DW = WIDE ? 4 : 1;                    // packed dwords per thread
    const int64_t units_per_row = K / (16 * DW);
    const int64_t total = M * units_per_row;
    unsigned nbad = 0;
    for (int64_t d = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; d < total;
         d += (int64_t)gridDim.x * blockDim.x) {
        const int64_t m = d / units_per_row;
        const int64_t r = d - m * units_per_row;
        const int64_t blk = r / (8 / DW);              // 8 dwords per block
        const int g0 = (int)(r % (8 / DW)) * 4 * DW;    // first block byte of this unit
        const int8_t *src = w + m * K + blk * kBlock + g0;
        uint32_t out[DW];
        uint32_t v[4][DW];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if constexpr (WIDE) {
                const uint4 q = *reinterpret_cast<const uint4 *>(src + 32 * i);
                v[i][0] = q.x;
                v[i][1] = q.y;
                v[i][2] = q.z;
                v[i][3] = q.w;
            } else {
                v[i][0] = *reinterpret_cast<const uint32_t *>(src + 32 * i);
            }
        }
#pragma unroll
        for (int t = 0; t < DW; ++t) {
            out[t] = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    int code = (int)(int8_t)(v[i][t] >> (8 * e)) + 1;   // -1,0,+1 -> 0,1,2
                    if ((unsigned)code > 2u) {
                        ++nbad;
                        code = 3;
                    }
                    out[t] |= (uint32_t)code << (8 * e + 6 - 2 * i);
                }
        }
        uint8_t *dst = packed + m * (K / 4) + blk * kBlockBytes + g0;
        if constexpr (WIDE)
            *reinterpret_cast<uint4 *>(dst) = uint4{out[0], out[1], out[2], out[3]};
        else
            *reinterpret_cast<uint32_t *>(dst) = out[0];
    }
    if (nbad) atomicAdd(bad, nbad);
}

hipError_t launch_pack(const int8_t *w, int64_t M, int64_t K, uint8_t *packed,
                       unsigned *bad, hipStream_t st) {
    const bool wide = (reinterpret_cast<uintptr_t>(w) & 15) == 0;
    const int64_t total = M * (K / (wide ? 64 : 16));
    int64_t blocks = (total + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    if (wide)
        hipLaunchKernelGGL(pack_i2s_kernel<1>, dim3((unsigned)blocks), dim3(256), 0, st, w, M, K,
                           packed, bad);
    else
        hipLaunchKernelGGL(pack_i2s_kernel<0>, dim3((unsigned)blocks), dim3(256), 0, st, w, M, K,
                           packed, bad);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Per-token quantisation [P1 §4-5]: s = 127 / max(max|x|, 1e-5),
// q = clamp(round_half_even(x*s), -128, 127) [P4], plus sum(q).
// One 256-thread workgroup per token; 16-byte loads (4 fp32 or 8 bf16).
// s is the correctly rounded fp32 quotient: the division is done in binary64
// and rounded once to binary32, which equals the correctly rounded binary32
// quotient of the two fp32 operands (53 >= 2*24 + 2).
// ---------------------------------------------------------------------------
template <int BF16>
struct Vec16;   // 16 bytes of activations widened to fp32

template <>
struct Vec16<0> {
    static constexpr int kElems = 4;
    __device__ static void load(const void *base, int64_t i, float *v) {
        const float4 f = reinterpret_cast<const float4 *>(base)[i];
        v[0] = f.x; v[1] = f.y; v[2] = f.z; v[3] = f.w;
    }
    __device__ static void widen(const uint4 u, float *v) {
        v[0] = __uint_as_float(u.x); v[1] = __uint_as_float(u.y);
        v[2] = __uint_as_float(u.z); v[3] = __uint_as_float(u.w);
    }
};

template <>
struct Vec16<1> {
    static constexpr int kElems = 8;
    __device__ static void load(const void *base, int64_t i, float *v) {
        widen(reinterpret_cast<const uint4 *>(base)[i], v);
    }
    __device__ static void widen(const uint4 u, float *v) {
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            v[2 * j] = __uint_as_float(w[j] << 16);            // low half = lower element
            v[2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
        }
    }
};

constexpr int kQuantThreads = 256;   // one workgroup per token
constexpr int kQuantWaves = kQuantThreads / 64;

// Rows longer than 16 pieces per thread (fp32 tokens above K = 16384): two
// passes over the row (absmax, then quantise).
template <int BF16>
__global__ __launch_bounds__(kQuantThreads) void quant_act_kernel(
    const void *__restrict__ x, int64_t K, int8_t *__restrict__ xq,
    float *__restrict__ xs, int32_t *__restrict__ xsum) {
    using V = Vec16<BF16>;
    constexpr int E = V::kElems;
    __shared__ float red_f[kQuantWaves];
    __shared__ int red_i[kQuantWaves];
    const int64_t n = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const char *row = reinterpret_cast<const char *>(x) + n * K * (BF16 ? 2 : 4);
    const int64_t nvec = K / E;

    float a = 0.0f;
    for (int64_t i = tid; i < nvec; i += kQuantThreads) {
        float v[E];
        V::load(row, i, v);
#pragma unroll
        for (int e = 0; e < E; ++e) a = fmaxf(a, fabsf(v[e]));
    }
    a = wave_max_f32(a);
    if (lane == 0) red_f[wv] = a;
    __syncthreads();
    a = red_f[0];
#pragma unroll
    for (int w = 1; w < kQuantWaves; ++w) a = fmaxf(a, red_f[w]);
    const float s = quant_scale(a);

    int8_t *qrow = xq + n * K;
    int sum = 0;
    for (int64_t i = tid; i < nvec; i += kQuantThreads) {
        float v[E];
        V::load(row, i, v);
        uint32_t packedq[E / 4];
#pragma unroll
        for (int j = 0; j < E / 4; ++j) {
            packedq[j] = pack_low_bytes(quant_bits(v[4 * j], s), quant_bits(v[4 * j + 1], s),
                                        quant_bits(v[4 * j + 2], s), quant_bits(v[4 * j + 3], s));
            sum = sum_codes4(packedq[j], sum);
        }
        if (E == 8) {
            reinterpret_cast<uint2 *>(qrow)[i] = make_uint2(packedq[0], packedq[E / 4 - 1]);
        } else {
            reinterpret_cast<uint32_t *>(qrow)[i] = packedq[0];
        }
    }
    sum = wave_sum_i32(sum);
    if (lane == 0) red_i[wv] = sum;
    __syncthreads();
    if (tid == 0) {
        xs[n] = s;
        int t = 0;
#pragma unroll
        for (int w = 0; w < kQuantWaves; ++w) t += red_i[w];
        xsum[n] = t;
    }
}

// The same per-token quantisation with the row held in registers: every
// thread issues the loads of all its R 16-byte pieces at once (clamped,
// always-valid addresses; a repeated last piece cannot change the absmax and
// is not emitted), so a token costs one memory round trip instead of one per
// piece and pass.  A workgroup holds TPB tokens of kQuantThreads / TPB
// threads each (the launcher's choice below).  Identical arithmetic,
// identical bits.
template <int BF16, int R, int TPB>
__global__ __launch_bounds__(kQuantThreads) void quant_act_regs_kernel(
    const void *__restrict__ x, int64_t N, int64_t K, int8_t *__restrict__ xq,
    float *__restrict__ xs, int32_t *__restrict__ xsum) {
    using V = Vec16<BF16>;
    constexpr int E = V::kElems;
    constexpr int T = kQuantThreads / TPB;   // threads per token
    constexpr int TW = T / 64;               // waves per token
    static_assert(TW >= 1 && TPB * TW == kQuantWaves, "whole waves per token");
    __shared__ float red_f[kQuantWaves];
    __shared__ int red_i[kQuantWaves];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int slot = tid / T, lt = tid - slot * T;   // this thread's token in the block
    const int64_t nb = (int64_t)blockIdx.x * TPB + slot;
    const bool valid = nb < N;                       // a ragged last block: loads stay in bounds
    const int64_t n = valid ? nb : N - 1;
    const char *row = reinterpret_cast<const char *>(x) + n * K * (BF16 ? 2 : 4);
    const int nvec = (int)(K / E);

    uint4 raw[R];   // the pieces as loaded; widened where used
#pragma unroll
    for (int r = 0; r < R; ++r)
        raw[r] = reinterpret_cast<const uint4 *>(row)[min(lt + r * T, nvec - 1)];
    float a = 0.0f;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        float v[E];
        V::widen(raw[r], v);
#pragma unroll
        for (int e = 0; e < E; ++e) a = fmaxf(a, fabsf(v[e]));
    }
    a = wave_max_f32(a);   // every lane receives the wave's maximum
    if constexpr (TW > 1) {
        if (lane == 0) red_f[wv] = a;
        __syncthreads();
        a = red_f[slot * TW];
#pragma unroll
        for (int w = 1; w < TW; ++w) a = fmaxf(a, red_f[slot * TW + w]);
    }
    const float s = quant_scale(a);

    int8_t *qrow = xq + n * K;
    int sum = 0;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int i = lt + r * T;
        if (i < nvec) {
            float v[E];
            V::widen(raw[r], v);
            uint32_t packedq[E / 4];
#pragma unroll
            for (int j = 0; j < E / 4; ++j) {
                packedq[j] = pack_low_bytes(quant_bits(v[4 * j], s), quant_bits(v[4 * j + 1], s),
                                            quant_bits(v[4 * j + 2], s), quant_bits(v[4 * j + 3], s));
                sum = sum_codes4(packedq[j], sum);
            }
            if (valid) {
                if (E == 8) {
                    reinterpret_cast<uint2 *>(qrow)[i] = make_uint2(packedq[0], packedq[E / 4 - 1]);
                } else {
                    reinterpret_cast<uint32_t *>(qrow)[i] = packedq[0];
                }
            }
        }
    }
    sum = wave_sum_i32(sum);   // every lane receives the wave's sum
    if constexpr (TW > 1) {
        if (lane == 0) red_i[wv] = sum;
        __syncthreads();
        if (lt == 0 && valid) {
            xs[n] = s;
            int t = 0;
#pragma unroll
            for (int w = 0; w < TW; ++w) t += red_i[slot * TW + w];
            xsum[n] = t;
        }
    } else if (lt == 0 && valid) {   // one wave per token: no exchange, no barrier
        xs[n] = s;
        xsum[n] = sum;
    }
}

#ifndef BITNET_QUANT_ROUND
#define BITNET_QUANT_ROUND 1
#endif

template <int BF16, int TPB>
static hipError_t launch_quant_tpb(const void *x, int64_t N, int64_t K, int8_t *xq, float *xs,
                                   int32_t *xsum, hipStream_t st) {
    constexpr int T = kQuantThreads / TPB;   // threads per token
    const int64_t per = (K / Vec16<BF16>::kElems + T - 1) / T;
    const dim3 g((unsigned)((N + TPB - 1) / TPB)), b(kQuantThreads);
    if (per <= 1) hipLaunchKernelGGL((quant_act_regs_kernel<BF16, 1, TPB>), g, b, 0, st, x, N, K, xq, xs, xsum);
    else if (per <= 2) hipLaunchKernelGGL((quant_act_regs_kernel<BF16, 2, TPB>), g, b, 0, st, x, N, K, xq, xs, xsum);
    else if (per <= 4) hipLaunchKernelGGL((quant_act_regs_kernel<BF16, 4, TPB>), g, b, 0, st, x, N, K, xq, xs, xsum);
    else if (per <= 8) hipLaunchKernelGGL((quant_act_regs_kernel<BF16, 8, TPB>), g, b, 0, st, x, N, K, xq, xs, xsum);
    else hipLaunchKernelGGL((quant_act_regs_kernel<BF16, 16, TPB>), g, b, 0, st, x, N, K, xq, xs, xsum);
    return hipGetLastError();
}

// Tokens per workgroup: one wave per token (four per workgroup) for rows of
// at most 256 16-byte pieces (K <= 2048 bf16), so a token needs no
// cross-wave exchange and no barrier (4096 x 1024 bf16: 5.35 -> 4.98 us);
// longer rows one token per workgroup, and at least two once a launch has
// more tokens than 2048 one-token workgroups (8 per CU) would hold in one
// resident round; each thread then holds more pieces, all loaded at once.
template <int BF16>
static hipError_t launch_quant_t(const void *x, int64_t N, int64_t K, int8_t *xq, float *xs,
                                 int32_t *xsum, hipStream_t st) {
    const int64_t pieces = K / Vec16<BF16>::kElems;
    int tpb = pieces <= 256 ? 4 : 1;
    if (BITNET_QUANT_ROUND && N > 2048 && tpb < 2) tpb = 2;
    // at most 16 pieces per thread in registers; longer rows stream twice
    while (tpb > 1 && pieces > (int64_t)16 * (kQuantThreads / tpb)) tpb /= 2;
    if (pieces > (int64_t)16 * kQuantThreads) {
        hipLaunchKernelGGL(quant_act_kernel<BF16>, dim3((unsigned)N), dim3(kQuantThreads), 0, st, x,
                           K, xq, xs, xsum);
        return hipGetLastError();
    }
    if (tpb == 4) return launch_quant_tpb<BF16, 4>(x, N, K, xq, xs, xsum, st);
    if (tpb == 2) return launch_quant_tpb<BF16, 2>(x, N, K, xq, xs, xsum, st);
    return launch_quant_tpb<BF16, 1>(x, N, K, xq, xs, xsum, st);
}

hipError_t launch_quant(const void *x, int bf16, int64_t N, int64_t K,
                        int8_t *xq, float *xs, int32_t *xsum, hipStream_t st) {
    return bf16 ? launch_quant_t<1>(x, N, K, xq, xs, xsum, st)
                : launch_quant_t<0>(x, N, K, xq, xs, xsum, st);
}

}  // namespace bitnet
