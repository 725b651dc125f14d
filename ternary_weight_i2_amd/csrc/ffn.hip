// ffn.hip -- the squared-ReLU gated FFN activation between the gate/up and
// down projections, quantised for the down projection.
//
// Pages: [P4] "bitnet.rs", "Forward Pass" (the FFN computes
// ffn_sub_norm(sqrelu(gate(x)) * up(x)) and feeds it to down); [P1]
// "BitNet 딥다이브" §4-5 (per-token absmax int8 activations).
//
// One workgroup per token.  Pass 1: each thread takes runs of 32 channels,
// forms h = (relu(g)^2) * u in fp32, keeps h in LDS and sums h^2 over its run
// in binary64 in index order (the squares of fp32 values are exact in
// binary64).  One thread then adds the run sums in index order and forms the
// factor c = fp32(1 / sqrt(sum / F + eps)); this fixed order makes the factor,
// and so every int8 code, independent of the launch shape.  Pass 2: v =
// (h * c) * gamma over the same runs (kept in LDS) and its absmax; pass 3: the
// scale and the codes, with the same arithmetic as the stand-alone activation
// quantiser.  Every pass works on whole 32-channel runs with 16-byte loads,
// so a thread's loads are in flight together.
#include "common.h"

namespace bitnet {

constexpr int kFfnThreads = 256;

__global__ __launch_bounds__(kFfnThreads) void ffn_act_quant_kernel(
    const float *__restrict__ g, const float *__restrict__ u, const float *__restrict__ gamma,
    float eps, int F, int8_t *__restrict__ xq, float *__restrict__ xs,
    int32_t *__restrict__ xsum) {
    // h[F] in LDS column-major over the runs -- channel j of run r at
    // j * nruns + r -- so the lanes of a wave (consecutive runs) hit
    // consecutive banks; then the run sums (double)
    extern __shared__ float hl[];
    double *runs = reinterpret_cast<double *>(hl + F); // F is a multiple of 128: 8-byte aligned
    __shared__ float c_tok, red_f[kFfnThreads / 64];
    __shared__ int red_i[kFfnThreads / 64];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int64_t row = (int64_t)blockIdx.x * F;
    const float4 *g4 = reinterpret_cast<const float4 *>(g + row);
    const float4 *u4 = reinterpret_cast<const float4 *>(u + row);
    const int nruns = F / 32;

    // The gain of the thread's first run is loaded with g and u, so pass 2
    // needs no second memory round trip when every run fits one thread
    // (F <= 8192); further runs load theirs in pass 2.
    float4 gm0[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
        gm0[i] = gamma && tid < nruns ? reinterpret_cast<const float4 *>(gamma)[tid * 8 + i]
                                      : make_float4(1.0f, 1.0f, 1.0f, 1.0f);

    for (int r = tid; r < nruns; r += kFfnThreads) {
        double part = 0.0;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float4 gv = g4[r * 8 + i], uv = u4[r * 8 + i];
            const float gg[4] = {gv.x, gv.y, gv.z, gv.w}, uu[4] = {uv.x, uv.y, uv.z, uv.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float rl = gg[e] > 0.0f ? gg[e] : 0.0f;
                const float h = (rl * rl) * uu[e];
                hl[(i * 4 + e) * nruns + r] = h;
                part += (double)h * (double)h;
            }
        }
        runs[r] = part;
    }
    __syncthreads();
    if (tid == 0) {
        // the run sums in index order; the LDS reads go out 32 at a time so
        // the chain of adds does not wait on one read per step
        double ss = 0.0;
        int r = 0;
        for (; r + 32 <= nruns; r += 32) {
            double t[32];
#pragma unroll
            for (int i = 0; i < 32; ++i) t[i] = runs[r + i];
#pragma unroll
            for (int i = 0; i < 32; ++i) ss += t[i];
        }
        for (; r < nruns; ++r) ss += runs[r];
        c_tok = (float)(1.0 / sqrt(ss / (double)F + (double)eps));
    }
    __syncthreads();
    const float c = c_tok;
    // Pass 2: v = (h * c) * gamma over the thread's own runs (16-byte loads of
    // the gain, all eight of a run in flight), kept in LDS in place of h.
    float amax = 0.0f;
    for (int r = tid; r < nruns; r += kFfnThreads) {
        float4 gm[8];
#pragma unroll
        for (int i = 0; i < 8; ++i)
            gm[i] = r == tid ? gm0[i]
                  : gamma    ? reinterpret_cast<const float4 *>(gamma)[r * 8 + i]
                             : make_float4(1.0f, 1.0f, 1.0f, 1.0f);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float ga[4] = {gm[i].x, gm[i].y, gm[i].z, gm[i].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int k = (i * 4 + e) * nruns + r;
                const float t = hl[k] * c;
                const float v = gamma ? t * ga[e] : t;
                hl[k] = v;
                amax = fmaxf(amax, fabsf(v));
            }
        }
    }
    amax = wave_max_f32(amax);
    if (lane == 0) red_f[wv] = amax;
    __syncthreads();
    float a = red_f[0];
#pragma unroll
    for (int i = 1; i < kFfnThreads / 64; ++i) a = fmaxf(a, red_f[i]);
    const float s = quant_scale(a);
    // Pass 3: codes of the thread's runs, 32 bytes per run in two stores.
    int sum = 0;
    int8_t *q = xq + row;
    for (int r = tid; r < nruns; r += kFfnThreads) {
        int w[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            uint32_t packed4 = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int v = quant_one(hl[(i * 4 + e) * nruns + r], s);
                sum += v;
                packed4 |= (uint32_t)(uint8_t)(int8_t)v << (8 * e);
            }
            w[i] = (int)packed4;
        }
        int4 *dst = reinterpret_cast<int4 *>(q + r * 32);
        dst[0] = make_int4(w[0], w[1], w[2], w[3]);
        dst[1] = make_int4(w[4], w[5], w[6], w[7]);
    }
    sum = wave_sum_i32(sum);
    if (lane == 0) red_i[wv] = sum;
    __syncthreads();
    if (tid == 0) {
        int t = 0;
#pragma unroll
        for (int i = 0; i < kFfnThreads / 64; ++i) t += red_i[i];
        xs[blockIdx.x] = s;
        xsum[blockIdx.x] = t;
    }
}

hipError_t launch_ffn_act_quant(const float *g, const float *u, const float *gamma, float eps,
                                int64_t N, int64_t F, int8_t *xq, float *xs, int32_t *xsum,
                                hipStream_t st) {
    const size_t lds = (size_t)F * sizeof(float) + (size_t)(F / 32) * sizeof(double);
    hipLaunchKernelGGL(ffn_act_quant_kernel, dim3((unsigned)N), dim3(kFfnThreads), lds, st, g, u,
                       gamma, eps, (int)F, xq, xs, xsum);
    return hipGetLastError();
}

}  // namespace bitnet
