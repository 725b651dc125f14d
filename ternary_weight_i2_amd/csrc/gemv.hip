// gemv.hip -- host side of the decode GEMV on the vector ALUs: lane split and
// launch geometry (the kernel template is in gemv_valu.h).
#include "gemv_valu.h"

#ifdef BITNET_STAMPS
#include <atomic>
#include <mutex>
#include <vector>
#endif

namespace bitnet {

// Lanes per row (a power of two in {8,16,32,64}; each lane then takes
// J = ceil(C/LPR) <= 8 of the row's C chunks).  A launch small enough to fit
// in kWaveBudget waves is latency-bound: it takes the most lanes per row that
// keep at least 3/4 of them busy, so each lane's serial chain of chunks is
// short.  A larger launch is throughput-bound: it takes the fewest lanes per
// row (more rows per wave) among those that leave the fewest lanes idle.
constexpr int64_t kWaveBudget = 2048;
static int pick_lpr(int C, int64_t rows) {
    for (int l = 64; l >= 8; l /= 2) {
        const int j = (C + l - 1) / l;
        if (j <= 8 && rows * l <= kWaveBudget * 64 && 4 * C >= 3 * l * j) return l;
    }
    int best = 64;
    double best_eff = -1.0;
    for (int l = 8; l <= 64; l *= 2) {
        const int j = (C + l - 1) / l;
        if (j > 8) continue;
        const double eff = (double)C / (double)(l * j);
        if (eff > best_eff + 1e-9) {
            best_eff = eff;
            best = l;
        }
    }
    return best;
}

// Launch geometry of a decode GEMV launch.
struct GemvGeometry {
    int lpr;           // lanes per row
    int rows_per_wg;   // rows per workgroup
    int per;           // tokens per pass
    bool long_rows;    // 16-wave workgroups, one row per wave in each row group
};
// Long rows (a whole wave per row and more than four chunks per lane, i.e.
// K > 16384) in a launch of at least 4096 rows take 16-wave workgroups, each
// wave one row per row group: the token is staged (int8) or quantised (bf16:
// the whole row then fits the prologue's registers, read once per workgroup
// instead of twice) by a quarter as many workgroups as with four waves.  A
// workgroup takes as many row groups as keep every workgroup resident in
// one round (the down projection 8192x28672: 256 workgroups of 32 rows;
// large layer stack at N = 1, int8 tokens 380 -> 365 us per step, fused
// bf16 455 -> 418 us).
static GemvGeometry gemv_geometry(int64_t K, int64_t total_rows, int mode) {
    GemvGeometry g;
    const int C = (int)(K >> 6);
    g.lpr = BITNET_GEMV_LPR ? BITNET_GEMV_LPR : pick_lpr(C, total_rows);
    g.long_rows = g.lpr == 64 && C > 4 * 64 && total_rows >= 4096;
    if (g.long_rows) {
        // as many row groups per wave as keep every workgroup resident in one
        // round (one 16-wave workgroup per CU at this kernel's register count)
        const int64_t round = (int64_t)kGemvWavesLong * 256;
        const int64_t iters = (total_rows + round - 1) / round;
        g.rows_per_wg = (int)(kGemvWavesLong * (iters < 1 ? 1 : iters));
        g.per = (int)(kLdsBytes / K) < 2 ? 1 : 2;
        return g;
    }
    const int rows_per_iter = kGemvWaves * (64 / g.lpr);   // rows per workgroup row-group step
    // Row groups per workgroup: one (every load in flight at once, a single
    // scheduling round) unless that would need more than ~1024 workgroups.
    const int64_t target = BITNET_GEMV_TARGET_WGS;
    int64_t iters = (total_rows + rows_per_iter * target - 1) / (rows_per_iter * target);
    if (iters < 1) iters = 1;
    g.rows_per_wg = (int)(rows_per_iter * iters);
    g.per = (int)(kLdsBytes / K);
    if (g.per > 2) g.per = 2;   // passes of at most two tokens (more run on MFMA)
    return g;
}

#ifdef BITNET_STAMPS
// Launch slots of the instrumented build, taken in launch order (at capture
// time for a captured graph) and wrapping after kStampSlots launches.  A slot
// is kStampSubs sub-slots on 128-byte lines of their own ([start, end] in
// the first 16 bytes); workgroup b stamps sub-slot b % kStampSubs, so the
// atomics of one launch spread over 64 lines instead of queueing on one.
constexpr int kStampSlots = 512;
constexpr int kStampStride = 16;   // unsigned long longs per sub-slot (128 bytes)
constexpr int kStampSlotLen = kStampSubs * kStampStride;
__device__ unsigned long long g_stamps[kStampSlots * kStampSlotLen];
static unsigned long long *g_stamps_addr[64];
static std::mutex g_stamps_mu;
static std::atomic<int> g_stamp_next{0};

static unsigned long long *stamps_base() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
    std::lock_guard<std::mutex> lock(g_stamps_mu);
    if (!g_stamps_addr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(g_stamps)) != hipSuccess) return nullptr;
        g_stamps_addr[dev] = static_cast<unsigned long long *>(p);
    }
    return g_stamps_addr[dev];
}

unsigned long long *stamp_slot() {
    unsigned long long *b = stamps_base();
    return b ? b + (size_t)(g_stamp_next++ % kStampSlots) * kStampSlotLen : nullptr;
}

__global__ void stamps_clear_kernel(unsigned long long *s) {
    const int i = blockIdx.x * 256 + threadIdx.x;   // sub-slot
    if (i < kStampSlots * kStampSubs) {
        s[(size_t)i * kStampStride] = ~0ull;
        s[(size_t)i * kStampStride + 1] = 0ull;
    }
}

int stamps_reset(int rewind, hipStream_t st) {
    unsigned long long *b = stamps_base();
    if (!b) return -1;
    if (rewind) g_stamp_next.store(0);
    hipLaunchKernelGGL(stamps_clear_kernel, dim3(kStampSlots * kStampSubs / 256), dim3(256), 0, st, b);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

// [min start, max end] over the sub-slots of each launch since the rewind
int stamps_read(unsigned long long *out, int max_launches) {
    unsigned long long *b = stamps_base();
    if (!b || max_launches < 0) return -1;
    const int used = g_stamp_next.load();
    int n = used < kStampSlots ? used : kStampSlots;
    if (n > max_launches) n = max_launches;
    if (hipDeviceSynchronize() != hipSuccess) return -1;
    std::vector<unsigned long long> h((size_t)n * kStampSlotLen);
    if (n && hipMemcpy(h.data(), b, h.size() * sizeof(unsigned long long), hipMemcpyDeviceToHost) !=
                 hipSuccess)
        return -1;
    for (int i = 0; i < n; ++i) {
        unsigned long long lo = ~0ull, hi = 0;
        for (int j = 0; j < kStampSubs; ++j) {
            const unsigned long long *q = &h[(size_t)i * kStampSlotLen + (size_t)j * kStampStride];
            if (q[0] < lo) lo = q[0];
            if (q[1] > hi) hi = q[1];
        }
        out[2 * i] = lo;
        out[2 * i + 1] = hi;
    }
    return n;
}
#endif

hipError_t launch_gemv_valu(const GemvMat *mats, int nmats, int64_t K, int64_t N,
                            int mode, const void *x, const float *xs,
                            const int32_t *xsum, int8_t *xq_out, float *xs_out,
                            int32_t *xsum_out, hipStream_t st) {
    int64_t total_rows = 0;
    for (int i = 0; i < nmats; ++i) total_rows += mats[i].M;
    const GemvGeometry geo = gemv_geometry(K, total_rows, mode);
    const int C = (int)(K >> 6);
    const int lpr = geo.lpr, rows_per_wg = geo.rows_per_wg, per = geo.per;
    const int esize = mode == 0 ? 1 : (mode == 1 ? 4 : 2);
    for (int64_t n0 = 0; n0 < N; n0 += per) {
        const int nt = (int)((N - n0) < per ? (N - n0) : per);
        GemvKernelArgs a{};
        int wg = 0;
        for (int i = 0; i < nmats; ++i) {
            a.mat[i] = mats[i];
            a.mat[i].wg_begin = wg;
            if (mats[i].dot) a.mat[i].dot = mats[i].dot + n0 * mats[i].M;
            if (mats[i].y) a.mat[i].y = mats[i].y + n0 * mats[i].M;
            wg += (mats[i].M + rows_per_wg - 1) / rows_per_wg;
        }
        a.nmats = nmats;
        a.K = (int)K;
        a.ntok = nt;
        a.rows_per_wg = rows_per_wg;
        a.x = reinterpret_cast<const char *>(x) + n0 * K * esize;
        if (mode == 0) {
            a.xs_in = xs + n0;
            a.xsum_in = xsum + n0;
        } else {
            a.xq_out = xq_out ? xq_out + n0 * K : nullptr;
            a.xs_out = xs_out ? xs_out + n0 : nullptr;
            a.xsum_out = xsum_out ? xsum_out + n0 : nullptr;
        }
        if (wg == 0) continue;
#ifdef BITNET_STAMPS
        a.stamp = stamp_slot();
#endif
        hipError_t e;
        const unsigned g = (unsigned)wg;
        // J <= 4: short-row kernels with exactly 3 or 4 chunk slots
        const int jn = (C + lpr - 1) / lpr;
        const int sr = nt == 1 && jn <= 4 ? (jn <= 3 ? 3 : 4) : 0;
        const bool lr = geo.long_rows;
        if (nt == 1)
            e = mode == 0 ? launch_gemv_nt<1, 0>(a, lpr, sr, lr, g, st)
              : mode == 1 ? launch_gemv_nt<1, 1>(a, lpr, sr, lr, g, st)
                          : launch_gemv_nt<1, 2>(a, lpr, sr, lr, g, st);
        else
            e = mode == 0 ? launch_gemv_nt<2, 0>(a, lpr, sr, lr, g, st)
              : mode == 1 ? launch_gemv_nt<2, 1>(a, lpr, sr, lr, g, st)
                          : launch_gemv_nt<2, 2>(a, lpr, sr, lr, g, st);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace bitnet
