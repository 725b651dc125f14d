// abi.hip -- the C ABI of libbitnet_i2s.so (declared in include/bitnet_i2s.h):
// host-side argument validation, error reporting and kernel dispatch.
#include <stdarg.h>
#include <stdio.h>

#include <mutex>
#include <string>

#include "bitnet_i2s.h"
#include "common.h"

#define BITNET_API extern "C" __attribute__((visibility("default")))

#ifndef BITNET_VALU_MAX_N
#define BITNET_VALU_MAX_N 2   // decode token counts served by the vector-ALU GEMV (MFMA above)
#endif

namespace {

thread_local std::string g_last_error;

int fail(int status, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return status;
}

int ok() {
    g_last_error.clear();
    return BITNET_OK;
}

int hip_fail(const char *where, hipError_t e) {
    return fail(BITNET_E_HIP, "%s: %s (%d)", where, hipGetErrorString(e), (int)e);
}

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

int check_k(const char *fn, int64_t K) {
    if (K <= 0 || K % bitnet::kBlock != 0 || K > BITNET_MAX_K)
        return fail(BITNET_E_SHAPE, "%s: K=%lld must be a positive multiple of 128 and <= %d",
                    fn, (long long)K, BITNET_MAX_K);
    return BITNET_OK;
}

// Device-side count of non-ternary weights seen by the packer.  Each device
// holds its own copy; its address is looked up once per device with
// hipGetSymbolAddress and only that address is used from the host.
__device__ unsigned g_pack_bad;
constexpr int kMaxDevices = 64;
void *g_pack_bad_addr[kMaxDevices];
std::mutex g_pack_mu;

int pack_counter(int dev, unsigned **out) {
    if (dev < 0 || dev >= kMaxDevices)
        return fail(BITNET_E_HIP, "bitnet_pack_i2s: device index %d unsupported", dev);
    if (!g_pack_bad_addr[dev]) {
        void *p = nullptr;
        hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(g_pack_bad));
        if (e != hipSuccess) return hip_fail("bitnet_pack_i2s: hipGetSymbolAddress", e);
        g_pack_bad_addr[dev] = p;
    }
    *out = static_cast<unsigned *>(g_pack_bad_addr[dev]);
    return BITNET_OK;
}

// Scratch of the one-time weight conversion calls (AbsMean partial sums, the
// scale, the non-finite count and max|w|).  Like the pack counter: one copy
// per device, its address looked up once per device, and the calls that use
// it serialised by g_pack_mu and synchronised before they return.
struct ConvScratch {
    uint32_t digits[bitnet::kConvPartials * bitnet::kConvDigits];   // AbsMean partial sums
    double partial[bitnet::kConvPartials];                          // max|w| per workgroup
    float alpha;
    unsigned bad;
    float wmax;
};
__device__ ConvScratch g_conv;
void *g_conv_addr[kMaxDevices];

int conv_scratch(const char *fn, ConvScratch **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(fn, e);
    if (dev < 0 || dev >= kMaxDevices)
        return fail(BITNET_E_HIP, "%s: device index %d unsupported", fn, dev);
    if (!g_conv_addr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(g_conv));
        if (e != hipSuccess) return hip_fail(fn, e);
        g_conv_addr[dev] = p;
    }
    *out = static_cast<ConvScratch *>(g_conv_addr[dev]);
    return BITNET_OK;
}

int check_matmul(const char *fn, const uint8_t *packed, int64_t M, int64_t K,
                 const int8_t *xq, const float *xs, const int32_t *xsum, int64_t N,
                 int64_t max_n, const int32_t *dot, const float *y) {
    if (M < 0 || N < 0)
        return fail(BITNET_E_SHAPE, "%s: negative size M=%lld N=%lld", fn, (long long)M,
                    (long long)N);
    if (M > 0x7fffffffLL)
        return fail(BITNET_E_SHAPE, "%s: M=%lld exceeds 2^31-1", fn, (long long)M);
    if (N > max_n)
        return fail(BITNET_E_SHAPE, "%s: N=%lld exceeds %lld", fn, (long long)N,
                    (long long)max_n);
    if (int s = check_k(fn, K)) return s;
    if (M == 0 || N == 0) return BITNET_OK;
    if (!packed || !xq || !xs || !xsum)
        return fail(BITNET_E_NULL, "%s: packed, xq, x_scale and x_sum are required", fn);
    if (!dot && !y) return fail(BITNET_E_NULL, "%s: dot and y are both NULL", fn);
    if (!aligned(packed, 16) || !aligned(xq, 16))
        return fail(BITNET_E_ALIGN, "%s: packed and xq must be 16-byte aligned", fn);
    if (!aligned(xs, 4) || !aligned(xsum, 4) || (dot && !aligned(dot, 4)) ||
        (y && !aligned(y, 4)))
        return fail(BITNET_E_ALIGN, "%s: x_scale, x_sum, dot, y must be 4-byte aligned", fn);
    return BITNET_OK;
}

}  // namespace

BITNET_API int bitnet_abi_version(void) { return BITNET_ABI_VERSION; }

BITNET_API const char *bitnet_last_error(void) { return g_last_error.c_str(); }

BITNET_API int bitnet_pack_i2s(const int8_t *w, int64_t M, int64_t K, uint8_t *packed,
                               void *stream) {
    const char *fn = "bitnet_pack_i2s";
    if (M < 0) return fail(BITNET_E_SHAPE, "%s: negative M=%lld", fn, (long long)M);
    if (int s = check_k(fn, K)) return s;
    if (M == 0) return ok();
    if (!w || !packed) return fail(BITNET_E_NULL, "%s: w and packed are required", fn);
    if (!aligned(w, 4) || !aligned(packed, 16))
        return fail(BITNET_E_ALIGN, "%s: w must be 4-byte and packed 16-byte aligned", fn);
    hipStream_t st = static_cast<hipStream_t>(stream);
    std::lock_guard<std::mutex> lock(g_pack_mu);
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail("bitnet_pack_i2s: hipGetDevice", e);
    unsigned *bad = nullptr;
    if (int s = pack_counter(dev, &bad)) return s;
    if ((e = hipMemsetAsync(bad, 0, sizeof(unsigned), st)) != hipSuccess)
        return hip_fail("bitnet_pack_i2s: clear counter", e);
    if ((e = bitnet::launch_pack(w, M, K, packed, bad, st)) != hipSuccess)
        return hip_fail("bitnet_pack_i2s: launch", e);
    unsigned nbad = 0;
    if ((e = hipMemcpyAsync(&nbad, bad, sizeof nbad, hipMemcpyDeviceToHost, st)) != hipSuccess)
        return hip_fail("bitnet_pack_i2s: read counter", e);
    if ((e = hipStreamSynchronize(st)) != hipSuccess)
        return hip_fail("bitnet_pack_i2s: synchronize", e);
    if (nbad)
        return fail(BITNET_E_VALUE, "%s: %u weight(s) outside {-1,0,+1}", fn, nbad);
    return ok();
}

BITNET_API int bitnet_absmean_i2s(const void *w, int dtype, int64_t M, int64_t K,
                                  uint8_t *packed, float *alpha, void *stream) {
    const char *fn = "bitnet_absmean_i2s";
    if (dtype != BITNET_F32 && dtype != BITNET_BF16)
        return fail(BITNET_E_DTYPE, "%s: unknown dtype %d", fn, dtype);
    if (M < 1) return fail(BITNET_E_SHAPE, "%s: M=%lld, need at least one row", fn, (long long)M);
    if (int s = check_k(fn, K)) return s;
    if (M > (1LL << 40) / K)
        return fail(BITNET_E_SHAPE, "%s: M*K exceeds 2^40 weights", fn);
    if (!w || !packed || !alpha) return fail(BITNET_E_NULL, "%s: w, packed and alpha are required", fn);
    if (!aligned(w, 16) || !aligned(packed, 16))
        return fail(BITNET_E_ALIGN, "%s: w and packed must be 16-byte aligned", fn);
    hipStream_t st = static_cast<hipStream_t>(stream);
    std::lock_guard<std::mutex> lock(g_pack_mu);
    ConvScratch *sc = nullptr;
    if (int s = conv_scratch(fn, &sc)) return s;
    hipError_t e = hipMemsetAsync(&sc->bad, 0, sizeof(unsigned), st);
    const int bf16 = dtype == BITNET_BF16;
    if (e == hipSuccess) e = bitnet::launch_absmean_alpha(w, bf16, M * K, sc->digits, &sc->alpha, st);
    if (e == hipSuccess)
        e = bitnet::launch_ternary_pack(w, bf16, 0, M, K, &sc->alpha, packed, &sc->bad, nullptr,
                                        nullptr, st);
    struct { float alpha; unsigned bad; } res{};
    if (e == hipSuccess) e = hipMemcpyAsync(&res, &sc->alpha, sizeof res, hipMemcpyDeviceToHost, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    if (e != hipSuccess) return hip_fail(fn, e);
    if (res.bad) return fail(BITNET_E_VALUE, "%s: %u non-finite weight(s)", fn, res.bad);
    *alpha = res.alpha;
    return ok();
}

BITNET_API int bitnet_pack_i2s_f32(const float *w, int64_t M, int64_t K, uint8_t *packed,
                                   float *w_max, void *stream) {
    const char *fn = "bitnet_pack_i2s_f32";
    if (M < 0) return fail(BITNET_E_SHAPE, "%s: negative M=%lld", fn, (long long)M);
    if (int s = check_k(fn, K)) return s;
    if (M == 0) {
        if (w_max) *w_max = 0.0f;
        return ok();
    }
    if (!w || !packed) return fail(BITNET_E_NULL, "%s: w and packed are required", fn);
    if (!aligned(w, 16) || !aligned(packed, 16))
        return fail(BITNET_E_ALIGN, "%s: w and packed must be 16-byte aligned", fn);
    hipStream_t st = static_cast<hipStream_t>(stream);
    std::lock_guard<std::mutex> lock(g_pack_mu);
    ConvScratch *sc = nullptr;
    if (int s = conv_scratch(fn, &sc)) return s;
    hipError_t e = hipMemsetAsync(&sc->bad, 0, sizeof(unsigned), st);
    if (e == hipSuccess)
        e = bitnet::launch_ternary_pack(w, 0, 1, M, K, nullptr, packed, &sc->bad, sc->partial,
                                        &sc->wmax, st);
    struct { unsigned bad; float wmax; } res{};
    if (e == hipSuccess) e = hipMemcpyAsync(&res, &sc->bad, sizeof res, hipMemcpyDeviceToHost, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    if (e != hipSuccess) return hip_fail(fn, e);
    if (res.bad) return fail(BITNET_E_VALUE, "%s: %u non-finite weight(s)", fn, res.bad);
    if (w_max) *w_max = res.wmax;
    return ok();
}

BITNET_API int bitnet_quant_act_i8(const void *x, int dtype, int64_t N, int64_t K, int8_t *xq,
                                   float *x_scale, int32_t *x_sum, void *stream) {
    const char *fn = "bitnet_quant_act_i8";
    if (dtype != BITNET_F32 && dtype != BITNET_BF16)
        return fail(BITNET_E_DTYPE, "%s: unknown dtype %d", fn, dtype);
    if (N < 0 || N > 0x7fffffffLL)
        return fail(BITNET_E_SHAPE, "%s: N=%lld out of range", fn, (long long)N);
    if (int s = check_k(fn, K)) return s;
    if (N == 0) return ok();
    if (!x || !xq || !x_scale || !x_sum)
        return fail(BITNET_E_NULL, "%s: x, xq, x_scale and x_sum are required", fn);
    if (!aligned(x, 16) || !aligned(xq, 16) || !aligned(x_scale, 4) || !aligned(x_sum, 4))
        return fail(BITNET_E_ALIGN, "%s: x and xq must be 16-byte aligned", fn);
    hipError_t e = bitnet::launch_quant(x, dtype == BITNET_BF16, N, K, xq, x_scale, x_sum,
                                        static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail("bitnet_quant_act_i8: launch", e);
    return ok();
}

BITNET_API int bitnet_gemv_i2s_i8(const uint8_t *packed, float w_scale, int64_t M, int64_t K,
                                  const int8_t *xq, const float *x_scale,
                                  const int32_t *x_sum, int64_t N, int32_t *dot, float *y,
                                  void *stream) {
    const char *fn = "bitnet_gemv_i2s_i8";
    if (int s = check_matmul(fn, packed, M, K, xq, x_scale, x_sum, N, BITNET_GEMV_MAX_N, dot, y))
        return s;
    if (M == 0 || N == 0) return ok();
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t e;
    if (N <= BITNET_VALU_MAX_N) {
        bitnet::GemvMat m{packed, dot, y, w_scale, (int)M, 0};
        e = bitnet::launch_gemv_valu(&m, 1, K, N, 0, xq, x_scale, x_sum, nullptr, nullptr,
                                     nullptr, st);
    } else {
        bitnet::GemmMat m{packed, dot, y, w_scale, (int)M, 0};
        e = bitnet::launch_gemv_mfma(&m, 1, K, xq, x_scale, x_sum, N, st);
    }
    if (e != hipSuccess) return hip_fail("bitnet_gemv_i2s_i8: launch", e);
    return ok();
}

BITNET_API int bitnet_gemv_i2s_lut(const uint8_t *packed, float w_scale, int64_t M, int64_t K,
                                   const int8_t *xq, const float *x_scale,
                                   const int32_t *x_sum, int64_t N, int32_t *dot, float *y,
                                   void *stream) {
    const char *fn = "bitnet_gemv_i2s_lut";
    if (int s = check_matmul(fn, packed, M, K, xq, x_scale, x_sum, N, BITNET_GEMV_MAX_N, dot, y))
        return s;
    if (K > BITNET_LUT_MAX_K)
        return fail(BITNET_E_SHAPE, "%s: K=%lld exceeds %d", fn, (long long)K, BITNET_LUT_MAX_K);
    if (M == 0 || N == 0) return ok();
    hipError_t e = bitnet::launch_gemv_lut(packed, w_scale, M, K, xq, x_scale, x_sum, N, dot, y,
                                           static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail("bitnet_gemv_i2s_lut: launch", e);
    return ok();
}

BITNET_API int bitnet_gemm_i2s_i8(const uint8_t *packed, float w_scale, int64_t M, int64_t K,
                                  const int8_t *xq, const float *x_scale,
                                  const int32_t *x_sum, int64_t N, int32_t *dot, float *y,
                                  void *stream) {
    const char *fn = "bitnet_gemm_i2s_i8";
    if (int s = check_matmul(fn, packed, M, K, xq, x_scale, x_sum, N, BITNET_GEMM_MAX_N, dot, y))
        return s;
    if (M == 0 || N == 0) return ok();
    const bitnet::GemmMat m{packed, dot, y, w_scale, (int)M, 0};
    hipError_t e = bitnet::launch_gemm_mfma(&m, 1, K, xq, x_scale, x_sum, N,
                                            static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail("bitnet_gemm_i2s_i8: launch", e);
    return ok();
}

// Validate a host array of matrix descriptors (shared by the grouped calls).
static int check_mats(const char *fn, const bitnet_i2s_matrix *mats, int n_mats) {
    if (n_mats < 1 || n_mats > BITNET_MAX_GROUP)
        return fail(BITNET_E_SHAPE, "%s: n_mats=%d outside [1, %d]", fn, n_mats,
                    BITNET_MAX_GROUP);
    if (!mats) return fail(BITNET_E_NULL, "%s: mats is NULL", fn);
    for (int i = 0; i < n_mats; ++i) {
        const bitnet_i2s_matrix &m = mats[i];
        if (m.M < 0 || m.M > 0x7fffffffLL)
            return fail(BITNET_E_SHAPE, "%s: mats[%d].M=%lld out of range", fn, i, (long long)m.M);
        if (m.M > 0) {
            if (!m.packed) return fail(BITNET_E_NULL, "%s: mats[%d].packed is NULL", fn, i);
            if (!m.dot && !m.y)
                return fail(BITNET_E_NULL, "%s: mats[%d] has neither dot nor y", fn, i);
            if (!aligned(m.packed, 16))
                return fail(BITNET_E_ALIGN, "%s: mats[%d].packed must be 16-byte aligned", fn, i);
            if ((m.dot && !aligned(m.dot, 4)) || (m.y && !aligned(m.y, 4)))
                return fail(BITNET_E_ALIGN, "%s: mats[%d] outputs must be 4-byte aligned", fn, i);
        }
    }
    return BITNET_OK;
}

BITNET_API int bitnet_ffn_act_quant_i8(const float *g, const float *u, const float *gamma,
                                      float eps, int64_t N, int64_t F, int8_t *xq,
                                      float *x_scale, int32_t *x_sum, void *stream) {
    const char *fn = "bitnet_ffn_act_quant_i8";
    if (N < 0) return fail(BITNET_E_SHAPE, "%s: negative N=%lld", fn, (long long)N);
    if (N > 0x7fffffffLL) return fail(BITNET_E_SHAPE, "%s: N=%lld exceeds 2^31-1", fn, (long long)N);
    if (int s = check_k(fn, F)) return s;
    if (!(eps > 0.0f) || !(eps < 3.4e38f))
        return fail(BITNET_E_VALUE, "%s: eps must be positive and finite", fn);
    if (N == 0) return ok();
    if (!g || !u || !xq || !x_scale || !x_sum)
        return fail(BITNET_E_NULL, "%s: g, u, xq, x_scale and x_sum are required", fn);
    if (!aligned(g, 16) || !aligned(u, 16) || (gamma && !aligned(gamma, 16)) ||
        !aligned(xq, 16) || !aligned(x_scale, 4) || !aligned(x_sum, 4))
        return fail(BITNET_E_ALIGN, "%s: g, u, gamma and xq must be 16-byte aligned", fn);
    hipError_t e = bitnet::launch_ffn_act_quant(g, u, gamma, eps, N, F, xq, x_scale, x_sum,
                                                static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(fn, e);
    return ok();
}

BITNET_API int bitnet_gemv_i2s_i8_group(const bitnet_i2s_matrix *mats, int n_mats, int64_t K,
                                        const int8_t *xq, const float *x_scale,
                                        const int32_t *x_sum, int64_t N, void *stream) {
    const char *fn = "bitnet_gemv_i2s_i8_group";
    if (int s = check_mats(fn, mats, n_mats)) return s;
    if (N < 0 || N > BITNET_GEMV_MAX_N)
        return fail(BITNET_E_SHAPE, "%s: N=%lld outside [0, %d]", fn, (long long)N,
                    BITNET_GEMV_MAX_N);
    if (int s = check_k(fn, K)) return s;
    int64_t rows = 0;
    for (int i = 0; i < n_mats; ++i) rows += mats[i].M;
    if (N == 0 || rows == 0) return ok();
    if (!xq || !x_scale || !x_sum)
        return fail(BITNET_E_NULL, "%s: xq, x_scale and x_sum are required", fn);
    if (!aligned(xq, 16) || !aligned(x_scale, 4) || !aligned(x_sum, 4))
        return fail(BITNET_E_ALIGN, "%s: xq must be 16-byte and x_scale/x_sum 4-byte aligned", fn);
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t e = hipSuccess;
    if (N <= BITNET_VALU_MAX_N) {
        bitnet::GemvMat gm[bitnet::kMaxMats];
        for (int i = 0; i < n_mats; ++i)
            gm[i] = bitnet::GemvMat{mats[i].packed, mats[i].dot, mats[i].y, mats[i].w_scale,
                                    (int)mats[i].M, 0};
        e = bitnet::launch_gemv_valu(gm, n_mats, K, N, 0, xq, x_scale, x_sum, nullptr, nullptr,
                                     nullptr, st);
    } else {
        bitnet::GemmMat mm[bitnet::kMaxMats];
        for (int i = 0; i < n_mats; ++i)
            mm[i] = bitnet::GemmMat{mats[i].packed, mats[i].dot, mats[i].y, mats[i].w_scale,
                                    (int)mats[i].M, 0};
        e = bitnet::launch_gemv_mfma(mm, n_mats, K, xq, x_scale, x_sum, N, st);
    }
    if (e != hipSuccess) return hip_fail(fn, e);
    return ok();
}

BITNET_API int bitnet_gemm_i2s_i8_group(const bitnet_i2s_matrix *mats, int n_mats, int64_t K,
                                        const int8_t *xq, const float *x_scale,
                                        const int32_t *x_sum, int64_t N, void *stream) {
    const char *fn = "bitnet_gemm_i2s_i8_group";
    if (int s = check_mats(fn, mats, n_mats)) return s;
    if (N < 0 || N > BITNET_GEMM_MAX_N)
        return fail(BITNET_E_SHAPE, "%s: N=%lld outside [0, %d]", fn, (long long)N,
                    BITNET_GEMM_MAX_N);
    if (int s = check_k(fn, K)) return s;
    bitnet::GemmMat gm[bitnet::kMaxMats];
    int64_t rows = 0;
    for (int i = 0; i < n_mats; ++i) {
        gm[i] = bitnet::GemmMat{mats[i].packed, mats[i].dot, mats[i].y, mats[i].w_scale,
                                (int)mats[i].M, 0};
        rows += mats[i].M;
    }
    if (N == 0 || rows == 0) return ok();
    if (!xq || !x_scale || !x_sum)
        return fail(BITNET_E_NULL, "%s: xq, x_scale and x_sum are required", fn);
    if (!aligned(xq, 16) || !aligned(x_scale, 4) || !aligned(x_sum, 4))
        return fail(BITNET_E_ALIGN, "%s: xq must be 16-byte and x_scale/x_sum 4-byte aligned", fn);
    hipError_t e = bitnet::launch_gemm_mfma(gm, n_mats, K, xq, x_scale, x_sum, N,
                                            static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(fn, e);
    return ok();
}

static int linear_impl(const char *fn, const void *x, int dtype, int64_t N, int64_t K,
                       const bitnet_i2s_matrix *mats, int n_mats, int8_t *xq, float *x_scale,
                       int32_t *x_sum, void *stream) {
    if (dtype != BITNET_F32 && dtype != BITNET_BF16)
        return fail(BITNET_E_DTYPE, "%s: unknown dtype %d", fn, dtype);
    if (N < 0 || N > BITNET_GEMM_MAX_N)
        return fail(BITNET_E_SHAPE, "%s: N=%lld outside [0, %d]", fn, (long long)N,
                    BITNET_GEMM_MAX_N);
    if (int s = check_k(fn, K)) return s;
    if (int s = check_mats(fn, mats, n_mats)) return s;
    bitnet::GemvMat gm[bitnet::kMaxMats];
    for (int i = 0; i < n_mats; ++i)
        gm[i] = bitnet::GemvMat{mats[i].packed, mats[i].dot, mats[i].y, mats[i].w_scale,
                                (int)mats[i].M, 0};
    if (N == 0) return ok();
    if (!x) return fail(BITNET_E_NULL, "%s: x is NULL", fn);
    if (!aligned(x, 16) || (xq && !aligned(xq, 16)) || (x_scale && !aligned(x_scale, 4)) ||
        (x_sum && !aligned(x_sum, 4)))
        return fail(BITNET_E_ALIGN, "%s: x/xq must be 16-byte and x_scale/x_sum 4-byte aligned", fn);
    if (N > BITNET_LINEAR_FUSED_MAX_N && (!xq || !x_scale || !x_sum))
        return fail(BITNET_E_NULL, "%s: N > %d needs the xq, x_scale and x_sum buffers", fn,
                    BITNET_LINEAR_FUSED_MAX_N);
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t e;
    if (N <= BITNET_LINEAR_FUSED_MAX_N) {
        e = bitnet::launch_gemv_valu(gm, n_mats, K, N, dtype == BITNET_BF16 ? 2 : 1, x, nullptr,
                                     nullptr, xq, x_scale, x_sum, st);
    } else if (N <= BITNET_GEMV_MAX_N) {
        e = bitnet::launch_quant(x, dtype == BITNET_BF16, N, K, xq, x_scale, x_sum, st);
        if (e == hipSuccess) {
            bitnet::GemmMat mm[bitnet::kMaxMats];
            for (int i = 0; i < n_mats; ++i)
                mm[i] = bitnet::GemmMat{gm[i].packed, gm[i].dot, gm[i].y, gm[i].alpha, gm[i].M, 0};
            e = bitnet::launch_gemv_mfma(mm, n_mats, K, xq, x_scale, x_sum, N, st);
        }
    } else {
        e = bitnet::launch_quant(x, dtype == BITNET_BF16, N, K, xq, x_scale, x_sum, st);
        if (e == hipSuccess) {
            bitnet::GemmMat mm[bitnet::kMaxMats];
            for (int i = 0; i < n_mats; ++i)
                mm[i] = bitnet::GemmMat{gm[i].packed, gm[i].dot, gm[i].y, gm[i].alpha, gm[i].M, 0};
            e = bitnet::launch_gemm_mfma(mm, n_mats, K, xq, x_scale, x_sum, N, st);
        }
    }
    if (e != hipSuccess) return hip_fail(fn, e);
    return ok();
}

BITNET_API int bitnet_linear_i2s(const void *x, int dtype, int64_t N, int64_t K,
                                 const bitnet_i2s_matrix *mats, int n_mats, int8_t *xq,
                                 float *x_scale, int32_t *x_sum, void *stream) {
    return linear_impl("bitnet_linear_i2s", x, dtype, N, K, mats, n_mats, xq, x_scale, x_sum,
                       stream);
}

#ifdef BITNET_STAMPS
// Instrumented build only (include/bitnet_i2s_stamps.h).
namespace bitnet {
int stamps_reset(int rewind, hipStream_t st);
int stamps_read(unsigned long long *out, int max_launches);
}  // namespace bitnet

BITNET_API int bitnet_stamps_reset(int rewind, void *stream) {
    if (bitnet::stamps_reset(rewind, static_cast<hipStream_t>(stream)) != 0)
        return fail(BITNET_E_HIP, "bitnet_stamps_reset: no stamp slots on this device");
    return ok();
}

BITNET_API int bitnet_stamps_read(uint64_t *out, int max_launches) {
    if (!out && max_launches > 0) return -1;
    return bitnet::stamps_read(reinterpret_cast<unsigned long long *>(out), max_launches);
}
#endif
