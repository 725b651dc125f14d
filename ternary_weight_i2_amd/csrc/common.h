// common.h -- device helpers and launcher declarations shared by the HIP
// translation units of libbitnet_i2s.so (library-internal; not installed).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bitnet {

// I2_S block: 128 weights in 32 bytes; byte j of a block holds the 2-bit codes
// of block positions j, j+32, j+64, j+96 in bits 7-6, 5-4, 3-2, 1-0.
constexpr int kBlock = 128;
constexpr int kBlockBytes = 32;
constexpr int kXcds = 8;   // MI355X: 8 XCDs (own L2 each); workgroups dealt round-robin

typedef int v4i __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int dot4(int a, int b, int c) {
    // v_dot4_i32_i8: c + sum of the four signed byte products
    return __builtin_amdgcn_sdot4(a, b, c, false);
}

// Cross-lane moves through DPP (no LDS round trip).  Inside a row of 16
// lanes: quad_perm [1,0,3,2] and [2,3,0,1] swap neighbours at distance 1 and
// 2; row_half_mirror reads lane 7-i of each 8-lane half row; row_mirror reads
// lane 15-i of the row.  Across rows (gfx9 DPP): row_bcast:15 hands lane 15 of
// each row to the next row, row_bcast:31 hands lane 31 to rows 2 and 3.
constexpr int kDppXor1 = 0xB1;
constexpr int kDppXor2 = 0x4E;
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppMirror = 0x140;
constexpr int kDppRowBcast15 = 0x142;
constexpr int kDppRowBcast31 = 0x143;
template <int CTRL>
__device__ __forceinline__ int dpp_i32(int v) {
    return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, true);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
    return __int_as_float(dpp_i32<CTRL>(__float_as_int(v)));
}
// A cross-row move into the rows of ROWMASK only; the other rows receive 0.
template <int CTRL, int ROWMASK>
__device__ __forceinline__ int dpp_rows_i32(int v) {
    return __builtin_amdgcn_update_dpp(0, v, CTRL, ROWMASK, 0xF, false);
}

// Sum over each aligned group of L lanes (L = 8, 16, 32 or 64).  Once
// neighbours at distance 1 and 2 are added every lane holds its quad's sum,
// so mirroring within 8 and then 16 lanes pairs whole quads and then whole
// halves: for L <= 16 every lane of the group receives the sum.  Groups of 32
// and 64 lanes then add whole rows with row_bcast: the sum is complete in the
// group's last row of 16 lanes only (lanes 16..31 of a 32-lane group, 48..63
// of the wave).
template <int L>
__device__ __forceinline__ int group_sum_i32(int v) {
    static_assert(L == 8 || L == 16 || L == 32 || L == 64, "group of 8..64 lanes");
    v += dpp_i32<kDppXor1>(v);
    v += dpp_i32<kDppXor2>(v);
    v += dpp_i32<kDppHalfMirror>(v);
    if constexpr (L >= 16) v += dpp_i32<kDppMirror>(v);
    if constexpr (L >= 32) v += dpp_rows_i32<kDppRowBcast15, 0xA>(v);   // rows 1, 3 += rows 0, 2
    if constexpr (L >= 64) v += dpp_rows_i32<kDppRowBcast31, 0xC>(v);   // rows 2, 3 += rows 0-1
    return v;
}
// Wave-wide sum, returned to every lane (read from lane 63).
__device__ __forceinline__ int wave_sum_i32(int v) {
    return __builtin_amdgcn_readlane(group_sum_i32<64>(v), 63);
}
// Wave-wide maximum of non-negative values, returned to every lane (fmaxf
// ignores a NaN operand; the rows a cross-row move skips receive 0, which
// cannot raise the maximum).
__device__ __forceinline__ float wave_max_f32(float v) {
    v = fmaxf(v, dpp_f32<kDppXor1>(v));
    v = fmaxf(v, dpp_f32<kDppXor2>(v));
    v = fmaxf(v, dpp_f32<kDppHalfMirror>(v));
    v = fmaxf(v, dpp_f32<kDppMirror>(v));
    v = fmaxf(v, __int_as_float(dpp_rows_i32<kDppRowBcast15, 0xA>(__float_as_int(v))));
    v = fmaxf(v, __int_as_float(dpp_rows_i32<kDppRowBcast31, 0xC>(__float_as_int(v))));
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}
// 64-bit lane moves (two 32-bit DPP moves) and the wave-wide sum of 64-bit
// integers, returned to every lane (read from lane 63).
template <int CTRL>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
    const uint32_t lo = (uint32_t)dpp_i32<CTRL>((int)(uint32_t)v);
    const uint32_t hi = (uint32_t)dpp_i32<CTRL>((int)(uint32_t)(v >> 32));
    return (uint64_t)hi << 32 | lo;
}
template <int CTRL, int ROWMASK>
__device__ __forceinline__ uint64_t dpp_rows_u64(uint64_t v) {
    const uint32_t lo = (uint32_t)dpp_rows_i32<CTRL, ROWMASK>((int)(uint32_t)v);
    const uint32_t hi = (uint32_t)dpp_rows_i32<CTRL, ROWMASK>((int)(uint32_t)(v >> 32));
    return (uint64_t)hi << 32 | lo;
}
__device__ __forceinline__ uint64_t readlane63_u64(uint64_t v) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, 63);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), 63);
    return (uint64_t)hi << 32 | lo;
}
__device__ __forceinline__ uint64_t wave_sum_u64(uint64_t v) {
    v += dpp_u64<kDppXor1>(v);
    v += dpp_u64<kDppXor2>(v);
    v += dpp_u64<kDppHalfMirror>(v);
    v += dpp_u64<kDppMirror>(v);
    v += dpp_rows_u64<kDppRowBcast15, 0xA>(v);
    v += dpp_rows_u64<kDppRowBcast31, 0xC>(v);
    return readlane63_u64(v);
}

// s_waitcnt immediate that waits until at most `v` vector-memory operations of
// this wave are outstanding and ignores the other counters (gfx9 encoding:
// vmcnt[3:0], expcnt[6:4], lgkmcnt[11:8], vmcnt[5:4] in bits 15:14).
template <int v>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(v >= 0 && v < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((v & 0xF) | (0x7 << 4) | (0xF << 8) | ((v >> 4) << 14));
}

// One LDS-DMA load: 16 bytes per lane from `g` to LDS address M0 + 16*lane.
// Issued through inline asm so the compiler does not attach its conservative
// "wait for every outstanding load" to later LDS reads; the kernel waits with
// explicit vmcnt counts instead.  M0 is set here and used by nothing else in
// the kernels that call this.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const void *g, uint32_t lds_addr) {
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
                 :
                 : "v"(g), "s"(lds_addr)
                 : "memory", "m0");
}
#pragma clang diagnostic pop

// LDS byte address (what M0 takes) of a pointer into a __shared__ array: the
// low 32 bits of its generic address.
__device__ __forceinline__ uint32_t lds_addr_of(const void *p) {
    return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)p);
}

// Per-token quantisation arithmetic, shared by the stand-alone quantiser and
// the fused decode prologue so both produce identical bits:
//   s = 127 / max(amax, 1e-5), the correctly rounded fp32 quotient (computed
//   in binary64 and rounded once: 53 >= 2*24 + 2 makes that exact), and
//   q = clamp(round_half_even(x * s), -128, 127) with x * s one fp32 product.
__device__ __forceinline__ float quant_scale(float amax) {
    const float denom = amax > 1e-5f ? amax : 1e-5f;
    return (float)(127.0 / (double)denom);
}
// quant_bits gives q in the low byte of its result: adding 1.5 * 2^23 to the
// fp32 product rounds it to an integer, half to even, and leaves that integer
// in the low mantissa bits -- the low byte is its two's complement int8.  No
// clamp is needed for finite tokens: |x| <= max(amax, 1e-5) and s is that
// bound's 127 / d rounded, so |x * s| <= 127 (1 + 2^-24)^2 < 127.5 rounds to
// at most 127 in magnitude.  Two VALU operations, with no conversion to int
// and no shifts for packing.
__device__ __forceinline__ uint32_t quant_bits(float v, float s) {
#pragma clang fp contract(off)
    const float t = v * s;   // rounded on its own: never fused with the add
    return __float_as_uint(t + 12582912.0f);
}
// Low bytes of four words -> one word (b0 in byte 0): three v_perm_b32.
__device__ __forceinline__ uint32_t pack_low_bytes(uint32_t b0, uint32_t b1, uint32_t b2,
                                                   uint32_t b3) {
    const uint32_t lo = __builtin_amdgcn_perm(b1, b0, 0x0c0c0400u);   // b0.0 b1.0 0 0
    const uint32_t hi = __builtin_amdgcn_perm(b3, b2, 0x0c0c0400u);   // b2.0 b3.0 0 0
    return __builtin_amdgcn_perm(hi, lo, 0x05040100u);
}
// Sum of the four int8 codes of a packed word, added to acc.
__device__ __forceinline__ int sum_codes4(uint32_t packed, int acc) {
    return __builtin_amdgcn_sdot4((int)packed, 0x01010101, acc, false);
}

// Grouped decode launch: up to kMaxMats matrices that share K and the same
// tokens; workgroups [wg_begin, next wg_begin) serve matrix i.
constexpr int kMaxMats = 8;
struct GemvMat {
    const uint8_t *packed;
    int32_t *dot;
    float *y;
    float alpha;
    int M;
    int wg_begin;
};
struct GemvArgs {
    GemvMat mat[kMaxMats];
    int nmats;
    int K;
    int ntok;
    int rows_per_wg;
    const void *x;          // int8 xq (mode 0), fp32 (mode 1) or bf16 (mode 2) tokens
    const float *xs_in;     // mode 0: per-token scale
    const int32_t *xsum_in; // mode 0: per-token sum of xq
    int8_t *xq_out;         // modes 1/2, optional: quantised tokens
    float *xs_out;          // modes 1/2, optional
    int32_t *xsum_out;      // modes 1/2, optional
};

// ---- launchers (each returns the hipError_t of its launch) ---------------
hipError_t launch_pack(const int8_t *w, int64_t M, int64_t K, uint8_t *packed,
                       unsigned *bad, hipStream_t st);
hipError_t launch_quant(const void *x, int bf16, int64_t N, int64_t K,
                        int8_t *xq, float *xs, int32_t *xsum, hipStream_t st);
// Decode GEMV on the vector ALUs for any N (tokens are processed in passes of
// at most 2).  mode 0: x is int8 xq with xs/xsum given; mode 1/2: x is fp32 /
// bf16 and is quantised inside the kernel (xq_out/xs_out/xsum_out optional).
hipError_t launch_gemv_valu(const GemvMat *mats, int nmats, int64_t K, int64_t N,
                            int mode, const void *x, const float *xs,
                            const int32_t *xsum, int8_t *xq_out, float *xs_out,
                            int32_t *xsum_out, hipStream_t st);
// Decode matmul by table lookup (per-token nibble-group tables in LDS, then
// lookups); 1 <= N, K <= 8192 (the tables take 16*K bytes of LDS).
hipError_t launch_gemv_lut(const uint8_t *packed, float alpha, int64_t M, int64_t K,
                           const int8_t *xq, const float *xs, const int32_t *xsum, int64_t N,
                           int32_t *dot, float *y, hipStream_t st);
// Prefill launch over up to kMaxMats matrices that share K and the tokens;
// output tiles [tile_begin, next tile_begin) belong to matrix i.
struct GemmMat {
    const uint8_t *packed;
    int32_t *dot;
    float *y;
    float alpha;
    int M;
    int tile_begin;
};
struct GemmArgs {
    GemmMat mat[kMaxMats];
    int nmats;
    int K;
    int N;
    const int8_t *xq;
    const float *xs;
    const int32_t *xsum;
};
// Batched decode (1..64 tokens) on MFMA, weights streamed once: every matrix
// of `mats` (M > 0) times the same quantised tokens, in one launch.
hipError_t launch_gemv_mfma(const GemmMat *mats, int nmats, int64_t K, const int8_t *xq,
                            const float *xs, const int32_t *xsum, int64_t N, hipStream_t st);
// Prefill (any token count) on int8 MFMA: every matrix of `mats` (M > 0)
// times the same quantised tokens, in one launch.
hipError_t launch_gemm_mfma(const GemmMat *mats, int nmats, int64_t K, const int8_t *xq,
                            const float *xs, const int32_t *xsum, int64_t N, hipStream_t st);

// Squared-ReLU gated FFN activation + sub-norm + int8 quantisation, one
// workgroup per token (F a multiple of 128, at most 32768).
hipError_t launch_ffn_act_quant(const float *g, const float *u, const float *gamma, float eps,
                                int64_t N, int64_t F, int8_t *xq, float *xs, int32_t *xsum,
                                hipStream_t st);

// One-time weight conversion (AbsMean ternariser, sign/threshold packer).
constexpr int kConvPartials = 1024;   // workgroups of the AbsMean and max reductions
constexpr int kConvDigits = 12;       // 32-bit digits of one exact partial sum of |w|
hipError_t launch_absmean_alpha(const void *w, int bf16, int64_t n, uint32_t *partial,
                                float *alpha, hipStream_t st);
hipError_t launch_ternary_pack(const void *w, int bf16, int mode, int64_t M, int64_t K,
                               const float *alpha, uint8_t *packed, unsigned *bad,
                               double *part, float *wmax, hipStream_t st);

}  // namespace bitnet
