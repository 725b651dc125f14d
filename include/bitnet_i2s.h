/*
 * bitnet_i2s.h -- C ABI of libbitnet_i2s.so, the MI355X (gfx950) BitNet b1.58
 * W2A8 matmul: ternary weights packed as I2_S, per-token absmax int8
 * activations, exact int32 dots and fp32 scaled outputs.
 *
 * Sources (web pages, cited by key and section):
 *   [P1] "BitNet 딥다이브 -- 작은 숫자를 빠른 연산으로 바꾸는 추론 엔진"
 *        (fiv.co.kr/repos/BitNet-deep-dive.html)
 *   [P2] "[분석/검증-3] BitNet.cpp ARM 커널 재작성 : 스칼라 폴백구현을 통한
 *        최종 검증" (uno-kim.tistory.com/459)
 *   [P3] "[기술 분석 보고서] ARM64 모바일 환경에서의 1.58-bit 양자화 모델 추론
 *        붕괴 원인 분석 및 C++ 커널 역공학을 통한 해결" (uno-kim.tistory.com/461)
 *   [P4] "bitnet.rs -- BitNet b1.58 Inference Engine in Rust",
 *        section "Mathematical Foundation"
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Notation: M = output rows (weight rows), K = reduction length, N = tokens.
 *    K must be a positive multiple of 128 (one I2_S block, [P1 §4-2]) and at
 *    most BITNET_MAX_K.
 *  - All pointers except `stream` are DEVICE pointers to caller-owned memory,
 *    row-major and densely packed.  The library never allocates, frees or
 *    retains caller memory and keeps no handles; it is reentrant.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Every
 *    call only enqueues work and returns without synchronising, except
 *    bitnet_pack_i2s (see there).
 *  - Arguments are validated on the host before anything is enqueued.  On any
 *    non-zero return nothing has been launched and no output written (except
 *    BITNET_E_VALUE / BITNET_E_HIP after a launch, documented per call).
 *    bitnet_last_error() then describes the failure.
 *  - M == 0 or N == 0 is a valid no-op returning BITNET_OK.
 *  - Results are deterministic: integer sums are exact and order-free, so
 *    repeated calls produce bit-identical int32 and fp32 outputs.
 */
#ifndef BITNET_I2S_H
#define BITNET_I2S_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BITNET_ABI_VERSION 2
#define BITNET_MAX_K 32768          /* largest supported reduction length   */
#define BITNET_GEMV_MAX_N 64        /* largest token count of the decode call */
#define BITNET_GEMM_MAX_N (1 << 21) /* largest token count of the prefill call */
#define BITNET_MAX_GROUP 8          /* matrices per bitnet_linear_i2s call     */
#define BITNET_LINEAR_FUSED_MAX_N 2 /* bitnet_linear_i2s: one fused launch up to this N */
#define BITNET_LUT_MAX_K 8192       /* largest K of the table-lookup decode call */

typedef enum {
    BITNET_OK = 0,
    BITNET_E_NULL = 1,   /* a required pointer is NULL                        */
    BITNET_E_SHAPE = 2,  /* negative size, K % 128 != 0, K or N out of range  */
    BITNET_E_ALIGN = 3,  /* a pointer lacks the alignment stated below        */
    BITNET_E_DTYPE = 4,  /* unknown activation dtype                          */
    BITNET_E_VALUE = 5,  /* pack saw a weight outside {-1, 0, +1}             */
    BITNET_E_HIP = 6     /* HIP launch/runtime error (text in last_error)     */
} bitnet_status;

typedef enum { BITNET_F32 = 0, BITNET_BF16 = 1 } bitnet_dtype;

/*
 * bitnet_pack_i2s -- ternary int8 weights -> I2_S bytes  [P1 §1-1, §4-2]
 *
 *   w       [M][K] int8, every entry in {-1, 0, +1}; 4-byte aligned.
 *   packed  [M][K/4] uint8 output; 16-byte aligned.  Weight (m, k) is stored
 *           as code w+1 (-1 -> 0b00, 0 -> 0b01, +1 -> 0b10 [P1 §1-1]) in byte
 *           m*K/4 + 32*(k/128) + (k%128)%32, at bit 6 - 2*((k%128)/32):
 *           byte j of a 128-weight block carries elements j, j+32, j+64, j+96,
 *           the first in bits 7-6 [P1 §4-2].  Code 0b11 is never written.
 *
 * Packing is a one-time, offline step, so this call synchronises `stream` to
 * read back a device-side count of non-ternary inputs and returns
 * BITNET_E_VALUE if there were any; the contents of `packed` are then
 * unspecified.  Calls on one device serialise on that count internally.
 */
int bitnet_pack_i2s(const int8_t *w, int64_t M, int64_t K, uint8_t *packed,
                    void *stream);

/*
 * bitnet_quant_act_i8 -- per-token absmax int8 quantisation  [P1 §4-5; P4]
 *
 *   x        [N][K] activations, fp32 (dtype BITNET_F32) or bf16 (BITNET_BF16);
 *            16-byte aligned.  bf16 is widened exactly to fp32 first.
 *   xq       [N][K] int8 output, 16-byte aligned.
 *   x_scale  [N] fp32 output: s_n = 127 / max(max_k |x[n][k]|, 1e-5), the
 *            correctly rounded fp32 quotient (a multiplier, not 1/s).
 *   x_sum    [N] int32 output: sum_k xq[n][k] (needed by the raw-code dot).
 *
 * xq[n][k] = clamp(round_half_even(x[n][k] * s_n), -128, 127) with x*s a
 * single fp32 product (only -127..127 is reachable).  Non-finite inputs give
 * unspecified results.
 */
int bitnet_quant_act_i8(const void *x, int dtype, int64_t N, int64_t K,
                        int8_t *xq, float *x_scale, int32_t *x_sum,
                        void *stream);

/*
 * bitnet_gemv_i2s_i8 -- decode matmul, 1 <= N <= BITNET_GEMV_MAX_N tokens
 * bitnet_gemm_i2s_i8 -- prefill matmul, 0 <= N <= BITNET_GEMM_MAX_N (int8 MFMA)
 *
 *   packed   [M][K/4] I2_S weights (as written by bitnet_pack_i2s), 16-byte
 *            aligned.  A slot holding code 0b11 gives unspecified results.
 *   w_scale  per-tensor weight scale alpha (AbsMean, weight = code-1 times
 *            alpha [P1 §6-2; P4]).
 *   xq, x_scale, x_sum  as produced by bitnet_quant_act_i8 for N tokens;
 *            xq 16-byte aligned.
 *   dot      [N][M] int32 output or NULL:
 *              dot[n][m] = sum_k (code(m,k) - 1) * xq[n][k]
 *            computed as the raw-code sum minus x_sum[n], the exact offset
 *            correction of [P2 §3; P3 §3.2] (never the zero-mean shortcut).
 *   y        [N][M] fp32 output or NULL: y[n][m] = dot[n][m] * w_scale /
 *            x_scale[n], the caller-side scaling of [P2 §3] (relative error
 *            below 1e-6; exactly 0 where dot is 0).
 *   At least one of dot / y must be non-NULL.
 *
 * gemv returns BITNET_E_SHAPE for N > BITNET_GEMV_MAX_N, gemm for
 * N > BITNET_GEMM_MAX_N; both for M > 2^31-1.
 */
int bitnet_gemv_i2s_i8(const uint8_t *packed, float w_scale, int64_t M,
                       int64_t K, const int8_t *xq, const float *x_scale,
                       const int32_t *x_sum, int64_t N, int32_t *dot, float *y,
                       void *stream);

int bitnet_gemm_i2s_i8(const uint8_t *packed, float w_scale, int64_t M,
                       int64_t K, const int8_t *xq, const float *x_scale,
                       const int32_t *x_sum, int64_t N, int32_t *dot, float *y,
                       void *stream);

/*
 * bitnet_gemv_i2s_lut -- the decode matmul of bitnet_gemv_i2s_i8 computed by
 * table lookup instead of unpacking the codes [P1 §4-3, §4-4 (the LUT route:
 * tables are built from the activations alone, then, after a barrier, the
 * weights index them); P1 §11-2 (T-MAC)].  For each token the call tabulates,
 * for every pair of 2-bit fields sharing a nibble of an I2_S byte, the 16
 * raw-code sums c_hi * x_first + c_lo * x_second, then sums one table entry
 * per nibble of each row; D = that sum minus x_sum[n].
 *
 * Arguments, layouts, outputs and errors are those of bitnet_gemv_i2s_i8
 * (identical dot and y, bit for bit), plus BITNET_E_SHAPE for
 * K > BITNET_LUT_MAX_K (the tables of a token live in 16*K bytes of LDS).
 * Weights are read once per token (no reuse across tokens): meant for N = 1.
 */
int bitnet_gemv_i2s_lut(const uint8_t *packed, float w_scale, int64_t M,
                        int64_t K, const int8_t *xq, const float *x_scale,
                        const int32_t *x_sum, int64_t N, int32_t *dot, float *y,
                        void *stream);

/*
 * bitnet_linear_i2s -- fused decode linear: quantise tokens and multiply them
 * by up to BITNET_MAX_GROUP I2_S matrices that share them, in one launch.
 * [P1 §4-5 (per-token scale), §4-3 (a weight block reused for several
 * activation columns); P2 §3; P3 §3.2]
 *
 *   x        [N][K] fp32 or bf16 tokens (as bitnet_quant_act_i8), 16-byte aligned.
 *   mats     host array of n_mats descriptors, read during the call only:
 *              packed [M][K/4] I2_S (16-byte aligned), M, w_scale, and the
 *              outputs dot [N][M] int32 / y [N][M] fp32 (either may be NULL,
 *              not both, unless M == 0).
 *   xq, x_scale, x_sum   optional outputs (may be NULL when
 *              N <= BITNET_LINEAR_FUSED_MAX_N): the
 *              quantised tokens exactly as bitnet_quant_act_i8 writes them.
 *              Required for larger N (they then carry the tokens between the
 *              quantiser and the MFMA kernels).
 *
 * N <= BITNET_LINEAR_FUSED_MAX_N: one launch quantises and multiplies (the
 * vector-ALU GEMV; at more tokens it is ALU-bound and slower than the two
 * launches below).  Up to BITNET_GEMV_MAX_N:
 * quantiser, then one batched-decode MFMA launch for all matrices.  Larger N
 * (prefill): quantiser, then one grouped MFMA GEMM launch for all matrices.
 * Every output equals what bitnet_quant_act_i8 followed by
 * bitnet_gemv_i2s_i8 (N <= BITNET_GEMV_MAX_N) or bitnet_gemm_i2s_i8 on each
 * matrix produces, bit for bit.
 * 0 <= N <= BITNET_GEMM_MAX_N; 1 <= n_mats <= BITNET_MAX_GROUP.
 */
typedef struct {
    const uint8_t *packed;
    int64_t M;
    float w_scale;
    int32_t *dot;
    float *y;
} bitnet_i2s_matrix;

int bitnet_linear_i2s(const void *x, int dtype, int64_t N, int64_t K,
                      const bitnet_i2s_matrix *mats, int n_mats, int8_t *xq,
                      float *x_scale, int32_t *x_sum, void *stream);

/*
 * bitnet_ffn_act_quant_i8 -- the squared-ReLU gated FFN activation that feeds
 * the down projection, quantised for it.  [P4 "Forward Pass":
 * inner = ffn_sub_norm(sqrelu(gate(x)) * up(x)), out = down(inner); P1 §4-5]
 *
 *   g, u     device [N][F] fp32: the gate and up projections' y outputs
 *            (16-byte aligned); F a multiple of 128, F <= BITNET_MAX_K.
 *   gamma    device [F] fp32 gain of the sub-norm (16-byte aligned), or NULL for 1.
 *   eps      the sub-norm's epsilon (positive, finite; else BITNET_E_VALUE).
 *   xq, x_scale, x_sum   outputs as bitnet_quant_act_i8 writes them, ready
 *            for bitnet_gemv_i2s_i8 / bitnet_gemm_i2s_i8 with the down weights.
 *
 * Per token: h = (relu(g)^2) * u in fp32; ss = the sum of the F squares h^2
 * (each exact in binary64) computed exactly and rounded once to binary64,
 * to nearest-even -- no summation order enters; c = fp32(1 / sqrt(ss / F +
 * eps)); v = (h * c) * gamma in fp32; then per-token absmax int8 quantisation
 * of v.  0 <= N < 2^31; N == 0 is a no-op.
 */
int bitnet_ffn_act_quant_i8(const float *g, const float *u, const float *gamma, float eps,
                            int64_t N, int64_t F, int8_t *xq, float *x_scale,
                            int32_t *x_sum, void *stream);

/*
 * bitnet_gemv_i2s_i8_group -- decode matmul (N <= BITNET_GEMV_MAX_N tokens,
 * already quantised) of several I2_S matrices that share the tokens: one
 * launch for all of them: the vector-ALU GEMV when N <= 2, else the
 * batched-decode MFMA kernel.  [P1 §2-1, §4-3; P2 §3; P3 §3.2]
 *
 *   mats, xq, x_scale, x_sum   as bitnet_gemm_i2s_i8_group.
 *
 * Outputs equal bitnet_gemv_i2s_i8 on each matrix, bit for bit.
 * 0 <= N <= BITNET_GEMV_MAX_N; N == 0 or all M == 0 is a no-op.
 */
int bitnet_gemv_i2s_i8_group(const bitnet_i2s_matrix *mats, int n_mats, int64_t K,
                             const int8_t *xq, const float *x_scale,
                             const int32_t *x_sum, int64_t N, void *stream);

/*
 * bitnet_gemm_i2s_i8_group -- prefill matmul of several I2_S matrices that
 * share one block of quantised tokens, in one MFMA launch (e.g. q/k/v, or
 * gate/up, of a layer).  [P1 §4-5 (a separate prefill path), §4-3 (one
 * token block reused by every weight row); P2 §3; P3 §3.2]
 *
 *   mats     host array of n_mats descriptors (1 <= n_mats <=
 *            BITNET_MAX_GROUP), read during the call only: packed [M][K/4]
 *            I2_S (16-byte aligned), M, w_scale, outputs dot [N][M] int32 /
 *            y [N][M] fp32 (either may be NULL, not both, unless M == 0).
 *   xq, x_scale, x_sum   the tokens as bitnet_quant_act_i8 writes them
 *            (xq 16-byte aligned).
 *
 * Outputs equal bitnet_gemm_i2s_i8 on each matrix, bit for bit.
 * 0 <= N <= BITNET_GEMM_MAX_N; N == 0 or all M == 0 is a no-op.
 */
int bitnet_gemm_i2s_i8_group(const bitnet_i2s_matrix *mats, int n_mats, int64_t K,
                             const int8_t *xq, const float *x_scale,
                             const int32_t *x_sum, int64_t N, void *stream);

/*
 * bitnet_absmean_i2s -- one-time conversion of full-precision weights to I2_S
 * with the AbsMean ternariser.  [P1 §6-2; P4 "Ternary Weight Quantisation
 * (AbsMean)"; layout P1 §1-1, §4-2]
 *
 *   w       device [M][K] fp32 or bf16 (dtype BITNET_F32 / BITNET_BF16),
 *           16-byte aligned; M >= 1.
 *   packed  device [M][K/4] I2_S output, 16-byte aligned.
 *   alpha   HOST pointer; receives the per-tensor scale
 *           alpha = max(mean |w| over all M*K weights, 1e-5): the sum of |w|
 *           computed exactly and rounded once to binary64 (so it depends on
 *           no summation order), divided by M*K in binary64, rounded to fp32.
 *           Use it as w_scale of the matmul calls.
 *
 * Each weight becomes q = clip(round-half-even(w / alpha), -1, 1), w / alpha
 * one fp32 division, stored as code q + 1.  Synchronises `stream`
 * (the scale is returned on the host); calls are serialised inside the
 * library.  Non-finite weights -> BITNET_E_VALUE (packed then unspecified);
 * M * K above 2^40 -> BITNET_E_SHAPE.
 */
int bitnet_absmean_i2s(const void *w, int dtype, int64_t M, int64_t K,
                       uint8_t *packed, float *alpha, void *stream);

/*
 * bitnet_pack_i2s_f32 -- pack float weights that are already ternary in value
 * (e.g. q * scale) by sign: |v| < 1e-6 (compared in binary64) -> code 1,
 * v > 0 -> code 2, v < 0 -> code 0.  [P1 §4-2 (the float packer), §1-1]
 *
 *   w       device [M][K] fp32, 16-byte aligned.
 *   packed  device [M][K/4] I2_S output, 16-byte aligned.
 *   w_max   HOST pointer or NULL; receives max |w| (0 for M == 0).
 *
 * Synchronises `stream`; M == 0 is a no-op.  Non-finite weights ->
 * BITNET_E_VALUE (packed then unspecified).
 */
int bitnet_pack_i2s_f32(const float *w, int64_t M, int64_t K, uint8_t *packed,
                        float *w_max, void *stream);

/* Thread-local description of the last non-OK status on this thread
 * (empty string if none).  The pointer stays valid until the next call on
 * the same thread. */
const char *bitnet_last_error(void);

/* BITNET_ABI_VERSION of the built library. */
int bitnet_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif
