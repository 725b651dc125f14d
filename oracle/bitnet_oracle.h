/*
 * bitnet_oracle.h -- plain CPU oracle for the BitNet b1.58 W2A8 (I2_S) matmul.
 *
 * TEST INFRASTRUCTURE ONLY.  This header and bitnet_oracle.c are the slow,
 * obviously-correct reference that the GPU library is checked against.  Only
 * the tests, the smoke check and the benchmark's CPU-baseline leg may load it.
 * It shares no code, header, table or constant with the GPU library
 * (ternary_weight_i2_amd/csrc, include/bitnet_i2s.h) and includes neither.
 *
 * Sources (web pages; cited by key and section):
 *   [P1] "BitNet 딥다이브 -- 작은 숫자를 빠른 연산으로 바꾸는 추론 엔진"
 *        (fiv.co.kr/repos/BitNet-deep-dive.html)
 *   [P2] "[분석/검증-3] BitNet.cpp ARM 커널 재작성 : 스칼라 폴백구현을 통한
 *        최종 검증" (uno-kim.tistory.com/459)
 *   [P3] "[기술 분석 보고서] ARM64 모바일 환경에서의 1.58-bit 양자화 모델 추론
 *        붕괴 원인 분석 및 C++ 커널 역공학을 통한 해결" (uno-kim.tistory.com/461)
 *   [P4] "bitnet.rs -- BitNet b1.58 Inference Engine in Rust"
 *        (shadowgraph.io/ryancinsight/bitnetrs), section "Mathematical Foundation"
 *
 * Notation: M output rows (weight rows), K reduction length, N tokens.
 * Weights W[M][K] are ternary int8 in {-1,0,+1}; activations are per-token.
 * All arrays are row-major host memory owned by the caller.
 */
#ifndef BITNET_ORACLE_H
#define BITNET_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Code map of [P1 §1-1]: weight -1 -> code 0, 0 -> 1, +1 -> 2.  Returns -1 for
 * any weight outside {-1,0,+1} (no code exists for it). */
int orc_code_of_weight(int w);
/* Inverse map [P1 §1-1, §8]: code c in {0,1,2} -> c - 1.  Code 3 is never
 * produced by the packer; returns 99 for it (and for anything > 3). */
int orc_weight_of_code(int c);

/* I2_S packing [P1 §4-2]: K must be a multiple of 128 (block size 128).
 * packed gets M*K/4 bytes.  Returns the number of weights that are not
 * ternary (those bytes are left with code 3 in their slot so they are
 * detectable); 0 means success. */
int64_t orc_pack_i2s(const int8_t *w, int64_t M, int64_t K, uint8_t *packed);

/* Inverse of the packing, element by element [P1 §8; P2 §3].  Returns the
 * number of slots holding code 3 (those weights are written as 99). */
int64_t orc_unpack_i2s(const uint8_t *packed, int64_t M, int64_t K, int8_t *w);

/* bf16 -> fp32 (exact: the 16 bf16 bits become the high half of the fp32). */
float orc_bf16_to_f32(uint16_t h);

/* Per-token absmax int8 quantisation [P1 §4-5; P4 "8-bit Activation
 * Quantisation"]: a = max_k |x|, s = 127 / max(a, 1e-5) (fp32 division),
 * q = clamp(round-half-even(x * s), -128, 127), qsum = sum_k q.
 * x_f32 is [N][K] fp32. */
void orc_quant_act_f32(const float *x, int64_t N, int64_t K,
                       int8_t *q, float *s, int32_t *qsum);
/* Same, for bf16 input bits [N][K] (converted exactly to fp32 first). */
void orc_quant_act_bf16(const uint16_t *x, int64_t N, int64_t K,
                        int8_t *q, float *s, int32_t *qsum);

/* The definition [P1 §1-1; P4 "Quantised Forward Pass"]:
 * D[n][m] = sum_k W[m][k] * q[n][k], accumulated in int64. */
void orc_dot_def(const int8_t *w, const int8_t *q, int64_t M, int64_t K,
                 int64_t N, int64_t *D);

/* The pages' packed formulation [P2 §3; P3 §3.2, §4]: walk the packed row
 * block by block, byte by byte, multiply the raw codes 0/1/2 by the
 * activations at offsets k, k+32, k+64, k+96 to get R[n][m]; then apply the
 * exact offset correction D = R - qsum[n].  Writes both R and D. */
void orc_dot_raw(const uint8_t *packed, const int8_t *q, const int32_t *qsum,
                 int64_t M, int64_t K, int64_t N, int64_t *R, int64_t *D);

/* Lookup-table route to the same raw-code dot [P1 §4-3 (the LUT path's entry
 * condition), §4-4 (its order: the table is built from the activations
 * before any lookup, with a barrier between the two phases); P1 §11-2
 * (T-MAC, the lookup-based low-bit method it follows)].  A weight group is the two
 * 2-bit fields of one nibble of an I2_S byte: the high nibble of byte t pairs
 * the activations at (block start + t mod 32) and 32 places after, the low
 * nibble those 64 and 96 places after.  Group g = 2t (high) or 2t + 1 (low)
 * of a row of K weights; there are K/2 groups.
 * orc_lut_tables: for one token q[K], table[g][c] (16 entries per group,
 * c = 4*c_hi + c_lo over raw codes 0..3) = c_hi * x_first + c_lo * x_second.
 * orc_dot_lut: per token, build the tables, then R[n][m] = sum over the
 * row's nibbles of table[g][nibble]; D = R - qsum[n] as in orc_dot_raw. */
void orc_lut_tables(const int8_t *q, int64_t K, int32_t *table);
void orc_dot_lut(const uint8_t *packed, const int8_t *q, const int32_t *qsum,
                 int64_t M, int64_t K, int64_t N, int64_t *R, int64_t *D);

/* Dequantising epilogue [P2 §3 (scale left to the caller); P1 §4-5; P4]:
 * y[n][m] = D[n][m] * alpha / s[n], in double. */
void orc_epilogue(const int64_t *D, double alpha, const float *s,
                  int64_t M, int64_t N, double *y);

/* Whole matmul on packed weights, split over nthreads threads by output row:
 * per row, unpack every weight (orc_weight_of_code of the slot's code), form
 * D by the definition, then y by the epilogue.  D and/or y may be NULL.
 * rows [row0, row0+nrows) only (the rest of D/y untouched; D/y are still
 * indexed [n][m] with full M).  Returns the number of code-3 slots seen. */
int64_t orc_linear_i2s(const uint8_t *packed, int64_t M, int64_t K,
                       const int8_t *q, int64_t N, const float *s, float alpha,
                       int64_t row0, int64_t nrows,
                       int64_t *D, double *y, int nthreads);

/* The sum of n finite, non-negative binary64 values, computed exactly and
 * rounded once to binary64 (to nearest, ties to even): the result does not
 * depend on the order of the values.  Returns -1 if a value is negative or
 * not finite.  Used by the AbsMean scale and the FFN sub-norm below. */
double orc_exact_sum(const double *x, int64_t n);

/* AbsMean ternarisation of full-precision weights [P1 §6-2; P4 "Ternary
 * Weight Quantisation (AbsMean)"], over all n weights of a tensor:
 *   alpha = max(mean |w|, 1e-5): the exactly rounded binary64 sum of |w|
 *           (orc_exact_sum), divided by n in binary64, rounded once to fp32,
 *           then the 1e-5 floor (fp32);
 *   q     = clip(round-half-even(w / alpha), -1, 1), w / alpha one fp32
 *           division.
 * Returns alpha; orc_absmean_ternary writes q.  Non-finite weights make alpha
 * NaN (the caller treats that as an error). */
float orc_absmean_alpha_f32(const float *w, int64_t n);
float orc_absmean_alpha_bf16(const uint16_t *w, int64_t n);
void orc_absmean_ternary_f32(const float *w, int64_t n, float alpha, int8_t *q);
void orc_absmean_ternary_bf16(const uint16_t *w, int64_t n, float alpha, int8_t *q);

/* Sign/threshold ternary of float weights, as the packer of [P1 §4-2] reads
 * them: |v| < 1e-6 (compared in binary64, the constant as written) -> 0,
 * v > 0 -> +1, v < 0 -> -1.  *wmax (if not NULL) gets max |v|.  Returns the
 * number of non-finite weights (their q is left 0). */
int64_t orc_sign_ternary_f32(const float *w, int64_t n, int8_t *q, float *wmax);

/* Squared-ReLU gated FFN activation feeding the down projection [P4
 * "Forward Pass": inner = ffn_sub_norm(sqrelu(gate(x)) (x) up(x)),
 * out = down(inner)], per token n over F channels (F a multiple of 32):
 *   r_k = max(g_k, 0);  h_k = (r_k * r_k) * u_k                    (fp32)
 *   ss  = sum of h_k^2 (each exact in binary64), computed exactly and
 *         rounded once to binary64 (orc_exact_sum): no summation order
 *   c   = fp32(1 / sqrt(ss / F + eps))   (binary64, one final rounding)
 *   v_k = (h_k * c) * gamma_k            (fp32; gamma NULL means 1)
 * then v is quantised per token exactly as orc_quant_act_f32 does.
 * v (if not NULL) receives the normalised activations [N][F]. */
void orc_ffn_act_quant(const float *g, const float *u, const float *gamma, float eps,
                       int64_t N, int64_t F, int8_t *q, float *s, int32_t *qsum,
                       float *v);

#ifdef __cplusplus
}
#endif
#endif
