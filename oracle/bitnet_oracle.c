/*
 * bitnet_oracle.c -- plain, slow CPU oracle for the BitNet b1.58 W2A8 (I2_S)
 * matmul.  TEST INFRASTRUCTURE ONLY: loaded by the tests, the smoke check and
 * the benchmark's CPU-baseline leg, never by the library.  No SIMD
 * intrinsics, no blocking, no code shared with the GPU path.  Page keys
 * [P1]..[P4] are listed in bitnet_oracle.h.
 *
 * Built with: gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math -fPIC -shared
 * (no FMA contraction: every float operation below is a single IEEE-754
 * binary32 or binary64 operation, as written).
 */
#define _POSIX_C_SOURCE 200809L
#include "bitnet_oracle.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

/* Block size of the I2_S layout on the x86 path [P1 §4-2]; the packed files
 * the pages work with always use 128 [P2 §3]. */
#define ORC_QK 128

int orc_code_of_weight(int w)
{
    /* [P1 §1-1] table: -1 -> 0 (bits 00), 0 -> 1 (01), +1 -> 2 (10). */
    if (w == -1) return 0;
    if (w == 0) return 1;
    if (w == 1) return 2;
    return -1;
}

int orc_weight_of_code(int c)
{
    /* Inverse of the same table; the worked byte of [P1 §8] takes c - 1. */
    if (c >= 0 && c <= 2) return c - 1;
    return 99;
}

int64_t orc_pack_i2s(const int8_t *w, int64_t M, int64_t K, uint8_t *packed)
{
    /* [P1 §4-2]: a block holds 128 consecutive weights of a row in 32 bytes.
     * Position p of the block (0..127) is stored in byte (p mod 32) of the
     * block, in the 2-bit field that starts at bit 6 - 2*(p div 32): the four
     * weights p, p+32, p+64, p+96 share one byte, the first in the top bits.
     * Blocks follow each other along the row and rows are contiguous, so the
     * block of weight (m, k) starts at byte m*K/4 + 32*(k div 128). */
    int64_t nonternary = 0;
    memset(packed, 0, (size_t)(M * K / 4));
    for (int64_t m = 0; m < M; m++) {
        for (int64_t k = 0; k < K; k++) {
            int c = orc_code_of_weight(w[m * K + k]);
            if (c < 0) {           /* not ternary: mark the slot with code 3 */
                nonternary++;
                c = 3;
            }
            int64_t blk = k / ORC_QK;
            int64_t p = k % ORC_QK;
            int64_t at = m * (K / 4) + blk * 32 + p % 32;
            int bit = 6 - 2 * (int)(p / 32);
            packed[at] = (uint8_t)(packed[at] | (c << bit));
        }
    }
    return nonternary;
}

int64_t orc_unpack_i2s(const uint8_t *packed, int64_t M, int64_t K, int8_t *w)
{
    /* For weight (m, k): block b = k / 128 of row m starts at byte
     * m*(K/4) + 32*b [P2 §3: row offset, 32 bytes per block]; inside the
     * block, position p = k % 128 lives in byte p % 32 at bits
     * (6 - 2*(p/32)) .. +1, i.e. group 0 in bits 7-6 [P1 §8; P3 §4]. */
    int64_t bad = 0;
    for (int64_t m = 0; m < M; m++) {
        for (int64_t k = 0; k < K; k++) {
            int64_t b = k / ORC_QK;
            int64_t p = k % ORC_QK;
            uint8_t byte = packed[m * (K / 4) + 32 * b + (p % 32)];
            int shift = 6 - 2 * (int)(p / 32);
            int code = (byte >> shift) & 3;
            int wv = orc_weight_of_code(code);
            if (wv == 99) bad++;
            w[m * K + k] = (int8_t)wv;
        }
    }
    return bad;
}

float orc_bf16_to_f32(uint16_t h)
{
    uint32_t bits = (uint32_t)h << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return f;
}

static void quant_row(const float *x, int64_t K, int8_t *q, float *s_out,
                      int32_t *qsum_out)
{
    /* [P1 §4-5]: s = 127 / max(max|x|, 1e-5); q = round(x*s), clamped to the
     * int8 range [P4: clip to [-128, 127]], stored as int8.  Round is IEEE
     * round-half-to-even (rintf in the default rounding mode). */
    float a = 0.0f;
    for (int64_t k = 0; k < K; k++) {
        float v = fabsf(x[k]);
        if (v > a) a = v;
    }
    float denom = a > 1e-5f ? a : 1e-5f;
    float s = 127.0f / denom;
    int32_t sum = 0;
    for (int64_t k = 0; k < K; k++) {
        float t = x[k] * s;
        float r = rintf(t);
        if (r > 127.0f) r = 127.0f;
        if (r < -128.0f) r = -128.0f;
        q[k] = (int8_t)r;
        sum += (int32_t)q[k];
    }
    *s_out = s;
    *qsum_out = sum;
}

void orc_quant_act_f32(const float *x, int64_t N, int64_t K, int8_t *q,
                       float *s, int32_t *qsum)
{
    for (int64_t n = 0; n < N; n++)
        quant_row(x + n * K, K, q + n * K, s + n, qsum + n);
}

void orc_quant_act_bf16(const uint16_t *x, int64_t N, int64_t K, int8_t *q,
                        float *s, int32_t *qsum)
{
    float *row = (float *)malloc((size_t)K * sizeof(float));
    if (!row) return;
    for (int64_t n = 0; n < N; n++) {
        for (int64_t k = 0; k < K; k++) row[k] = orc_bf16_to_f32(x[n * K + k]);
        quant_row(row, K, q + n * K, s + n, qsum + n);
    }
    free(row);
}

void orc_dot_def(const int8_t *w, const int8_t *q, int64_t M, int64_t K,
                 int64_t N, int64_t *D)
{
    /* D = W_q @ x_q, an integer dot with no float multiply [P1 §1-1; P4]. */
    for (int64_t n = 0; n < N; n++) {
        for (int64_t m = 0; m < M; m++) {
            int64_t acc = 0;
            for (int64_t k = 0; k < K; k++)
                acc += (int64_t)w[m * K + k] * (int64_t)q[n * K + k];
            D[n * M + m] = acc;
        }
    }
}

void orc_dot_raw(const uint8_t *packed, const int8_t *q, const int32_t *qsum,
                 int64_t M, int64_t K, int64_t N, int64_t *R, int64_t *D)
{
    /* [P2 §3; P3 §3.1-§4]: the packed row is read one byte at a time.  Byte t
     * of the row belongs to block t div 32; its four 2-bit fields, taken from
     * the top bits down, pair with the activations 0, 32, 64 and 96 places
     * after (block start + t mod 32).  The raw codes 0/1/2 are what gets
     * multiplied [P3 §3.2], so the sum over the row is
     * R = sum((w+1)*x) = sum(w*x) + sum(x), and the exact dot is
     * D = R - sum(x)  (the zero-mean shortcut of [P3 §3.2] is not taken). */
    int64_t bytes_per_row = K / 4;
    for (int64_t n = 0; n < N; n++) {
        const int8_t *act = q + n * K;
        for (int64_t m = 0; m < M; m++) {
            const uint8_t *rowbytes = packed + m * bytes_per_row;
            int64_t raw = 0;
            for (int64_t t = 0; t < bytes_per_row; t++) {
                int64_t base = (t / 32) * ORC_QK + (t % 32);
                for (int field = 0; field < 4; field++) {
                    int code = (rowbytes[t] >> (6 - 2 * field)) & 3;
                    raw += (int64_t)code * (int64_t)act[base + 32 * field];
                }
            }
            R[n * M + m] = raw;
            D[n * M + m] = raw - (int64_t)qsum[n];
        }
    }
}

/* ---- lookup-table route ------------------------------------------------ */

void orc_lut_tables(const int8_t *q, int64_t K, int32_t *table)
{
    /* Phase one of the LUT method [P1 §4-4]: every value a group of two
     * raw codes can contribute is tabulated from the activations alone. */
    for (int64_t t = 0; t < K / 4; t++) {
        int64_t base = (t / 32) * ORC_QK + (t % 32);
        for (int half = 0; half < 2; half++) {
            int64_t first = base + 64 * half;   /* fields 0,1 or fields 2,3 */
            int32_t xa = q[first], xb = q[first + 32];
            int32_t *entry = table + (2 * t + half) * 16;
            for (int c_hi = 0; c_hi < 4; c_hi++)
                for (int c_lo = 0; c_lo < 4; c_lo++)
                    entry[4 * c_hi + c_lo] = c_hi * xa + c_lo * xb;
        }
    }
}

void orc_dot_lut(const uint8_t *packed, const int8_t *q, const int32_t *qsum,
                 int64_t M, int64_t K, int64_t N, int64_t *R, int64_t *D)
{
    /* Phase two [P1 §4-4]: only after the whole table exists, each packed
     * byte is split into its two nibbles and each nibble indexes its group's
     * table; the lookups add up to the raw-code sum R, corrected as in the
     * unpack route. */
    int64_t bytes_per_row = K / 4;
    int32_t *table = (int32_t *)malloc((size_t)(K / 2) * 16 * sizeof(int32_t));
    if (!table) abort();
    for (int64_t n = 0; n < N; n++) {
        orc_lut_tables(q + n * K, K, table);
        for (int64_t m = 0; m < M; m++) {
            const uint8_t *rowbytes = packed + m * bytes_per_row;
            int64_t raw = 0;
            for (int64_t t = 0; t < bytes_per_row; t++) {
                raw += table[(2 * t) * 16 + (rowbytes[t] >> 4)];
                raw += table[(2 * t + 1) * 16 + (rowbytes[t] & 15)];
            }
            R[n * M + m] = raw;
            D[n * M + m] = raw - (int64_t)qsum[n];
        }
    }
    free(table);
}

void orc_epilogue(const int64_t *D, double alpha, const float *s, int64_t M,
                  int64_t N, double *y)
{
    /* The integer dot leaves the scales to the caller [P2 §3]; the weight is
     * q*alpha [P1 §6-2] and the activation is q/s [P1 §4-5], so the output is
     * D * alpha / s. */
    for (int64_t n = 0; n < N; n++)
        for (int64_t m = 0; m < M; m++)
            y[n * M + m] = (double)D[n * M + m] * alpha / (double)s[n];
}

/* ---- threaded driver over output rows ---------------------------------- */

typedef struct {
    const uint8_t *packed;
    int64_t M, K, N;
    const int8_t *q;
    const float *s;
    double alpha;
    int64_t r0, r1;
    int64_t *D;
    double *y;
    int64_t bad;
} orc_job;

static void *linear_worker(void *arg)
{
    orc_job *j = (orc_job *)arg;
    int8_t *wrow = (int8_t *)malloc((size_t)j->K);
    if (!wrow) return NULL;
    for (int64_t m = j->r0; m < j->r1; m++) {
        /* unpack row m weight by weight (same addressing as orc_unpack_i2s) */
        for (int64_t k = 0; k < j->K; k++) {
            int64_t b = k / ORC_QK, p = k % ORC_QK;
            uint8_t byte = j->packed[m * (j->K / 4) + 32 * b + (p % 32)];
            int wv = orc_weight_of_code((byte >> (6 - 2 * (int)(p / 32))) & 3);
            if (wv == 99) { j->bad++; wv = 0; }
            wrow[k] = (int8_t)wv;
        }
        for (int64_t n = 0; n < j->N; n++) {
            int64_t acc = 0;
            const int8_t *qn = j->q + n * j->K;
            for (int64_t k = 0; k < j->K; k++)
                acc += (int64_t)wrow[k] * (int64_t)qn[k];
            if (j->D) j->D[n * j->M + m] = acc;
            if (j->y) j->y[n * j->M + m] = (double)acc * j->alpha / (double)j->s[n];
        }
    }
    free(wrow);
    return NULL;
}

int64_t orc_linear_i2s(const uint8_t *packed, int64_t M, int64_t K,
                       const int8_t *q, int64_t N, const float *s, float alpha,
                       int64_t row0, int64_t nrows, int64_t *D, double *y,
                       int nthreads)
{
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if (nrows < nthreads) nthreads = nrows > 0 ? (int)nrows : 1;
    orc_job jobs[256];
    pthread_t tids[256];
    int64_t per = nrows / nthreads, rem = nrows % nthreads, r = row0;
    for (int t = 0; t < nthreads; t++) {
        int64_t cnt = per + (t < rem ? 1 : 0);
        jobs[t] = (orc_job){packed, M, K, N, q, s, (double)alpha, r, r + cnt, D, y, 0};
        r += cnt;
    }
    for (int t = 1; t < nthreads; t++)
        pthread_create(&tids[t], NULL, linear_worker, &jobs[t]);
    linear_worker(&jobs[0]);
    int64_t bad = jobs[0].bad;
    for (int t = 1; t < nthreads; t++) {
        pthread_join(tids[t], NULL);
        bad += jobs[t].bad;
    }
    return bad;
}

/* ---- exactly rounded sum of non-negative binary64 values ---- */

/* A fixed-point integer wide enough to hold any sum of finite binary64
 * values exactly: bit i stands for 2^(i - 1074), the weight of the smallest
 * subnormal.  1074 + 1024 bits cover every finite value, and 206 more leave
 * room for far more than 2^63 addends of the largest one. */
#define ORC_ACC_DIGITS 72
typedef struct {
    uint32_t d[ORC_ACC_DIGITS];
} orc_acc;

/* a += v * 2^(bitpos - 1074), with the carry propagated at once */
static void acc_add_u32_at(orc_acc *a, int64_t bitpos, uint32_t v)
{
    int64_t j = bitpos / 32;
    uint64_t t = (uint64_t)v << (bitpos % 32);   /* below 2^63 */
    uint64_t carry = 0;
    for (; j < ORC_ACC_DIGITS && (t != 0 || carry != 0); j++) {
        uint64_t s = (uint64_t)a->d[j] + (t & 0xffffffffu) + carry;
        a->d[j] = (uint32_t)s;
        carry = s >> 32;
        t >>= 32;
    }
}

/* a += x for a finite x >= 0, exactly */
static void acc_add(orc_acc *a, double x)
{
    if (x == 0.0) return;
    int e;
    double f = frexp(x, &e);                      /* x = f * 2^e, 0.5 <= f < 1 */
    uint64_t m = (uint64_t)ldexp(f, 53);          /* x = m * 2^(e - 53), exactly */
    int64_t pos = (int64_t)e - 53 + 1074;
    while (pos < 0) {                             /* a subnormal: m ends in zeros */
        m >>= 1;
        pos++;
    }
    acc_add_u32_at(a, pos, (uint32_t)(m & 0xffffffffu));
    acc_add_u32_at(a, pos + 32, (uint32_t)(m >> 32));
}

static int acc_bit(const orc_acc *a, int64_t i)
{
    return (int)((a->d[i / 32] >> (i % 32)) & 1u);
}

/* the accumulated value rounded once to binary64, to nearest, ties to even */
static double acc_round(const orc_acc *a)
{
    int64_t top = -1;
    for (int64_t i = (int64_t)ORC_ACC_DIGITS * 32 - 1; i >= 0; i--) {
        if (acc_bit(a, i)) {
            top = i;
            break;
        }
    }
    if (top < 0) return 0.0;
    if (top < 53) {                               /* below 2^53 units: exact */
        uint64_t v = 0;
        for (int64_t i = top; i >= 0; i--) v = 2 * v + (uint64_t)acc_bit(a, i);
        return ldexp((double)v, -1074);
    }
    uint64_t keep = 0;                            /* the 53 leading bits */
    for (int64_t i = top; i > top - 53; i--) keep = 2 * keep + (uint64_t)acc_bit(a, i);
    int round = acc_bit(a, top - 53);
    int sticky = 0;
    for (int64_t i = top - 54; i >= 0 && !sticky; i--) sticky = acc_bit(a, i);
    if (round && (sticky || (keep & 1u))) keep++;
    return ldexp((double)keep, (int)(top - 52 - 1074));
}

double orc_exact_sum(const double *x, int64_t n)
{
    orc_acc acc;
    memset(&acc, 0, sizeof acc);
    for (int64_t i = 0; i < n; i++) {
        if (!(x[i] >= 0.0) || isinf(x[i])) return -1.0;
        acc_add(&acc, x[i]);
    }
    return acc_round(&acc);
}

/* ---- AbsMean ternariser and sign/threshold ternary (weight conversion) ---- */

static float absmean_from_sum(double sum, int64_t n)
{
    /* [P1 §6-2]: abs_mean = max(mean(abs(w)), 1e-5); [P4]: alpha_W = mean|W| */
    float a = (float)(sum / (double)n);
    return a > 1e-5f ? a : 1e-5f;
}

/* Non-finite weights make the result NaN (the caller reports an error). */
float orc_absmean_alpha_f32(const float *w, int64_t n)
{
    orc_acc acc;
    memset(&acc, 0, sizeof acc);
    for (int64_t i = 0; i < n; i++) {
        if (!isfinite(w[i])) return NAN;
        acc_add(&acc, fabs((double)w[i]));
    }
    return absmean_from_sum(acc_round(&acc), n);
}

float orc_absmean_alpha_bf16(const uint16_t *w, int64_t n)
{
    orc_acc acc;
    memset(&acc, 0, sizeof acc);
    for (int64_t i = 0; i < n; i++) {
        float v = orc_bf16_to_f32(w[i]);
        if (!isfinite(v)) return NAN;
        acc_add(&acc, fabs((double)v));
    }
    return absmean_from_sum(acc_round(&acc), n);
}

static int8_t ternary_of(float v, float alpha)
{
    /* [P1 §6-2; P4]: q = clip(round(w / alpha), -1, 1); the division is one
     * fp32 operation and round is half-to-even (rintf, default mode). */
    float t = v / alpha;
    float r = rintf(t);
    if (r > 1.0f) r = 1.0f;
    if (r < -1.0f) r = -1.0f;
    return (int8_t)r;
}

void orc_absmean_ternary_f32(const float *w, int64_t n, float alpha, int8_t *q)
{
    for (int64_t i = 0; i < n; i++) q[i] = ternary_of(w[i], alpha);
}

void orc_absmean_ternary_bf16(const uint16_t *w, int64_t n, float alpha, int8_t *q)
{
    for (int64_t i = 0; i < n; i++) q[i] = ternary_of(orc_bf16_to_f32(w[i]), alpha);
}

int64_t orc_sign_ternary_f32(const float *w, int64_t n, int8_t *q, float *wmax)
{
    /* [P1 §4-2]: near-zero (fabs < 1e-6) -> code 1, positive -> code 2,
     * negative -> code 0; here as the ternary value (code - 1). */
    int64_t bad = 0;
    float m = 0.0f;
    for (int64_t i = 0; i < n; i++) {
        float v = w[i];
        if (!isfinite(v)) {
            bad++;
            q[i] = 0;
            continue;
        }
        if (fabs((double)v) < 1e-6) q[i] = 0;
        else q[i] = v > 0.0f ? 1 : -1;
        if (fabsf(v) > m) m = fabsf(v);
    }
    if (wmax) *wmax = m;
    return bad;
}

/* ---- squared-ReLU gated FFN activation + sub-norm + quantisation ---- */

void orc_ffn_act_quant(const float *g, const float *u, const float *gamma, float eps,
                       int64_t N, int64_t F, int8_t *q, float *s, int32_t *qsum,
                       float *v)
{
    float *h = malloc((size_t)F * sizeof *h);
    float *nv = malloc((size_t)F * sizeof *nv);
    for (int64_t n = 0; n < N; n++) {
        const float *gn = g + n * F, *un = u + n * F;
        /* [P4]: sqrelu(gate) (x) up -- squared ReLU of the gate times up */
        for (int64_t k = 0; k < F; k++) {
            float r = gn[k] > 0.0f ? gn[k] : 0.0f;
            float r2 = r * r;
            h[k] = r2 * un[k];
        }
        /* ffn_sub_norm: RMS normalisation over the F channels.  Every h^2 is
         * exact in binary64 (24-bit significands); their sum is taken exactly
         * and rounded once, so it does not depend on any summation order. */
        orc_acc acc;
        memset(&acc, 0, sizeof acc);
        for (int64_t k = 0; k < F; k++) acc_add(&acc, (double)h[k] * (double)h[k]);
        double ss = acc_round(&acc);
        float c = (float)(1.0 / sqrt(ss / (double)F + (double)eps));
        for (int64_t k = 0; k < F; k++) {
            float t = h[k] * c;
            nv[k] = gamma ? t * gamma[k] : t;
        }
        if (v) memcpy(v + n * F, nv, (size_t)F * sizeof *nv);
        quant_row(nv, F, q + n * F, s + n, qsum + n);
    }
    free(h);
    free(nv);
}
