// exact_sum.h -- exactly rounded binary64 sums of non-negative values whose
// bits are known exactly (squares of fp32 values; magnitudes of fp32 values),
// for the FFN sub-norm and the AbsMean scale.  The result is the exact sum
// rounded once to nearest-even, so it depends on no summation order and a
// reduction may be split across lanes, waves and workgroups freely.
//
// Pages: [P4] "bitnet.rs", "Forward Pass" (ffn_sub_norm of the squared-ReLU
// gated product) and "Mathematical Foundation" (AbsMean, mean |W|); [P1]
// "BitNet 딥다이브" §6-2 (AbsMean).  Neither fixes a summation order; every
// h^2 of an fp32 h and every |w| of an fp32 w is exact in binary64, so the
// exact sum is well defined and taken here.
//
// Two schemes:
//  * Window sums (squares).  An fp32 h = m * 2^(e) with m < 2^24 gives
//    h^2 = v * 2^(P - 298), v = m^2 < 2^48, P in [0, 506].  With T the top bit
//    position of the largest square of a token, level 1 keeps every square's
//    bits at positions >= b1 = T - kWin exactly in a 128-bit integer (unit
//    2^b1) and counts the squares that have bits below b1.  If the count
//    cannot carry into the round bit, the level-1 integer decides the
//    rounding; otherwise further levels add the next kWin bits of every
//    square into an exact big integer until no square has bits left below.
//  * Digit sums (magnitudes).  Nine 32-bit digits held in 64-bit lanes, in
//    units of 2^-149 (carry-save; no carries while accumulating), cover every
//    finite fp32 |w| = m * 2^P' (P' in [0, 253], m < 2^24) with no window and
//    no second level.  The AbsMean kernel gathers the magnitudes in exact
//    binary64 buckets first and folds those into the digits (convert.hip);
//    mag_normalise and mag_round turn digit sums into one binary64 value.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bitnet {

constexpr int kWin = 112;        // bits per window level (sums of 2^15 terms fit in 128)
constexpr int kBigDigits = 32;   // 32-bit digits of the slow path's exact integer

struct U128 {
    uint64_t lo, hi;
};

__host__ __device__ __forceinline__ void add128(U128 &a, const U128 &b) {
    const uint64_t lo = a.lo + b.lo;
    a.hi += b.hi + (lo < a.lo ? 1u : 0u);
    a.lo = lo;
}

// h -> (v, P): h^2 = v * 2^(P - 298) exactly (v = 0 for h = 0).
__host__ __device__ __forceinline__ void square_parts(float h, uint64_t &v, int &P) {
    uint32_t bits;
    __builtin_memcpy(&bits, &h, 4);
    bits &= 0x7fffffffu;
    const uint32_t E = bits >> 23, mant = bits & 0x7fffffu;
    const uint64_t m = E ? (mant | 0x800000u) : mant;
    v = m * m;
    P = E ? 2 * (int)E - 2 : 0;
}

// Position (in units of 2^-298) of the top bit of v * 2^P, v > 0.
__host__ __device__ __forceinline__ int top_position(uint64_t v, int P) {
    return P + 63 - __builtin_clzll(v);
}

// Bits [b, b + kWin) of x = v * 2^P (all bits >= b when !masked), as an
// integer in units of 2^b; *rem is set when x has bits below b.
__host__ __device__ __forceinline__ U128 window_bits(uint64_t v, int P, int b, bool masked,
                                                     bool *rem) {
    U128 r{0, 0};
    const int d = P - b;
    if (d >= 0) {
        *rem = false;
        if (d < 64) {
            r.lo = v << d;
            r.hi = d ? v >> (64 - d) : 0;
        } else if (d < 128) {
            r.hi = v << (d - 64);
        }
        if (masked) {
            if (d >= kWin) r = U128{0, 0};
            else r.hi &= (1ull << (kWin - 64)) - 1;
        }
    } else {
        const int s = -d;
        if (s < 64) {
            r.lo = v >> s;
            *rem = (v & ((1ull << s) - 1)) != 0;
        } else {
            *rem = v != 0;
        }
    }
    return r;
}

// The same as window_bits, without branches (one straight sequence of selects
// per square, so the lanes of a wave never diverge) and with the square's
// parts formed from the fp32 value here: adds the window bits of h^2 to acc
// and counts a square with bits below b in cnt.  Shift counts are kept in
// 0..63 so every shift is defined; out-of-range cases are selected away.
template <bool MASKED>
__host__ __device__ __forceinline__ void window_add(float h, int b, U128 &acc, uint32_t &cnt) {
    uint32_t bits;
    __builtin_memcpy(&bits, &h, 4);
    bits &= 0x7fffffffu;
    const uint32_t E = bits >> 23;
    const uint32_t m = (bits & 0x7fffffu) | (E ? 0x800000u : 0u);
    const uint64_t v = (uint64_t)m * m;
    const int d = (E ? 2 * (int)E - 2 : 0) - b;
    // bits below b: v >> s, s = -d (all of v when s >= 64)
    const int s = d < 0 ? -d : 0;
    const uint64_t vr = s < 64 ? v >> (s & 63) : 0;
    const uint64_t below = s == 0 ? 0 : (s < 64 ? v << ((64 - s) & 63) : v);
    // the rest shifted up by l = d (<= 112 at level 1)
    const int l = d > 0 ? d : 0;
    uint64_t lo = l < 64 ? vr << (l & 63) : 0;
    uint64_t hi = l == 0 ? 0 : (l < 64 ? vr >> ((64 - l) & 63) : (l < 128 ? vr << ((l - 64) & 63) : 0));
    if (MASKED) {
        hi &= (1ull << (kWin - 64)) - 1;
        if (l >= kWin) lo = hi = 0;
    }
    const uint64_t nlo = acc.lo + lo;
    acc.hi += hi + (nlo < lo ? 1u : 0u);
    acc.lo = nlo;
    cnt += below != 0 ? 1u : 0u;
}

// Level 1 on the FP64 units.  With b the window's bottom position, the
// square x = h^2 (exact in binary64) is split into three parts that are
// exact multiples of 2^(b+75), 2^(b+37) and 2^b, each below 2^38 of its unit
// (x < 2^(b+113) at level 1): part k = floor(x_k / u_k) * u_k with x_k what
// the higher parts left, formed as fl(fl(x_k + sigma) - sigma), sigma =
// 2^52 * u_k (x_k rounded to a multiple of u_k, exact), minus u_k where that
// rounded up; x_k minus the part is exact.  Every part, and every sum of at
// most 2^15 of them, is an integer multiple of its unit below 2^53 units, so
// the three per-bin double accumulators are exact in any order.  What is left
// below 2^b marks the square in cnt.  bin_unit(k) gives the scales.
struct Bins3 {
    double s[3];
};
__host__ __device__ __forceinline__ double pos_scale(int pos) {   // 2^(pos - 298)
    return __builtin_ldexp(1.0, pos - 298);
}
__host__ __device__ __forceinline__ void window_add_f64(float h, const double *unit,
                                                       const double *sigma, Bins3 &acc,
                                                       uint32_t &cnt) {
    const double hd = (double)h;
    double x = hd * hd;
#pragma unroll
    for (int k = 0; k < 3; ++k) {
        double q = (x + sigma[k]) - sigma[k];
        q = q > x ? q - unit[k] : q;
        x = x - q;
        acc.s[k] += q;
    }
    cnt += x != 0.0 ? 1u : 0u;
}
// The exact integer sum_k bins[k] / unit_k * 2^(shift_k), shift = 75, 37, 0,
// unit_k = 2^(b + shift_k - 298) (each bins[k] an integer multiple of its
// unit below 2^53 units).
__host__ __device__ __forceinline__ U128 bins_to_u128(const double *bins, int b) {
    U128 r{0, 0};
    const int shift[3] = {75, 37, 0};
#pragma unroll
    for (int k = 0; k < 3; ++k) {
        const double n = bins[k] * __builtin_ldexp(1.0, 298 - b - shift[k]);   // exact
        const double nh = __builtin_floor(n * 0x1p-32);
        const uint64_t v = ((uint64_t)(uint32_t)nh << 32) | (uint32_t)(n - nh * 0x1p32);
        const int sh = shift[k];
        const U128 t = sh == 0 ? U128{v, 0}
                     : sh < 64 ? U128{v << sh, v >> (64 - sh)}
                               : U128{0, v << (sh - 64)};
        add128(r, t);
    }
    return r;
}

__host__ __device__ __forceinline__ int top_bit128(const U128 &a) {
    return a.hi ? 127 - __builtin_clzll(a.hi) : 63 - __builtin_clzll(a.lo);
}
__host__ __device__ __forceinline__ uint64_t shr128(const U128 &a, int s) {   // low 64 bits of a >> s
    if (s == 0) return a.lo;
    if (s < 64) return (a.lo >> s) | (a.hi << (64 - s));
    return a.hi >> (s - 64);
}
__host__ __device__ __forceinline__ bool low_bits_zero128(const U128 &a, int s) {   // a mod 2^s == 0
    if (s <= 0) return true;
    if (s < 64) return (a.lo & ((1ull << s) - 1)) == 0;
    if (a.lo) return false;
    return s == 64 || (a.hi & ((1ull << (s - 64)) - 1)) == 0;
}
// a mod 2^s + c > 2^s ?  (0 < s < 128, c >= 0 small)
__host__ __device__ __forceinline__ bool may_carry128(const U128 &a, int s, uint64_t c) {
    if (c == 0) return false;
    // room = 2^s - (a mod 2^s); carry possible when c > room
    if (s < 64) {
        const uint64_t low = a.lo & ((1ull << s) - 1);
        return c > (1ull << s) - low;
    }
    const uint64_t hmask = s == 64 ? 0 : (1ull << (s - 64)) - 1;
    const uint64_t lh = a.hi & hmask;
    if (lh != hmask) return false;   // room >= 2^64 > c
    // high part of the low bits all ones: room = 2^64 - a.lo
    return a.lo != 0 && c > (~a.lo) + 1;
}

// Level 1: A = sum of the window integers (unit 2^(b - 298)), cnt = number of
// squares with bits below b.  If the rounding of the exact sum is decided,
// writes it to *ss and returns true.  A >= 2^kWin (the largest square alone).
__host__ __device__ __forceinline__ bool round_level1(const U128 &A, uint64_t cnt, int b,
                                                      double *ss) {
    const int t = top_bit128(A);
    const int r = t - 53;                     // round-bit index (>= kWin - 53)
    if (may_carry128(A, r, cnt)) return false;
    uint64_t keep = shr128(A, r + 1);         // 53 bits
    const bool rb = (shr128(A, r) & 1u) != 0;
    const bool sticky = cnt != 0 || !low_bits_zero128(A, r);
    if (rb && (sticky || (keep & 1u))) ++keep;
    *ss = __builtin_ldexp((double)keep, r + 1 + b - 298);
    return true;
}

// ---- slow path: an exact big integer, 32-bit digits, least significant first
// big = big * 2^kWin + a
__host__ __device__ __forceinline__ void big_shift_add(uint32_t *big, const U128 &a) {
    const int ds = kWin / 32, bs = kWin % 32;   // 3 digits and 16 bits
    for (int i = kBigDigits - 1; i >= 0; --i) {
        const int j = i - ds;
        uint64_t v = 0;
        if (j >= 0) v = (uint64_t)big[j] << bs;
        if (j - 1 >= 0 && bs) v |= (uint64_t)big[j - 1] >> (32 - bs);
        big[i] = (uint32_t)v;
    }
    const uint32_t add[4] = {(uint32_t)a.lo, (uint32_t)(a.lo >> 32), (uint32_t)a.hi,
                             (uint32_t)(a.hi >> 32)};
    uint64_t carry = 0;
    for (int i = 0; i < kBigDigits; ++i) {
        const uint64_t s = (uint64_t)big[i] + (i < 4 ? add[i] : 0u) + carry;
        big[i] = (uint32_t)s;
        carry = s >> 32;
    }
}
__host__ __device__ __forceinline__ int big_bit(const uint32_t *big, int i) {
    return (int)((big[i >> 5] >> (i & 31)) & 1u);
}
// The exact integer big (unit 2^(b - 298)) rounded once to binary64.
__host__ __device__ __forceinline__ double big_round(const uint32_t *big, int b) {
    int top = -1;
    for (int i = kBigDigits - 1; i >= 0 && top < 0; --i)
        if (big[i]) top = 32 * i + 31 - __builtin_clz(big[i]);
    if (top < 0) return 0.0;
    uint64_t keep = 0;
    const int lo = top - 52;
    for (int i = top; i >= lo && i >= 0; --i) keep = 2 * keep + (uint64_t)big_bit(big, i);
    if (lo <= 0) return __builtin_ldexp((double)keep, b - 298);   // at most 53 bits: exact
    const int rb = big_bit(big, lo - 1);
    int sticky = 0;
    for (int i = lo - 2; i >= 0 && !sticky; --i) sticky = big_bit(big, i);
    if (rb && (sticky || (keep & 1u))) ++keep;
    return __builtin_ldexp((double)keep, lo + b - 298);
}

// ---- digit sums of fp32 magnitudes (AbsMean) ----
constexpr int kMagDigits = 9;     // 288 bits >= 24 + 253
constexpr int kMagNorm = 12;      // normalised digits of a (workgroup or total) sum

// Carry-save digits (each < 2^64) -> normalised 32-bit digits.
__host__ __device__ __forceinline__ void mag_normalise(const uint64_t *d, int nd, uint32_t *out) {
    uint64_t carry = 0;
    for (int i = 0; i < kMagNorm; ++i) {
        const uint64_t x = (i < nd ? d[i] : 0);
        const uint64_t lo = (x & 0xffffffffu) + (carry & 0xffffffffu);
        out[i] = (uint32_t)lo;
        carry = (x >> 32) + (carry >> 32) + (lo >> 32);
    }
}

// Normalised digits (units 2^-149) rounded once to binary64.
__host__ __device__ __forceinline__ double mag_round(const uint32_t *n) {
    // Word-level: the top three words form a 96-bit window W (bit 0 of W has
    // weight 2^(32*(ti-2)-149); words below index 0 count as zero), of which
    // the 53 bits from W's top bit are kept; the round bit and the sticky bit
    // (the rest of W and every lower word) decide round-to-nearest-even.
    // Every index below is a compile-time one (unrolled), so nothing goes to
    // scratch memory.
    int ti = -1;
#pragma unroll
    for (int i = 0; i < kMagNorm; ++i)
        if (n[i]) ti = i;
    if (ti < 0) return 0.0;
    uint32_t w2 = 0, w1 = 0, w0 = 0, below = 0;
#pragma unroll
    for (int i = 0; i < kMagNorm; ++i) {
        if (i == ti) w2 = n[i];
        if (i == ti - 1) w1 = n[i];
        if (i == ti - 2) w0 = n[i];
        if (i < ti - 2) below |= n[i];
    }
    const uint64_t hi = (uint64_t)w2 << 32 | w1;
    const int s = 95 - __builtin_clz(w2) - 52;   // low bits of W dropped: 12..43
    uint64_t keep;
    int rb, sticky;
    if (s <= 32) {
        keep = (hi << (32 - s)) | ((uint64_t)w0 >> s);
        rb = (int)((w0 >> (s - 1)) & 1u);
        sticky = (s > 1 && (w0 & ((1u << (s - 1)) - 1u)) != 0) || below != 0;
    } else {
        keep = hi >> (s - 32);
        rb = (int)((hi >> (s - 33)) & 1u);
        sticky = (s > 33 && (hi & ((1ull << (s - 33)) - 1ull)) != 0) || w0 != 0 || below != 0;
    }
    if (rb && (sticky || (keep & 1u))) ++keep;
    return __builtin_ldexp((double)keep, 32 * (ti - 2) + s - 149);
}

}  // namespace bitnet
