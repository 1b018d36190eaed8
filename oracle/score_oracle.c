/*
 * score_oracle.c -- plain CPU definition of the FP8 and MXFP4 MQA indexer
 * logits that feed the exact top-k (the scorer of the K3.1 decode indexer).
 *
 * TEST INFRASTRUCTURE ONLY.  The tests, the smoke check and the benchmark's
 * CPU-baseline leg may load this library; the product path (libtopk) never
 * does, and the two share no code, header, table or constant.
 *
 * Source: vLLM API page "vllm.models.kimi_k3.nvidia.specialized_decode.
 * cutedsl.dsa.indexer": the module docstring (the logit of query row t and
 * key i at the stock logits path's precision) and IndexerScore (the epilogue: each head's
 * relu(q . k) rounded to BF16, the heads weighted by BF16 FMAs in two BF16x2
 * sums, then one BF16 add, then the key's UE8M0 scale; each 8 keys' largest
 * order-preserving key into a side array).
 *
 * What is computed, literally:
 *   d_h   = sum over the 128 dims of q[h][c] * key[c]   (FP8 E4M3 values, exact)
 *   r_h   = bf16(fp32(max(d_h, 0)))                        (the head's FP32 value, then BF16)
 *   a_j   = 0; for h = j, j + 4, ..., j + 28: a_j = bf16(r_h * w_h + a_j)   (j = 0..3)
 *   total = bf16(bf16(a_0 + a_2) + bf16(a_1 + a_3))
 *   logit = bf16(total * 2^(s - 127))                      (s: the key's UE8M0 byte)
 * Every bf16(.) rounds the exact value once, to nearest with ties to even.
 * The sums are exact in long double (an FP8 product has at most 8
 * significant bits and 2^-18 <= |product| <= 448^2, so 128 of them span at
 * most 43 bits; an FMA of BF16 values spans at most 64 bits unless its
 * terms differ by more than 2^48, which no input here reaches).
 *
 * Readings (also in the design notes):
 *  - E4M3 is the OCP "fn" format: bias 7, no infinities, S.1111.111 is NaN
 *    (never an input).
 *  - The head's value is the MMA's FP32 result; its summation order is the
 *    hardware's.  The definition takes the exact dot product rounded once to
 *    FP32.  oracle_mqa_logit also returns the interval that a dot product
 *    within +-delta * sum_c |q[h][c] * key[c]| of the exact one allows, and
 *    lets each BF16 FMA round either way when its exact result lies within
 *    half an FP32 unit of a BF16 midpoint (an FMA computed in FP32 and then
 *    rounded to BF16 may do so); the rest of the chain is monotone, so the
 *    interval bounds every result those allowances permit.
 *  - UE8M0 byte s scales by 2^(s - 127); 255 (NaN) is never an input.
 *
 * The MXFP4 logits (the same page: the FP4 cache's E2M1 keys with a UE8M0
 * scale per 32 values, the FP4 query with its own scales, both applied
 * inside the block-scaled MMA, and no scale after the head sum):
 *   d_h   = sum over blocks b of 2^(sq[h][b] + sk[b] - 254) *
 *           sum over the 32 dims c of block b of q[h][c] * key[c]   (E2M1 values, exact)
 *   then r_h, a_j and total as above, and logit = total, -0 written as +0.
 * Byte j of a row holds dims 2j (low nibble) and 2j + 1 (high nibble).  The
 * long double sums are exact while one head's products span less than 2^50
 * (scales within 40 of each other).
 */
#include <float.h>
#include <math.h>
#include <stdint.h>
#include <string.h>

#define HEADS 32
#define DIM 128

/* OCP FP8 E4M3: sign, 4 exponent bits (bias 7), 3 mantissa bits;
 * exponent field 0 holds the subnormals m * 2^-9. */
long double oracle_e4m3(uint8_t x)
{
    const int e = (x >> 3) & 15, m = x & 7;
    long double v;
    if ((x & 0x7F) == 0x7F)
        return NAN;
    if (e == 0)
        v = ldexpl((long double)m, -9);
    else
        v = ldexpl(1.0L + m / 8.0L, e - 7);
    return (x & 0x80) ? -v : v;
}

/* OCP FP4 E2M1 (the low 4 bits of the argument): sign, 2 exponent bits
 * (bias 1), 1 mantissa bit; exponent field 0 holds the subnormal m / 2. */
long double oracle_e2m1(uint8_t nibble)
{
    const int e = (nibble >> 1) & 3, m = nibble & 1;
    long double v;
    if (e == 0)
        v = m / 2.0L;
    else
        v = ldexpl(1.0L + m / 2.0L, e - 1);
    return (nibble & 8) ? -v : v;
}

/* The BF16 value of a pattern (its bits are the top half of an FP32). */
long double oracle_bf16_value(uint16_t bits)
{
    const uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (long double)f;
}

/* Round a real to the nearest BF16 (8 significant bits, FP32's exponent
 * range), ties to even, and return its bits.  Above the largest finite
 * BF16 (after rounding) the result is infinity. */
uint16_t oracle_bf16_round(long double x)
{
    if (x != x)
        return 0x7FC0;
    const int neg = signbit(x) != 0;
    long double a = fabsl(x);
    uint16_t bits;
    if (a == 0) {
        bits = 0;
    } else {
        int e;
        frexpl(a, &e);              /* a in [2^(e-1), 2^e) */
        int qe = e - 8;             /* the spacing of 8-bit values in that binade */
        if (qe < -133)
            qe = -133;              /* below 2^-126 the spacing stays 2^-133 */
        const long double q = ldexpl(1.0L, qe);
        const long double r = nearbyintl(a / q) * q;   /* to nearest, ties to even */
        if (r >= ldexpl(1.0L, 128)) {
            bits = 0x7F80;
        } else {
            const float f = (float)r;                   /* exact: 8 significant bits */
            uint32_t u;
            memcpy(&u, &f, sizeof u);
            bits = (uint16_t)(u >> 16);
        }
    }
    return neg ? (uint16_t)(bits | 0x8000u) : bits;
}

/* The nearest FP32 of a real (ties to even). */
static long double fp32_round(long double x)
{
    return (long double)(float)x;
}

static long double bf16r(long double x)
{
    return oracle_bf16_value(oracle_bf16_round(x));
}

/* One BF16 FMA a * b + c of BF16 values, its rounding allowance included:
 * lo/hi are the results of rounding the exact value to BF16 directly and
 * through FP32 (the same unless the exact value lies within half an FP32
 * unit of a BF16 midpoint). */
static void fma_bf16(long double ab_c, long double *lo, long double *hi)
{
    const long double d = bf16r(ab_c), t = bf16r(fp32_round(ab_c));
    *lo = d < t ? d : t;
    *hi = d < t ? t : d;
}

/* The logit from the heads' dot products dd[h] and the sums of their
 * products' magnitudes ss[h]: the definition's BF16 pattern (*exact) and the
 * interval [*lo, *hi] (BF16 patterns, lo <= hi in value) that dot products
 * within delta times those sums, and the FMA rounding allowance, permit.
 * sc scales the BF16 total (the FP8 key scale; 1 for MXFP4, whose scales
 * are in the dot products); with clear_neg_zero a -0 logit is written +0. */
static void logit_of_heads(const long double *dd, const long double *ss, const uint16_t *w,
                           double delta, long double sc, int clear_neg_zero, uint16_t *exact,
                           uint16_t *lo, uint16_t *hi)
{
    long double r[HEADS], rlo[HEADS], rhi[HEADS];
    for (int h = 0; h < HEADS; ++h) {
        const long double d = dd[h], s = ss[h];
        const long double dl = d - (long double)delta * s, dh = d + (long double)delta * s;
        r[h] = bf16r(fp32_round(d > 0 ? d : 0));
        rlo[h] = bf16r(fp32_round(dl > 0 ? dl : 0));
        rhi[h] = bf16r(fp32_round(dh > 0 ? dh : 0));
    }
    long double a[4] = {0, 0, 0, 0}, al[4] = {0, 0, 0, 0}, ah[4] = {0, 0, 0, 0};
    for (int i = 0; i < HEADS / 4; ++i) {
        for (int j = 0; j < 4; ++j) {
            const int h = j + 4 * i;
            const long double wh = oracle_bf16_value(w[h]);
            long double l1, h1, l2, h2;
            a[j] = bf16r(r[h] * wh + a[j]);
            /* monotone in r (by the sign of w) and in the accumulator */
            const long double xl = (wh >= 0 ? rlo[h] : rhi[h]) * wh + al[j];
            const long double xh = (wh >= 0 ? rhi[h] : rlo[h]) * wh + ah[j];
            fma_bf16(xl, &l1, &h1);
            fma_bf16(xh, &l2, &h2);
            al[j] = l1;
            ah[j] = h2;
        }
    }
    const long double t = bf16r(bf16r(a[0] + a[2]) + bf16r(a[1] + a[3]));
    const long double tl = bf16r(bf16r(al[0] + al[2]) + bf16r(al[1] + al[3]));
    const long double th = bf16r(bf16r(ah[0] + ah[2]) + bf16r(ah[1] + ah[3]));
    *exact = oracle_bf16_round(t * sc);
    *lo = oracle_bf16_round(tl * sc);
    *hi = oracle_bf16_round(th * sc);
    if (clear_neg_zero) {
        if (*exact == 0x8000)
            *exact = 0;
        if (*lo == 0x8000)
            *lo = 0;
        if (*hi == 0x8000)
            *hi = 0;
    }
}

/* The logit of one query row (q: HEADS x DIM E4M3 bytes, w: HEADS BF16
 * patterns) and one key (DIM E4M3 bytes, UE8M0 scale byte), as the BF16
 * pattern of the definition (*exact) and the interval [*lo, *hi] (BF16
 * patterns, lo <= hi in value) that a dot product within delta times the
 * sum of the products' magnitudes, and the FMA rounding allowance, permit. */
void oracle_mqa_logit(const uint8_t *q, const uint16_t *w, const uint8_t *key, uint8_t scale,
                      double delta, uint16_t *exact, uint16_t *lo, uint16_t *hi)
{
    long double dd[HEADS], ss[HEADS];
    for (int h = 0; h < HEADS; ++h) {
        long double d = 0, s = 0;
        for (int c = 0; c < DIM; ++c) {
            const long double p = oracle_e4m3(q[h * DIM + c]) * oracle_e4m3(key[c]);
            d += p;
            s += fabsl(p);
        }
        dd[h] = d;
        ss[h] = s;
    }
    const long double sc = ldexpl(1.0L, (int)scale - 127);
    logit_of_heads(dd, ss, w, delta, sc, 0, exact, lo, hi);
}

/* Dim c of a row of E2M1 nibbles (byte c / 2, the low nibble for even c). */
static long double e2m1_dim(const uint8_t *row, int c)
{
    return oracle_e2m1((uint8_t)((row[c / 2] >> (4 * (c % 2))) & 15));
}

/* The MXFP4 logit of one query row (q: HEADS x DIM / 2 E2M1 bytes, q_scale:
 * HEADS x 4 UE8M0 bytes, one per 32 dims of a head, w: HEADS BF16 patterns)
 * and one key (DIM / 2 E2M1 bytes, key_scale: 4 UE8M0 bytes), with the
 * interval of oracle_mqa_logit. */
void oracle_mxfp4_logit(const uint8_t *q, const uint8_t *q_scale, const uint16_t *w,
                        const uint8_t *key, const uint8_t *key_scale, double delta,
                        uint16_t *exact, uint16_t *lo, uint16_t *hi)
{
    long double dd[HEADS], ss[HEADS];
    for (int h = 0; h < HEADS; ++h) {
        long double d = 0, s = 0;
        for (int c = 0; c < DIM; ++c) {
            const int b = c / 32;  /* the block of 32 dims that one scale byte covers */
            const long double bs = ldexpl(1.0L, (int)q_scale[h * 4 + b] + (int)key_scale[b] - 254);
            const long double p = e2m1_dim(q + h * (DIM / 2), c) * e2m1_dim(key, c) * bs;
            d += p;
            s += fabsl(p);
        }
        dd[h] = d;
        ss[h] = s;
    }
    logit_of_heads(dd, ss, w, delta, 1.0L, 1, exact, lo, hi);
}

/* The logits of rows x keys of one request: row t's query at q + t *
 * HEADS * DIM, its weights at w + t * HEADS; key i at keys + i * DIM, its
 * scale scales[i]; outputs row-major [rows, nkeys] (patterns). */
void oracle_mqa_logits(const uint8_t *q, const uint16_t *w, int32_t rows, const uint8_t *keys,
                       const uint8_t *scales, int32_t nkeys, double delta, uint16_t *exact,
                       uint16_t *lo, uint16_t *hi)
{
    for (int32_t t = 0; t < rows; ++t)
        for (int32_t i = 0; i < nkeys; ++i) {
            const int64_t o = (int64_t)t * nkeys + i;
            oracle_mqa_logit(q + (int64_t)t * HEADS * DIM, w + (int64_t)t * HEADS,
                             keys + (int64_t)i * DIM, scales[i], delta, exact + o, lo + o,
                             hi + o);
        }
}

/* The MXFP4 logits of rows x keys of one request: row t's query at q + t *
 * HEADS * DIM / 2, its scales at q_scale + t * HEADS * 4, its weights at w +
 * t * HEADS; key i at keys + i * DIM / 2, its scales at key_scales + i * 4;
 * outputs row-major [rows, nkeys] (patterns). */
void oracle_mxfp4_logits(const uint8_t *q, const uint8_t *q_scale, const uint16_t *w,
                         int32_t rows, const uint8_t *keys, const uint8_t *key_scales,
                         int32_t nkeys, double delta, uint16_t *exact, uint16_t *lo, uint16_t *hi)
{
    for (int32_t t = 0; t < rows; ++t)
        for (int32_t i = 0; i < nkeys; ++i) {
            const int64_t o = (int64_t)t * nkeys + i;
            oracle_mxfp4_logit(q + (int64_t)t * HEADS * (DIM / 2), q_scale + (int64_t)t * HEADS * 4,
                               w + (int64_t)t * HEADS, keys + (int64_t)i * (DIM / 2),
                               key_scales + (int64_t)i * 4, delta, exact + o, lo + o, hi + o);
        }
}
