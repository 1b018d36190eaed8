/*
 * score_driver.c -- runs the scorer oracle (oracle/score_oracle.c) over
 * exactly sized heap buffers on random FP8 and MXFP4 inputs, every byte
 * value and the scales' whole range included, for a build with
 * -fsanitize=address,undefined.  Test infrastructure: the pins check the
 * results; this only has to finish cleanly.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

long double oracle_e4m3(uint8_t x);
long double oracle_e2m1(uint8_t nibble);
long double oracle_bf16_value(uint16_t bits);
uint16_t oracle_bf16_round(long double x);
void oracle_mqa_logits(const uint8_t *q, const uint16_t *w, int32_t rows, const uint8_t *keys,
                       const uint8_t *scales, int32_t nkeys, double delta, uint16_t *exact,
                       uint16_t *lo, uint16_t *hi);
void oracle_mxfp4_logits(const uint8_t *q, const uint8_t *q_scale, const uint16_t *w,
                         int32_t rows, const uint8_t *keys, const uint8_t *key_scales,
                         int32_t nkeys, double delta, uint16_t *exact, uint16_t *lo, uint16_t *hi);

static uint64_t state = 0x2545F4914F6CDD1Dull;
static uint32_t next(void)
{
    state ^= state << 13;
    state ^= state >> 7;
    state ^= state << 17;
    return (uint32_t)(state >> 16);
}

static void *must(size_t bytes)
{
    void *p = malloc(bytes ? bytes : 1);
    if (!p) {
        fprintf(stderr, "out of memory\n");
        exit(2);
    }
    return p;
}

int main(void)
{
    volatile long double sink = 0;
    for (int i = 0; i < 256; ++i)
        sink += oracle_e4m3((uint8_t)i) == oracle_e4m3((uint8_t)i);  /* NaN codes compare false */
    for (int i = 0; i < 16; ++i)
        sink += oracle_e2m1((uint8_t)i);
    for (int i = 0; i < 65536; ++i)
        sink += oracle_bf16_round(oracle_bf16_value((uint16_t)i)) == (uint16_t)i;
    for (int trial = 0; trial < 6; ++trial) {
        const int rows = 1 + trial % 3, nk = 1 + (int)(next() % 40);
        uint8_t *q8 = must((size_t)rows * 32 * 128), *k8 = must((size_t)nk * 128);
        uint8_t *s8 = must((size_t)nk), *q4 = must((size_t)rows * 32 * 64);
        uint8_t *qs = must((size_t)rows * 32 * 4), *k4 = must((size_t)nk * 64);
        uint8_t *ks = must((size_t)nk * 4);
        uint16_t *w = must((size_t)rows * 32 * 2);
        uint16_t *ex = must((size_t)rows * nk * 2), *lo = must((size_t)rows * nk * 2);
        uint16_t *hi = must((size_t)rows * nk * 2);
        for (int i = 0; i < rows * 32 * 128; ++i) {
            uint8_t b = (uint8_t)next();
            q8[i] = (b & 0x7F) == 0x7F ? (uint8_t)(b ^ 1) : b;
        }
        for (int i = 0; i < nk * 128; ++i) {
            uint8_t b = (uint8_t)next();
            k8[i] = (b & 0x7F) == 0x7F ? (uint8_t)(b ^ 1) : b;
        }
        for (int i = 0; i < nk; ++i)
            s8[i] = (uint8_t)(next() % 255);
        for (int i = 0; i < rows * 32 * 64; ++i)
            q4[i] = (uint8_t)next();
        for (int i = 0; i < nk * 64; ++i)
            k4[i] = (uint8_t)next();
        for (int i = 0; i < rows * 32 * 4; ++i)
            qs[i] = (uint8_t)(107 + next() % 40);
        for (int i = 0; i < nk * 4; ++i)
            ks[i] = (uint8_t)(107 + next() % 40);
        for (int i = 0; i < rows * 32; ++i)
            w[i] = (uint16_t)next();
        oracle_mqa_logits(q8, w, rows, k8, s8, nk, trial % 2 ? 0x1p-10 : 0.0, ex, lo, hi);
        oracle_mxfp4_logits(q4, qs, w, rows, k4, ks, nk, trial % 2 ? 0x1p-20 : 0.0, ex, lo, hi);
        free(q8); free(k8); free(s8); free(q4); free(qs); free(k4); free(ks);
        free(w); free(ex); free(lo); free(hi);
    }
    printf("score driver done (%d)\n", (int)(sink != 0));
    return 0;
}
