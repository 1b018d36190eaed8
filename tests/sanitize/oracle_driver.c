/*
 * oracle_driver.c -- runs every function of oracle/topk_oracle.c over
 * exactly sized heap buffers (so that AddressSanitizer sees any access
 * past them) on random rows, edge lengths and edge k, for a build with
 * -fsanitize=address,undefined.  Test infrastructure: the results are
 * checked by the pins, not here; this only has to finish cleanly.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

uint16_t oracle_key(uint16_t bits);
int oracle_is_nan(uint16_t bits);
uint16_t oracle_block_key(const uint16_t *x8);
void oracle_keys(const uint16_t *bits, int64_t count, uint16_t *keys);
int32_t oracle_row_elements(int32_t v, int32_t mode);
int32_t oracle_row_keys(const uint16_t *row, int32_t v, int32_t mode, uint16_t *keys);
int oracle_threshold(const uint16_t *keys, int32_t n, int32_t k, uint16_t *T,
                     int32_t *count_gt, int32_t *count_eq);
int oracle_topk_row(const uint16_t *row, int32_t valid_len, int32_t width, int32_t k,
                    int32_t mode, const int32_t *pages, int32_t page_size, int32_t *out);
int oracle_topk_rows(const uint16_t *logits, int64_t row_stride, const int32_t *valid_len,
                     int32_t row_begin, int32_t row_end, int32_t width, int32_t k,
                     int32_t mode, const int32_t *pages, int64_t pages_stride,
                     int32_t page_size, int32_t *out);
int oracle_topk_row_ordered(const uint16_t *row, int32_t valid_len, int32_t width, int32_t k,
                            int32_t mode, const int32_t *pages, int32_t page_size,
                            int32_t *out, int32_t *ids, int32_t *valid);
int oracle_topk_rows_ordered(const uint16_t *logits, int64_t row_stride,
                             const int32_t *valid_len, int32_t row_begin, int32_t row_end,
                             int32_t width, int32_t k, int32_t mode, const int32_t *pages,
                             int64_t pages_stride, int32_t page_size, int32_t *out,
                             int32_t *ids, int32_t *valid);
void oracle_vector_maxima(const uint16_t *row, int32_t valid_len, int32_t width,
                          uint16_t *tops);

static uint64_t state = 0x9E3779B97F4A7C15ull;
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
    uint32_t i;
    int trial;
    uint16_t keys[65536];
    uint16_t all[65536];
    for (i = 0; i < 65536; ++i)
        all[i] = (uint16_t)i;
    oracle_keys(all, 65536, keys);
    for (i = 0; i < 65536; ++i)
        (void)oracle_is_nan((uint16_t)i);
    for (trial = 0; trial < 200; ++trial) {
        const int32_t width = (int32_t)(next() % 700);
        const int32_t rows = 1 + (int32_t)(next() % 3);
        const int32_t mode = (int32_t)(next() % 2);
        const int32_t pad = (int32_t)(next() % 3) * 8;
        const int64_t stride = (int64_t)((width + 7) / 8 * 8 + pad);
        const int32_t k = 1 + (int32_t)(next() % (trial % 5 == 0 ? 2048 : 40));
        const int32_t psz = 1 << (next() % 8);
        const int32_t npg = (width + psz - 1) / psz;
        const int64_t pstride = npg + (int64_t)(next() % 3);
        uint16_t *logits = must(sizeof(uint16_t) * (size_t)(rows * stride));
        int32_t *vl = must(sizeof(int32_t) * (size_t)rows);
        int32_t *pages = must(sizeof(int32_t) * (size_t)(rows * pstride));
        int32_t *out = must(sizeof(int32_t) * (size_t)rows * (size_t)k);
        int32_t *ids = must(sizeof(int32_t) * (size_t)rows * (size_t)k);
        int32_t *valid = must(sizeof(int32_t) * (size_t)rows);
        uint16_t *tops = must(sizeof(uint16_t) * (size_t)((width + 7) / 8));
        uint16_t *rk = must(sizeof(uint16_t) * (size_t)(width ? width : 1));
        int32_t r, j;
        for (j = 0; j < rows * stride; ++j)
            logits[j] = (uint16_t)((trial % 3 == 0) ? (0x3F80 + next() % 4) : next());
        for (r = 0; r < rows; ++r) {
            const uint32_t c = next() % 6;
            vl[r] = c == 0 ? -3 : c == 1 ? width + 5 : c == 2 ? 0 : (int32_t)(next() % (width + 1));
            for (j = 0; j < pstride; ++j)
                pages[r * pstride + j] = (int32_t)(next() % 1000);
        }
        (void)oracle_topk_rows(logits, stride, vl, 0, rows, width, k, mode,
                               (trial & 1) ? pages : NULL, pstride, psz, out);
        (void)oracle_topk_rows_ordered(logits, stride, vl, 0, rows, width, k, mode,
                                       (trial & 2) ? pages : NULL, pstride, psz, out, ids,
                                       valid);
        for (r = 0; r < rows; ++r) {
            const int32_t v = vl[r] < 0 ? 0 : (vl[r] > width ? width : vl[r]);
            const int32_t n = oracle_row_keys(logits + r * stride, v, mode, rk);
            uint16_t T;
            int32_t gt, eq;
            if (n > 0)
                (void)oracle_threshold(rk, n, k, &T, &gt, &eq);
            (void)oracle_row_elements(v, mode);
            if (width > 0) {
                (void)oracle_topk_row(logits + r * stride, vl[r], width, k, mode, NULL, 64, out);
                (void)oracle_topk_row_ordered(logits + r * stride, vl[r], width, k, mode, NULL,
                                              64, out, ids, valid);
                oracle_vector_maxima(logits + r * stride, vl[r], width, tops);
            }
            if (v >= 8)
                (void)oracle_block_key(logits + r * stride);
        }
        free(logits);
        free(vl);
        free(pages);
        free(out);
        free(ids);
        free(valid);
        free(tops);
        free(rk);
    }
    printf("oracle driver done\n");
    return 0;
}
