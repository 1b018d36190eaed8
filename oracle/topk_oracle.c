/*
 * topk_oracle.c -- plain CPU definition of exact per-row top-k over BF16
 * logits.
 *
 * TEST INFRASTRUCTURE ONLY.  The tests, the smoke check and the benchmark's
 * CPU-baseline leg may load this library; the product path (libtopk) never
 * does, and the two share no code, header, table or constant.
 *
 * It is deliberately slow and literal: every row is turned into its element
 * keys, the (key, index) pairs are fully sorted with the C library's qsort,
 * and the first k are taken.  No blocking, sampling or radix logic.
 *
 * Sources (the web pages this follows):
 *  [DTK] vLLM API page "vllm.models.deepseek_v41.nvidia.specialized_decode.
 *        attention.decode_topk_cute", module docstring, paragraph
 *        "What this module computes" (result definition, token and block
 *        elements, pinned newest block, -inf blocks, padding).
 *  [SGL] sglang PR #39305 "[dsv4.1] Exact bf16 consumer top-k adapted from
 *        DeepSelect", section "What is kept from DeepSelect" (the 16-bit
 *        order-preserving value order).
 *  [K3]  vLLM API page "vllm.models.kimi_k3.nvidia.specialized_decode.
 *        cutedsl.dsa.indexer", IndexerSelect.emit (block-table transform)
 *        and the short-context bypass in IndexerSelect.kernel (length
 *        clamped at zero); IndexerScore's epilogue (the side array of each
 *        8 logits' largest key).
 *
 * Readings where the pages leave a point open (each also listed in the
 * design notes):
 *  - NaN order: NaNs are ordinary keys ([DTK] compares only through the
 *    key), so positive NaNs rank above +inf and negative NaNs below -inf.
 *  - Block max with a NaN: the result is the canonical positive NaN, bits
 *    0x7FFF, whose key is 0xFFFF.
 *  - Block max of +0 and -0: taken in key order (+0 above -0).
 *  - Ties at the k-th key: any choice is correct; this oracle keeps the
 *    lowest indices (stable order by index), the checker accepts any.
 *  - valid_len is clamped to [0, width].
 *  - Rows with n <= k: indices 0..n-1 in order, then -1; in block mode a
 *    selected -inf block is written as -1 in this case too.
 *  - Page transform: out = pages[r][i / P] * P + i % P for every i >= 0;
 *    -1 stays -1.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_TOKEN 0
#define ORACLE_BLOCK 1

/* [SGL] value order: a negative BF16 pattern (sign bit set) has all 16 bits
 * inverted, a non-negative one only its sign bit, so that unsigned order of
 * the result is the value order (negatives reversed and below positives,
 * -0 just below +0). */
uint16_t oracle_key(uint16_t bits)
{
    if (bits & 0x8000u)
        return (uint16_t)(bits ^ 0xFFFFu);
    return (uint16_t)(bits ^ 0x8000u);
}

/* BF16 NaN: exponent field all ones and a non-zero mantissa. */
int oracle_is_nan(uint16_t bits)
{
    return ((bits & 0x7F80u) == 0x7F80u) && ((bits & 0x007Fu) != 0u);
}

/* [DTK] block element: the NaN-propagating maximum of 8 aligned logits,
 * compared through the key.  Reading: a block holding any NaN evaluates to
 * the canonical positive NaN 0x7FFF. */
uint16_t oracle_block_key(const uint16_t *x8)
{
    int i;
    uint16_t best;
    for (i = 0; i < 8; ++i)
        if (oracle_is_nan(x8[i]))
            return oracle_key(0x7FFFu);
    best = oracle_key(x8[0]);
    for (i = 1; i < 8; ++i) {
        uint16_t k = oracle_key(x8[i]);
        if (k > best)
            best = k;
    }
    return best;
}

/* Keys of an array of BF16 patterns (for the checker and the pins). */
void oracle_keys(const uint16_t *bits, int64_t count, uint16_t *keys)
{
    int64_t i;
    for (i = 0; i < count; ++i)
        keys[i] = oracle_key(bits[i]);
}

static int32_t clamp_len(int32_t v, int32_t width)
{
    if (v < 0)
        return 0;
    if (v > width)
        return width;
    return v;
}

/* Number of elements of a row with v valid logits: one per logit in token
 * mode, one per (possibly partial) group of 8 in block mode [DTK]. */
int32_t oracle_row_elements(int32_t v, int32_t mode)
{
    if (mode == ORACLE_BLOCK)
        return (v + 7) / 8;
    return v;
}

/* The element keys of one row ([DTK]): token mode, the key of each of the
 * first v logits; block mode, the block key of each aligned group of 8,
 * except the newest block (the last one), whose key is that of +inf (bits
 * 0x7F80) whatever it holds.  Returns n. */
int32_t oracle_row_keys(const uint16_t *row, int32_t v, int32_t mode,
                        uint16_t *keys)
{
    int32_t n = oracle_row_elements(v, mode);
    int32_t i;
    if (mode == ORACLE_TOKEN) {
        for (i = 0; i < n; ++i)
            keys[i] = oracle_key(row[i]);
        return n;
    }
    for (i = 0; i + 1 < n; ++i)
        keys[i] = oracle_block_key(row + (int64_t)8 * i);
    if (n > 0)
        keys[n - 1] = oracle_key(0x7F80u);
    return n;
}

typedef struct {
    uint16_t key;
    int32_t index;
} oracle_item;

/* Larger key first; equal keys by ascending index. */
static int by_key_desc(const void *pa, const void *pb)
{
    const oracle_item *a = (const oracle_item *)pa;
    const oracle_item *b = (const oracle_item *)pb;
    if (a->key != b->key)
        return a->key > b->key ? -1 : 1;
    if (a->index != b->index)
        return a->index < b->index ? -1 : 1;
    return 0;
}

/* The k-th largest key T of keys[0:n] (n > k >= 1), and how many keys are
 * above it and equal to it.  Plain full sort. Returns 0, or -1 if n <= k
 * or k < 1 (no threshold then). */
int oracle_threshold(const uint16_t *keys, int32_t n, int32_t k,
                     uint16_t *T, int32_t *count_gt, int32_t *count_eq)
{
    oracle_item *items;
    int32_t i, gt = 0, eq = 0;
    uint16_t t;
    if (k < 1 || n <= k)
        return -1;
    items = (oracle_item *)malloc(sizeof(oracle_item) * (size_t)n);
    if (!items)
        return -2;
    for (i = 0; i < n; ++i) {
        items[i].key = keys[i];
        items[i].index = i;
    }
    qsort(items, (size_t)n, sizeof(oracle_item), by_key_desc);
    t = items[k - 1].key;
    free(items);
    for (i = 0; i < n; ++i) {
        if (keys[i] > t)
            ++gt;
        else if (keys[i] == t)
            ++eq;
    }
    *T = t;
    *count_gt = gt;
    *count_eq = eq;
    return 0;
}

/* One row of the result ([DTK] "What this module computes"):
 *  n <= k : 0, 1, ..., n-1, then -1 up to k (the short-row case; [K3]
 *           bypass writes the same pattern);
 *  n >  k : the indices of the first k items of the (key desc, index asc)
 *           order, i.e. every key above the k-th key and the lowest-index
 *           keys equal to it.
 * Block mode then writes -1 for every selected element whose key is that of
 * -inf (bits 0xFF80).  Finally, with a block table, each index i >= 0
 * becomes pages[i / P] * P + i % P ([K3] IndexerSelect.emit).
 * Returns 0, or -2 on allocation failure. */
int oracle_topk_row(const uint16_t *row, int32_t valid_len, int32_t width,
                    int32_t k, int32_t mode, const int32_t *pages,
                    int32_t page_size, int32_t *out)
{
    int32_t v = clamp_len(valid_len, width);
    int32_t n, j, cnt;
    uint16_t *keys;
    uint16_t neg_inf_key = oracle_key(0xFF80u);
    keys = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)(width > 0 ? width : 1));
    if (!keys)
        return -2;
    n = oracle_row_keys(row, v, mode, keys);
    if (n <= k) {
        for (j = 0; j < n; ++j)
            out[j] = j;
        cnt = n;
    } else {
        oracle_item *items = (oracle_item *)malloc(sizeof(oracle_item) * (size_t)n);
        if (!items) {
            free(keys);
            return -2;
        }
        for (j = 0; j < n; ++j) {
            items[j].key = keys[j];
            items[j].index = j;
        }
        qsort(items, (size_t)n, sizeof(oracle_item), by_key_desc);
        for (j = 0; j < k; ++j)
            out[j] = items[j].index;
        free(items);
        cnt = k;
    }
    if (mode == ORACLE_BLOCK)
        for (j = 0; j < cnt; ++j)
            if (keys[out[j]] == neg_inf_key)
                out[j] = -1;
    for (j = cnt; j < k; ++j)
        out[j] = -1;
    if (pages)
        for (j = 0; j < k; ++j)
            if (out[j] >= 0)
                out[j] = pages[out[j] / page_size] * page_size + out[j] % page_size;
    free(keys);
    return 0;
}

/* Rows [row_begin, row_end) of a [rows, row_stride] BF16 matrix into
 * out[rows, k].  pages (may be NULL) is [rows, pages_stride].  Returns 0 or
 * the first row's error. */
int oracle_topk_rows(const uint16_t *logits, int64_t row_stride,
                     const int32_t *valid_len, int32_t row_begin,
                     int32_t row_end, int32_t width, int32_t k, int32_t mode,
                     const int32_t *pages, int64_t pages_stride,
                     int32_t page_size, int32_t *out)
{
    int32_t r;
    for (r = row_begin; r < row_end; ++r) {
        const int32_t *prow = pages ? pages + (int64_t)r * pages_stride : NULL;
        int rc = oracle_topk_row(logits + (int64_t)r * row_stride, valid_len[r],
                                 width, k, mode, prow, page_size,
                                 out + (int64_t)r * k);
        if (rc)
            return rc;
    }
    return 0;
}

static int by_index_asc(const void *pa, const void *pb)
{
    const int32_t a = *(const int32_t *)pa, b = *(const int32_t *)pb;
    return a < b ? -1 : (a > b ? 1 : 0);
}

/* The deterministic ordered result of one row ([K3] IndexerSelect class
 * docstring and its ordered output pass: the selected keys in key order,
 * that is by ascending element index, ties at the threshold going to the
 * lowest indices; -1 past the row's count; the counts in `valid`; the
 * logical element indices in `ids`):
 *  ids[0:c]  the selected element indices in ascending order, where the
 *            selection is the first c = min(n, k) items of the (key desc,
 *            index asc) order (all n elements when n <= k), then -1 up to k;
 *  out[j]    -1 where ids[j] is -1 or, in block mode, where the element's
 *            key is that of -inf (the [DTK] -1 rule); otherwise ids[j]
 *            through the block table, as in oracle_topk_row;
 *  *valid    c.
 * ids may be NULL.  Returns 0, or -2 on allocation failure. */
int oracle_topk_row_ordered(const uint16_t *row, int32_t valid_len, int32_t width,
                            int32_t k, int32_t mode, const int32_t *pages,
                            int32_t page_size, int32_t *out, int32_t *ids,
                            int32_t *valid)
{
    int32_t v = clamp_len(valid_len, width);
    int32_t n, j, cnt;
    uint16_t *keys;
    int32_t *sel;
    uint16_t neg_inf_key = oracle_key(0xFF80u);
    keys = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)(width > 0 ? width : 1));
    sel = (int32_t *)malloc(sizeof(int32_t) * (size_t)(k > 0 ? k : 1));
    if (!keys || !sel) {
        free(keys);
        free(sel);
        return -2;
    }
    n = oracle_row_keys(row, v, mode, keys);
    if (n <= k) {
        for (j = 0; j < n; ++j)
            sel[j] = j;
        cnt = n;
    } else {
        oracle_item *items = (oracle_item *)malloc(sizeof(oracle_item) * (size_t)n);
        if (!items) {
            free(keys);
            free(sel);
            return -2;
        }
        for (j = 0; j < n; ++j) {
            items[j].key = keys[j];
            items[j].index = j;
        }
        qsort(items, (size_t)n, sizeof(oracle_item), by_key_desc);
        for (j = 0; j < k; ++j)
            sel[j] = items[j].index;
        free(items);
        cnt = k;
        qsort(sel, (size_t)cnt, sizeof(int32_t), by_index_asc);
    }
    for (j = 0; j < k; ++j) {
        int32_t i = j < cnt ? sel[j] : -1;
        int32_t o = i;
        if (i >= 0 && mode == ORACLE_BLOCK && keys[i] == neg_inf_key)
            o = -1;
        if (o >= 0 && pages)
            o = pages[o / page_size] * page_size + o % page_size;
        out[j] = o;
        if (ids)
            ids[j] = i;
    }
    *valid = cnt;
    free(keys);
    free(sel);
    return 0;
}

/* oracle_topk_row_ordered over rows [row_begin, row_end) of a
 * [rows, row_stride] BF16 matrix: out and ids [rows, k], valid [rows]
 * (ids may be NULL).  Returns 0 or the first row's error. */
int oracle_topk_rows_ordered(const uint16_t *logits, int64_t row_stride,
                             const int32_t *valid_len, int32_t row_begin,
                             int32_t row_end, int32_t width, int32_t k, int32_t mode,
                             const int32_t *pages, int64_t pages_stride,
                             int32_t page_size, int32_t *out, int32_t *ids,
                             int32_t *valid)
{
    int32_t r;
    for (r = row_begin; r < row_end; ++r) {
        const int32_t *prow = pages ? pages + (int64_t)r * pages_stride : NULL;
        int rc = oracle_topk_row_ordered(logits + (int64_t)r * row_stride, valid_len[r],
                                         width, k, mode, prow, page_size,
                                         out + (int64_t)r * k,
                                         ids ? ids + (int64_t)r * k : NULL, valid + r);
        if (rc)
            return rc;
    }
    return 0;
}

/* [K3] IndexerScore epilogue: the side array of vector maxima.  tops[j],
 * for every j < ceil(width / 8), is the largest key among logits 8j ..
 * 8j+7 that lie below the clamped valid length, or 0 when none does (the
 * epilogue starts each lane's maximum at 0 and folds in only the keys it
 * stores).  A plain loop over the logits. */
void oracle_vector_maxima(const uint16_t *row, int32_t valid_len, int32_t width,
                          uint16_t *tops)
{
    int32_t v = clamp_len(valid_len, width);
    int32_t nv = (width + 7) / 8;
    int32_t j, i;
    for (j = 0; j < nv; ++j) {
        uint16_t best = 0;
        for (i = 8 * j; i < 8 * j + 8 && i < v; ++i) {
            uint16_t k = oracle_key(row[i]);
            if (k > best)
                best = k;
        }
        tops[j] = best;
    }
}
