/*
 * libtopk.h -- exact per-row top-k of BF16 logits on AMD Instinct MI355X
 * (gfx950).  Plain C ABI: no C++ types, no exceptions, no torch types.
 *
 * What is computed (vLLM API page "vllm.models.deepseek_v41.nvidia.
 * specialized_decode.attention.decode_topk_cute", module docstring,
 * paragraph "What this module computes"):
 *
 *   For each row r, with v = valid_len[r] clamped to [0, width]:
 *   - TOPK_MODE_TOKEN: the row has n = v elements, element i is logit i.
 *   - TOPK_MODE_BLOCK: the row has n = ceil(v / 8) elements; element b is
 *     the NaN-propagating maximum of logits 8b .. 8b+7, except the newest
 *     element n-1, which counts as +inf whatever it holds.  A block holding
 *     a NaN evaluates to the canonical positive NaN.
 *   Elements are compared through the order-preserving 16-bit key of their
 *   BF16 bits, key(x) = x ^ (x has its sign bit set ? 0xFFFF : 0x8000)
 *   (sglang PR #39305, section "What is kept from DeepSelect"), so the
 *   selection is exact: positive NaNs rank above +inf, negative NaNs below
 *   -inf, -0 just below +0.
 *   - n >  k: out[r] holds, in no particular order, the indices of k
 *     elements such that no unselected element has a larger key (every key
 *     above the k-th largest, then enough keys equal to it).
 *   - n <= k: out[r] = 0, 1, ..., n-1, then -1 up to k.  Token rows with
 *     n <= k read no logits (vLLM kimi_k3 indexer page, IndexerSelect,
 *     short-context bypass).
 *   - Block mode writes -1 in place of every selected block whose key is
 *     that of -inf.
 *   - With a block table, every index i >= 0 is written as
 *     pages[r][i >> log2(P)] * P + (i & (P - 1)), P = page_size (vLLM
 *     kimi_k3 indexer page, IndexerSelect.emit); -1 stays -1.
 *
 * Layout and ownership.  Every pointer argument except block_table and
 * options is device memory owned by the caller; the library never frees
 * or retains it past the call.  logits is row-major [rows, row_stride]
 * BF16 bit patterns, 16-byte aligned, row_stride a multiple of 8
 * elements; valid_len is int32 [rows]; out is int32 [rows, k], row-major;
 * pages is int32 [rows, pages_row_stride].
 *
 * Execution.  The call enqueues its kernels on `stream` (a hipStream_t;
 * NULL = the default stream) and returns without waiting.  It allocates
 * nothing on the hot path: rows wider than one workgroup's share (16384
 * tokens, 4096 blocks) use a per-(device, stream) scratch buffer that the
 * library allocates on first use for that stream and replaces by a larger
 * one, after synchronizing that stream, when a call needs more.  The scratch
 * is never cleared: every word a call reads there was written earlier in
 * the same call.  Under graph capture nothing is allocated: a captured call
 * needs a scratch buffer set up beforehand (by an earlier call on the stream
 * or by topk_reserve_scratch), and otherwise fails with TOPK_ERR_UNSUPPORTED.
 * A captured graph keeps the scratch address, so a buffer once used under
 * capture (or reserved) is never replaced: a later call that would need
 * more fails with TOPK_ERR_UNSUPPORTED (and a reason) instead of freeing
 * memory a graph may still use.  Calls that overlap on one stream's scratch are serialized
 * by the stream; calls on different streams get different scratch buffers;
 * a graph replayed on another stream still uses the scratch of the stream
 * it was captured on.
 *
 * Errors.  Argument errors are reported before anything is enqueued, by
 * a negative status; out is then untouched.  Values are never errors:
 * valid_len outside [0, width] is clamped and NaNs are ordinary keys.
 */
#ifndef LIBTOPK_H
#define LIBTOPK_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TOPK_MAX_K 2048
#define TOPK_MAX_WIDTH (1 << 20)

enum topk_mode {
    TOPK_MODE_TOKEN = 0, /* one element per logit */
    TOPK_MODE_BLOCK = 1  /* one element per aligned group of 8 logits */
};

enum topk_status {
    TOPK_OK = 0,
    TOPK_ERR_INVALID_ARG = -1, /* null pointer, k outside [1, 2048], bad
                                  mode, width outside [0, 2^20], rows < 0,
                                  row_stride < width, bad block table */
    TOPK_ERR_MISALIGNED = -2,  /* logits not 16-byte aligned, or
                                  row_stride not a multiple of 8 */
    TOPK_ERR_HIP = -3,         /* a HIP runtime call or launch failed;
                                  topk_last_error() has the detail */
    TOPK_ERR_UNSUPPORTED = -4  /* valid arguments this library cannot
                                  serve; topk_last_error() names the
                                  reason */
};

/* Per-row path codes written when topk_options_t.path_codes is set. */
enum topk_path {
    TOPK_PATH_SHORT = 0,         /* n <= k: 0..n-1 then -1 */
    TOPK_PATH_SAMPLED = 1,       /* sampled cutoff, k-th key above it */
    TOPK_PATH_SAMPLED_TIES = 2,  /* sampled cutoff equal to the k-th key */
    TOPK_PATH_DIRECT_FORCED = 3, /* direct radix, requested */
    TOPK_PATH_DIRECT_MISJUDGED = 4, /* direct radix: fewer than k keys at
                                       or above the sampled cutoff */
    TOPK_PATH_DIRECT_OVERFLOW = 5,  /* direct radix: more survivors above
                                       the cutoff than the buffers hold */
    TOPK_PATH_TOPS = 6,             /* vector-max bound: only the vectors
                                       whose maximum reaches it loaded */
    TOPK_PATH_DIRECT_DENSE = 7      /* direct radix: a row given vector
                                       maxima with fewer than 2k vectors,
                                       too wide for the sampled registers */
};

/* Optional block table of the page transform (host struct; `pages` is a
 * device pointer). */
typedef struct topk_block_table {
    const int32_t *pages;     /* device int32 [rows, row_stride]          */
    int64_t row_stride;       /* entries between rows; >= ceil(width/P)   */
    int32_t page_size;        /* P: tokens per page, a power of two >= 1  */
} topk_block_table_t;

/* Test and diagnosis options (host struct). */
typedef struct topk_options {
    int32_t force_direct;     /* 1: every row takes the direct radix path */
    int32_t *path_codes;      /* device int32 [rows] or NULL: topk_path   */
} topk_options_t;

/* Exact top-k of every row (see above).
 *   logits       device BF16 bits [rows, row_stride], 16-byte aligned
 *   row_stride   elements between rows; multiple of 8; >= width
 *   valid_len    device int32 [rows]; clamped to [0, width]
 *   rows         >= 0 (0: nothing is enqueued)
 *   width        logits per row, 0 .. 2^20
 *   k            1 .. 2048
 *   mode         TOPK_MODE_TOKEN or TOPK_MODE_BLOCK
 *   block_table  host pointer to a table descriptor, or NULL
 *   out          device int32 [rows, k]
 *   stream       hipStream_t, NULL for the default stream
 * Returns TOPK_OK or a negative topk_status. */
int topk_bf16_rows(const uint16_t *logits, int64_t row_stride,
                   const int32_t *valid_len, int32_t rows, int32_t width,
                   int32_t k, int32_t mode,
                   const topk_block_table_t *block_table, int32_t *out,
                   void *stream);

/* topk_bf16_rows with test and diagnosis options (NULL = none). */
int topk_bf16_rows_ex(const uint16_t *logits, int64_t row_stride,
                      const int32_t *valid_len, int32_t rows, int32_t width,
                      int32_t k, int32_t mode,
                      const topk_block_table_t *block_table, int32_t *out,
                      const topk_options_t *options, void *stream);

/* topk_bf16_rows for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same arguments, results and errors as topk_bf16_rows.  It
 * calls no allocating routine: rows wider than one workgroup's share use a
 * fixed 16 MiB scratch array that the library's code object holds on every
 * device it runs on, for the life of the process (its address is looked up
 * once per device, on the first call there).  Rows are processed in batches
 * that fit it; a single row needs at most 64 members' slices of 32,320
 * bytes (about 2.1 MB), so no call is refused for size
 * (TOPK_ERR_UNSUPPORTED would name the reason).  Every call on one device
 * shares that device's array: calls that overlap in time on one device, on
 * any streams, race and must be serialized by the caller.
 * Nothing in the array needs clearing between calls: every word a call
 * reads there was written earlier in the same call. */
int topk_bf16_rows_noalloc(const uint16_t *logits, int64_t row_stride,
                           const int32_t *valid_len, int32_t rows,
                           int32_t width, int32_t k, int32_t mode,
                           const topk_block_table_t *block_table,
                           int32_t *out, void *stream);

/* topk_bf16_rows given each row's vector maxima: the largest key of every
 * aligned group of 8 logits, a side array 1/8 of the row that a scorer can
 * write as it stores the logits (vLLM API page "vllm.models.kimi_k3.nvidia.
 * specialized_decode.cutedsl.dsa.indexer", IndexerScore's epilogue).  The
 * result is exactly that of topk_bf16_rows; only the route differs (the same
 * page, IndexerSelect passes 1 and 2): the k-th largest maximum, low, is the
 * largest key of k different groups, so the k-th key is at least low, and
 * every key at or above low lies in a group whose maximum reaches low.  Only
 * those groups (about k on smooth data) are loaded, so a row reads its
 * maxima and about 16 k bytes of logits instead of 2 v bytes.
 *   tops         device uint16 [rows, tops_stride]: tops[r][j], for every
 *                j < ceil(v / 8) (v the clamped valid length), must be the
 *                largest key (the order-preserving key above) among logits
 *                8j .. 8j+7 of row r that lie below v, as
 *                topk_bf16_vector_maxima writes it; entries from ceil(v / 8)
 *                on are not read.  A side array that breaks this gives an
 *                unspecified selection (never an access out of bounds).
 *   tops_stride  entries between rows: a multiple of 8 (16-byte rows; tops
 *                itself 16-byte aligned), at least ceil(width / 8)
 *   options      as for topk_bf16_rows_ex, or NULL
 * Other arguments as for topk_bf16_rows.  Which rows use the maxima: token
 * rows, for an unforced call, when ceil(width / 8) lies between 2k and
 * 32768 (width up to 262144, one workgroup per row).  There a row with
 * n <= k is short as always; a row with fewer than 2k vectors (where the
 * k-th largest maximum bounds loosely) takes the sampled path if it has at
 * most 16384 logits, else the direct path (TOPK_PATH_DIRECT_DENSE); every
 * other row takes the bound (TOPK_PATH_TOPS), or the direct path when a
 * wave lists more than 256 hot groups, the survivors overflow, or low is 0.
 * Other calls (block mode, whose -inf and NaN blocks are found only by
 * reading every block; other widths; a forced direct path) ignore tops and
 * run as topk_bf16_rows_ex, and tops may then be NULL.  Returns TOPK_OK or a
 * negative topk_status; asynchronous like topk_bf16_rows. */
int topk_bf16_rows_tops(const uint16_t *logits, int64_t row_stride,
                        const int32_t *valid_len, int32_t rows, int32_t width,
                        int32_t k, int32_t mode, const uint16_t *tops,
                        int64_t tops_stride,
                        const topk_block_table_t *block_table, int32_t *out,
                        const topk_options_t *options, void *stream);

/* The side array topk_bf16_rows_tops reads, for callers whose scorer does
 * not write it: tops[r][j] = the largest key among logits 8j .. 8j+7 of row
 * r below its clamped valid length, 0 where none is, for every
 * j < ceil(width / 8); the rest of the 16-byte word holding entry
 * ceil(width / 8) - 1 is written as 0.  Arguments as for topk_bf16_rows;
 * tops and tops_stride as for topk_bf16_rows_tops.  One kernel that reads
 * every valid logit once.  Returns TOPK_OK or a negative topk_status;
 * asynchronous. */
int topk_bf16_vector_maxima(const uint16_t *logits, int64_t row_stride,
                            const int32_t *valid_len, int32_t rows,
                            int32_t width, uint16_t *tops,
                            int64_t tops_stride, void *stream);

/* The FP8 MQA indexer logits the selection runs on, with their side array
 * of vector maxima (vLLM API page "vllm.models.kimi_k3.nvidia.
 * specialized_decode.cutedsl.dsa.indexer": the module docstring's logit of
 * query row t and key i at the stock logits path's precision, and IndexerScore's epilogue).
 * Row t belongs to request t / qpr, whose keys it shares with the other
 * rows of the request; for every key i below the row's clamped valid
 * length v:
 *   logits[t][i] = bf16(2^(s - 127) * sum over heads h of
 *                       bf16(relu(q[t][h] . key[i])) * w[t][h])
 * where the dot product runs over the 128 dims in FP8 E4M3 (OCP, bias 7)
 * and is taken as the matrix cores' FP32 result, s is the key's UE8M0 byte,
 * and the sum is formed as the page states: four BF16 accumulators a_j, each
 * a_j = bf16(r_h * w_h + a_j) over heads h = j, j+4, ..., j+28 in that
 * order, then bf16(bf16(a_0 + a_2) + bf16(a_1 + a_3)); every bf16() rounds
 * to nearest, ties to even.  tops[t][j] = the largest order-preserving key
 * among logits 8j .. 8j+7 of row t below v, for j < ceil(v / 8): exactly
 * the side array topk_bf16_rows_tops reads (pass logits with row stride
 * logits_stride and the same tops).  Nothing else is written.
 *   q            device FP8 E4M3 [rows, 32, 128], 16-byte aligned (the
 *                query's MX scale 1; fold its scale into w)
 *   w            device BF16 [rows, 32] head weights, 4-byte aligned
 *   keys         device FP8 E4M3 [requests, key_stride, 128], 16-byte
 *                aligned: request r's key i at keys + (r * key_stride + i)
 *                * 128
 *   key_scale    device uint8 [requests, key_stride]: UE8M0 bytes 0..254
 *                (2^(s - 127); 255 is not a scale)
 *   key_stride   keys per request slot, >= width
 *   valid_len    device int32 [rows]: keys row t scores, clamped to
 *                [0, width]
 *   rows         query rows, a multiple of qpr; qpr in [1, 8]
 *   width        keys per row at most, <= TOPK_MAX_WIDTH
 *   logits       device BF16 [rows, logits_stride], logits_stride >= width
 *   tops         device uint16 [rows, tops_stride], tops_stride >=
 *                ceil(width / 8) (a multiple of 8 and 16-byte rows to feed
 *                topk_bf16_rows_tops)
 * The matrix cores' FP8 dot product may differ from the exact one by a few
 * units of the largest product's precision (their accumulation order and
 * width are the hardware's); a logit then differs from the one of the exact
 * dot products by at most what that allows after the BF16 roundings (also,
 * an FMA whose exact result lies within half an FP32 unit of a BF16 midpoint
 * may round either way).  Returns TOPK_OK or a negative topk_status
 * (TOPK_ERR_INVALID_ARG, TOPK_ERR_MISALIGNED, TOPK_ERR_HIP); asynchronous on
 * `stream`, allocates nothing. */
int topk_fp8_mqa_logits(const uint8_t *q, const uint16_t *w, const uint8_t *keys,
                        const uint8_t *key_scale, int64_t key_stride,
                        const int32_t *valid_len, int32_t rows, int32_t qpr,
                        int32_t width, uint16_t *logits, int64_t logits_stride,
                        uint16_t *tops, int64_t tops_stride, void *stream);

/* The same logits and side array from an MXFP4 indexer cache (the same
 * page: IndexerScore's FP4 path, whose block-scaled MMA applies the scales
 * and whose epilogue applies none after the head sum):
 *   logits[t][i] = sum over heads h of bf16(relu(d(t, h, i))) * w[t][h],
 *   d(t, h, i) = sum over blocks b = 0..3 of 2^(qs[t][h][b] + ks[i][b] - 254)
 *                * (sum over dims c of block b (32 dims) of q[t][h][c] * key[i][c])
 * with the head chain, the BF16 roundings and tops exactly as for
 * topk_fp8_mqa_logits (the four accumulators, the pairing), no scale after
 * the sum, and a -0 logit written as +0.  Elements are OCP FP4 E2M1 (values
 * 0, 0.5, 1, 1.5, 2, 3, 4, 6 and their negatives), two a byte: dim 2j in
 * the low nibble of byte j, 2j + 1 in the high nibble.
 *   q            device E2M1 [rows, 32, 64], 16-byte aligned
 *   q_scale      device UE8M0 [rows, 32, 4]: head h's scale of dims 32b ..
 *                32b + 31 at byte (t * 32 + h) * 4 + b (a caller folding a
 *                per-row query scale folds it into w instead)
 *   w            device BF16 [rows, 32] head weights, 4-byte aligned
 *   keys         device E2M1 [requests, key_stride, 64], 16-byte aligned
 *   key_scale    device UE8M0 [requests, key_stride, 4]: key i's scale of
 *                dims 32b .. 32b + 31 at byte (r * key_stride + i) * 4 + b
 * and the other arguments as for topk_fp8_mqa_logits.  The matrix cores'
 * block-scaled FP32 sums may differ from the exact dot product in its last
 * FP32 bits (when the blocks' scales differ); a logit then differs from
 * that of the exact dot products only where a BF16 rounding decides it.
 * Returns TOPK_OK or a negative topk_status; asynchronous on `stream`,
 * allocates nothing. */
int topk_mxfp4_mqa_logits(const uint8_t *q, const uint8_t *q_scale, const uint16_t *w,
                          const uint8_t *keys, const uint8_t *key_scale, int64_t key_stride,
                          const int32_t *valid_len, int32_t rows, int32_t qpr,
                          int32_t width, uint16_t *logits, int64_t logits_stride,
                          uint16_t *tops, int64_t tops_stride, void *stream);

/* Deterministic ordered top-k of every row (vLLM API page
 * "vllm.models.kimi_k3.nvidia.specialized_decode.cutedsl.dsa.indexer",
 * IndexerSelect: the selected keys in key order with -1 past the row's
 * count, the counts in `valid`, the logical key indices in `ids`).  The
 * selection is that of topk_bf16_rows with the ties at the k-th key taken
 * from the lowest element indices, which makes the result unique:
 *   ids[r, 0:c]  the selected element indices in ascending order, c =
 *                min(n, k), then -1 up to k (for n <= k: 0..n-1, then -1);
 *   out[r, j]    ids[r, j] through the block table when one is given; -1
 *                where ids[r, j] is -1 and, in block mode, where the
 *                element is a -inf block;
 *   valid[r]     c.
 * Arguments as for topk_bf16_rows, plus
 *   valid        device int32 [rows], or NULL (not written)
 *   ids          device int32 [rows, k], or NULL (not written)
 * Costs over topk_bf16_rows: rows up to 16384 tokens or 4096 blocks are
 * ordered from the registers that hold them; wider rows are ordered from
 * the survivor lists their members wrote (no further read of the row, no
 * further launch; a row that leaves the sampled path is read once more).
 * Scratch as for topk_bf16_rows.  Returns TOPK_OK or a negative
 * topk_status; asynchronous like topk_bf16_rows. */
int topk_bf16_rows_ordered(const uint16_t *logits, int64_t row_stride,
                           const int32_t *valid_len, int32_t rows, int32_t width,
                           int32_t k, int32_t mode,
                           const topk_block_table_t *block_table, int32_t *out,
                           int32_t *valid, int32_t *ids, void *stream);

/* topk_bf16_rows_ordered with test and diagnosis options (NULL = none). */
int topk_bf16_rows_ordered_ex(const uint16_t *logits, int64_t row_stride,
                              const int32_t *valid_len, int32_t rows,
                              int32_t width, int32_t k, int32_t mode,
                              const topk_block_table_t *block_table,
                              int32_t *out, int32_t *valid, int32_t *ids,
                              const topk_options_t *options, void *stream);

/* A static string naming a status code. */
const char *topk_status_string(int status);

/* Detail of the last error on the calling thread ("" if none). */
const char *topk_last_error(void);

/* Size the scratch of `stream` on the current device for calls of up to
 * `rows` rows of this width, k and mode (ordered or not: the same scratch),
 * so that such calls can then be captured into HIP graphs (vLLM kimi_k3
 * indexer page, the indexer's `reserve` of its logits scratch before
 * capture).  Nothing is allocated when every row fits one workgroup.  A
 * reserved scratch is never replaced by a call (a call that needs more
 * fails with TOPK_ERR_UNSUPPORTED and a reason); further reservations grow
 * it, for several call shapes, until a call under capture has used it:
 * from then on nothing replaces it, and a larger reservation fails too.
 * Not under graph capture.  Synchronizes the stream when it replaces a
 * buffer.  Returns TOPK_OK or a negative topk_status. */
int topk_reserve_scratch(int32_t rows, int32_t width, int32_t k, int32_t mode,
                         int32_t ordered, void *stream);

/* Release every scratch buffer the library holds, reserved ones included
 * (synchronizes the streams they belong to).  Graphs captured with them
 * must not be replayed afterwards.  Optional; for tests and clean
 * shutdown. */
int topk_release_scratch(void);

#ifdef __cplusplus
}
#endif

#endif /* LIBTOPK_H */
