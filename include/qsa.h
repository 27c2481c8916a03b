/*
 * qsa.h -- C ABI of libqsa: QSA attention over an int8 KV cache on AMD Instinct MI355X (gfx950).
 *
 * The decode path for one layer is four calls on one stream:
 *   qsa_block_scores -> qsa_topk -> qsa_attn_chunk -> qsa_attn_merge
 * or the same work as one call in three launches, qsa_decode_layer (plus qsa_block_index when cells are
 * appended); the prompt path is one call, qsa_prompt_attn.
 *
 * Sources for what each call computes (pull requests against one inference engine):
 *   [1888] "#1888 QSA decode attention: split each query's cells across blocks on the int8 mma path"
 *   [2075] "#2075 QSA decode attention: PR #540's two-cells-per-step chunk kernel on every CUDA card and a
 *          bounded merge"
 *   [2806] "#2806 sycl: decode QSA selection and attention in fewer, shorter launches"
 *   [1367] "#1367 prompt attention: STRATA_PROMPT_ATTN_IMMA=1 - the int8-KV kernel on INT8 tensor cores"
 *
 * Conventions for every call:
 *   - Every array argument is DEVICE memory owned by the caller (the struct arguments themselves -- qsa_pool,
 *     qsa_partials, the pool array -- are read on the host during the call and may be freed afterwards). The
 *     library never allocates, keeps no state between calls, never synchronises, and is thread-safe.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and runs asynchronously.
 *   - Arguments are validated first. On any error the call returns a negative qsa_status and has launched
 *     nothing -- the convention of [1888] "What changed", where the split launcher returns false with nothing
 *     launched when the case is unsupported or the partials would not fit the caller's scratch.
 *   - sm_scale (the calls that take one) may be any finite value; inf or NaN returns QSA_ERR_RANGE.
 *   - Values that live in device memory (positions, ids, counts, pool indices) cannot be checked on the host;
 *     the kernels treat out-of-range values as "no cell" and never read outside the pool (documented per call).
 *   - Supported shapes: head_dim in {64, 128, 192, 256}; block_cells == 64; n_q_heads a multiple of n_kv_heads with
 *     at most 8 q heads per KV head; at most 65,535 KV heads (a launch grid dimension). Anything else returns
 *     QSA_ERR_UNSUPPORTED.
 *
 * Layouts (row-major):
 *   K and V codes   int8  [n_kv_heads][capacity][head_dim]
 *   K and V scales  float [n_kv_heads][capacity][head_dim / 64]   value = scale * code, one scale per 64-dim group
 *   block index     float [n_kv_heads][ceil(capacity / 64)][head_dim]
 *   q               float [n_rows][n_q_heads][head_dim]           q head h uses KV head h / (n_q_heads / n_kv_heads)
 *   pos             int32 [n_rows]                                 a row at position p sees cells 0..p
 */
#ifndef QSA_H
#define QSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    QSA_OK = 0,
    QSA_ERR_NULL = -1,        /* a required pointer is NULL */
    QSA_ERR_SHAPE = -2,       /* inconsistent or negative sizes */
    QSA_ERR_UNSUPPORTED = -3, /* a shape this library does not implement (head_dim, block size, GQA ratio) */
    QSA_ERR_SCRATCH = -4,     /* the caller's partials or scratch buffer is too small */
    QSA_ERR_RANGE = -5,       /* a size argument outside its range (n_valid > capacity, cell range, k, ...) */
    QSA_ERR_LAUNCH = -6       /* the HIP runtime reported an error for a launch */
} qsa_status;

typedef void *qsa_stream_t; /* hipStream_t */

typedef struct {
    int32_t n_q_heads;
    int32_t n_kv_heads;
    int32_t head_dim;    /* 64, 128, 192 or 256 */
    int32_t block_cells; /* must be 64 */
} qsa_dims;

/* One int8 KV pool (one slot's cache). Cells c < n_valid are valid; c in [n_valid, capacity) are never read.
 * v_bits selects the V format: 8 (or 0) = int8 V codes like K; 4 = K8V4, the cache format the pages list beside
 * int8 (#1888, "What changed": formats left alone; #2075, "Bit for bit": parity cases per KV format) without its
 * layout -- V codes are signed 4-bit integers (-7..7), two per byte (dim 2j in the low nibble, 2j + 1 in the high
 * one), v is [n_kv_heads][capacity][head_dim / 2] bytes, and v_scale is as for int8. K8V4 is supported by the decode
 * calls and the prompt call at head_dim 128, 192 and 256 (QSA_ERR_UNSUPPORTED at 64); the pools of one call must
 * share a format. */
typedef struct {
    const int8_t *k;
    const float *k_scale;
    const int8_t *v;
    const float *v_scale;
    const float *index; /* block index from qsa_block_index; read only by the selection calls */
    int32_t capacity;
    int32_t n_valid;
    int32_t v_bits;     /* 8 (or 0): int8 V; 4: K8V4 */
} qsa_pool;

/* Split-K chunk partials ("partials in the decode scratch", [1888] "What changed"), owned by the caller.
 *   m, l   float [n_rows][n_q_heads][max_chunks]            running max (natural-log units) and sum of e^(t - m)
 *   o      float [n_rows][n_q_heads][max_chunks][head_dim]  sum of e^(t - m) * v (not normalised)
 *   empty  uint8 [n_rows][n_q_heads][max_chunks]            1 when the chunk holds no visible cell ([2075] Summary)
 * An empty chunk is written as m = -inf, l = 0, o = 0, empty = 1. */
typedef struct {
    float *m;
    float *l;
    float *o;
    uint8_t *empty;
    int32_t max_chunks;
} qsa_partials;

/* Block index ("indexer", appended per row next to K/V in [2806] "Extra Notes"; its content is not given there):
 * index[g][b][:] = mean over the block's valid cells c (64b <= c < min(64b + 64, n_valid)) of the dequantised key
 * k_scale[g][c][d/64] * k[g][c][d]. Recomputes every block that holds a cell of [cell_begin, cell_end); blocks
 * with no valid cell are written as zeros. Requires 0 <= cell_begin <= cell_end <= capacity (QSA_ERR_RANGE).
 * pool->index is ignored; `index` is the output, laid out [n_kv][ceil(capacity/64)][head_dim]. */
qsa_status qsa_block_index(const qsa_pool *pool, qsa_dims dims, int32_t cell_begin, int32_t cell_end, float *index,
                           qsa_stream_t stream);

/* Append path: K/V and indexer appends per row ([2806] "What it leaves alone" and "What changed": a window's K/V and
 * indexer appends; per-slot appends as a follow-up). Row i encodes k_new[i] and v_new[i] ([n_rows][n_kv_heads]
 * [head_dim] f32) into cell cells[i] (device memory) of every KV head of pool pools[row_pool[i]] (row_pool NULL =
 * pool 0), writing codes and scales through the pool's pointers, which must therefore be writable. The pages give
 * the int8 format with per-64-dim scales but not its encoder; the encoding is symmetric absmax per (cell, KV head,
 * 64-dim group): amax = max |x|, scale = amax / 127, code = rint(x * (127 / amax)) clamped to [-127, 127], all in
 * fp32 with correctly rounded division and round-half-to-even; amax = 0 gives scale 0 and zero codes. Then, for
 * every pool with a non-NULL index, the index row of each block that received a cell is recomputed as
 * qsa_block_index does (after all rows are written, so rows may share a block). The pools' n_valid must already
 * count the new cells: a row whose cell is outside [0, n_valid) or whose device-side row_pool value is out of
 * range writes nothing. Rows must name distinct (pool, cell) pairs: two rows naming the same one race and may
 * leave a mix of both encodings. Two launches. */
qsa_status qsa_kv_append(const qsa_pool *pools, int32_t n_pools, const int32_t *row_pool, qsa_dims dims,
                         const float *k_new, const float *v_new, const int32_t *cells, int32_t n_rows,
                         qsa_stream_t stream);

/* Block scores ([2806] Summary table, block-score row: one sum per (query, KV head) per block):
 * scores[i][g][b] = (sum over the q heads h of KV head g of q[i][h]) . pool->index[g][b], for every block whose
 * first cell is visible (64b <= pos[i]) and valid (64b < n_valid); -inf for every other b < n_blocks.
 * scores is [n_rows][n_kv_heads][n_blocks]; n_blocks (the row width) may exceed ceil(n_valid/64) but not
 * ceil(capacity/64) (QSA_ERR_RANGE). pool->index must be non-NULL. */
qsa_status qsa_block_scores(const float *q, const int32_t *pos, int32_t n_rows, const qsa_pool *pool, qsa_dims dims,
                            int32_t n_blocks, float *scores, qsa_stream_t stream);

/* Scratch bytes qsa_topk needs (0: the radix passes run in LDS, one workgroup per row). */
size_t qsa_topk_scratch_bytes(int32_t n_rows, int32_t width, int32_t k);

/* Radix top-k per row ([2806] Summary table, top-k row: 8-bit digits, one digit found per pass by a work-group
 * scan over 256 bins; integer-exact). For each of the n_rows rows of `scores` [n_rows][width]: the k largest
 * finite scores, ties broken toward the lower index, written to ids [n_rows][k] in ascending index order and
 * padded with -1; counts [n_rows] = min(k, number of finite scores). -0.0 ranks equal to +0.0; -inf is
 * ineligible; NaN is not a supported score (it ranks above +inf). Requires 1 <= k <= width <= 16384
 * (QSA_ERR_RANGE / QSA_ERR_UNSUPPORTED). scratch may be NULL when qsa_topk_scratch_bytes returns 0. */
qsa_status qsa_topk(const float *scores, int32_t n_rows, int32_t width, int32_t k, int32_t *ids, int32_t *counts,
                    void *scratch, size_t scratch_bytes, qsa_stream_t stream);

/* Split-K chunk attention over int8 K/V ([1888] Summary and "What changed": one query's cells split over chunks,
 * partials in a scratch; [2075] Summary: chunks with no cell are marked empty).
 * For each row i, q head h and chunk j < n_chunks, over the chunk's cells c -- valid (c < n_valid) and visible
 * (c <= pos[i]) -- with t_c = sm_scale * sum_grp k_scale[g][c][grp] * sum_{d in grp} q[i][h][d] * k[g][c][d]:
 *   m = max t_c,  l = sum e^(t_c - m),  o[d] = sum e^(t_c - m) * v_scale[g][c][d/64] * v[g][c][d].
 * Sparse mode (ids != NULL): ids [n_rows][n_kv][k] and counts [n_rows][n_kv] are qsa_topk's output; the
 *   count c = counts[i][g] (clamped to [0, k]) selected blocks of row (i, g) are cut into n_chunks contiguous runs
 *   in list order, the first (c mod n_chunks) runs one block longer. Negative ids and ids past the pool are
 *   skipped. blocks_per_chunk is ignored.
 * Dense mode (ids == NULL): chunk j covers blocks [j * blocks_per_chunk, (j + 1) * blocks_per_chunk).
 * Pools: row i reads pools[row_pool[i]] (row_pool NULL = pool 0 for every row; at most 8 pools). A row whose
 *   device-side row_pool value is outside [0, n_pools) writes only empty chunks.
 * Requires 1 <= n_chunks <= out->max_chunks (else QSA_ERR_SCRATCH), 0 <= n_valid <= capacity for every pool. */
qsa_status qsa_attn_chunk(const float *q, const int32_t *pos, int32_t n_rows, const qsa_pool *pools, int32_t n_pools,
                          const int32_t *row_pool, qsa_dims dims, const int32_t *ids, const int32_t *counts, int32_t k,
                          int32_t blocks_per_chunk, int32_t n_chunks, float sm_scale, const qsa_partials *out,
                          qsa_stream_t stream);

/* Log-sum-exp merge of chunk partials ([1888] "What changed": splits merged in split order; [2075] Summary and
 * "Bit for bit": chunks marked empty are skipped; [2806] Summary table, merge row: only the chunks the call
 * reaches are folded). For each row i and q head h, over chunks j < n_active[i] (n_active NULL = n_chunks;
 * values are clamped to [0, n_chunks]) that are not marked empty: M = max m_j, L = sum e^(m_j - M) l_j,
 * out[i][h][:] = sum e^(m_j - M) o_j / L, lse[i][h] = M + ln L (lse may be NULL). A row with no such chunk gets
 * out = 0 and lse = -inf. out is [n_rows][n_q_heads][head_dim]. Requires 1 <= n_chunks (QSA_ERR_RANGE),
 * n_chunks <= in->max_chunks (QSA_ERR_SCRATCH) and n_rows * n_q_heads <= INT32_MAX (QSA_ERR_UNSUPPORTED). */
qsa_status qsa_attn_merge(const qsa_partials *in, int32_t n_rows, qsa_dims dims, int32_t n_chunks,
                          const int32_t *n_active, float *out, float *lse, qsa_stream_t stream);

/* Scratch bytes qsa_prompt_attn needs for n_q queries starting at position pos0 (0 if the arguments are invalid).
 * Covers any pool and V format: the call sees at most pos0 + n_q cells. */
size_t qsa_prompt_scratch_bytes(int32_t n_q, int32_t pos0, qsa_dims dims);

/* Prompt-chunk attention on int8 matrix cores ([1367] "What it does"): dense causal attention for n_q queries at
 * positions pos0 .. pos0 + n_q - 1 over the pool's cells c <= pos (and c < n_valid). With head_dim 128 both
 * products run on the int8 K/V codes as stored (K8V4 pools: the 4-bit V codes widened to int8 in LDS); q (scaled per
 * query and head) is split into three exact 8-bit parts and the probabilities times v_scale (scaled per KV head)
 * into four, so every int32 sum is exact. Head_dim 64, 192 and 256 (int8, and K8V4 at 192 and 256) give the same
 * attention through the chunk attention kernel in dense mode and the merge, 64 queries at a time (much slower: each
 * query reads its own cells). out [n_q][n_q_heads][head_dim]; sm_scale multiplies q . k. Requires pos0 >= 0 and
 * pos0 + n_q - 1 <= INT32_MAX (QSA_ERR_RANGE), a supported head_dim and V format (QSA_ERR_UNSUPPORTED: K8V4 at
 * head_dim 64), n_q * n_q_heads <= INT32_MAX (QSA_ERR_UNSUPPORTED) and
 * scratch_bytes >= qsa_prompt_scratch_bytes (QSA_ERR_SCRATCH). */
qsa_status qsa_prompt_attn(const float *q, int32_t n_q, int32_t pos0, const qsa_pool *pool, qsa_dims dims,
                           float sm_scale, float *out, void *scratch, size_t scratch_bytes, qsa_stream_t stream);

/* Block scores and radix top-k in one launch ([2806] Summary), one workgroup per (row, KV head) holding its score
 * row in LDS: the same scores as qsa_block_scores (same fp32 arithmetic in the same order) over n_blocks columns
 * of each row's pool (pools[row_pool[i]], row_pool NULL = pool 0), and the same ids and counts as qsa_topk with k.
 * ids [n_rows][n_kv][k] and counts [n_rows][n_kv] are required; scores [n_rows][n_kv][n_blocks] may be NULL. A row
 * whose device-side row_pool value is out of range has no eligible block. Requires every pool to carry K, V, both
 * scales and an index, 1 <= k <= n_blocks <= 16,384 and n_blocks <= ceil(capacity / 64) for every pool. */
qsa_status qsa_decode_select(const float *q, const int32_t *pos, int32_t n_rows, const qsa_pool *pools,
                             int32_t n_pools, const int32_t *row_pool, qsa_dims dims, int32_t n_blocks, int32_t k,
                             float *scores, int32_t *ids, int32_t *counts, qsa_stream_t stream);

/* Scratch bytes qsa_decode_layer needs for score rows of n_blocks columns (0 if the arguments are invalid). */
size_t qsa_decode_layer_scratch_bytes(int32_t n_rows, qsa_dims dims, int32_t n_blocks, int32_t k, int32_t n_chunks);

/* One decode layer in three launches ([2806] Summary: fewer, shorter launches per layer): the selection, then
 * qsa_attn_chunk in sparse mode with n_chunks, then qsa_attn_merge over all n_chunks. With n_blocks <= 1,024 and
 * k <= 256 the first launch writes the score rows only and every chunk workgroup takes its row's top-k itself;
 * otherwise the first launch is qsa_decode_select. For every row i (pool
 * pools[row_pool[i]], row_pool NULL = pool 0) and KV head g it computes the same scores, ids and counts as
 * qsa_block_scores + qsa_topk, and the same output as qsa_attn_chunk + qsa_attn_merge on them:
 *   out [n_rows][n_q_heads][head_dim]; lse [n_rows][n_q_heads] (may be NULL).
 * scores [n_rows][n_kv][n_blocks], ids [n_rows][n_kv][k] and counts [n_rows][n_kv] are optional outputs (NULL:
 * kept in scratch). Requires every pool to carry K, V, both scales and an index, 1 <= k <= n_blocks <= 16,384,
 * n_blocks <= ceil(capacity / 64) for every pool, n_chunks >= 1, and scratch_bytes >=
 * qsa_decode_layer_scratch_bytes for n_blocks (QSA_ERR_SCRATCH); scratch holds the chunk partials (and scores, ids
 * and counts when they are not asked for). Calls sharing one scratch buffer must be ordered on one stream. */
qsa_status qsa_decode_layer(const float *q, const int32_t *pos, int32_t n_rows, const qsa_pool *pools, int32_t n_pools,
                            const int32_t *row_pool, qsa_dims dims, int32_t n_blocks, int32_t k, int32_t n_chunks,
                            float sm_scale, float *out, float *lse, float *scores, int32_t *ids, int32_t *counts,
                            void *scratch, size_t scratch_bytes, qsa_stream_t stream);

/* Bytes of device scratch qsa_decode_layer_noalloc may use: qsa_decode_layer_scratch_bytes of its arguments must not
 * exceed this (8 MiB: the verify window's 4 rows at 16 chunks need 0.8 MiB, 32 rows of 24 heads at 16 chunks 6.3 MiB). */
#define QSA_NOALLOC_SCRATCH_BYTES (8u << 20)

/* qsa_decode_layer for callers that cannot allocate device memory (code under HIP graph capture, serving loops or
 * harnesses that forbid hipMalloc): the same launches, arithmetic and outputs, with the scratch taken from a
 * file-scope device array of QSA_NOALLOC_SCRATCH_BYTES that each GPU holds from the first call on it until the
 * process ends. The caller still passes every input and output. Calls no hipMalloc/hipFree or allocating routine.
 * Returns QSA_ERR_SCRATCH, having launched nothing, when qsa_decode_layer_scratch_bytes(n_rows, dims, n_blocks, k,
 * n_chunks) > QSA_NOALLOC_SCRATCH_BYTES; QSA_ERR_LAUNCH if the array's device address cannot be obtained. Every
 * call on one GPU shares that GPU's array (it keeps the last call's contents; nothing in it must start at zero):
 * calls that may overlap on one GPU -- on different streams, or from different threads -- race and must be ordered
 * by the caller. The library's otherwise stateless convention does not hold for this call. */
qsa_status qsa_decode_layer_noalloc(const float *q, const int32_t *pos, int32_t n_rows, const qsa_pool *pools,
                                    int32_t n_pools, const int32_t *row_pool, qsa_dims dims, int32_t n_blocks,
                                    int32_t k, int32_t n_chunks, float sm_scale, float *out, float *lse,
                                    float *scores, int32_t *ids, int32_t *counts, qsa_stream_t stream);

/* Static, human-readable name of a status code. */
const char *qsa_status_str(qsa_status status);

#ifdef __cplusplus
}
#endif

#endif /* QSA_H */
