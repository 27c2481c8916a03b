/*
 * QSA reference oracle -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, single-threaded FP64 CPU statement of what QSA attention over an int8 KV cache computes. Only the
 * test suite, the smoke check and the benchmark's CPU-baseline leg may load this file's library; the GPU product
 * path never does, and this file shares no code, header, table or helper with it.
 *
 * Sources (the pages are pull requests against one inference engine):
 *   [1888] "#1888 QSA decode attention: split each query's cells across blocks on the int8 mma path"
 *   [2075] "#2075 QSA decode attention: PR #540's two-cells-per-step chunk kernel on every CUDA card and a
 *          bounded merge"
 *   [V100] "qsa_prompt_attn: tensor-core kernel for Volta (sm_70, mma.m8n8k4)"
 *   [2806] "#2806 sycl: decode QSA selection and attention in fewer, shorter launches"
 *   [1367] "#1367 prompt attention: STRATA_PROMPT_ATTN_IMMA=1 - the int8-KV kernel on INT8 tensor cores"
 *
 * Once the selection is fixed the attention is exactly softmax attention over the selected visible cells; split-K,
 * the online softmax and the log-sum-exp merge are ways to reach that result faster. So orc_attn_* below is the
 * plain definition (two passes: max, then sum of exponentials), and orc_chunk_partials / orc_merge exist only to
 * check the GPU's intermediate buffers. The pages never give the block-score formula or the content of the
 * per-block "indexer"; orc_block_index and orc_block_scores take the plainest reading consistent with the pages:
 * the mean dequantised key of each (KV head, block), dotted with the sum of the KV head's q heads.
 *
 * Layouts (row-major, all host memory):
 *   codes   int8  [n_kv][cap][d]        scales f32 [n_kv][cap][d/64]   (dequantised value = scale * code)
 *   q       f32   [n_rows][n_qh][d]     pos    i32 [n_rows]            (a query at pos sees cells 0..pos)
 *   index   f64   [n_kv][r_blocks][d]   scores f64 [n_rows][n_kv][n_blocks]
 *   ids     i32   [n_rows][n_kv][k]     counts i32 [n_rows][n_kv]
 *   partials m,l  f64 [n_rows][n_qh][S], o f64 [n_rows][n_qh][S][d], empty u8 [n_rows][n_qh][S]
 * q head h belongs to KV head h / (n_qh / n_kv) (grouped-query attention).
 *
 * Parity status per function is stated in each comment; all but the block-score/index reading are pinned by the
 * CPU tests (brute force, closed forms, split invariance, full sort). The score formula itself cannot be pinned
 * against the pages, which print none: parity unpinned for orc_block_index/orc_block_scores as a reading of the
 * pages (they are pinned against an independent evaluation of the same reading).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_GROUP 64

typedef struct {
    const int8_t *k, *v;
    const float *ks, *vs;
    int32_t capacity, n_valid;
    int32_t v_bits;   /* 8: int8 V codes [n_kv][cap][d]; 4: bytes [n_kv][cap][d/2], two signed 4-bit codes each */
} orc_pool;

static double deq(const int8_t *codes, const float *scales, int32_t cap, int32_t d, int32_t g, int32_t c, int32_t e)
{
    const int32_t ng = d / ORC_GROUP;
    return (double)scales[((int64_t)g * cap + c) * ng + e / ORC_GROUP] * (double)codes[((int64_t)g * cap + c) * d + e];
}

/* Dequantised value of V. v_bits = 4 is the K8V4 cache the pages list beside int8 ([1888] "What changed", formats
 * left alone; [2075] "Bit for bit", parity cases by KV format) without giving its layout. Reading: V codes are signed
 * 4-bit integers (two's complement nibbles, -7..7 written), two per byte -- dim 2j in the low nibble, 2j + 1 in the
 * high one -- with the same per-64-dim fp32 scales as int8 V. Pinned against an independent numpy unpacking. */
static double deq_v(const orc_pool *p, int32_t d, int32_t g, int32_t c, int32_t e)
{
    if (p->v_bits != 4) return deq(p->v, p->vs, p->capacity, d, g, c, e);
    const int32_t ng = d / ORC_GROUP;
    const uint8_t byte = (uint8_t)p->v[((int64_t)g * p->capacity + c) * (d / 2) + e / 2];
    int32_t nib = (e & 1) ? (byte >> 4) : (byte & 15);
    if (nib >= 8) nib -= 16;
    return (double)p->vs[((int64_t)g * p->capacity + c) * ng + e / ORC_GROUP] * (double)nib;
}

/* Per-block key summary ("indexer"): [2806] names an indexer that is appended per row next to K/V, without its
 * content. Reading: r[g][b] = mean over the block's valid cells (c < n_valid) of the dequantised key. A block
 * with no valid cell gets r = 0. Parity unpinned against the pages (reading). */
void orc_block_index(const int8_t *k, const float *ks, int32_t n_kv, int32_t cap, int32_t n_valid, int32_t d,
                     int32_t block, int32_t r_blocks, double *r)
{
    for (int32_t g = 0; g < n_kv; g++)
        for (int32_t b = 0; b < r_blocks; b++) {
            double *out = r + ((int64_t)g * r_blocks + b) * d;
            int32_t c0 = b * block, c1 = c0 + block;
            if (c1 > n_valid) c1 = n_valid;
            for (int32_t e = 0; e < d; e++) out[e] = 0.0;
            if (c1 <= c0) continue;
            for (int32_t c = c0; c < c1; c++)
                for (int32_t e = 0; e < d; e++) out[e] += deq(k, ks, cap, d, g, c, e);
            for (int32_t e = 0; e < d; e++) out[e] /= (double)(c1 - c0);
        }
}

/* Block scores: [2806] Summary table (STRATA_QSA_SCORES_TRANSPOSED row) sums one value per (query, KV head) per
 * block. Reading: s[i][g][b] = (sum of the q heads of KV head g) . r[g][b], for blocks whose first cell is visible
 * to the query (64b <= pos_i) and holds valid cells (64b < n_valid); every other entry of the row is -inf. */
void orc_block_scores(const float *q, const int32_t *pos, int32_t n_rows, int32_t n_qh, int32_t n_kv, int32_t d,
                      const double *r, int32_t r_blocks, int32_t n_valid, int32_t block, int32_t n_blocks, double *s)
{
    const int32_t G = n_qh / n_kv;
    double *qt = (double *)malloc(sizeof(double) * (size_t)d);
    for (int32_t i = 0; i < n_rows; i++)
        for (int32_t g = 0; g < n_kv; g++) {
            for (int32_t e = 0; e < d; e++) {
                double acc = 0.0;
                for (int32_t h = g * G; h < (g + 1) * G; h++) acc += (double)q[((int64_t)i * n_qh + h) * d + e];
                qt[e] = acc;
            }
            for (int32_t b = 0; b < n_blocks; b++) {
                double *out = s + ((int64_t)i * n_kv + g) * n_blocks + b;
                int64_t first = (int64_t)b * block;
                if (first > pos[i] || first >= n_valid || b >= r_blocks) { *out = -INFINITY; continue; }
                double acc = 0.0;
                const double *rb = r + ((int64_t)g * r_blocks + b) * d;
                for (int32_t e = 0; e < d; e++) acc += qt[e] * rb[e];
                *out = acc;
            }
        }
    free(qt);
}

typedef struct { double s; int32_t b; } orc_key;

static int orc_key_cmp(const void *pa, const void *pb)
{
    const orc_key *a = (const orc_key *)pa, *b = (const orc_key *)pb;
    if (a->s > b->s) return -1;           /* larger score first */
    if (a->s < b->s) return 1;
    return (a->b > b->b) - (a->b < b->b); /* equal scores: lower block index first */
}

static int orc_int_cmp(const void *pa, const void *pb)
{
    int32_t a = *(const int32_t *)pa, b = *(const int32_t *)pb;
    return (a > b) - (a < b);
}

/* Top-k per row: the k highest-scoring eligible (finite) blocks, ties to the lower block index, returned in
 * ascending block order and padded with -1; counts = min(k, eligible). [2806] Summary table: the radix top-k
 * is integer-exact ("the same ids"), and at 1K context every block is taken (kernel table note). Defined here by a
 * full sort on (score descending, index ascending). Pinned by the CPU tests against an independent stable sort. */
void orc_topk(const double *s, int32_t n_rows, int32_t width, int32_t k, int32_t *ids, int32_t *counts)
{
    orc_key *keys = (orc_key *)malloc(sizeof(orc_key) * (size_t)(width > 0 ? width : 1));
    for (int32_t row = 0; row < n_rows; row++) {
        int32_t n = 0;
        for (int32_t b = 0; b < width; b++) {
            double v = s[(int64_t)row * width + b];
            if (v > -INFINITY) { keys[n].s = v; keys[n].b = b; n++; }
        }
        qsort(keys, (size_t)n, sizeof(orc_key), orc_key_cmp);
        int32_t take = n < k ? n : k;
        int32_t *out = ids + (int64_t)row * k;
        for (int32_t j = 0; j < take; j++) out[j] = keys[j].b;
        qsort(out, (size_t)take, sizeof(int32_t), orc_int_cmp);
        for (int32_t j = take; j < k; j++) out[j] = -1;
        counts[row] = take;
    }
    free(keys);
}

/* The visible cell set of (row i, KV head g): the cells of the row's selected blocks (or of every block when ids is
 * NULL) that are valid (c < n_valid) and causally visible (c <= pos_i). [2075] "Bit for bit": masked cells stay
 * out of the sums. Writes the cells in the order they are visited and returns their count. */
static int32_t visible_cells(const orc_pool *p, int32_t block, int32_t pos_i, const int32_t *sel, int32_t n_sel,
                             int32_t b_begin, int32_t b_end, int32_t *cells)
{
    int32_t n = 0;
    int32_t nb = sel ? n_sel : b_end - b_begin;
    for (int32_t j = 0; j < nb; j++) {
        int32_t b = sel ? sel[j] : b_begin + j;
        int64_t first = (int64_t)b * block;
        if (b < 0 || first >= p->n_valid) continue;   /* ids past the valid cells name no cell */
        for (int32_t c = (int32_t)first; c < first + block; c++)
            if (c < p->n_valid && c <= pos_i) cells[n++] = c;
    }
    return n;
}

/* Attention of one (query row, q head) over a given cell list, in two plain passes: the logits
 * t_c = sm_scale * (q . dequantised k_c), their max M, then out = sum_c e^(t_c - M) v_c / sum_c e^(t_c - M) and
 * lse = M + ln(sum). An empty list gives out = 0 and lse = -inf. */
static void attend(const float *qrow, const orc_pool *p, int32_t g, int32_t d, const int32_t *cells, int32_t n,
                   double sm_scale, double *t, double *out, double *lse)
{
    for (int32_t e = 0; e < d; e++) out[e] = 0.0;
    if (n == 0) { *lse = -INFINITY; return; }
    double M = -INFINITY;
    for (int32_t j = 0; j < n; j++) {
        double acc = 0.0;
        for (int32_t e = 0; e < d; e++) acc += (double)qrow[e] * deq(p->k, p->ks, p->capacity, d, g, cells[j], e);
        t[j] = sm_scale * acc;
        if (t[j] > M) M = t[j];
    }
    double L = 0.0;
    for (int32_t j = 0; j < n; j++) {
        double w = exp(t[j] - M);
        L += w;
        for (int32_t e = 0; e < d; e++) out[e] += w * deq_v(p, d, g, cells[j], e);
    }
    for (int32_t e = 0; e < d; e++) out[e] /= L;
    *lse = M + log(L);
}

/* Softmax attention of one (row i, q head h) over its visible selected cells. ids/counts NULL = dense (every
 * valid visible cell). Pinned by brute force, closed forms and the split-invariance tests. */
void orc_attn_one(const float *q, const int32_t *pos, int32_t i, int32_t h, const int8_t *k, const float *ks,
                  const int8_t *v, const float *vs, int32_t cap, int32_t n_valid, int32_t n_qh, int32_t n_kv,
                  int32_t d, int32_t block, const int32_t *ids, const int32_t *counts, int32_t topk, double sm_scale,
                  double *out, double *lse, int32_t v_bits)
{
    orc_pool p = {k, v, ks, vs, cap, n_valid, v_bits};
    const int32_t G = n_qh / n_kv, g = h / G;
    int32_t max_cells = ids ? topk * block : ((n_valid + block - 1) / block) * block;
    int32_t *cells = (int32_t *)malloc(sizeof(int32_t) * (size_t)(max_cells > 0 ? max_cells : 1));
    double *t = (double *)malloc(sizeof(double) * (size_t)(max_cells > 0 ? max_cells : 1));
    int32_t n;
    if (ids) {
        const int32_t *sel = ids + ((int64_t)i * n_kv + g) * topk;
        int32_t n_sel = counts ? counts[(int64_t)i * n_kv + g] : topk;
        n = visible_cells(&p, block, pos[i], sel, n_sel, 0, 0, cells);
    } else {
        n = visible_cells(&p, block, pos[i], NULL, 0, 0, (n_valid + block - 1) / block, cells);
    }
    attend(q + ((int64_t)i * n_qh + h) * d, &p, g, d, cells, n, sm_scale, t, out, lse);
    free(cells);
    free(t);
}

/* All rows and heads: out [n_rows][n_qh][d], lse [n_rows][n_qh]. */
void orc_attn(const float *q, const int32_t *pos, int32_t n_rows, const int8_t *k, const float *ks, const int8_t *v,
              const float *vs, int32_t cap, int32_t n_valid, int32_t n_qh, int32_t n_kv, int32_t d, int32_t block,
              const int32_t *ids, const int32_t *counts, int32_t topk, double sm_scale, double *out, double *lse,
              int32_t v_bits)
{
    for (int32_t i = 0; i < n_rows; i++)
        for (int32_t h = 0; h < n_qh; h++)
            orc_attn_one(q, pos, i, h, k, ks, v, vs, cap, n_valid, n_qh, n_kv, d, block, ids, counts, topk,
                         sm_scale, out + ((int64_t)i * n_qh + h) * d, lse + (int64_t)i * n_qh + h, v_bits);
}

/* Chunk partials, for checking a split-K chunk kernel's scratch: [1888] "What changed" (one split of one query's
 * cells writes partials to the decode scratch) and [2075] Summary (chunks with no cell are marked empty).
 * Chunking rule (the pages leave it open; up to 20 splits per query in [1888] Summary): with ids, chunk j of row
 * (i, g) takes a contiguous run of the row's selected blocks -- the count c of selected blocks is cut into S runs,
 * the first c mod S runs one block longer; without ids, chunk j covers blocks [j*bpc, (j+1)*bpc).
 * m_j = max logit, l_j = sum e^(t - m_j), o_j = sum e^(t - m_j) v; an empty chunk is (-inf, 0, 0) with mark 1. */
void orc_chunk_partials(const float *q, const int32_t *pos, int32_t n_rows, const int8_t *k, const float *ks,
                        const int8_t *v, const float *vs, int32_t cap, int32_t n_valid, int32_t n_qh, int32_t n_kv,
                        int32_t d, int32_t block, const int32_t *ids, const int32_t *counts, int32_t topk,
                        int32_t bpc, int32_t n_chunks, double sm_scale, double *m, double *l, double *o,
                        uint8_t *empty, int32_t v_bits)
{
    orc_pool p = {k, v, ks, vs, cap, n_valid, v_bits};
    const int32_t G = n_qh / n_kv;
    int32_t max_blocks = ids ? topk : bpc;
    int32_t *cells = (int32_t *)malloc(sizeof(int32_t) * (size_t)(max_blocks * block + 1));
    double *t = (double *)malloc(sizeof(double) * (size_t)(max_blocks * block + 1));
    for (int32_t i = 0; i < n_rows; i++)
        for (int32_t h = 0; h < n_qh; h++) {
            const int32_t g = h / G;
            const float *qrow = q + ((int64_t)i * n_qh + h) * d;
            for (int32_t j = 0; j < n_chunks; j++) {
                int32_t n;
                if (ids) {
                    int32_t cnt = counts[(int64_t)i * n_kv + g];
                    int32_t base = cnt / n_chunks, rem = cnt % n_chunks;
                    int32_t len = base + (j < rem ? 1 : 0);
                    int32_t start = j * base + (j < rem ? j : rem);
                    n = visible_cells(&p, block, pos[i], ids + ((int64_t)i * n_kv + g) * topk + start, len, 0, 0,
                                      cells);
                } else {
                    n = visible_cells(&p, block, pos[i], NULL, 0, j * bpc, (j + 1) * bpc, cells);
                }
                int64_t idx = ((int64_t)i * n_qh + h) * n_chunks + j;
                double *oj = o + idx * d;
                for (int32_t e = 0; e < d; e++) oj[e] = 0.0;
                if (n == 0) {
                    m[idx] = -INFINITY; l[idx] = 0.0; empty[idx] = 1;
                    continue;
                }
                double mj = -INFINITY;
                for (int32_t c = 0; c < n; c++) {
                    double dot = 0.0;
                    for (int32_t e = 0; e < d; e++) dot += (double)qrow[e] * deq(p.k, p.ks, cap, d, g, cells[c], e);
                    t[c] = sm_scale * dot;
                    if (t[c] > mj) mj = t[c];
                }
                double lj = 0.0;
                for (int32_t c = 0; c < n; c++) {
                    double w = exp(t[c] - mj);
                    lj += w;
                    for (int32_t e = 0; e < d; e++) oj[e] += w * deq_v(&p, d, g, cells[c], e);
                }
                m[idx] = mj; l[idx] = lj; empty[idx] = 0;
            }
        }
    free(cells); free(t);
}

/* Log-sum-exp merge of chunk partials: [1888] "What changed" (the splits of each query and head merged in split
 * order) and [2075] Summary / "Bit for bit" (the merge skips chunks marked empty); [2806] Summary table,
 * STRATA_ATTN_MERGE_ACTIVE row (only the chunks the selection reaches are folded). Folds chunks [0, n_active[i])
 * (all S when n_active is NULL) in chunk order, skipping marked ones: M = max m_j,
 * out = sum e^(m_j - M) o_j / sum e^(m_j - M) l_j, lse = M + ln(sum e^(m_j - M) l_j); no chunk -> 0 and -inf. */
void orc_merge(const double *m, const double *l, const double *o, const uint8_t *empty, int32_t n_rows,
               int32_t n_qh, int32_t n_chunks, int32_t d, const int32_t *n_active, double *out, double *lse)
{
    for (int32_t i = 0; i < n_rows; i++) {
        int32_t na = n_active ? n_active[i] : n_chunks;
        if (na > n_chunks) na = n_chunks;
        for (int32_t h = 0; h < n_qh; h++) {
            int64_t base = ((int64_t)i * n_qh + h) * n_chunks;
            double *orow = out + ((int64_t)i * n_qh + h) * d;
            double M = -INFINITY;
            for (int32_t j = 0; j < na; j++)
                if (!empty[base + j] && m[base + j] > M) M = m[base + j];
            for (int32_t e = 0; e < d; e++) orow[e] = 0.0;
            if (M == -INFINITY) { lse[(int64_t)i * n_qh + h] = -INFINITY; continue; }
            double L = 0.0;
            for (int32_t j = 0; j < na; j++) {
                if (empty[base + j]) continue;
                double w = exp(m[base + j] - M);
                L += w * l[base + j];
                for (int32_t e = 0; e < d; e++) orow[e] += w * o[(base + j) * d + e];
            }
            for (int32_t e = 0; e < d; e++) orow[e] /= L;
            lse[(int64_t)i * n_qh + h] = M + log(L);
        }
    }
}

/* The exact 24-bit operand split of [1367] "What it does" (Operands): an operand is scaled so its largest
 * magnitude maps to 127, then X = rint(x * 65536) is written as 65536*h + 256*l + m with three 8-bit digits.
 * The pages take h and l signed and m unsigned; every exact digit split names the same integer X, and this one
 * writes balanced signed digits (h, l, m all in [-128, 127]), which is what a signed x signed byte product needs.
 * orc_split24 returns 0 on success and -1 if some X cannot be written with three such digits. */
int orc_split24(const int32_t *X, int64_t n, int32_t *h, int32_t *l, int32_t *m)
{
    for (int64_t j = 0; j < n; j++) {
        int64_t x = X[j];
        int64_t d0 = ((x % 256) + 256) % 256;     /* residue in [0, 256) */
        if (d0 >= 128) d0 -= 256;                 /* balanced: [-128, 128) */
        int64_t r1 = (x - d0) / 256;
        int64_t d1 = ((r1 % 256) + 256) % 256;
        if (d1 >= 128) d1 -= 256;
        int64_t d2 = (r1 - d1) / 256;
        if (d2 < -128 || d2 > 127) return -1;
        h[j] = (int32_t)d2; l[j] = (int32_t)d1; m[j] = (int32_t)d0;
    }
    return 0;
}

/* Scaling step of the same split: x' = x * 127 / amax, X = rint(x' * 65536) (round half to even). */
void orc_quant24(const double *x, int64_t n, double amax, int32_t *X)
{
    for (int64_t j = 0; j < n; j++) {
        double xs = amax > 0.0 ? x[j] * 127.0 / amax : 0.0;
        X[j] = (int32_t)nearbyint(xs * 65536.0);
    }
}

/* int8 encode of one 64-dim scale group, the write side of the int8 KV pool ([2806] "Extra Notes": K/V appended
 * per row, with per-64-dim scales, [1888] Summary). The pages name the format but not its encoder; reading:
 * symmetric absmax per (cell, KV head, group) -- amax = max |x|, scale = amax / 127, code = rint(x * (127 / amax))
 * clamped to [-127, 127], and amax = 0 gives scale 0 and all-zero codes. The quantised code is an integer decided by
 * floating point, so it is decided here in fp32 with the same three roundings the GPU makes (127 / amax, the
 * product, rint half-to-even); nothing else in this file is fp32. Pinned by brute force (nearest code over all 255),
 * exact recovery of power-of-two grids, and the reconstruction bound. */
void orc_encode_group(const float *x, int32_t n, int8_t *codes, float *scale)
{
    float amax = 0.0f;
    for (int32_t e = 0; e < n; e++) {
        const float a = fabsf(x[e]);
        if (a > amax) amax = a;
    }
    if (amax == 0.0f) {
        for (int32_t e = 0; e < n; e++) codes[e] = 0;
        *scale = 0.0f;
        return;
    }
    const float inv = 127.0f / amax;
    for (int32_t e = 0; e < n; e++) {
        float c = rintf(x[e] * inv);
        if (c > 127.0f) c = 127.0f;
        if (c < -127.0f) c = -127.0f;
        codes[e] = (int8_t)c;
    }
    *scale = amax / 127.0f;
}

/* The same encoder for the 4-bit V codes of a K8V4 pool (reading, as above): scale = amax / 7,
 * code = rint(x * (7 / amax)) clamped to [-7, 7], in fp32. */
void orc_encode_group4(const float *x, int32_t n, int8_t *codes, float *scale)
{
    float amax = 0.0f;
    for (int32_t e = 0; e < n; e++) {
        const float a = fabsf(x[e]);
        if (a > amax) amax = a;
    }
    if (amax == 0.0f) {
        for (int32_t e = 0; e < n; e++) codes[e] = 0;
        *scale = 0.0f;
        return;
    }
    const float inv = 7.0f / amax;
    for (int32_t e = 0; e < n; e++) {
        float c = rintf(x[e] * inv);
        if (c > 7.0f) c = 7.0f;
        if (c < -7.0f) c = -7.0f;
        codes[e] = (int8_t)c;
    }
    *scale = amax / 7.0f;
}

/* Append of n_rows new cells to one pool: row i writes cell cells[i] of every KV head, K from k_new and V from v_new
 * ([n_rows][n_kv][d] f32), one orc_encode_group per 64-dim group (orc_encode_group4 for a K8V4 pool's V). Rows whose cell is outside [0, n_valid) are
 * skipped (n_valid is the pool's count after the append). Index rows are recomputed by orc_block_index. */
void orc_kv_append(int8_t *k, float *ks, int8_t *v, float *vs, int32_t n_kv, int32_t cap, int32_t n_valid, int32_t d,
                   const float *k_new, const float *v_new, const int32_t *cells, int32_t n_rows, int32_t v_bits)
{
    int8_t c4[ORC_GROUP];
    const int32_t ng = d / ORC_GROUP;
    for (int32_t i = 0; i < n_rows; i++) {
        const int32_t c = cells[i];
        if (c < 0 || c >= n_valid || c >= cap) continue;
        for (int32_t g = 0; g < n_kv; g++) {
            const int64_t src = ((int64_t)i * n_kv + g) * d, dst = ((int64_t)g * cap + c);
            for (int32_t t = 0; t < ng; t++) {
                orc_encode_group(k_new + src + t * ORC_GROUP, ORC_GROUP, k + dst * d + t * ORC_GROUP, ks + dst * ng + t);
                if (v_bits != 4) {
                    orc_encode_group(v_new + src + t * ORC_GROUP, ORC_GROUP, v + dst * d + t * ORC_GROUP, vs + dst * ng + t);
                } else {   /* pack two 4-bit codes per byte, dim 2j low */
                    orc_encode_group4(v_new + src + t * ORC_GROUP, ORC_GROUP, c4, vs + dst * ng + t);
                    for (int32_t e = 0; e < ORC_GROUP; e += 2)
                        v[dst * (d / 2) + (t * ORC_GROUP + e) / 2] = (int8_t)(uint8_t)((c4[e] & 15) | ((c4[e + 1] & 15) << 4));
                }
            }
        }
    }
}
