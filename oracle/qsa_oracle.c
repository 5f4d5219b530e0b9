/*
 * qsa_oracle.c - plain CPU oracle for sparse-attention block selection.
 *
 * TEST INFRASTRUCTURE ONLY. Only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py may load this library. The product path (the
 * HIP library under sparse_attention_block_scores_amd/) never calls it and
 * shares no code, header, table or helper with it.
 *
 * What it computes, written out as plainly as possible:
 *
 *  1. Block scores (Strata pull #1091 "qsa_select: FP32 tiled block scores
 *     below sm_80", section What: each row of the contraction is one
 *     (query, indexer head) pair over a 128-wide key, and each head's dot
 *     product goes through a relu before the heads are added up):
 *         s[q][b] = sum_h w[q][h] * max(0, sum_d q[q][h][d] * k[b][d])
 *     in double. Every float*float product is exact in double (24+24 <= 53
 *     significand bits), so the only rounding is the double summation.
 *
 *  2. Block top-k by full sort (Strata pull #2093 "sm_75: the prompt path's
 *     top-k with one full read of the scores", section Beschreibung, step 3;
 *     Strata pull #3987, section Approach). Every cell carries its block's
 *     key; cells are ordered by key descending, ties by cell index ascending;
 *     the first min(width, cells) cells are the selection, written in
 *     ascending cell order and padded with -1.
 *
 *  3. The same selection by the threshold rule the pages describe: T = the
 *     width-th largest cell key, `above` = cells with key > T, a tie budget
 *     of width - above filled from the lowest cell upward, emitted in order.
 *     T is found by counting (a binary search over the order-preserving
 *     32-bit image of the float keys), not by sorting, so that forms 2 and 3
 *     are two independent computations of one definition.
 *
 *  4. Attention over the selected cells, the consumer of the selection
 *     (iree-org/wave issue #1257 "NSA: LDS optimization for block-gather in
 *     selection attention", sections Problem and Per-block LDS staging: each
 *     query attends to the key/value pairs of the cells it selected, and the
 *     query heads of one group share one key/value head). For query q, query
 *     head h and its key/value head g = h / (n_heads / kv_heads):
 *         s_c = scale * sum_d q[q][h][d] * k[c][g][d]     for each listed c
 *         out[q][h][:] = sum_c exp(s_c) * v[c][g][:] / sum_c exp(s_c)
 *         lse[q][h]    = log(sum_c exp(s_c))
 *     over the entries c of row q of the id list that lie in [0, n_cells)
 *     (others select nothing). A query that selects nothing gets out = 0 and
 *     lse = -inf. Every exp(s_c) is taken as exp(s_c - max s) * exp(max s),
 *     the same ratios without overflow.
 *
 * Visible cells: on a decode call every cell of the n_blocks blocks; on a
 * prompt call the cells of the first min(max(active[q], 0), n_blocks) blocks
 * of query q. The *_cells entry points take a cell count per query instead,
 * cells [0, min(max(cells[q], 0), n_blocks * block_size)), so the last visible
 * block may hold fewer than block_size cells; every visible cell still carries
 * its block's key.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define EXPORT __attribute__((visibility("default")))

/* ---------------------------------------------------------------- scores */

EXPORT void oracle_block_scores(const float *q, const float *k, const float *w,
                                double *s, int64_t ld, int nq, int heads,
                                int head_dim, int n_blocks)
{
#pragma omp parallel for collapse(2) schedule(static)
    for (int iq = 0; iq < nq; ++iq) {
        for (int b = 0; b < n_blocks; ++b) {
            double total = 0.0;
            for (int h = 0; h < heads; ++h) {
                const float *qrow = q + ((int64_t)iq * heads + h) * head_dim;
                const float *krow = k + (int64_t)b * head_dim;
                double dot = 0.0;
                for (int d = 0; d < head_dim; ++d)
                    dot += (double)qrow[d] * (double)krow[d];
                double relu = dot > 0.0 ? dot : 0.0;
                total += (double)w[(int64_t)iq * heads + h] * relu;
            }
            s[(int64_t)iq * ld + b] = total;
        }
    }
}

/* The same score for a list of (query, block) pairs, for spot checks of
 * outputs too large to recompute whole. */
EXPORT void oracle_block_scores_at(const float *q, const float *k, const float *w,
                                   int heads, int head_dim,
                                   const int32_t *qi, const int32_t *bi, int n,
                                   double *out)
{
#pragma omp parallel for schedule(static)
    for (int i = 0; i < n; ++i) {
        double total = 0.0;
        for (int h = 0; h < heads; ++h) {
            const float *qrow = q + ((int64_t)qi[i] * heads + h) * head_dim;
            const float *krow = k + (int64_t)bi[i] * head_dim;
            double dot = 0.0;
            for (int d = 0; d < head_dim; ++d)
                dot += (double)qrow[d] * (double)krow[d];
            double relu = dot > 0.0 ? dot : 0.0;
            total += (double)w[(int64_t)qi[i] * heads + h] * relu;
        }
        out[i] = total;
    }
}

/* ----------------------------------------------------------- common bits */

static int visible_blocks(int n_blocks, const int32_t *active, int iq)
{
    if (!active)
        return n_blocks;
    int a = active[iq];
    if (a < 0)
        a = 0;
    if (a > n_blocks)
        a = n_blocks;
    return a;
}

/* Visible cells of query iq: a cell count when `cells` is given, else whole
 * visible blocks. */
static int64_t visible_cells(int n_blocks, int block_size, const int32_t *active, const int32_t *cells, int iq)
{
    const int64_t all = (int64_t)n_blocks * block_size;
    if (cells) {
        int64_t c = cells[iq];
        return c < 0 ? 0 : (c > all ? all : c);
    }
    return (int64_t)visible_blocks(n_blocks, active, iq) * block_size;
}

/* --------------------------------------------------- top-k by full sort */

typedef struct {
    float key;
    int32_t cell;
} cell_t;

static int by_key_desc_then_cell(const void *pa, const void *pb)
{
    const cell_t *a = (const cell_t *)pa, *b = (const cell_t *)pb;
    if (a->key > b->key)
        return -1;
    if (a->key < b->key)
        return 1;
    return (a->cell > b->cell) - (a->cell < b->cell);
}

static int by_int_asc(const void *pa, const void *pb)
{
    int32_t a = *(const int32_t *)pa, b = *(const int32_t *)pb;
    return (a > b) - (a < b);
}

static void topk_sort(const float *scores, int64_t ld, int nq, int n_blocks, int block_size, int width,
                      const int32_t *active, const int32_t *vcells, int32_t *ids, int32_t *counts)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int iq = 0; iq < nq; ++iq) {
        const int64_t ncells = visible_cells(n_blocks, block_size, active, vcells, iq);
        int32_t *out = ids + (int64_t)iq * width;
        cell_t *cells = (cell_t *)malloc((size_t)(ncells > 0 ? ncells : 1) * sizeof(cell_t));
        for (int64_t c = 0; c < ncells; ++c) {
            cells[c].key = scores[(int64_t)iq * ld + c / block_size];
            cells[c].cell = (int32_t)c;
        }
        qsort(cells, (size_t)ncells, sizeof(cell_t), by_key_desc_then_cell);
        const int64_t m = ncells < width ? ncells : width;
        for (int64_t i = 0; i < m; ++i)
            out[i] = cells[i].cell;
        qsort(out, (size_t)m, sizeof(int32_t), by_int_asc);
        for (int64_t i = m; i < width; ++i)
            out[i] = -1;
        if (counts)
            counts[iq] = (int32_t)m;
        free(cells);
    }
}

EXPORT void oracle_topk_sort(const float *scores, int64_t ld, int nq, int n_blocks,
                             int block_size, int width, const int32_t *active,
                             int32_t *ids, int32_t *counts)
{
    topk_sort(scores, ld, nq, n_blocks, block_size, width, active, NULL, ids, counts);
}

EXPORT void oracle_topk_sort_cells(const float *scores, int64_t ld, int nq, int n_blocks,
                                   int block_size, int width, const int32_t *cells,
                                   int32_t *ids, int32_t *counts)
{
    topk_sort(scores, ld, nq, n_blocks, block_size, width, NULL, cells, ids, counts);
}

/* ------------------------------------------- top-k by the threshold rule */

/* Order-preserving image of a float in uint32: a > b  <=>  image(a) > image(b),
 * with -0.0 and +0.0 mapped to one value (they compare equal as floats). */
/* Visible cells of block b when the first ncells cells are visible. */
static int64_t cells_of(int b, int block_size, int64_t ncells)
{
    const int64_t rest = ncells - (int64_t)b * block_size;
    return rest < block_size ? rest : block_size;
}

static uint32_t ordered_image(float f)
{
    uint32_t bits;
    memcpy(&bits, &f, sizeof bits);
    if (bits == 0x80000000u)
        bits = 0u;
    return (bits & 0x80000000u) ? ~bits : (bits | 0x80000000u);
}

static void topk_rule(const float *scores, int64_t ld, int nq, int n_blocks, int block_size, int width,
                      const int32_t *active, const int32_t *vcells, int32_t *ids, int32_t *counts)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int iq = 0; iq < nq; ++iq) {
        const int64_t ncells = visible_cells(n_blocks, block_size, active, vcells, iq);
        const int nb = (int)((ncells + block_size - 1) / block_size);
        const float *row = scores + (int64_t)iq * ld;
        int32_t *out = ids + (int64_t)iq * width;
        const int64_t m = ncells < width ? ncells : width;
        int64_t written = 0;
        if (m > 0) {
            /* T = the m-th largest cell key: the largest t with
             * #{cells : image(key) >= t} >= m, by binary search on t. */
            uint64_t lo = 0, hi = 0xFFFFFFFFull; /* answer in [lo, hi] */
            while (lo < hi) {
                uint64_t mid = lo + (hi - lo + 1) / 2;
                int64_t n_ge = 0;
                for (int b = 0; b < nb; ++b)
                    if ((uint64_t)ordered_image(row[b]) >= mid)
                        n_ge += cells_of(b, block_size, ncells);
                if (n_ge >= m)
                    lo = mid;
                else
                    hi = mid - 1;
            }
            const uint32_t T = (uint32_t)lo;
            int64_t above = 0;
            for (int b = 0; b < nb; ++b)
                if (ordered_image(row[b]) > T)
                    above += cells_of(b, block_size, ncells);
            int64_t budget = m - above;
            for (int64_t c = 0; c < ncells; ++c) {
                uint32_t key = ordered_image(row[c / block_size]);
                if (key > T) {
                    out[written++] = (int32_t)c;
                } else if (key == T && budget > 0) {
                    out[written++] = (int32_t)c;
                    --budget;
                }
            }
        }
        for (int64_t i = written; i < width; ++i)
            out[i] = -1;
        if (counts)
            counts[iq] = (int32_t)written;
    }
}

EXPORT void oracle_topk_rule(const float *scores, int64_t ld, int nq, int n_blocks,
                             int block_size, int width, const int32_t *active,
                             int32_t *ids, int32_t *counts)
{
    topk_rule(scores, ld, nq, n_blocks, block_size, width, active, NULL, ids, counts);
}

EXPORT void oracle_topk_rule_cells(const float *scores, int64_t ld, int nq, int n_blocks,
                                   int block_size, int width, const int32_t *cells,
                                   int32_t *ids, int32_t *counts)
{
    topk_rule(scores, ld, nq, n_blocks, block_size, width, NULL, cells, ids, counts);
}

/* ------------------------------------------------- selection attention */

EXPORT void oracle_selection_attention(const float *q, const float *k, const float *v,
                                       const int32_t *ids, int64_t ld_ids, int nq,
                                       int n_heads, int kv_heads, int head_dim,
                                       int n_cells, int width, double scale,
                                       double *out, double *lse)
{
    const int group = n_heads / kv_heads;
#pragma omp parallel for collapse(2) schedule(dynamic, 4)
    for (int iq = 0; iq < nq; ++iq) {
        for (int h = 0; h < n_heads; ++h) {
            const int g = h / group;
            const float *qrow = q + ((int64_t)iq * n_heads + h) * head_dim;
            const int32_t *list = ids + (int64_t)iq * ld_ids;
            double *o = out + ((int64_t)iq * n_heads + h) * head_dim;
            double *s = malloc(sizeof(double) * (size_t)(width > 0 ? width : 1));
            /* logits of the listed cells (NAN marks an entry that selects nothing) */
            double top = -INFINITY;
            for (int i = 0; i < width; ++i) {
                const int32_t c = list[i];
                if (c < 0 || c >= n_cells) {
                    s[i] = NAN;
                    continue;
                }
                const float *krow = k + ((int64_t)c * kv_heads + g) * head_dim;
                double dot = 0.0;
                for (int d = 0; d < head_dim; ++d)
                    dot += (double)qrow[d] * (double)krow[d];
                s[i] = scale * dot;
                if (s[i] > top)
                    top = s[i];
            }
            for (int d = 0; d < head_dim; ++d)
                o[d] = 0.0;
            double total = 0.0;
            for (int i = 0; i < width; ++i) {
                if (isnan(s[i]))
                    continue;
                const double e = exp(s[i] - top);
                const float *vrow = v + ((int64_t)list[i] * kv_heads + g) * head_dim;
                total += e;
                for (int d = 0; d < head_dim; ++d)
                    o[d] += e * (double)vrow[d];
            }
            if (total > 0.0) {
                for (int d = 0; d < head_dim; ++d)
                    o[d] /= total;
                if (lse)
                    lse[(int64_t)iq * n_heads + h] = top + log(total);
            } else if (lse) {
                lse[(int64_t)iq * n_heads + h] = -INFINITY;
            }
            free(s);
        }
    }
}
