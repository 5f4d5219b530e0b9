/*
 * qsa.h - C ABI of libqsa.so: sparse-attention block selection on MI355X
 * (gfx950).
 *
 * Two steps make up the selection an indexer runs before sparse attention:
 *
 *  1. Block scores (Strata pull #1091 "qsa_select: FP32 tiled block scores
 *     below sm_80", section What). For query q and key block b,
 *         score[q][b] = sum_h w[q][h] * max(0, dot(q[q][h][:], k[b][:]))
 *     with a 128-wide indexer key: a dense FP32 contraction over rows of
 *     (query, indexer head), a relu per head, and a weighted head sum.
 *
 *  2. Block top-k (Strata pull #3987, section Approach; Strata pull #2093
 *     "sm_75: the prompt path's top-k with one full read of the scores",
 *     section Beschreibung). Each block holds `block_size` cells and every
 *     cell carries its block's score as its key. The selection is the first
 *     min(width, visible cells) cells in the order (key descending, cell id
 *     ascending): a threshold T (the width-th largest cell key), every cell
 *     above T, and a tie budget of cells equal to T filled from the lowest
 *     block (then lowest cell) upward. Cells are written in ascending order.
 *     -0.0 and +0.0 are equal keys. Keys must be finite (NaN and Inf are
 *     outside the contract: results are unspecified but the call is safe).
 *
 * Calls. A decode call carries no active-block count: all n_blocks blocks are
 * visible to every query. A prompt call may carry a per-query active-block
 * count: query q sees blocks [0, min(max(active[q], 0), n_blocks)). The
 * *_cells entry points take, for either call, a per-query count of visible
 * CELLS that stays in device memory, so the last visible block may be partial
 * and the length can change between calls without the host knowing it (the
 * launches depend only on the host arguments, so a stream capture replays).
 *
 * Memory and streams. Every pointer argument except `opt` and `out` structs
 * is caller-owned DEVICE memory; the library never allocates or frees device
 * memory, and the only device memory of its own is the fixed workspace array
 * of qsa_block_topk_noalloc (one per GPU, for callers that cannot allocate).
 * All work is enqueued on `stream` (a hipStream_t; NULL = the default
 * stream) and the calls return without synchronising. Nothing is printed.
 * Host-side state: the first call that takes the exact chunked split raises
 * one kernel's dynamic-LDS limit (a kernel attribute, set once per process;
 * concurrent first calls are safe), and the first allocation-free call on a
 * device looks up that device's array. Nothing else persists between calls.
 *
 * Errors. Arguments are checked on the host before anything is launched; a
 * call that returns anything but QSA_OK has enqueued nothing. QSA_EHIP means
 * a launch failed (work enqueued before the failure may still run).
 *
 * Workspace. The top-k needs a scratch area of qsa_topk_workspace_bytes()
 * bytes, 256-byte aligned. It needs no set-up: every call writes what it
 * reads back (qsa_workspace_init() zero-fills one all the same, for callers
 * that want defined contents). Calls that may run concurrently (two streams)
 * need separate workspaces.
 */
#ifndef QSA_H
#define QSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum qsa_status {
    QSA_OK = 0,
    QSA_EINVAL = 1,        /* argument out of range, inconsistent or misaligned */
    QSA_EUNSUPPORTED = 2,  /* valid request the library does not implement */
    QSA_EWORKSPACE = 3,    /* workspace NULL, misaligned or too small */
    QSA_EHIP = 4           /* a HIP launch or runtime call failed */
} qsa_status;

/* The kind of call. Entry points take it as an int32_t `call` (as
 * qsa_status_str takes its code), so that any value a caller passes is a
 * valid argument and anything else is rejected with QSA_EINVAL. */
typedef enum qsa_call {
    QSA_DECODE = 0,  /* no active-block count: every block is visible */
    QSA_PROMPT = 1   /* optional per-query active-block count */
} qsa_call;

/* Top-k path choice. AUTO is what production callers use; the others force a
 * path for tests and measurements. Every path returns the same ids. A forced
 * ONEREAD with rows of more than 64 * 16,384 blocks, or a selection of more
 * than 4,095 blocks (2 * (r + 1) over the 8,192-block cap of its flagged
 * pass), and a forced FILTER with more than 1,024 chunks per row, take SPLIT
 * (qsa_topk_plan_get shows the path taken). */
enum {
    QSA_PATH_AUTO = 0,
    QSA_PATH_SPLIT = 1,    /* exact chunked split: per-chunk stage A, per-query stage B */
    QSA_PATH_ONEREAD = 2,  /* sampled bound, one read by one workgroup per query; a flagged query
                              takes the exact rule in one more read of its row */
    QSA_PATH_FILTER = 3    /* sampled bound and one read spread over chunk workgroups (first launch),
                              per-query selection over their candidates (second launch) */
};

/* Sampling of the one-read path's lower bound (results never depend on it). */
enum {
    QSA_SAMPLE_AUTO = 0,
    QSA_SAMPLE_STRIDE = 1, /* every 32nd block (one key per 128-byte line) */
    QSA_SAMPLE_LINES = 2   /* 32 consecutive blocks out of every 1,024 */
};

/* Optional knobs; pass NULL for the defaults. Zero-initialise and set only
 * what is needed. None of them changes a result. */
typedef struct qsa_options {
    int32_t topk_path;      /* QSA_PATH_* */
    int32_t chunk_blocks;   /* SPLIT chunk size in blocks: 0 = auto, else 64..15360, multiple of 4 */
    int32_t sample;         /* QSA_SAMPLE_* */
    int32_t force_fallback; /* ONEREAD, FILTER: every query is flagged (the exact rule over its whole row) */
    int32_t filter_blocks;  /* FILTER chunk size in blocks: 0 = auto, else 1024, 2048, 4096 or 8192 */
    int32_t reserved[3];    /* must be zero */
} qsa_options;

/* The launch plan the top-k would use; exported so host code and tests can
 * inspect the dispatch without a GPU. Sizes are for the largest query. */
typedef struct qsa_topk_plan {
    int32_t path;            /* QSA_PATH_SPLIT, QSA_PATH_ONEREAD or QSA_PATH_FILTER */
    int32_t r_blocks;        /* blocks a full selection touches: ceil(min(width, n_blocks*bs) / bs) */
    int32_t chunk_blocks;    /* SPLIT chunk size: the fewest chunks of <= 4,104 blocks, equal sizes */
    int32_t n_chunks;        /* SPLIT chunks per query */
    int32_t split_threads;   /* SPLIT workgroup size */
    int32_t stage_b_lds;     /* 1 if stage B keeps its candidates in LDS */
    int32_t oneread_blocks;  /* ONEREAD blocks streamed per batch (halved for short rows) */
    int32_t cap;             /* ONEREAD, FILTER candidate cap per query (blocks) */
    int32_t sample_stride;   /* 32 */
    int32_t sample_mode;     /* QSA_SAMPLE_STRIDE or QSA_SAMPLE_LINES */
    int32_t ks;              /* sample rank of the bound: 2*r_blocks/32 + 16 */
    int32_t filter_blocks;   /* FILTER blocks per chunk workgroup */
    int32_t filter_chunks;   /* FILTER chunks of the longest row */
    int32_t filter_slot;     /* FILTER candidates a chunk may keep */
    int32_t filter_groups;   /* FILTER first-launch workgroups */
    int32_t reserved;
    uint64_t workspace_bytes;
} qsa_topk_plan;

/*
 * qsa_block_scores - step 1 (Strata pull #1091, section What).
 *
 *   q       [nq][n_heads][head_dim] float, row-major, 16-byte aligned
 *   k       [n_blocks][head_dim]    float, row-major, 16-byte aligned
 *   w       [nq][n_heads]           float
 *   scores  [nq][ld_scores]         float output; columns >= n_blocks untouched
 *   head_dim must be 128 (else QSA_EUNSUPPORTED); 1 <= n_heads <= 64;
 *   nq >= 1, n_blocks >= 1, ld_scores >= n_blocks.
 *   FP32 inputs, FP32 matrix-core products with FP32 accumulation.
 */
qsa_status qsa_block_scores(const float *q, const float *k, const float *w,
                            float *scores, int64_t ld_scores,
                            int32_t nq, int32_t n_heads, int32_t head_dim,
                            int32_t n_blocks, void *stream);

/*
 * qsa_block_scores_bf16 - step 1 with BF16 q and k: the lower-precision
 * tensor-core scorer that Strata pull #1091 names as an existing switch in its
 * opening description; the score itself is that pull's section What.
 *
 *   q       [nq][n_heads][head_dim] bfloat16 (raw 16-bit IEEE bfloat16
 *           values), row-major, 16-byte aligned
 *   k       [n_blocks][head_dim]    bfloat16, row-major, 16-byte aligned
 *   w, scores, shapes, limits and errors as qsa_block_scores; in addition
 *   ld_scores must be below 2^24 (else QSA_EUNSUPPORTED).
 *   Products of BF16 values on the BF16 matrix cores, exact in FP32, with
 *   FP32 accumulation: the scores of the BF16-rounded inputs. Ids selected
 *   from them agree with the FP32 path's only within the rounding of the
 *   inputs.
 */
qsa_status qsa_block_scores_bf16(const void *q, const void *k, const float *w,
                                 float *scores, int64_t ld_scores,
                                 int32_t nq, int32_t n_heads, int32_t head_dim,
                                 int32_t n_blocks, void *stream);

/* Bytes of workspace qsa_block_topk / qsa_select need for these sizes and
 * options (0 if the arguments are invalid). */
size_t qsa_topk_workspace_bytes(int32_t nq, int32_t n_blocks, int32_t block_size,
                                int32_t width, int32_t call, const qsa_options *opt);

/* Fill the plan for these arguments (host only; no GPU needed). */
qsa_status qsa_topk_plan_get(int32_t nq, int32_t n_blocks, int32_t block_size,
                             int32_t width, int32_t call, const qsa_options *opt,
                             qsa_topk_plan *out);

/* Zero-fill `bytes` of workspace on `stream` (a kernel, not a memset). */
qsa_status qsa_workspace_init(void *workspace, size_t bytes, void *stream);

/*
 * qsa_block_topk - step 2 (Strata pull #3987, section Approach; Strata pull
 * #2093, section Beschreibung).
 *
 *   scores         [nq][ld_scores] float; only columns < n_blocks are read
 *   active_blocks  [nq] int32, PROMPT only (NULL = every block visible);
 *                  non-NULL with QSA_DECODE is QSA_EINVAL
 *   cell_ids       [nq][width] int32 output: selected cell ids b*block_size+j,
 *                  ascending, then -1 up to width
 *   counts         [nq] int32 output or NULL: min(width, visible cells)
 *   workspace      qsa_topk_workspace_bytes(...) bytes (see above)
 *   1 <= block_size, 1 <= width, n_blocks * block_size < 2^31, nq >= 1.
 */
qsa_status qsa_block_topk(const float *scores, int64_t ld_scores, int32_t nq,
                          int32_t n_blocks, int32_t block_size, int32_t width,
                          int32_t call, const int32_t *active_blocks,
                          int32_t *cell_ids, int32_t *counts,
                          void *workspace, size_t workspace_bytes, void *stream,
                          const qsa_options *opt);

/*
 * qsa_block_topk_cells - qsa_block_topk with a cell-granular visible length
 * read on the device, for decode and prompt calls alike. Strata pull #3987,
 * section Approach, derives the split from the context length on the device;
 * Strata pull #1091, section What, keeps a separate tail block, so a context
 * need not end on a block boundary.
 *
 *   visible_cells  [nq] int32 device, or NULL (every cell visible): query q
 *                  sees cells [0, min(max(visible_cells[q], 0),
 *                  n_blocks * block_size)); every visible cell carries its
 *                  block's score as its key, cells past the count do not
 *                  exist for the selection.
 *   cell_ids, counts, workspace, stream, opt: as qsa_block_topk (the same
 *   workspace size); counts[q] = min(width, visible cells of q).
 */
qsa_status qsa_block_topk_cells(const float *scores, int64_t ld_scores, int32_t nq,
                                int32_t n_blocks, int32_t block_size, int32_t width,
                                int32_t call, const int32_t *visible_cells,
                                int32_t *cell_ids, int32_t *counts,
                                void *workspace, size_t workspace_bytes, void *stream,
                                const qsa_options *opt);

/*
 * qsa_block_topk_noalloc - qsa_block_topk for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): the same selection with the default options, its
 * workspace taken from a fixed array of QSA_NOALLOC_SCRATCH_BYTES per GPU
 * inside the library (held until the process ends) instead of a caller's
 * buffer. Nothing is allocated; the first call on a device zero-fills that
 * device's array on `stream` (nothing depends on it: every call writes what
 * it reads back).
 *
 *   Arguments and results as qsa_block_topk without workspace and options.
 *   A call whose workspace (qsa_topk_workspace_bytes with NULL options) is
 *   larger than QSA_NOALLOC_SCRATCH_BYTES returns QSA_EUNSUPPORTED and
 *   enqueues nothing.
 *   Every call on one GPU shares that GPU's array: calls that may overlap on
 *   one GPU (several streams, several host threads) race and must be ordered
 *   by the caller.
 */
#define QSA_NOALLOC_SCRATCH_BYTES (16u << 20)
qsa_status qsa_block_topk_noalloc(const float *scores, int64_t ld_scores, int32_t nq,
                                  int32_t n_blocks, int32_t block_size, int32_t width,
                                  int32_t call, const int32_t *active_blocks,
                                  int32_t *cell_ids, int32_t *counts, void *stream);

/*
 * qsa_select - qsa_block_scores followed by qsa_block_topk on the scores it
 * wrote (`scores` is the caller's buffer and holds the scores afterwards).
 * Same argument rules as the two calls above.
 */
qsa_status qsa_select(const float *q, const float *k, const float *w,
                      int32_t n_heads, int32_t head_dim,
                      float *scores, int64_t ld_scores, int32_t nq, int32_t n_blocks,
                      int32_t block_size, int32_t width, int32_t call,
                      const int32_t *active_blocks, int32_t *cell_ids, int32_t *counts,
                      void *workspace, size_t workspace_bytes, void *stream,
                      const qsa_options *opt);

/* qsa_select with the cell-granular visible length of qsa_block_topk_cells. */
qsa_status qsa_select_cells(const float *q, const float *k, const float *w,
                            int32_t n_heads, int32_t head_dim,
                            float *scores, int64_t ld_scores, int32_t nq, int32_t n_blocks,
                            int32_t block_size, int32_t width, int32_t call,
                            const int32_t *visible_cells, int32_t *cell_ids, int32_t *counts,
                            void *workspace, size_t workspace_bytes, void *stream,
                            const qsa_options *opt);

/*
 * qsa_selection_attention - attention of every query head over the cells its
 * query selected: the consumer of the selection (iree-org/wave issue #1257
 * "NSA: LDS optimization for block-gather in selection attention", sections
 * Problem and Per-block LDS staging). The heads of one group,
 * g = h / (n_heads / kv_heads), share key/value head g:
 *     s_c        = scale * q[q][h][:] . k[c][g][:]   for each listed cell c
 *     out[q][h]  = sum_c exp(s_c) v[c][g][:] / sum_c exp(s_c)
 *     lse[q][h]  = log(sum_c exp(s_c))
 *
 *   q      [nq][n_heads][head_dim]    bfloat16 (raw 16-bit values), 16-byte aligned
 *   k, v   [n_cells][kv_heads][head_dim] bfloat16, 16-byte aligned
 *   ids    [nq][ld_ids] int32 device; entries 0 .. width-1 of each row are the
 *          query's list (the cell_ids of qsa_block_topk fit as they are); an
 *          entry outside [0, n_cells) selects nothing
 *   out    [nq][n_heads][head_dim] float output, 16-byte aligned
 *   lse    [nq][n_heads] float output (natural log), or NULL
 *   A query that selects no cell gets out = 0 and lse = -inf. Only the listed
 *   cells' rows of k and v are read into the result (they must be finite);
 *   other rows may hold anything.
 *   head_dim must be 128 (else QSA_EUNSUPPORTED); n_heads a multiple of
 *   kv_heads; n_cells, width >= 1; ld_ids >= width; scale finite.
 *   Products of bfloat16 values with FP32 accumulation, FP32 softmax.
 *   workspace: qsa_selection_attention_workspace_bytes() bytes, 256-byte
 *   aligned (may be NULL when that is 0): per-chunk partial results, written
 *   and read within the call; its contents need no set-up. Calls that may
 *   overlap need separate workspaces. The size function also returns 0 for
 *   sizes the call rejects (it then fails with QSA_EINVAL).
 */
size_t qsa_selection_attention_workspace_bytes(int32_t nq, int32_t n_heads, int32_t kv_heads, int32_t width);
qsa_status qsa_selection_attention(const void *q, const void *k, const void *v,
                                   const int32_t *ids, int64_t ld_ids, float *out, float *lse,
                                   int32_t nq, int32_t n_heads, int32_t kv_heads, int32_t head_dim,
                                   int32_t n_cells, int32_t width, float scale,
                                   void *workspace, size_t workspace_bytes, void *stream);

/*
 * qsa_selection_attention_shared - qsa_selection_attention for queries whose
 * neighbours select many of the same cells (iree-org/wave issue #1257
 * "NSA: LDS optimization for block-gather in selection attention", section
 * Shared block deduplication). Queries 2i and 2i+1 form a pair (with an odd
 * nq the last query is alone); a first launch merges the pair's two lists
 * into one list of distinct cells, each marked with the queries that listed
 * it, and the attention then gathers each distinct cell's key and value rows
 * once for both queries.
 *
 *   Arguments, results and the bfloat16/FP32 arithmetic as
 *   qsa_selection_attention; the sums may add the same terms in another
 *   order. Limits (else QSA_EUNSUPPORTED): n_heads / kv_heads <= 8 (a pair's
 *   heads fill one 16-column matrix-core tile), width <= 4096 (the merge's
 *   hash lives in LDS), n_cells < 2^30 (a merged entry packs the cell id and
 *   the two query marks into 32 bits). A query that lists a cell more than
 *   once counts it that often: a pair with such a repeat is not merged (each
 *   of its entries stays separate; the result is the same).
 *   workspace: qsa_selection_attention_shared_workspace_bytes() bytes,
 *   256-byte aligned, never 0 (the merged lists live there); written and read
 *   within the call, no set-up. The size function returns 0 for sizes the
 *   call rejects.
 */
size_t qsa_selection_attention_shared_workspace_bytes(int32_t nq, int32_t n_heads, int32_t kv_heads,
                                                      int32_t width);
qsa_status qsa_selection_attention_shared(const void *q, const void *k, const void *v,
                                          const int32_t *ids, int64_t ld_ids, float *out, float *lse,
                                          int32_t nq, int32_t n_heads, int32_t kv_heads, int32_t head_dim,
                                          int32_t n_cells, int32_t width, float scale,
                                          void *workspace, size_t workspace_bytes, void *stream);

/* Static text for a status code (a qsa_status; other values get a text too). */
const char *qsa_status_str(int32_t status);

#ifdef __cplusplus
}
#endif

#endif /* QSA_H */
