// qsa_api.hip - the C ABI of libqsa.so: argument checks, the top-k dispatch
// plan, workspace layout and the launches. Nothing here allocates device
// memory, synchronises or prints.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <mutex>

#include "qsa_internal.h"

namespace qsa {

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

qsa_status check_options(const qsa_options *opt)
{
    if (!opt)
        return QSA_OK;
    if (opt->reserved[0] != 0 || opt->reserved[1] != 0 || opt->reserved[2] != 0)
        return QSA_EINVAL;
    if (opt->filter_blocks != 0 && opt->filter_blocks != 1024 && opt->filter_blocks != 2048 &&
        opt->filter_blocks != 4096 && opt->filter_blocks != 8192)
        return QSA_EINVAL;
    if (opt->topk_path < QSA_PATH_AUTO || opt->topk_path > QSA_PATH_FILTER)
        return QSA_EINVAL;
    if (opt->chunk_blocks != 0 &&
        (opt->chunk_blocks < kMinChunk || opt->chunk_blocks > kMaxChunk || opt->chunk_blocks % 4 != 0))
        return QSA_EINVAL;
    if (opt->sample < QSA_SAMPLE_AUTO || opt->sample > QSA_SAMPLE_LINES)
        return QSA_EINVAL;
    if (opt->force_fallback != 0 && opt->force_fallback != 1)
        return QSA_EINVAL;
    return QSA_OK;
}

} // namespace

qsa_status make_topk_plan(int32_t nq, int32_t n_blocks, int32_t block_size, int32_t width,
                          int32_t call, const qsa_options *opt, TopkPlan &plan)
{
    memset(&plan, 0, sizeof plan);
    if (nq < 0 || n_blocks < 0 || block_size < 1 || width < 1)
        return QSA_EINVAL;
    if (call != QSA_DECODE && call != QSA_PROMPT)
        return QSA_EINVAL;
    if ((int64_t)n_blocks * block_size >= ((int64_t)1 << 31))
        return QSA_EINVAL;
    if (nq > 65535)
        return QSA_EUNSUPPORTED;
    const qsa_status os = check_options(opt);
    if (os != QSA_OK)
        return os;

    qsa_topk_plan &p = plan.pub;
    const int64_t cells = (int64_t)n_blocks * block_size;
    const int64_t wmax = cells < width ? cells : width;
    p.r_blocks = (int32_t)((wmax + block_size - 1) / block_size);

    // Split geometry: the fewest chunks of at most kChunkBound blocks, equal
    // sizes rounded up to a multiple of 4 (or the forced size).
    // (64-bit sums: n_blocks may be as large as 2^31 - 1 with one-cell blocks.)
    if (opt && opt->chunk_blocks) {
        p.chunk_blocks = opt->chunk_blocks;
    } else {
        const int64_t nb = n_blocks > 0 ? n_blocks : 1;
        const int64_t k = (nb + kChunkBound - 1) / kChunkBound;
        p.chunk_blocks = (int32_t)(((nb + k - 1) / k + 3) / 4 * 4);
    }
    p.n_chunks = n_blocks > 0 ? (int32_t)(((int64_t)n_blocks + p.chunk_blocks - 1) / p.chunk_blocks) : 1;
    p.split_threads = kSplitThreads;
    // Room for one block more per chunk: a query whose last visible block is
    // partial keeps r + 1 candidates per chunk (qsa_block_topk_cells).
    const int64_t cap_c = (int64_t)p.r_blocks + 1 < p.chunk_blocks ? (int64_t)p.r_blocks + 1 : p.chunk_blocks;
    plan.cand_stride = ((int64_t)p.n_chunks * (cap_c > 0 ? cap_c : 1) + 3) / 4 * 4;
    p.stage_b_lds = plan.cand_stride <= kStageBLdsWords ? 1 : 0;

    // One-read geometry: one workgroup streams each query's row in batches of
    // blocks (one slice per wave).
    p.oneread_blocks = oneread_short_slices(nq, n_blocks) ? kOneReadShortBatch : kOneReadBatch;
    p.cap = kOneReadCap;
    p.sample_stride = kSampleStride;
    p.sample_mode = (opt && opt->sample) ? opt->sample : QSA_SAMPLE_LINES;
    p.ks = (int32_t)(2 * (int64_t)p.r_blocks / kSampleStride + 16);

    // Filtered split geometry: chunks of 1,024-8,192 blocks, the largest size
    // that still gives about kFilterTargetGroups first-launch workgroups (or
    // the forced size), at most kFilterMaxChunks chunks per row. A chunk's
    // slot holds up to twice an even share of the candidate cap (at least
    // 512), so a row whose candidates fit the cap overflows no slot unless
    // they crowd into a few chunks.
    {
        int32_t fb = kFilterMaxChunk;
        if (opt && opt->filter_blocks) {
            fb = opt->filter_blocks;
        } else {
            const int64_t nb = n_blocks > 0 ? n_blocks : 1;
            while (fb > kFilterMinChunk && (int64_t)nq * ((nb + fb - 1) / fb) < kFilterTargetGroups)
                fb /= 2;
        }
        p.filter_blocks = fb;
        p.filter_chunks = n_blocks > 0 ? (int32_t)(((int64_t)n_blocks + fb - 1) / fb) : 1;
        const int32_t share = (2 * kOneReadCap + p.filter_chunks - 1) / p.filter_chunks;
        int32_t slot = (share + 63) / 64 * 64;
        slot = slot < 512 ? 512 : slot;
        p.filter_slot = slot < fb ? slot : fb;
        p.filter_groups = (int32_t)((int64_t)nq * p.filter_chunks);
    }

    // Dispatch (measured on MI355X; results never depend on it). A row that
    // fits one chunk is selected in LDS by one workgroup. Longer rows take a
    // sampled-bound path while its candidates are a small share of the row
    // (the bound keeps about 3r blocks); otherwise the split. Among those, up
    // to 16 queries with rows of at least 65,536 + 2,048 nq blocks spread
    // each row over chunk workgroups (the filtered split: there one workgroup
    // per query streams too long); the rest take one workgroup per query (one
    // read, one launch).
    int path = opt ? opt->topk_path : QSA_PATH_AUTO;
    if (path == QSA_PATH_AUTO) {
        if (n_blocks > kChunkBound && (int64_t)n_blocks >= (int64_t)kOneReadMinRatio * p.r_blocks)
            path = (nq <= kFilterMaxQueries &&
                    (int64_t)n_blocks >= (int64_t)kFilterMinBlocks + (int64_t)kFilterBlocksPerQuery * nq)
                       ? QSA_PATH_FILTER
                       : QSA_PATH_ONEREAD;
        else
            path = QSA_PATH_SPLIT;
    }
    if (path == QSA_PATH_ONEREAD && n_blocks > kOneReadMaxBatches * kOneReadBatch)
        path = QSA_PATH_SPLIT;  // per-batch counts of longer rows do not fit the LDS table
    // A query whose sampled bound fails is finished in LDS chunks, keeping up
    // to r + 1 blocks of each beside a list of as many (select_row_chunked).
    if (path == QSA_PATH_ONEREAD && 2 * ((int64_t)p.r_blocks + 1) > kOneReadCap)
        path = QSA_PATH_SPLIT;
    if (path == QSA_PATH_FILTER && p.filter_chunks > kFilterMaxChunks)
        path = QSA_PATH_SPLIT;  // stage B scans at most kFilterMaxChunks chunk headers
    p.path = path;

    // Workspace: only the split keeps candidates in global memory.
    TopkLayout &L = plan.lay;
    size_t off = 0;
    if (path == QSA_PATH_SPLIT) {
        const size_t q = (size_t)(nq > 0 ? nq : 1);
        L.split_keys = off;    off = align_up(off + q * (size_t)plan.cand_stride * 4);
        L.split_blocks = off;  off = align_up(off + q * (size_t)plan.cand_stride * 4);
    } else if (path == QSA_PATH_FILTER) {
        const size_t q = (size_t)(nq > 0 ? nq : 1);
        L.filter_heads = off; off = align_up(off + q * (size_t)p.filter_chunks * 16);
        L.filter_slots = off; off = align_up(off + q * (size_t)p.filter_chunks * 2 * (size_t)p.filter_slot * 4);
    } else {
        off = kAlign;  // nothing is kept; a minimal non-empty workspace
    }
    L.bytes = off;
    p.workspace_bytes = off;
    return QSA_OK;
}

namespace {

qsa_status check_topk_args(const float *scores, int64_t ld, int32_t nq, int32_t n_blocks,
                           int32_t call, const int32_t *active, const int32_t *cells,
                           const int32_t *ids, const int32_t *counts)
{
    if (nq > 0 && (!scores || !ids))
        return QSA_EINVAL;
    if (ld < n_blocks || ld < 1)
        return QSA_EINVAL;
    if (call == QSA_DECODE && active)
        return QSA_EINVAL;
    if (!aligned(scores, 4) || !aligned(ids, 4) || !aligned(counts, 4) || !aligned(active, 4) ||
        !aligned(cells, 4))
        return QSA_EINVAL;
    return QSA_OK;
}

TopkGeom make_geom(const float *scores, int64_t ld, int32_t nq, int32_t n_blocks, int32_t bs,
                   int32_t width, const int32_t *active, const int32_t *cells, int32_t *ids,
                   int32_t *counts)
{
    TopkGeom g;
    g.scores = scores;
    g.ld = ld;
    g.nq = nq;
    g.n_blocks = n_blocks;
    g.bs = bs;
    g.width = width;
    g.active = active;
    g.cells = cells;
    g.ids = ids;
    g.counts = counts;
    g.vec4 = (aligned(scores, 16) && ld % 4 == 0) ? 1 : 0;
    return g;
}

template <class T>
T *at(void *base, size_t off) { return reinterpret_cast<T *>(static_cast<char *>(base) + off); }

qsa_status run_topk(const TopkGeom &g, const TopkPlan &plan, void *ws, hipStream_t s,
                    const qsa_options *opt)
{
    const qsa_topk_plan &p = plan.pub;
    if (p.path == QSA_PATH_FILTER) {
        FilterArgs fa;
        fa.g = g;
        fa.heads = at<uint32_t>(ws, plan.lay.filter_heads);
        fa.slots = at<uint32_t>(ws, plan.lay.filter_slots);
        fa.chunk = p.filter_blocks;
        fa.n_chunks = p.filter_chunks;
        fa.slot = p.filter_slot;
        fa.mode = p.sample_mode;
        fa.force_flag = (opt && opt->force_fallback) ? 1 : 0;
        fa.xcd = (g.nq % 8 == 0) ? 1 : 0;
        return launch_filter(fa, s) == hipSuccess ? QSA_OK : QSA_EHIP;
    }
    if (p.path == QSA_PATH_ONEREAD) {
        OneReadArgs oa;
        oa.g = g;
        oa.mode = p.sample_mode;
        oa.force_flag = (opt && opt->force_fallback) ? 1 : 0;
        return launch_oneread(oa, s) == hipSuccess ? QSA_OK : QSA_EHIP;
    }
    const TopkLayout &L = plan.lay;
    SplitArgs sa;
    sa.g = g;
    sa.cand_keys = at<uint32_t>(ws, L.split_keys);
    sa.cand_blocks = at<int32_t>(ws, L.split_blocks);
    sa.cand_stride = plan.cand_stride;
    sa.chunk = p.chunk_blocks;
    sa.n_chunks = p.n_chunks;
    const int64_t stage_b = p.stage_b_lds ? plan.cand_stride : 0;
    sa.lds_words = p.chunk_blocks;
    sa.blk_words = (int32_t)stage_b;
    return launch_split(sa, s) == hipSuccess ? QSA_OK : QSA_EHIP;
}

qsa_status check_score_args(const float *q, const float *k, const float *w, const float *scores,
                            int64_t ld, int32_t nq, int32_t heads, int32_t head_dim, int32_t n_blocks)
{
    if (nq < 0 || n_blocks < 0 || heads < 1 || head_dim < 1)
        return QSA_EINVAL;
    if (ld < n_blocks || ld < 1)
        return QSA_EINVAL;
    if (head_dim != 128 || heads > 64)
        return QSA_EUNSUPPORTED;
    if (nq > 0 && n_blocks > 0 && (!q || !k || !w || !scores))
        return QSA_EINVAL;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(w, 4) || !aligned(scores, 4))
        return QSA_EINVAL;
    if ((int64_t)nq * 64 > 0x7fffffffLL)
        return QSA_EUNSUPPORTED;
    return QSA_OK;
}

} // namespace
} // namespace qsa

using namespace qsa;

namespace {

qsa_status topk_call(const float *scores, int64_t ld_scores, int32_t nq, int32_t n_blocks, int32_t block_size,
                     int32_t width, int32_t call, const int32_t *active, const int32_t *cells,
                     int32_t *cell_ids, int32_t *counts, void *workspace, size_t workspace_bytes,
                     void *stream, const qsa_options *opt)
{
    TopkPlan plan;
    qsa_status st = make_topk_plan(nq, n_blocks, block_size, width, call, opt, plan);
    if (st != QSA_OK)
        return st;
    st = check_topk_args(scores, ld_scores, nq, n_blocks, call, active, cells, cell_ids, counts);
    if (st != QSA_OK)
        return st;
    if (nq == 0)
        return QSA_OK;
    if (!workspace || !aligned(workspace, kAlign) || workspace_bytes < plan.lay.bytes)
        return QSA_EWORKSPACE;
    const TopkGeom g = make_geom(scores, ld_scores, nq, n_blocks, block_size, width, active, cells, cell_ids,
                                 counts);
    return run_topk(g, plan, workspace, (hipStream_t)stream, opt);
}

qsa_status select_call(const float *q, const float *k, const float *w, int32_t n_heads, int32_t head_dim,
                       float *scores, int64_t ld_scores, int32_t nq, int32_t n_blocks, int32_t block_size,
                       int32_t width, int32_t call, const int32_t *active, const int32_t *cells,
                       int32_t *cell_ids, int32_t *counts, void *workspace, size_t workspace_bytes,
                       void *stream, const qsa_options *opt)
{
    qsa_status st = check_score_args(q, k, w, scores, ld_scores, nq, n_heads, head_dim, n_blocks);
    if (st != QSA_OK)
        return st;
    TopkPlan plan;
    st = make_topk_plan(nq, n_blocks, block_size, width, call, opt, plan);
    if (st != QSA_OK)
        return st;
    st = check_topk_args(scores, ld_scores, nq, n_blocks, call, active, cells, cell_ids, counts);
    if (st != QSA_OK)
        return st;
    if (nq == 0)
        return QSA_OK;
    if (!workspace || !aligned(workspace, kAlign) || workspace_bytes < plan.lay.bytes)
        return QSA_EWORKSPACE;
    if (n_blocks > 0) {
        ScoreArgs a{q, k, w, scores, ld_scores, nq, n_heads, n_blocks};
        if (launch_scores(a, (hipStream_t)stream) != hipSuccess)
            return QSA_EHIP;
    }
    const TopkGeom g = make_geom(scores, ld_scores, nq, n_blocks, block_size, width, active, cells, cell_ids,
                                 counts);
    return run_topk(g, plan, workspace, (hipStream_t)stream, opt);
}

// ------------------------------------------------------------ static scratch
// The workspace of qsa_block_topk_noalloc: one fixed array per GPU, in device
// memory for as long as the library is loaded. In host code `scratch` names a
// host-side stand-in, never the device array: its device address comes from
// hipGetSymbolAddress, once per device, and only that address is used.
constexpr size_t kStaticScratchBytes = (size_t)QSA_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;

struct DeviceScratch {
    std::once_flag once;
    void *ptr = nullptr;
    hipError_t err = hipSuccess;
};

DeviceScratch g_scratch[kMaxDevices];

// The current device's scratch address; the first call on a device looks it
// up (with that device current) and zero-fills the array on `s` (a kernel,
// ordered before the caller's launches on the same stream).
qsa_status device_scratch(hipStream_t s, void **out)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return QSA_EHIP;
    DeviceScratch &d = g_scratch[dev];
    std::call_once(d.once, [&] {
        d.err = hipGetSymbolAddress(&d.ptr, HIP_SYMBOL(scratch));
        if (d.err == hipSuccess)
            d.err = launch_zero(d.ptr, kStaticScratchBytes, s);
        if (d.err != hipSuccess)
            d.ptr = nullptr;
    });
    if (d.err != hipSuccess || !d.ptr)
        return QSA_EHIP;
    *out = d.ptr;
    return QSA_OK;
}

} // namespace

extern "C" {

qsa_status qsa_block_topk_noalloc(const float *scores, int64_t ld_scores, int32_t nq, int32_t n_blocks,
                                  int32_t block_size, int32_t width, int32_t call, const int32_t *active_blocks,
                                  int32_t *cell_ids, int32_t *counts, void *stream)
{
    TopkPlan plan;
    qsa_status st = make_topk_plan(nq, n_blocks, block_size, width, call, nullptr, plan);
    if (st != QSA_OK)
        return st;
    st = check_topk_args(scores, ld_scores, nq, n_blocks, call, active_blocks, nullptr, cell_ids, counts);
    if (st != QSA_OK)
        return st;
    if (plan.lay.bytes > kStaticScratchBytes)
        return QSA_EUNSUPPORTED;  // the call needs more workspace than the fixed array holds
    if (nq == 0)
        return QSA_OK;
    void *ws = nullptr;
    st = device_scratch((hipStream_t)stream, &ws);
    if (st != QSA_OK)
        return st;
    const TopkGeom g = make_geom(scores, ld_scores, nq, n_blocks, block_size, width, active_blocks, nullptr,
                                 cell_ids, counts);
    return run_topk(g, plan, ws, (hipStream_t)stream, nullptr);
}

const char *qsa_status_str(int32_t status)
{
    switch (status) {
    case QSA_OK: return "ok";
    case QSA_EINVAL: return "invalid argument";
    case QSA_EUNSUPPORTED: return "unsupported argument";
    case QSA_EWORKSPACE: return "workspace missing, misaligned or too small";
    case QSA_EHIP: return "HIP launch failed";
    }
    return "unknown status";
}

qsa_status qsa_topk_plan_get(int32_t nq, int32_t n_blocks, int32_t block_size, int32_t width,
                             int32_t call, const qsa_options *opt, qsa_topk_plan *out)
{
    if (!out)
        return QSA_EINVAL;
    TopkPlan plan;
    const qsa_status st = make_topk_plan(nq, n_blocks, block_size, width, call, opt, plan);
    if (st == QSA_OK)
        *out = plan.pub;
    return st;
}

size_t qsa_topk_workspace_bytes(int32_t nq, int32_t n_blocks, int32_t block_size, int32_t width,
                                int32_t call, const qsa_options *opt)
{
    TopkPlan plan;
    if (make_topk_plan(nq, n_blocks, block_size, width, call, opt, plan) != QSA_OK)
        return 0;
    return plan.lay.bytes;
}

qsa_status qsa_workspace_init(void *workspace, size_t bytes, void *stream)
{
    if (!workspace || !aligned(workspace, kAlign))
        return QSA_EWORKSPACE;
    return launch_zero(workspace, bytes, (hipStream_t)stream) == hipSuccess ? QSA_OK : QSA_EHIP;
}

qsa_status qsa_block_scores(const float *q, const float *k, const float *w, float *scores,
                            int64_t ld_scores, int32_t nq, int32_t n_heads, int32_t head_dim,
                            int32_t n_blocks, void *stream)
{
    const qsa_status st = check_score_args(q, k, w, scores, ld_scores, nq, n_heads, head_dim, n_blocks);
    if (st != QSA_OK)
        return st;
    if (nq == 0 || n_blocks == 0)
        return QSA_OK;
    ScoreArgs a{q, k, w, scores, ld_scores, nq, n_heads, n_blocks};
    return launch_scores(a, (hipStream_t)stream) == hipSuccess ? QSA_OK : QSA_EHIP;
}

qsa_status qsa_block_scores_bf16(const void *q, const void *k, const float *w, float *scores,
                                 int64_t ld_scores, int32_t nq, int32_t n_heads, int32_t head_dim,
                                 int32_t n_blocks, void *stream)
{
    // The FP32 checks apply unchanged: the same shapes, 16-byte aligned rows.
    const qsa_status st = check_score_args(static_cast<const float *>(q), static_cast<const float *>(k), w, scores,
                                           ld_scores, nq, n_heads, head_dim, n_blocks);
    if (st != QSA_OK)
        return st;
    if (ld_scores >= (int64_t)1 << 24)
        return QSA_EUNSUPPORTED;  // the kernel addresses 32 score rows with 31-bit offsets
    if (nq == 0 || n_blocks == 0)
        return QSA_OK;
    ScoreArgs a{static_cast<const float *>(q), static_cast<const float *>(k), w, scores, ld_scores, nq, n_heads,
                n_blocks};
    return launch_scores_bf16(a, (hipStream_t)stream) == hipSuccess ? QSA_OK : QSA_EHIP;
}

qsa_status qsa_block_topk(const float *scores, int64_t ld_scores, int32_t nq, int32_t n_blocks,
                          int32_t block_size, int32_t width, int32_t call,
                          const int32_t *active_blocks, int32_t *cell_ids, int32_t *counts,
                          void *workspace, size_t workspace_bytes, void *stream,
                          const qsa_options *opt)
{
    return topk_call(scores, ld_scores, nq, n_blocks, block_size, width, call, active_blocks, nullptr,
                     cell_ids, counts, workspace, workspace_bytes, stream, opt);
}

qsa_status qsa_block_topk_cells(const float *scores, int64_t ld_scores, int32_t nq, int32_t n_blocks,
                                int32_t block_size, int32_t width, int32_t call,
                                const int32_t *visible_cells, int32_t *cell_ids, int32_t *counts,
                                void *workspace, size_t workspace_bytes, void *stream,
                                const qsa_options *opt)
{
    return topk_call(scores, ld_scores, nq, n_blocks, block_size, width, call, nullptr, visible_cells,
                     cell_ids, counts, workspace, workspace_bytes, stream, opt);
}

qsa_status qsa_select(const float *q, const float *k, const float *w, int32_t n_heads,
                      int32_t head_dim, float *scores, int64_t ld_scores, int32_t nq,
                      int32_t n_blocks, int32_t block_size, int32_t width, int32_t call,
                      const int32_t *active_blocks, int32_t *cell_ids, int32_t *counts,
                      void *workspace, size_t workspace_bytes, void *stream,
                      const qsa_options *opt)
{
    return select_call(q, k, w, n_heads, head_dim, scores, ld_scores, nq, n_blocks, block_size, width, call,
                       active_blocks, nullptr, cell_ids, counts, workspace, workspace_bytes, stream, opt);
}

qsa_status qsa_select_cells(const float *q, const float *k, const float *w, int32_t n_heads,
                            int32_t head_dim, float *scores, int64_t ld_scores, int32_t nq,
                            int32_t n_blocks, int32_t block_size, int32_t width, int32_t call,
                            const int32_t *visible_cells, int32_t *cell_ids, int32_t *counts,
                            void *workspace, size_t workspace_bytes, void *stream,
                            const qsa_options *opt)
{
    return select_call(q, k, w, n_heads, head_dim, scores, ld_scores, nq, n_blocks, block_size, width, call,
                       nullptr, visible_cells, cell_ids, counts, workspace, workspace_bytes, stream, opt);
}

size_t qsa_selection_attention_workspace_bytes(int32_t nq, int32_t n_heads, int32_t kv_heads, int32_t width)
{
    AttnPlan plan;
    if (!make_attn_plan(nq, n_heads, kv_heads, width, plan))
        return 0;
    return plan.bytes;
}

size_t qsa_selection_attention_shared_workspace_bytes(int32_t nq, int32_t n_heads, int32_t kv_heads,
                                                      int32_t width)
{
    AttnPlan plan;
    if (!make_attn_plan(nq, n_heads, kv_heads, width, plan, true))
        return 0;
    return plan.bytes;
}

} // extern "C"

namespace {

qsa_status attention_call(bool shared, const void *q, const void *k, const void *v, const int32_t *ids,
                          int64_t ld_ids, float *out, float *lse, int32_t nq, int32_t n_heads, int32_t kv_heads,
                          int32_t head_dim, int32_t n_cells, int32_t width, float scale, void *workspace,
                          size_t workspace_bytes, void *stream)
{
    if (nq < 0 || n_heads < 1 || kv_heads < 1 || n_heads % kv_heads != 0 || n_cells < 1 || width < 1 ||
        ld_ids < width || !isfinite(scale))
        return QSA_EINVAL;
    if (head_dim != 128)
        return QSA_EUNSUPPORTED;
    if (shared && (n_heads / kv_heads > kPairHeads || width > kPairMaxWidth || n_cells >= (1 << kPairIdBits)))
        return QSA_EUNSUPPORTED;
    AttnPlan plan;
    if (!make_attn_plan(nq, n_heads, kv_heads, width, plan, shared))
        return QSA_EINVAL;
    if (nq == 0)
        return QSA_OK;
    if (!q || !k || !v || !ids || !out)
        return QSA_EINVAL;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) || !aligned(ids, 4) ||
        !aligned(lse, 4))
        return QSA_EINVAL;
    if (plan.bytes > 0 && (!workspace || !aligned(workspace, kAlign) || workspace_bytes < plan.bytes))
        return QSA_EWORKSPACE;
    AttnArgs a{};
    a.q = static_cast<const uint16_t *>(q);
    a.k = static_cast<const uint16_t *>(k);
    a.v = static_cast<const uint16_t *>(v);
    a.out = out;
    a.lse = lse;
    a.part_ml = plan.n_chunks > 1 ? at<float2>(workspace, plan.ml_offset) : nullptr;
    a.part_o = plan.n_chunks > 1 ? at<float>(workspace, plan.o_offset) : nullptr;
    a.nq = nq;
    a.n_heads = n_heads;
    a.kv_heads = kv_heads;
    a.group = n_heads / kv_heads;
    a.hblocks = plan.hblocks;
    a.n_cells = n_cells;
    a.steps_per_wave = plan.steps_per_wave;
    a.n_chunks = plan.n_chunks;
    a.scale_log2 = (float)((double)scale * 1.4426950408889634);
    if (shared) {
        // The units walk the merged lists: twice the width, one row per pair.
        a.union_ids = at<int32_t>(workspace, plan.union_offset);
        a.union_len = at<int32_t>(workspace, plan.len_offset);
        a.ids = a.union_ids;
        a.ld_ids = 2 * (int64_t)width;
        a.width = 2 * width;
        a.src_ids = ids;
        a.src_ld = ld_ids;
        a.src_width = width;
        a.slot_bits = plan.slot_bits;
    } else {
        a.ids = ids;
        a.ld_ids = ld_ids;
        a.width = width;
    }
    return launch_attention(a, plan, (hipStream_t)stream) == hipSuccess ? QSA_OK : QSA_EHIP;
}

} // namespace

extern "C" {

qsa_status qsa_selection_attention(const void *q, const void *k, const void *v, const int32_t *ids,
                                   int64_t ld_ids, float *out, float *lse, int32_t nq, int32_t n_heads,
                                   int32_t kv_heads, int32_t head_dim, int32_t n_cells, int32_t width,
                                   float scale, void *workspace, size_t workspace_bytes, void *stream)
{
    return attention_call(false, q, k, v, ids, ld_ids, out, lse, nq, n_heads, kv_heads, head_dim, n_cells, width,
                          scale, workspace, workspace_bytes, stream);
}

qsa_status qsa_selection_attention_shared(const void *q, const void *k, const void *v, const int32_t *ids,
                                          int64_t ld_ids, float *out, float *lse, int32_t nq, int32_t n_heads,
                                          int32_t kv_heads, int32_t head_dim, int32_t n_cells, int32_t width,
                                          float scale, void *workspace, size_t workspace_bytes, void *stream)
{
    return attention_call(true, q, k, v, ids, ld_ids, out, lse, nq, n_heads, kv_heads, head_dim, n_cells, width,
                          scale, workspace, workspace_bytes, stream);
}

} // extern "C"
