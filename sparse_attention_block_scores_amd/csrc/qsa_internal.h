// qsa_internal.h - host/device argument blocks and host-side planning shared
// by the library's translation units (not part of the public ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/qsa.h"

namespace qsa {

// ---------------------------------------------------------------- top-k
constexpr int kSplitThreads = 512;        // workgroup of the exact split's stage A
constexpr int kSplitMergeThreads = 1024;  // workgroup of its stage B (one per query)
constexpr int kOneReadThreads = 1024;     // one workgroup per query on the one-read path
constexpr int kOneReadF4 = 4;             // float4 loads per lane and slice
constexpr int kOneReadBuffers = 2;        // slices in flight per lane
constexpr int kOneReadBatch = kOneReadThreads * kOneReadF4 * 4;  // blocks streamed per batch
constexpr int kOneReadMaxBatches = 64;    // the one-read path takes rows of up to 64 batches
// Short streams use slices half as long (kOneReadShortF4 float4 loads per
// lane): more slices per wave balance the waves' ends better. Measured on
// MI355X: 256 queries x 32,768 blocks 14.4 -> 13.5 us, 65,536 blocks equal
// or better, longer rows no gain; with 3 queries (a lone workgroup streams
// each row) 10,240 / 16,384 blocks 8.8 -> 8.3 / 9.4 -> 9.2 us but 32,768 /
// 64,512 blocks 0.2 / 0.4 us slower.
constexpr int kOneReadShortF4 = 2;
constexpr int kOneReadShortRow = 65536;     // many queries: rows up to this many blocks
constexpr int kOneReadShortFewRow = 16384;  // few queries: rows up to this many blocks
constexpr int kOneReadShortQueries = 64;    // "many"
constexpr int kOneReadShortBatch = kOneReadThreads * kOneReadShortF4 * 4;

inline bool oneread_short_slices(int32_t nq, int32_t n_blocks)
{
    return n_blocks <= kOneReadShortFewRow || (nq >= kOneReadShortQueries && n_blocks <= kOneReadShortRow);
}
constexpr int kChunkBound = 4104;         // split chunks: the fewest of at most this many blocks
constexpr int kMinChunk = 64;
constexpr int kMaxChunk = 15360;          // keeps a chunk's keys under 60 KB of LDS
constexpr int kStageBLdsWords = 15360;    // stage B keeps up to this many candidates (keys and blocks) in LDS
constexpr int kOneReadCap = 8192;         // one-read candidate cap per query (blocks)
constexpr int kOneReadSample = 4096;      // one-read sample: at most this many keys
constexpr int kOneReadMinRatio = 16;      // one-read when n_blocks >= this many times r_blocks ...
constexpr int kSampleStride = 32;

// Two-launch filtered split: stage A filters chunks of a row by the sampled
// bound (one 256-thread workgroup per chunk), stage B selects per query.
constexpr int kFilterThreads = 256;
constexpr int kFilterMinChunk = 1024;     // blocks per stage-A chunk: 1024 * (1, 2, 4 or 8)
constexpr int kFilterMaxChunk = 8192;
constexpr int kFilterMaxChunks = 1024;    // chunks per row (stage B scans one header per thread)
constexpr int kFilterTargetGroups = 512;  // stage-A workgroups the chunk size aims for
constexpr int kFilterMinBlocks = 65536;   // the dispatch's filtered split: rows of at least this many blocks ...
constexpr int kFilterBlocksPerQuery = 2048;  // ... plus this many per query ...
constexpr int kFilterMaxQueries = 16;     // ... in calls of at most this many queries
constexpr uint32_t kFilterOverflow = 0xFFFFFFFFu;  // header count of a chunk whose slot overflowed

// Workspace layout of the split (byte offsets, 256-byte aligned).
struct TopkLayout {
    size_t split_keys;      // u32 [nq][cand_stride]
    size_t split_blocks;    // i32 [nq][cand_stride]
    size_t filter_heads;    // u32 [nq][n_chunks][4]  (filtered split)
    size_t filter_slots;    // u32 [nq][n_chunks][2][slot]
    size_t bytes;
};

struct TopkPlan {
    qsa_topk_plan pub;
    int64_t cand_stride;    // split candidates per query, a multiple of 4
    TopkLayout lay;
};

// Fills `plan`; returns QSA_OK or the argument error.
qsa_status make_topk_plan(int32_t nq, int32_t n_blocks, int32_t block_size, int32_t width,
                          int32_t call, const qsa_options *opt, TopkPlan &plan);

struct TopkGeom {
    const float *scores;
    int64_t ld;
    int32_t nq;
    int32_t n_blocks;
    int32_t bs;
    int32_t width;
    const int32_t *active;  // nullable: visible blocks per query
    const int32_t *cells;   // nullable: visible cells per query (the last visible block may be partial)
    int32_t *ids;
    int32_t *counts;        // nullable
    int32_t vec4;           // rows are 16-byte aligned (float4 loads allowed)
};

struct SplitArgs {
    TopkGeom g;
    uint32_t *cand_keys;
    int32_t *cand_blocks;
    int64_t cand_stride;
    int32_t chunk;
    int32_t n_chunks;
    int32_t lds_words;      // stage A: dynamic LDS words for a chunk's keys (>= chunk)
    int32_t blk_words;      // stage B: LDS words for candidate keys, as many again for their blocks (0: read from the workspace)
};

struct OneReadArgs {
    TopkGeom g;
    int32_t mode;           // QSA_SAMPLE_STRIDE / QSA_SAMPLE_LINES
    int32_t force_flag;     // take the exact path for every query
};

struct FilterArgs {
    TopkGeom g;
    uint32_t *heads;        // [nq][n_chunks] x {count or kFilterOverflow, min key, max key, bound key}
    uint32_t *slots;        // [nq][n_chunks][2][slot]: candidate keys, then their block indices
    int32_t chunk;          // blocks per chunk
    int32_t n_chunks;       // chunks of the longest row
    int32_t slot;           // candidates a chunk may keep
    int32_t mode;           // QSA_SAMPLE_STRIDE / QSA_SAMPLE_LINES
    int32_t force_flag;     // every query takes the exact fallback
    int32_t xcd;            // 1: the chunks of a query run on one XCD (nq a multiple of 8)
};

hipError_t launch_zero(void *p, size_t bytes, hipStream_t s);
hipError_t launch_filter(const FilterArgs &a, hipStream_t s);
hipError_t launch_split(const SplitArgs &a, hipStream_t s);
hipError_t launch_oneread(const OneReadArgs &a, hipStream_t s);

// ---------------------------------------------------------------- scores
struct ScoreArgs {
    const float *q;
    const float *k;
    const float *w;
    float *scores;
    int64_t ld;
    int32_t nq;
    int32_t heads;
    int32_t n_blocks;
};

hipError_t launch_scores(const ScoreArgs &a, hipStream_t s);
// The same with q and k holding BF16 values (ScoreArgs' q and k point at them).
hipError_t launch_scores_bf16(const ScoreArgs &a, hipStream_t s);

// Attention of every query head over its query's selected cells.
constexpr int kAttnWaves = 8;             // waves per workgroup (one workgroup per CU)
constexpr int kAttnStepCells = 32;        // cells per wave step
constexpr int kAttnHeadBlock = 16;        // query heads per workgroup (one matrix-core column each)
constexpr int kAttnTargetGroups = 256;    // workgroups the chunking aims for (one per CU)
constexpr int kAttnMaxChunks = 16;        // chunks of one unit's list at most
// Shared-block attention: pairs of queries, each pair's lists merged first.
constexpr int kPairHeads = 8;             // heads of one query in a pair's 16 matrix-core columns
constexpr int kPairMaxWidth = 4096;       // longest list the merge's LDS hash takes
constexpr int kPairIdBits = 30;           // merged entry: cell id (low 30 bits) | which queries listed it

struct AttnPlan {
    int32_t shared;          // 1: pairs of queries over their merged lists
    int32_t pairs;           // shared: ceil(nq / 2)
    int32_t slot_bits;       // shared: log2 of the merge's hash slots
    size_t union_offset;     // shared: workspace: merged lists, [pairs][2 * width] int32
    size_t len_offset;       // shared: workspace: merged list lengths, [pairs] int32
    int32_t hblocks;         // blocks of up to 16 heads per key/value head
    int32_t steps_per_wave;  // 32-cell steps each wave takes
    int32_t n_chunks;        // chunks of the id list per (query, kv head, head block)
    int64_t units;           // nq * kv_heads * hblocks
    size_t ml_offset;        // workspace: (max, sum) per partial, float2
    size_t o_offset;         // workspace: 128 floats per partial
    size_t bytes;            // 0 when one chunk covers the list
};

struct AttnArgs {
    const uint16_t *q;       // [nq][n_heads][128] bfloat16
    const uint16_t *k;       // [n_cells][kv_heads][128] bfloat16
    const uint16_t *v;       // [n_cells][kv_heads][128] bfloat16
    const int32_t *ids;      // [nq][ld_ids]
    int64_t ld_ids;
    float *out;              // [nq][n_heads][128]
    float *lse;              // [nq][n_heads] or null
    float2 *part_ml;
    float *part_o;
    int32_t nq, n_heads, kv_heads, group, hblocks, n_cells, width, steps_per_wave, n_chunks;
    float scale_log2;        // softmax scale times log2(e)
    // Shared-block attention: ids are the merged lists (ld_ids = width = twice
    // the callers' width), src_ids the callers' lists.
    const int32_t *src_ids;  // [nq][src_ld]
    int64_t src_ld;
    int32_t src_width;
    int32_t slot_bits;
    int32_t *union_ids;      // [pairs][width]
    int32_t *union_len;      // [pairs]
};

bool make_attn_plan(int32_t nq, int32_t n_heads, int32_t kv_heads, int32_t width, AttnPlan &plan,
                    bool shared = false);
hipError_t launch_attention(const AttnArgs &a, const AttnPlan &plan, hipStream_t s);

} // namespace qsa
