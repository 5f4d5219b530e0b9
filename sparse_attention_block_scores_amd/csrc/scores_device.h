// scores_device.h - the indexer block scorer's building blocks on FP32 and
// BF16 matrix cores (gfx950), used by the scorer kernels.
//
// score[q][b] = sum_h w[q][h] * relu(dot(q[q][h][:], k[b][:])), K = 128
// (Strata pull #1091 "qsa_select: FP32 tiled block scores below sm_80",
// section What: rows of the contraction are (query, indexer head) pairs, the
// relu is per head and the heads are summed without leaving registers).
//
//  * Rows: each query's heads are padded to HP (a power of two up to 32, or
//    64) rows; padded rows have q = 0 and w = 0, so they add nothing. Each
//    wave keeps its MR 32-row tiles of q in VGPRs as the A operand of
//    v_mfma_f32_32x32x2_f32.
//  * K-index order: step s of the 64 MFMA steps contracts k-indices s (lanes
//    0-31) and 64+s (lanes 32-63), so every lane reads 64 consecutive floats
//    of its own q row and of its key row; the sum is the same dot product in
//    another order.
//  * Columns: key tiles of 32 blocks x 128 floats (16 KB) are staged in LDS,
//    double-buffered; the next tiles' global loads are in flight while the
//    current tile's 64*MR MFMAs run (16-wave workgroups stage pairs of tiles
//    with loads straight into LDS: score_tiles_dma). LDS rows are padded to
//    132 floats so the 128-bit LDS reads of 32 different key rows hit
//    distinct banks.
//  * Epilogue: the 32x32 accumulator puts rows 8*(v/4) + 4*(lane/32) + v%4
//    of column lane%32 in register v, so a query's head sum is a few in-lane
//    adds plus (for HP >= 8) one exchange with lane^32. Only scores leave
//    registers, through the caller's store(query, block, score).
#pragma once

#include "qsa_internal.h"

namespace qsa {

typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kHeadDim = 128;
constexpr int kTileBlocks = 32;
constexpr int kLdsRow = 132;  // floats per staged key row (128 + 4 pad)
// Fourth word of a raw buffer resource on gfx9-family GPUs (32-bit data
// format, no swizzle); with stride 0 an access at or past num_records bytes
// is dropped (stores) or reads zero (loads).
constexpr int kScoreBufferWord3 = 0x00020000;

// LDS of one scoring workgroup: two staged key tiles and the weights of its
// ROWS padded rows.
template <int ROWS>
struct ScoreLds {
    __attribute__((aligned(16))) float k[2][kTileBlocks * kLdsRow];
    float w[ROWS];
};

// max(x, 0) for a finite x, as an integer max of its bit pattern: negative
// values (and -0.0) have the sign bit set, so they compare below 0 and give
// +0.0; one instruction, where a float max would first quiet the operand.
__device__ __forceinline__ float relu(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

// x of this lane plus x of the lane 32 away (lanes l and l ^ 32 get the same
// sum): one cross-half swap of two copies.
__device__ __forceinline__ float half_sum(float x)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Epilogue of one key tile: relu, weight, head sum, store. acc[m] holds the
// 32x32 dot products of this wave's row tile m (rows 8*(v/4) + 4*(lane/32) +
// v%4 of column lane%32 in register v, the layout of every 32x32 matrix-core
// product); wgt(m, v) is the weight of acc[m][v]'s row; blk is the block of
// this lane's column.
template <int HP, int MR, bool MASKED = false, class Weight, class Store>
__device__ __forceinline__ void score_epilogue(const f32x16 (&acc)[MR], const ScoreArgs &a, int row0, int wv,
                                               int half, int blk, Weight wgt, Store store)
{
    const bool col_ok = blk < a.n_blocks;
    // MASKED: every lane calls store(qi, blk, s, ok, qb) (qb: the first
    // query of the row tile, wave-uniform) and the store itself drops the
    // lanes whose ok is false; else only valid lanes call store(qi, blk, s).
    auto emit = [&](int qi, float x, bool ok, int qb) {
        if constexpr (MASKED)
            store(qi, blk, x, ok, qb);
        else if (ok)
            store(qi, blk, x);
    };
    if constexpr (HP == 64) {
        float s = 0.f;
#pragma unroll
        for (int m = 0; m < MR; ++m)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                s += wgt(m, v) * relu(acc[m][v]);
            }
        s = half_sum(s);
        const int qi = (row0 + wv * MR * 32) / 64;
        emit(qi, s, half == 0 && col_ok && qi < a.nq, qi);
    } else {
#pragma unroll
        for (int m = 0; m < MR; ++m) {
            const int tile_row = (wv * MR + m) * 32;  // slab row of this tile's row 0
            const int q0 = (row0 + tile_row) / HP;    // first query of the tile
            if constexpr (HP >= 8) {
                constexpr int SLOTS = 32 / HP;
                float part[SLOTS];
#pragma unroll
                for (int s = 0; s < SLOTS; ++s)
                    part[s] = 0.f;
#pragma unroll
                for (int v = 0; v < 16; ++v)
                    part[(8 * (v >> 2)) / HP] += wgt(m, v) * relu(acc[m][v]);
#pragma unroll
                for (int s = 0; s < SLOTS; ++s) {
                    const float tot = half_sum(part[s]);
                    const int qi = q0 + s;
                    emit(qi, tot, half == 0 && col_ok && qi < a.nq, q0);
                }
            } else {
                // HP <= 4: a lane's rows cover whole queries; no exchange.
                constexpr int LS = 32 / HP;  // local slot index space
                float part[LS];
#pragma unroll
                for (int s = 0; s < LS; ++s)
                    part[s] = 0.f;
#pragma unroll
                for (int v = 0; v < 16; ++v)
                    part[(8 * (v >> 2)) / HP + (v & 3) / HP] += wgt(m, v) * relu(acc[m][v]);
#pragma unroll
                for (int v = 0; v < 16; v += HP) {
                    const int s = (8 * (v >> 2)) / HP + (v & 3) / HP;
                    const int qi = q0 + s + (4 * half) / HP;
                    emit(qi, part[s], col_ok && qi < a.nq, q0);
                }
            }
        }
    }
}

// Scores of key tiles [t0, t1) for the NW*MR*32 padded rows from row0: q rows
// of this wave into VGPRs, weights into LDS, then every tile through the
// MFMAs and the epilogue; store(qi, blk, score) receives each score. All
// threads call; the LDS is free again on return.
template <int HP, int MR, int NW, class Store>
__device__ __forceinline__ void score_tiles(const ScoreArgs &a, int row0, int t0, int t1, ScoreLds<NW * MR * 32> &sm,
                                            Store store)
{
    constexpr int NT = NW * 64;
    constexpr int ROWS = NW * MR * 32;
    static_assert(HP <= 32 || (HP == 64 && MR == 2), "64 heads need both row tiles of a wave");
    const int tid = threadIdx.x;
    const int lane = tid & 63, wv = tid >> 6;
    const int li = lane & 31, half = lane >> 5;
    const bool live = __builtin_amdgcn_readfirstlane(row0 + wv * MR * 32) < a.nq * HP;  // wave-uniform

    // Key tile t -> registers: 1024 float4 granules, 1024/NT per thread.
    constexpr int GPT = (kTileBlocks * kHeadDim / 4) / NT;
    float4 pre[GPT];
    auto load_tile = [&](int t) {
#pragma unroll
        for (int i = 0; i < GPT; ++i) {
            const int gidx = tid + NT * i;
            const int blk = t * kTileBlocks + (gidx >> 5);
            pre[i] = blk < a.n_blocks
                         ? reinterpret_cast<const float4 *>(a.k + (int64_t)blk * kHeadDim)[gidx & 31]
                         : make_float4(0.f, 0.f, 0.f, 0.f);
        }
    };
    auto store_tile = [&](float *dst) {
#pragma unroll
        for (int i = 0; i < GPT; ++i) {
            const int gidx = tid + NT * i;
            *reinterpret_cast<float4 *>(dst + (gidx >> 5) * kLdsRow + (gidx & 31) * 4) = pre[i];
        }
    };
    // The first tile's loads go out before q's and w's, so that their round
    // trips overlap (storing w waits for every load issued before it).
    load_tile(t0);

    // q rows of this wave -> VGPRs (A operand).
    float qa[MR][64];
#pragma unroll
    for (int m = 0; m < MR; ++m) {
        const int R = row0 + (wv * MR + m) * 32 + li;
        const int qi = R / HP, h = R % HP;
        const bool ok = qi < a.nq && h < a.heads;
        const float4 *src = reinterpret_cast<const float4 *>(
            a.q + ((int64_t)(ok ? qi : 0) * a.heads + (ok ? h : 0)) * kHeadDim + 64 * half);
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            const float4 v = ok ? src[u] : make_float4(0.f, 0.f, 0.f, 0.f);
            qa[m][4 * u + 0] = v.x;
            qa[m][4 * u + 1] = v.y;
            qa[m][4 * u + 2] = v.z;
            qa[m][4 * u + 3] = v.w;
        }
    }
    for (int r = tid; r < ROWS; r += NT) {
        const int R = row0 + r;
        const int qi = R / HP, h = R % HP;
        sm.w[r] = (qi < a.nq && h < a.heads) ? a.w[(int64_t)qi * a.heads + h] : 0.f;
    }

    // One key tile (staged at kt) through the MFMAs and the epilogue. A wave
    // whose rows are all padding skips both (it still stages key tiles and
    // meets every barrier).
    auto score_tile = [&](int t, const float *kt) {
        if (!live)
            return;
        f32x16 acc[MR];
#pragma unroll
        for (int m = 0; m < MR; ++m)
#pragma unroll
            for (int v = 0; v < 16; ++v)
                acc[m][v] = 0.f;
        const float *kb = kt + li * kLdsRow + 64 * half;
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            const float4 b = *reinterpret_cast<const float4 *>(kb + 4 * u);
            const float bv[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
            for (int e = 0; e < 4; ++e)
#pragma unroll
                for (int m = 0; m < MR; ++m)
                    acc[m] = __builtin_amdgcn_mfma_f32_32x32x2f32(qa[m][4 * u + e], bv[e], acc[m], 0, 0, 0);
        }
        score_epilogue<HP, MR>(
            acc, a, row0, wv, half, t * kTileBlocks + li,
            [&](int m, int v) { return sm.w[(wv * MR + m) * 32 + 8 * (v >> 2) + 4 * half + (v & 3)]; }, store);
    };

    store_tile(sm.k[0]);
    __syncthreads();
    for (int t = t0; t < t1; ++t) {
        const int cur = (t - t0) & 1;
        if (t + 1 < t1)
            load_tile(t + 1);
        score_tile(t, sm.k[cur]);
        if (t + 1 < t1)
            store_tile(sm.k[cur ^ 1]);
        __syncthreads();
    }
}


// The FP32 path of 16-wave workgroups with one row tile per wave (the
// prompt-call shapes): key tiles go from memory straight into LDS
// (buffer_load ... lds), so staging holds no registers and issues no LDS
// writes. Two pairs of tile buffers, kA and kB, are separate LDS arrays: the
// reads of one pair then need not wait for the loads into the other, and the
// barrier after a pair waits for them. One load instruction fills half a key
// row (64 lanes x 4 bytes, in lane order at the instruction's LDS base), so
// rows keep the 132-float padding of the register-staged path.
constexpr int kDmaTile = kTileBlocks * kLdsRow;  // floats per staged key tile

template <int HP, class Store>
__device__ __forceinline__ void score_tiles_dma(const ScoreArgs &a, int row0, int t0, int t1,
                                                float (&kA)[2][kDmaTile], float (&kB)[2][kDmaTile],
                                                float *w_lds, Store store)
{
    constexpr int NW = 16, MR = 1, NT = NW * 64, ROWS = NW * 32;
    static_assert(HP <= 32, "one row tile per wave");
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int li = lane & 31, half = lane >> 5;
    const bool live = __builtin_amdgcn_readfirstlane(row0 + wv * 32) < a.nq * HP;  // wave-uniform

    // Tiles tp and tp + 1 into dst: wave w loads key rows 2w and 2w + 1 of
    // each, half a row per instruction. The resource spans the pair's
    // visible blocks (none past the last: those read zero without a memory
    // access), so every offset stays below 32 KiB whatever n_blocks is.
    auto issue_pair = [&](int tp, float (&dst)[2][kDmaTile]) {
        const int64_t first = (int64_t)tp * kTileBlocks;
        const int64_t left = (int64_t)a.n_blocks - first;
        const int recs = left <= 0 ? 0 : (int)(left < 2 * kTileBlocks ? left : 2 * kTileBlocks) * kHeadDim * 4;
        const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<float *>(a.k + (left > 0 ? first : 0) * kHeadDim), (short)0, recs, kScoreBufferWord3);
#pragma unroll
        for (int d = 0; d < 2; ++d)
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                const int row = 2 * wv + (x >> 1), part = x & 1;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    r, (__attribute__((address_space(3))) void *)(&dst[d][row * kLdsRow + part * 64]), 4,
                    ((d * kTileBlocks + row) * kHeadDim + part * 64 + lane) * 4, 0, 0, 0);
            }
    };

    // The first pair's loads go out before q's and w's, so that their round
    // trips overlap (storing w waits for every load issued before it).
    issue_pair(t0, kA);

    // q rows of this wave -> VGPRs (A operand).
    float qa[64];
    {
        const int R = row0 + wv * 32 + li;
        const int qi = R / HP, h = R % HP;
        const bool ok = qi < a.nq && h < a.heads;
        const float4 *src = reinterpret_cast<const float4 *>(
            a.q + ((int64_t)(ok ? qi : 0) * a.heads + (ok ? h : 0)) * kHeadDim + 64 * half);
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            const float4 v = ok ? src[u] : make_float4(0.f, 0.f, 0.f, 0.f);
            qa[4 * u + 0] = v.x;
            qa[4 * u + 1] = v.y;
            qa[4 * u + 2] = v.z;
            qa[4 * u + 3] = v.w;
        }
    }
    for (int r = tid; r < ROWS; r += NT) {
        const int R = row0 + r;
        const int qi = R / HP, h = R % HP;
        w_lds[r] = (qi < a.nq && h < a.heads) ? a.w[(int64_t)qi * a.heads + h] : 0.f;
    }

    // One staged tile through the MFMAs and the epilogue. (Deferring each
    // epilogue past the next tile's matrix steps, with a second accumulator
    // set, measured slower here: C5 1,885 -> 1,917 us.)
    auto score_tile = [&](int t, const float *kt) {
        if (!live)
            return;
        f32x16 acc[MR];
#pragma unroll
        for (int v = 0; v < 16; ++v)
            acc[0][v] = 0.f;
        const float *kb = kt + li * kLdsRow + 64 * half;
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            const float4 b = *reinterpret_cast<const float4 *>(kb + 4 * u);
            const float bv[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
            for (int e = 0; e < 4; ++e)
                acc[0] = __builtin_amdgcn_mfma_f32_32x32x2f32(qa[4 * u + e], bv[e], acc[0], 0, 0, 0);
        }
        score_epilogue<HP, MR>(
            acc, a, row0, wv, half, t * kTileBlocks + li,
            [&](int m, int v) { return w_lds[wv * 32 + 8 * (v >> 2) + 4 * half + (v & 3)]; }, store);
    };

    __syncthreads();  // the first pair and the weights are in LDS
    for (int tb = t0; tb < t1; tb += 4) {
        issue_pair(tb + 2, kB);
        score_tile(tb, kA[0]);
        if (tb + 1 < t1)
            score_tile(tb + 1, kA[1]);
        __syncthreads();  // kB loaded; kA read by every wave
        if (tb + 2 >= t1)
            break;
        issue_pair(tb + 4, kA);
        score_tile(tb + 2, kB[0]);
        if (tb + 3 < t1)
            score_tile(tb + 3, kB[1]);
        __syncthreads();
    }
}


// ------------------------------------------------------------ BF16 inputs
// The same scores from BF16 q and k (16-bit IEEE bfloat16 bit patterns) on
// the BF16 matrix cores: v_mfma_f32_32x32x16_bf16 takes 8 consecutive
// k-indices per lane, so step u of the 8 steps contracts k-indices 8u..8u+7
// (lanes 0-31) and 64+8u..64+8u+7 (lanes 32-63): every lane again reads 64
// consecutive values of its own q row and key row. Products of two BF16
// values are exact in FP32 and accumulate in FP32; the epilogue is the FP32
// path's. In ScoreArgs, q and k then point at BF16 data.
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
constexpr int kLdsRowH = 136;  // BF16 values per staged key row (128 + 8 pad: 272-byte rows)

template <int ROWS>
struct ScoreLdsH {
    __attribute__((aligned(16))) uint16_t k[4][kTileBlocks * kLdsRowH];  // two pairs of key tiles
    float w[ROWS];
};

template <int HP, int MR, int NW, class Store>
__device__ __forceinline__ void score_tiles_bf16(const ScoreArgs &a, int row0, int t0, int t1,
                                                 ScoreLdsH<NW * MR * 32> &sm, Store store)
{
    constexpr int NT = NW * 64;
    constexpr int ROWS = NW * MR * 32;
    static_assert(HP <= 32 || (HP == 64 && MR == 2), "64 heads need both row tiles of a wave");
    const uint16_t *qh = reinterpret_cast<const uint16_t *>(a.q);
    const uint16_t *kh = reinterpret_cast<const uint16_t *>(a.k);
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    // Wave-uniform (scalar): the tile's first query, and with it the score
    // stores' buffer resource, stay in scalar registers.
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int li = lane & 31, half = lane >> 5;
    const bool live = __builtin_amdgcn_readfirstlane(row0 + wv * MR * 32) < a.nq * HP;  // wave-uniform

    // Key tile t -> registers: 8 KB per tile, CH bytes per thread. The loads
    // are unconditional (a block past the end re-reads the last block, and
    // its scores are never stored): a load under a branch would make the
    // compiler wait for every load in flight before the next use.
    constexpr int CH = kTileBlocks * kHeadDim * 2 / NT;  // bytes per thread: 32, 16 or 8 (256-1,024 threads)
    static_assert(CH == 16 || CH == 8 || CH == 32, "a tile splits into 8, 16 or 32 bytes per thread");
    constexpr int PS = CH < 16 ? CH : 16;                // bytes per load
    constexpr int GPT = CH / PS;                         // loads per thread
    constexpr int PPR = kHeadDim * 2 / PS;               // pieces per key row
    uint4 pre[GPT];
    auto load_tile = [&](int t) {
#pragma unroll
        for (int i = 0; i < GPT; ++i) {
            const int piece = tid * GPT + i;
            const int blk = min(t * kTileBlocks + piece / PPR, a.n_blocks - 1);
            const char *src = reinterpret_cast<const char *>(kh + (int64_t)blk * kHeadDim) + (piece % PPR) * PS;
            if constexpr (PS == 8) {
                const uint2 v = *reinterpret_cast<const uint2 *>(src);
                pre[i] = make_uint4(v.x, v.y, 0u, 0u);
            } else {
                pre[i] = *reinterpret_cast<const uint4 *>(src);
            }
        }
    };
    auto store_tile = [&](uint16_t *dst) {
#pragma unroll
        for (int i = 0; i < GPT; ++i) {
            const int piece = tid * GPT + i;
            char *d = reinterpret_cast<char *>(dst + (piece / PPR) * kLdsRowH) + (piece % PPR) * PS;
            if constexpr (PS == 8)
                *reinterpret_cast<uint2 *>(d) = make_uint2(pre[i].x, pre[i].y);
            else
                *reinterpret_cast<uint4 *>(d) = pre[i];
        }
    };

    // Key tiles go through LDS in pairs: the workgroup scores one pair from
    // one half of the LDS while the next pair, loaded a pair ago into
    // registers, is stored into the other half and the pair after it is
    // loaded; one barrier per pair (a tile is only 8 matrix-core steps here,
    // so a barrier per tile costs a visible share). The barrier orders LDS
    // only, leaving the loads in flight. The loop body has no branch around a
    // memory access, so the compiler waits for exactly the loads a step needs:
    // slots past the last tile score the last tile again with every store
    // dropped, loads of tiles past the end re-read the last one, and waves
    // whose rows are all padding score zero rows (their stores are dropped too).
    uint4 ring[2][GPT];
    auto load_into = [&](int t, uint4 (&dst)[GPT]) {
        load_tile(min(t, t1 - 1));
#pragma unroll
        for (int i = 0; i < GPT; ++i)
            dst[i] = pre[i];
    };
    auto store_from = [&](const uint4 (&src)[GPT], uint16_t *dst) {
#pragma unroll
        for (int i = 0; i < GPT; ++i)
            pre[i] = src[i];
        store_tile(dst);
    };
    // The first pair's loads go out before q's and w's, so that their round
    // trips overlap (storing w waits for every load issued before it).
    load_into(t0, ring[0]);
    load_into(t0 + 1, ring[1]);

    // q rows of this wave -> VGPRs (A operand): 64 BF16 values per lane.
    bf16x8 qa[MR][8];
#pragma unroll
    for (int m = 0; m < MR; ++m) {
        const int R = row0 + (wv * MR + m) * 32 + li;
        const int qi = R / HP, h = R % HP;
        const bool ok = qi < a.nq && h < a.heads;
        const uint4 *src = reinterpret_cast<const uint4 *>(
            qh + ((int64_t)(ok ? qi : 0) * a.heads + (ok ? h : 0)) * kHeadDim + 64 * half);
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const uint4 v = ok ? src[u] : make_uint4(0u, 0u, 0u, 0u);
            qa[m][u] = __builtin_bit_cast(bf16x8, v);
        }
    }
    for (int r = tid; r < ROWS; r += NT) {
        const int R = row0 + r;
        const int qi = R / HP, h = R % HP;
        sm.w[r] = (qi < a.nq && h < a.heads) ? a.w[(int64_t)qi * a.heads + h] : 0.f;
    }

    store_from(ring[0], sm.k[0]);
    store_from(ring[1], sm.k[1]);
    load_into(t0 + 2, ring[0]);
    load_into(t0 + 3, ring[1]);
    __syncthreads();

    // The q rows and the first tiles were loaded above; nothing of the
    // prologue is waited for inside the loop.
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    // This wave's weights, once, in registers.
    float wr[MR][16];
#pragma unroll
    for (int m = 0; m < MR; ++m)
#pragma unroll
        for (int v = 0; v < 16; ++v)
            wr[m][v] = sm.w[(wv * MR + m) * 32 + 8 * (v >> 2) + 4 * half + (v & 3)];
    (void)live;

    for (int tb = t0; tb < t1; tb += 4) {
#pragma unroll
        for (int pr = 0; pr < 2; ++pr) {      // pair tb + 2pr .. tb + 2pr + 1 in LDS half pr
#pragma unroll
            for (int d = 0; d < 2; ++d) {
                const int t = tb + 2 * pr + d;
                f32x16 acc[MR];
#pragma unroll
                for (int m = 0; m < MR; ++m)
#pragma unroll
                    for (int v = 0; v < 16; ++v)
                        acc[m][v] = 0.f;
                const uint16_t *kb = &sm.k[2 * pr + d][li * kLdsRowH + 64 * half];
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const bf16x8 b = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(kb + 8 * u));
#pragma unroll
                    for (int m = 0; m < MR; ++m)
                        acc[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[m][u], b, acc[m], 0, 0, 0);
                }
                // A slot past the last tile: its column test fails for every lane.
                const int blk = t < t1 ? t * kTileBlocks + li : a.n_blocks;
                score_epilogue<HP, MR, true>(acc, a, row0, wv, half, blk, [&](int m, int v) { return wr[m][v]; },
                                             store);
            }
            // The next pair (in the ring) into the other LDS half, and the
            // pair after it into the ring.
            const int tn = tb + 2 * pr + 2;
            store_from(ring[0], sm.k[2 * (pr ^ 1)]);
            store_from(ring[1], sm.k[2 * (pr ^ 1) + 1]);
            load_into(tn + 2, ring[0]);
            load_into(tn + 3, ring[1]);
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
            __builtin_amdgcn_s_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
        }
    }
}

// The BF16 path of 512-row workgroups (16 waves of one row tile, or 8 waves
// of two: each key operand read from LDS then feeds two matrix steps): key-
// tile pairs straight into LDS as in score_tiles_dma (a padded BF16 key row
// is one load instruction: 64 lanes x 4 bytes), kA and kB separate LDS arrays.
constexpr int kDmaTileH = kTileBlocks * kLdsRowH;  // BF16 values per staged key tile

template <int HP, int NW, int MR, class Store>
__device__ __forceinline__ void score_tiles_bf16_dma(const ScoreArgs &a, int row0, int t0, int t1,
                                                     uint16_t (&kA)[2][kDmaTileH], uint16_t (&kB)[2][kDmaTileH],
                                                     float *w_lds, Store store)
{
    constexpr int NT = NW * 64, ROWS = NW * MR * 32;
    constexpr int RPW = kTileBlocks / NW;  // key rows each wave loads per tile
    static_assert(HP <= 32, "whole queries inside a row tile");
    static_assert(RPW * NW == kTileBlocks, "waves split a tile's rows evenly");
    const uint16_t *qh = reinterpret_cast<const uint16_t *>(a.q);
    const uint16_t *kh = reinterpret_cast<const uint16_t *>(a.k);
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int li = lane & 31, half = lane >> 5;

    // Tiles tp and tp + 1 into dst: wave w loads key rows 2w and 2w + 1 of
    // each, a whole row per instruction; the resource spans the pair's
    // visible blocks (the rest reads zero without a memory access).
    auto issue_pair = [&](int tp, uint16_t (&dst)[2][kDmaTileH]) {
        const int64_t first = (int64_t)tp * kTileBlocks;
        const int64_t left = (int64_t)a.n_blocks - first;
        const int recs = left <= 0 ? 0 : (int)(left < 2 * kTileBlocks ? left : 2 * kTileBlocks) * kHeadDim * 2;
        const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint16_t *>(kh + (left > 0 ? first : 0) * kHeadDim), (short)0, recs, kScoreBufferWord3);
#pragma unroll
        for (int d = 0; d < 2; ++d)
#pragma unroll
            for (int x = 0; x < RPW; ++x) {
                const int row = RPW * wv + x;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    r, (__attribute__((address_space(3))) void *)(&dst[d][row * kLdsRowH]), 4,
                    ((d * kTileBlocks + row) * kHeadDim) * 2 + 4 * lane, 0, 0, 0);
            }
    };

    // The first pair's loads go out before q's and w's, so that their round
    // trips overlap (storing w waits for every load issued before it).
    issue_pair(t0, kA);

    // q rows of this wave -> VGPRs (A operand): 64 BF16 values per lane.
    bf16x8 qa[MR][8];
#pragma unroll
    for (int m = 0; m < MR; ++m) {
        const int R = row0 + (wv * MR + m) * 32 + li;
        const int qi = R / HP, h = R % HP;
        const bool ok = qi < a.nq && h < a.heads;
        const uint4 *src = reinterpret_cast<const uint4 *>(
            qh + ((int64_t)(ok ? qi : 0) * a.heads + (ok ? h : 0)) * kHeadDim + 64 * half);
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const uint4 v = ok ? src[u] : make_uint4(0u, 0u, 0u, 0u);
            qa[m][u] = __builtin_bit_cast(bf16x8, v);
        }
    }
    for (int r = tid; r < ROWS; r += NT) {
        const int R = row0 + r;
        const int qi = R / HP, h = R % HP;
        w_lds[r] = (qi < a.nq && h < a.heads) ? a.w[(int64_t)qi * a.heads + h] : 0.f;
    }

    __syncthreads();  // the first pair and the weights are in LDS
    // This wave's weights, once, in registers.
    float wr[MR][16];
#pragma unroll
    for (int m = 0; m < MR; ++m)
#pragma unroll
        for (int v = 0; v < 16; ++v)
            wr[m][v] = w_lds[(wv * MR + m) * 32 + 8 * (v >> 2) + 4 * half + (v & 3)];

    // One staged tile through the matrix cores and the epilogue (every lane
    // stores; the store drops what is not a score: MASKED). Waves whose rows
    // are all padding compute zero rows, whose stores are all dropped.
    auto score_tile = [&](int t, const uint16_t *kt) {
        f32x16 acc[MR];
#pragma unroll
        for (int m = 0; m < MR; ++m)
#pragma unroll
            for (int v = 0; v < 16; ++v)
                acc[m][v] = 0.f;
        const uint16_t *kb = kt + li * kLdsRowH + 64 * half;
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const bf16x8 b = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(kb + 8 * u));
#pragma unroll
            for (int m = 0; m < MR; ++m)
                acc[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[m][u], b, acc[m], 0, 0, 0);
        }
        score_epilogue<HP, MR, true>(acc, a, row0, wv, half, t * kTileBlocks + li,
                                     [&](int m, int v) { return wr[m][v]; }, store);
    };

    for (int tb = t0; tb < t1; tb += 4) {
        issue_pair(tb + 2, kB);
        score_tile(tb, kA[0]);
        if (tb + 1 < t1)
            score_tile(tb + 1, kA[1]);
        __syncthreads();  // kB loaded; kA read by every wave
        if (tb + 2 >= t1)
            break;
        issue_pair(tb + 4, kA);
        score_tile(tb + 2, kB[0]);
        if (tb + 3 < t1)
            score_tile(tb + 3, kB[1]);
        __syncthreads();
    }
}

} // namespace qsa
