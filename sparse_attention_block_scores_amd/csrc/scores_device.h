// scores_device.h - the indexer block scorer's building blocks on FP32
// matrix cores (gfx950), shared by the scorer kernel and the fused decode
// select.
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
//    double-buffered; the next tile's global loads are in flight while the
//    current tile's 64*MR MFMAs run. LDS rows are padded to 132 floats so the
//    128-bit LDS reads of 32 different key rows hit distinct banks.
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

// LDS of one scoring workgroup: two staged key tiles and the weights of its
// ROWS padded rows.
template <int ROWS>
struct ScoreLds {
    __attribute__((aligned(16))) float k[2][kTileBlocks * kLdsRow];
    float w[ROWS];
};

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

    load_tile(t0);
    store_tile(sm.k[0]);
    __syncthreads();

    for (int t = t0; t < t1; ++t) {
        const int cur = (t - t0) & 1;
        if (t + 1 < t1)
            load_tile(t + 1);

        // A wave whose rows are all padding skips the MFMAs and the epilogue
        // (it still stages key tiles and meets every barrier).
        if (live) {
            f32x16 acc[MR];
#pragma unroll
            for (int m = 0; m < MR; ++m)
#pragma unroll
                for (int v = 0; v < 16; ++v)
                    acc[m][v] = 0.f;
            const float *kb = &sm.k[cur][li * kLdsRow + 64 * half];
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

            // Epilogue: relu, weight, head sum, store.
            const int blk = t * kTileBlocks + li;
            const bool col_ok = blk < a.n_blocks;
            if constexpr (HP == 64) {
                float s = 0.f;
#pragma unroll
                for (int m = 0; m < MR; ++m)
#pragma unroll
                    for (int v = 0; v < 16; ++v) {
                        const int row = (wv * MR + m) * 32 + 8 * (v >> 2) + 4 * half + (v & 3);
                        s += sm.w[row] * fmaxf(acc[m][v], 0.f);
                    }
                s += __shfl_xor(s, 32, 64);
                const int qi = (row0 + wv * MR * 32) / 64;
                if (half == 0 && col_ok && qi < a.nq)
                    store(qi, blk, s);
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
                        for (int v = 0; v < 16; ++v) {
                            const int row = 8 * (v >> 2) + 4 * half + (v & 3);
                            part[(8 * (v >> 2)) / HP] += sm.w[tile_row + row] * fmaxf(acc[m][v], 0.f);
                        }
#pragma unroll
                        for (int s = 0; s < SLOTS; ++s) {
                            const float tot = part[s] + __shfl_xor(part[s], 32, 64);
                            const int qi = q0 + s;
                            if (half == 0 && col_ok && qi < a.nq)
                                store(qi, blk, tot);
                        }
                    } else {
                        // HP <= 4: a lane's rows cover whole queries; no exchange.
                        constexpr int LS = 32 / HP;  // local slot index space
                        float part[LS];
#pragma unroll
                        for (int s = 0; s < LS; ++s)
                            part[s] = 0.f;
#pragma unroll
                        for (int v = 0; v < 16; ++v) {
                            const int row = 8 * (v >> 2) + 4 * half + (v & 3);
                            part[(8 * (v >> 2)) / HP + (v & 3) / HP] += sm.w[tile_row + row] * fmaxf(acc[m][v], 0.f);
                        }
#pragma unroll
                        for (int v = 0; v < 16; v += HP) {
                            const int s = (8 * (v >> 2)) / HP + (v & 3) / HP;
                            const int qi = q0 + s + (4 * half) / HP;
                            if (col_ok && qi < a.nq)
                                store(qi, blk, part[s]);
                        }
                    }
                }
            }
        }

        if (t + 1 < t1)
            store_tile(sm.k[cur ^ 1]);
        __syncthreads();
    }
}

} // namespace qsa
