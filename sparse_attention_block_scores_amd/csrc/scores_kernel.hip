// scores_kernel.hip - indexer block scores on the matrix cores (gfx950):
// FP32 inputs on the FP32 matrix cores, or BF16 inputs on the BF16 ones.
//
// The contraction, its layout on the matrix cores and the epilogue are in
// scores_device.h. This kernel owns the grid:
//  * A workgroup owns a slab of NW*MR*32 padded rows (query, head) for its
//    whole life and a group of consecutive key tiles.
//  * Grid: slabs x column groups. Workgroup ids go round-robin over the 8
//    XCDs; ids are mapped so that all slabs of one column group run on the
//    same XCD and share its L2 for the key tiles.
#include <type_traits>

#include "scores_device.h"

namespace qsa {

namespace {

struct ScoreGrid {
    int32_t n_slabs;
    int32_t n_groups;
    int32_t tiles_per_group;
    int32_t n_tiles;
    int32_t xcd_map;
};

// The second bound is the waves per SIMD the register budget must allow:
// two 4-wave or two 8-wave workgroups per CU, or one 16-wave workgroup. With
// 1 or 2 heads the epilogue keeps a partial sum per row, and with two row
// tiles per wave (MR = 2) q takes twice the VGPRs: those get the larger
// budget of one 8-wave workgroup per CU instead of spilling.
template <int HP, int MR, int NW, bool BF16>
__global__ __launch_bounds__(NW * 64, NW >= 8 && HP >= 4 && MR == 1 ? 4 : 2) void scores_kernel(ScoreArgs a,
                                                                                              ScoreGrid grid)
{
    constexpr int ROWS = NW * MR * 32;
    using Lds = typename std::conditional<BF16, ScoreLdsH<ROWS>, ScoreLds<ROWS>>::type;

    int slab, grp;
    {
        const int g = blockIdx.x;
        if (grid.xcd_map) {
            const int xcd = g & 7, j = g >> 3;
            slab = j % grid.n_slabs;
            grp = xcd + 8 * (j / grid.n_slabs);
        } else {
            slab = g % grid.n_slabs;
            grp = g / grid.n_slabs;
        }
    }
    const int t0 = grp * grid.tiles_per_group;
    const int t1 = min(t0 + grid.tiles_per_group, grid.n_tiles);
    if (t0 >= t1)
        return;
    if constexpr (BF16) {
        // Unconditional buffer stores: a lane with nothing to store gets an
        // offset past the resource's end, which the hardware drops. (A store
        // under a branch would make the compiler wait for every memory access
        // in flight before the next tile's loads are used.) The resource
        // spans the score rows of the tile's queries; ld < 2^24 keeps its
        // size and every offset below 2^31.
        auto store = [&](int qi, int blk, float s, bool ok, int qb) {
            // A tile of padding rows (qb >= nq) gets an empty resource: every
            // store of it is dropped, and its base stays inside the matrix.
            const bool any = qb < a.nq;
            const int rows = any ? min(a.nq - qb, 32) : 0;
            const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
                a.scores + (int64_t)(any ? qb : 0) * a.ld, (short)0, rows * (int)a.ld * 4, kScoreBufferWord3);
            const int off = ok ? ((qi - qb) * (int)a.ld + blk) * 4 : (int)0x80000000;
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(s), r, off, 0, 0);
        };
        if constexpr ((NW == 16 && MR == 1) || (NW == 8 && MR == 2)) {
            __shared__ __attribute__((aligned(16))) uint16_t kA[2][kDmaTileH];
            __shared__ __attribute__((aligned(16))) uint16_t kB[2][kDmaTileH];
            __shared__ float w_lds[ROWS];
            score_tiles_bf16_dma<HP, NW, MR>(a, slab * ROWS, t0, t1, kA, kB, w_lds, store);
        } else {
            __shared__ Lds sm;
            score_tiles_bf16<HP, MR, NW>(a, slab * ROWS, t0, t1, sm, store);
        }
    } else if constexpr (NW == 16 && MR == 1) {
        // Key tiles straight into LDS (score_tiles_dma): two separate arrays.
        __shared__ __attribute__((aligned(16))) float kA[2][kDmaTile];
        __shared__ __attribute__((aligned(16))) float kB[2][kDmaTile];
        __shared__ float w_lds[ROWS];
        score_tiles_dma<HP>(a, slab * ROWS, t0, t1, kA, kB, w_lds,
                            [&](int qi, int blk, float s) { a.scores[(int64_t)qi * a.ld + blk] = s; });
    } else {
        __shared__ Lds sm;
        score_tiles<HP, MR, NW>(a, slab * ROWS, t0, t1, sm,
                                [&](int qi, int blk, float s) { a.scores[(int64_t)qi * a.ld + blk] = s; });
    }
}

// FP32 scores of long rows when every padded (query, head) row fits one
// 32-row tile (a few queries with few heads over a long context). The slab
// grid would leave one live wave per workgroup (the rest padding), scoring
// its column group's key tiles one after another. Here the workgroup stages
// the 32 q rows in LDS once (coalesced), every wave takes them as its A
// operand, and each wave scores key tiles of its own: a tile is loaded
// coalesced into the wave's LDS area (rows padded to 132 floats, as in the
// slab kernels) and read back as the B operand. Waves share nothing after
// the prologue, so the loop has no barrier. (Keeping the wave's next tile in
// flight in registers put that array in scratch memory; with up to 2,048
// tiles every wave has one tile, and two waves per SIMD overlap the rest.)
constexpr int kLongWaves = 8;
constexpr int kLongMinTiles = 1024;  // shorter rows keep the slab grid

template <int HP>
__global__ __launch_bounds__(kLongWaves * 64, 2) void scores_longrow_kernel(ScoreArgs a, int n_tiles, int tiles_per_wg)
{
    static_assert(HP <= 32, "every row inside one 32-row tile");
    constexpr int NT = kLongWaves * 64;
    __shared__ __attribute__((aligned(16))) float q_lds[kTileBlocks * kLdsRow];
    __shared__ __attribute__((aligned(16))) float k_lds[kLongWaves][kTileBlocks * kLdsRow];
    __shared__ float w_lds[32];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int li = lane & 31, half = lane >> 5;

    const int tb = (int)blockIdx.x * tiles_per_wg;
    const int te = min(tb + tiles_per_wg, n_tiles);
    int t = tb + wv;
    // q rows 0..31 of the tile (zero past nq x heads) and their weights.
    for (int f = tid; f < kTileBlocks * 32; f += NT) {
        const int r = f >> 5, c = f & 31, qi = r / HP, h = r % HP;
        const bool ok = qi < a.nq && h < a.heads;
        const float4 v = ok ? reinterpret_cast<const float4 *>(a.q + ((int64_t)qi * a.heads + h) * kHeadDim)[c]
                            : make_float4(0.f, 0.f, 0.f, 0.f);
        *reinterpret_cast<float4 *>(&q_lds[r * kLdsRow + 4 * c]) = v;
    }
    if (tid < 32) {
        const int qi = tid / HP, h = tid % HP;
        w_lds[tid] = (qi < a.nq && h < a.heads) ? a.w[(int64_t)qi * a.heads + h] : 0.f;
    }
    __syncthreads();
    float4 qa4[16];
    {
        const float *src = q_lds + li * kLdsRow + 64 * half;
#pragma unroll
        for (int u = 0; u < 16; ++u)
            qa4[u] = *reinterpret_cast<const float4 *>(src + 4 * u);
    }

    for (; t < te; t += kLongWaves) {
        // Tile t's 32 key rows (16 KiB, consecutive in memory) through
        // registers: lane l takes float4 l + 64u, u < 16 (row (l + 64u) / 32,
        // part (l + 64u) % 32). Rows past the last block read block
        // n_blocks - 1 (their scores are not stored).
        float4 nxt[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            const int f = lane + 64 * u;
            const int b = min(t * kTileBlocks + (f >> 5), a.n_blocks - 1);
            nxt[u] = reinterpret_cast<const float4 *>(a.k + (int64_t)b * kHeadDim)[f & 31];
        }
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            const int f = lane + 64 * u;
            *reinterpret_cast<float4 *>(&k_lds[wv][(f >> 5) * kLdsRow + 4 * (f & 31)]) = nxt[u];
        }
        f32x16 acc[1];
#pragma unroll
        for (int v = 0; v < 16; ++v)
            acc[0][v] = 0.f;
        const float *kb = &k_lds[wv][li * kLdsRow + 64 * half];
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            const float4 b = *reinterpret_cast<const float4 *>(kb + 4 * u);
            acc[0] = __builtin_amdgcn_mfma_f32_32x32x2f32(qa4[u].x, b.x, acc[0], 0, 0, 0);
            acc[0] = __builtin_amdgcn_mfma_f32_32x32x2f32(qa4[u].y, b.y, acc[0], 0, 0, 0);
            acc[0] = __builtin_amdgcn_mfma_f32_32x32x2f32(qa4[u].z, b.z, acc[0], 0, 0, 0);
            acc[0] = __builtin_amdgcn_mfma_f32_32x32x2f32(qa4[u].w, b.w, acc[0], 0, 0, 0);
        }
        score_epilogue<HP, 1>(
            acc, a, 0, 0, half, t * kTileBlocks + li,
            [&](int, int v) { return w_lds[8 * (v >> 2) + 4 * half + (v & 3)]; },
            [&](int q, int b, float x) { a.scores[(int64_t)q * a.ld + b] = x; });
    }
}

template <int HP>
hipError_t launch_longrow(const ScoreArgs &a, hipStream_t s)
{
    const int n_tiles = (a.n_blocks + kTileBlocks - 1) / kTileBlocks;
    // Up to 256 workgroups (one per CU), each a multiple of 8 tiles.
    const int per_wave = (n_tiles + 256 * kLongWaves - 1) / (256 * kLongWaves);
    const int tiles_per_wg = per_wave * kLongWaves;
    const int wgs = (n_tiles + tiles_per_wg - 1) / tiles_per_wg;
    hipLaunchKernelGGL((scores_longrow_kernel<HP>), dim3((unsigned)wgs), dim3(kLongWaves * 64), 0, s, a, n_tiles,
                       tiles_per_wg);
    return hipGetLastError();
}

template <int HP, int MR, int NW, bool BF16>
hipError_t launch_cfg(const ScoreArgs &a, hipStream_t s)
{
    constexpr int ROWS = NW * MR * 32;
    // One 8- or 16-wave workgroup per CU. With fewer rows than a 16-wave slab,
    // two 8-wave workgroups would fit a CU, but half as many of them, each
    // taking twice the key tiles, measured faster (16 queries x 16 heads x
    // 65,536 blocks: 45.0 -> 40.3 us FP32, 10.9 -> 10.1 us BF16): each
    // workgroup loads its slab's q rows once, and that prologue is a large
    // share of a short one. Four-wave workgroups (64 heads) go two per CU.
    constexpr int RESIDENT = NW >= 8 ? 256 : 512;
    ScoreGrid g;
    const int64_t rows = (int64_t)a.nq * HP;
    g.n_slabs = (int32_t)((rows + ROWS - 1) / ROWS);
    g.n_tiles = (a.n_blocks + kTileBlocks - 1) / kTileBlocks;
    // About RESIDENT workgroups cover the chip once.
    int groups = (int)((RESIDENT + g.n_slabs - 1) / g.n_slabs);
    groups = groups < 1 ? 1 : groups;
    groups = groups > g.n_tiles ? g.n_tiles : groups;
    g.tiles_per_group = (g.n_tiles + groups - 1) / groups;
    groups = (g.n_tiles + g.tiles_per_group - 1) / g.tiles_per_group;
    g.xcd_map = (groups % 8 == 0) ? 1 : 0;
    g.n_groups = groups;
    const int64_t wgs = (int64_t)g.n_slabs * groups;
    if (wgs > 0x7fffffff)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL((scores_kernel<HP, MR, NW, BF16>), dim3((unsigned)wgs), dim3(NW * 64), 0, s, a, g);
    return hipGetLastError();
}

// 64 heads: a wave holds a whole query (two 32-row tiles). Otherwise each
// wave holds one 32-row tile (a quarter of the VGPRs, four waves per SIMD);
// many rows take 16-wave workgroups, one per CU, which halves the key tiles
// each CU stages and the key traffic from L2 (BF16 with 8 or more heads:
// 8-wave workgroups of two row tiles per wave, the same 512-row slabs); few
// rows take 8-wave workgroups (as do 1 or 2 heads), whose 256 rows match the
// decode shapes.
template <int HP, bool BF16>
hipError_t launch_hp(const ScoreArgs &a, hipStream_t s)
{
    if constexpr (HP == 64) {
        return launch_cfg<HP, 2, 4, BF16>(a, s);
    } else {
        const int64_t rows = (int64_t)a.nq * HP;
        if constexpr (!BF16) {
            if (rows <= 32 && a.n_blocks >= kLongMinTiles * kTileBlocks)
                return launch_longrow<HP>(a, s);
        }
        if constexpr (HP >= 4) {  // 1 or 2 heads: the epilogue's partial sums need more VGPRs
            if (rows >= 16 * 512) {
                // BF16 with 8 or more heads: eight-wave workgroups of two row
                // tiles per wave (the same 512-row slabs), so each key-tile
                // operand read from LDS feeds two matrix steps (C5 239 -> 226
                // us); FP32 keeps one row tile per wave (its operand reads are
                // a quarter as frequent per cycle, and q takes 64 VGPRs a tile).
                if constexpr (BF16 && HP >= 8)
                    return launch_cfg<HP, 2, 8, BF16>(a, s);
                else
                    return launch_cfg<HP, 1, 16, BF16>(a, s);
            }
        }
        return launch_cfg<HP, 1, 8, BF16>(a, s);
    }
}

template <bool BF16>
hipError_t launch_heads(const ScoreArgs &a, hipStream_t s)
{
    const int h = a.heads;
    if (h <= 1) return launch_hp<1, BF16>(a, s);
    if (h <= 2) return launch_hp<2, BF16>(a, s);
    if (h <= 4) return launch_hp<4, BF16>(a, s);
    if (h <= 8) return launch_hp<8, BF16>(a, s);
    if (h <= 16) return launch_hp<16, BF16>(a, s);
    if (h <= 32) return launch_hp<32, BF16>(a, s);
    if (h <= 64) return launch_hp<64, BF16>(a, s);
    return hipErrorInvalidValue;
}

} // namespace

hipError_t launch_scores(const ScoreArgs &a, hipStream_t s) { return launch_heads<false>(a, s); }

hipError_t launch_scores_bf16(const ScoreArgs &a, hipStream_t s) { return launch_heads<true>(a, s); }

} // namespace qsa
