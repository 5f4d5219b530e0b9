// select_fused.hip - one launch for a small decode-call selection (gfx950).
//
// Scores of short rows and their top-k in one kernel (the scorer of Strata
// pull #1091, section What, then the selection rule of Strata pull #3987,
// section Approach). Decode calls carry few queries and, early in a
// context, few blocks; two launches (scores, then top-k) then cost more than
// the work. Here:
//  * every workgroup scores one or more key tiles of 32 blocks for all the
//    call's queries (the FP32 matrix-core contraction of scores_device.h) and
//    stores the scores with device-coherent (sc1) stores into the caller's
//    score matrix;
//  * each thread waits for its stores, and the workgroup takes one ticket;
//  * the workgroup that arrives last selects: wave w takes query w, holds
//    the query's block keys in registers (lane l: blocks [l*KPL, l*KPL+KPL)),
//    finds the threshold with radix digits over the keys' own range in a
//    histogram of its own in LDS, and writes the cells in block order from
//    one wave scan of (blocks above T, blocks equal to T).
// No device-scope fences (see the hand-off notes in topk_device.h). Rows up to
// kFusedMaxBlocks blocks, up to 16 queries (one wave each) and 32 heads.
#include "scores_device.h"
#include "topk_device.h"

namespace qsa {

namespace {

constexpr int kFusedKpl = kFusedMaxBlocks / kWave;  // keys per lane, at most

// One wave: the rank-th largest (1-based) of the valid keys k[j] (v[j]) held
// by the wave, and how many of them lie above it. hist is the wave's own
// 256-bin LDS histogram (any contents on entry). Digits are taken over the
// keys' own range, as in radix_select_range.
__device__ __forceinline__ void wave_select(const uint32_t (&k)[kFusedKpl], const bool (&v)[kFusedKpl],
                                            uint32_t rank, uint32_t *hist, uint32_t &T, uint32_t &n_above)
{
    const int lane = lane_id();
    uint32_t lo = 0xFFFFFFFFu, hi = 0u;
#pragma unroll
    for (int j = 0; j < kFusedKpl; ++j) {
        lo = v[j] ? min(lo, k[j]) : lo;
        hi = v[j] ? max(hi, k[j]) : hi;
    }
    lo = wave_min(lo);
    hi = wave_max(hi);
    uint32_t span = hi - lo, r = rank, above = 0;
    while (span != 0) {
        const int s = first_digit_shift(span);
#pragma unroll
        for (int i = 0; i < kBins / kWave; ++i)
            hist[lane + kWave * i] = 0u;
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
#pragma unroll
        for (int j = 0; j < kFusedKpl; ++j) {
            const uint32_t sub = k[j] - lo;
            if (v[j] && sub <= span)
                lds_add(&hist[sub >> s], 1u);
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
        uint32_t d, h;
        wave_pick(hist, r, d, h);
        r -= h;
        above += h;
        lo += d << s;
        span = (s == 0) ? 0u : min(span - (d << s), (1u << s) - 1u);
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
        __builtin_amdgcn_wave_barrier();  // every lane has read the bins before the next clear
    }
    T = lo;
    n_above = above;
}

template <int HP, int NW>
__global__ __launch_bounds__(NW * 64) void select_fused_kernel(FusedArgs a)
{
    constexpr int ROWS = NW * 32;
    __shared__ ScoreLds<ROWS> sm;
    __shared__ __attribute__((aligned(16))) uint32_t s_hist[NW][kBins];
    __shared__ uint32_t s_flag[1];

    // Scores of this workgroup's tiles, stored device-coherent.
    const ScoreArgs &sa = a.s;
    const int t0 = blockIdx.x * a.tiles_per_group;
    const int t1 = min(t0 + a.tiles_per_group, a.n_tiles);
    score_tiles<HP, 1, NW>(sa, 0, t0, t1, sm, [&](int qi, int blk, float s) {
        store_dev(reinterpret_cast<uint32_t *>(sa.scores + (int64_t)qi * sa.ld + blk), __float_as_uint(s));
    });
    if (!last_to_arrive(a.ticket, gridDim.x, s_flag))
        return;
    if (threadIdx.x == 0)
        store_dev(a.ticket, 0u);  // zero again for the next call

    // Selection: wave w takes queries w, w + NW, ...
    const int lane = lane_id(), wid = wave_id();
    const int n = sa.n_blocks;
    const int bs = a.bs;
    const int64_t cells = (int64_t)n * bs;
    const int wq = (int)(cells < a.width ? cells : (int64_t)a.width);
    const int r = (wq + bs - 1) / bs;
    const int last_unit = wq - bs * (r - 1);
    const int kpl = (n + kWave - 1) / kWave;
    for (int qi = wid; qi < sa.nq; qi += NW) {
        // The row as a buffer: every load is issued unconditionally (loads
        // past the row return zero without a memory access), all in flight
        // at once, with the device-coherent (sc1) cache policy.
        const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
            sa.scores + (int64_t)qi * sa.ld, (short)0, n * 4, kBufferWord3);
        uint32_t k[kFusedKpl];
        bool v[kFusedKpl];
        const int b0 = lane * kpl;
#pragma unroll
        for (int j = 0; j < kFusedKpl; ++j)
            k[j] = __builtin_amdgcn_raw_buffer_load_b32(rsrc, (b0 + j) * 4, 0, kBufferDevice);
#pragma unroll
        for (int j = 0; j < kFusedKpl; ++j) {
            v[j] = j < kpl && b0 + j < n;
            k[j] = v[j] ? key_of(__uint_as_float(k[j])) : 0u;
        }
        // With r >= n every block is taken (T = 0 lies below every finite key).
        uint32_t T = 0, above = 0;
        if (r < n)
            wave_select(k, v, (uint32_t)r, s_hist[wid], T, above);
        const uint32_t budget = (uint32_t)r - above;
        uint32_t gt = 0, tie = 0;
#pragma unroll
        for (int j = 0; j < kFusedKpl; ++j) {
            gt += v[j] && k[j] > T ? 1u : 0u;
            tie += v[j] && k[j] == T ? 1u : 0u;
        }
        const uint32_t packed = gt | (tie << 16);
        const uint32_t incl = wave_incl_sum(packed);
        const uint32_t before = incl - packed;
        uint32_t ties_before = before >> 16;
        const uint32_t ubs = (uint32_t)bs, shortfall = ubs - (uint32_t)last_unit;
        int32_t *out = a.ids + (int64_t)qi * a.width;
        uint32_t pos = ubs * ((before & 0xFFFFu) + min(ties_before, budget)) - (ties_before >= budget ? shortfall : 0u);
#pragma unroll
        for (int j = 0; j < kFusedKpl; ++j) {
            uint32_t c = 0;
            if (v[j] && k[j] > T) {
                c = ubs;
            } else if (v[j] && k[j] == T) {
                if (ties_before < budget)
                    c = ties_before == budget - 1u ? (uint32_t)last_unit : ubs;
                ++ties_before;
            }
            if (c != 0u) {
                write_cells(out, pos, c, (b0 + j) * bs, (uint32_t)wq);
                pos += c;
            }
        }
        for (int p = wq + lane; p < a.width; p += kWave)
            out[p] = -1;
        if (a.counts && lane == 0)
            a.counts[qi] = wq;
    }
}

template <int HP>
hipError_t launch_hp(const FusedArgs &a, int nw, hipStream_t s)
{
    const dim3 grid((unsigned)((a.n_tiles + a.tiles_per_group - 1) / a.tiles_per_group));
    if (nw <= 4)
        hipLaunchKernelGGL((select_fused_kernel<HP, 4>), grid, dim3(4 * 64), 0, s, a);
    else if (nw <= 8)
        hipLaunchKernelGGL((select_fused_kernel<HP, 8>), grid, dim3(8 * 64), 0, s, a);
    else
        hipLaunchKernelGGL((select_fused_kernel<HP, 16>), grid, dim3(16 * 64), 0, s, a);
    return hipGetLastError();
}

} // namespace

bool fused_select_fits(int32_t nq, int32_t heads, int32_t n_blocks)
{
    if (nq < 1 || nq > kFusedMaxQueries || heads < 1 || heads > 32 || n_blocks < 1 || n_blocks > kFusedMaxBlocks)
        return false;
    int hp = 1;
    while (hp < heads)
        hp *= 2;
    return (int64_t)nq * hp <= 16 * 32;
}

hipError_t launch_fused_select(FusedArgs a, hipStream_t s)
{
    int hp = 1;
    while (hp < a.s.heads)
        hp *= 2;
    const int rows_waves = (a.s.nq * hp + 31) / 32;
    const int nw = rows_waves > a.s.nq ? rows_waves : a.s.nq;
    a.n_tiles = (a.s.n_blocks + kTileBlocks - 1) / kTileBlocks;
    a.tiles_per_group = 1;
    switch (hp) {
    case 1: return launch_hp<1>(a, nw, s);
    case 2: return launch_hp<2>(a, nw, s);
    case 4: return launch_hp<4>(a, nw, s);
    case 8: return launch_hp<8>(a, nw, s);
    case 16: return launch_hp<16>(a, nw, s);
    case 32: return launch_hp<32>(a, nw, s);
    default: return hipErrorInvalidValue;
    }
}

} // namespace qsa
