// topk_select.h - per-query pieces of the block top-k shared by the one-read
// kernel and the two-launch filtered split (gfx950): the query's geometry,
// the sampled lower bound and the exact selection over a candidate list.
//
// These run once per workgroup and launch, so their instructions come from a
// cold instruction cache every time: loops stay rolled and each piece has one
// code path, which keeps the bytes fetched (and the time they take) small.
//
// The rule (Strata pull #3987, section Approach; Strata pull #2093 "sm_75:
// the prompt path's top-k with one full read of the scores", section
// Beschreibung): with r the blocks a selection touches, T is the r-th largest
// block key; blocks above T are taken, then blocks equal to T in ascending
// block order until r blocks are taken, the last of them possibly only in
// part.
#pragma once

#include "qsa_internal.h"
#include "topk_device.h"

namespace qsa {

struct QuerySel {
    int n_vis;      // visible blocks
    int wq;         // cells selected: min(width, visible cells)
    int r;          // blocks the selection touches, every block taken whole
    int last_unit;  // cells of the last block in (key desc, block asc) order
    int tail;       // cells of the last visible block when it is partial, else 0
};

// r and last_unit of a selection of w cells from whole blocks of bs cells.
__device__ __forceinline__ void set_width(QuerySel &s, int w, int bs)
{
    s.r = (w + bs - 1) / bs;
    s.last_unit = s.r > 0 ? w - bs * (s.r - 1) : 0;
}

// n_blocks * bs < 2^31 (checked on the host), so cell counts fit in int.
__device__ __forceinline__ QuerySel query_sel(const TopkGeom &g, int q)
{
    QuerySel s;
    int cells;
    if (g.cells) {
        const int all = g.n_blocks * g.bs;
        const int c = g.cells[q];
        cells = c < 0 ? 0 : (c > all ? all : c);
        s.n_vis = (cells + g.bs - 1) / g.bs;
        s.tail = cells - (s.n_vis - 1) * g.bs;
        s.tail = s.tail == g.bs ? 0 : s.tail;
    } else {
        int nv = g.n_blocks;
        if (g.active) {
            const int a = g.active[q];
            nv = a < 0 ? 0 : (a > g.n_blocks ? g.n_blocks : a);
        }
        s.n_vis = nv;
        s.tail = 0;
        cells = nv * g.bs;
    }
    s.wq = cells < g.width ? cells : g.width;
    set_width(s, s.wq, g.bs);
    return s;
}

// Visible cells of the query (the last visible block may be partial).
__device__ __forceinline__ int64_t visible_cells(const QuerySel &qs, int bs)
{
    return (int64_t)qs.n_vis * bs - (qs.tail != 0 ? bs - qs.tail : 0);
}

// A partial last visible block p (qs.tail cells). Counted as a whole block,
// p is the last of the blocks with its key in (key desc, block asc) order, so
// whole-block cells precede it exactly for the n_ge - 1 other blocks with key
// >= key(p). If fewer than wq such cells precede it, p is taken, and the
// selection is the whole-block selection of wq + bs - tail cells cut to its
// first wq cells in cell order (p's cells past the visible ones are the
// highest ids); otherwise p is not taken and the whole-block selection of wq
// cells is the selection. Every emit writes at most qs.wq cells.
__device__ __forceinline__ void widen_for_tail(QuerySel &qs, int bs, uint32_t n_ge)
{
    if (qs.tail != 0 && n_ge >= 1 && (int64_t)(n_ge - 1) * bs < qs.wq)
        set_width(qs, qs.wq + bs - qs.tail, bs);
}

// Cells 0 .. first-1, then -1 up to the width, and the count. This is the
// whole selection when every visible cell is selected, and when every visible
// block has the same key (ties go to the lowest cells).
template <int NT>
__device__ __forceinline__ void write_first_cells(const TopkGeom &g, int q, int first)
{
    int32_t *out = g.ids + (int64_t)q * g.width;
#pragma unroll 1
    for (int p = threadIdx.x; p < g.width; p += NT)
        out[p] = p < first ? p : -1;
    if (g.counts && threadIdx.x == 0)
        g.counts[q] = first;
}

// The sample of a row of n blocks for the lower bound (Strata pull #2093,
// section Beschreibung, step 1: every 32nd block, and KS = 2*r/32 + 16).
// QSA_SAMPLE_STRIDE takes every (32*P)-th block; QSA_SAMPLE_LINES takes 32
// consecutive blocks (one 128-byte line) out of every 1,024*P. P is 1 up to
// 131,072 blocks; longer rows take a proportionally sparser sample of at most
// 4,096 keys spread over the whole row, and KS = 2*r/(32*P) + 16 keeps the
// expected number of blocks above the bound where it is for P = 1.
struct SampleGeom {
    int ns;         // samples
    int period;     // P
    uint32_t ks;    // rank of the bound among the samples
    int stride;     // 1: every (32*P)-th block; 0: lines
};

__device__ __forceinline__ SampleGeom sample_geom(int n, int r, int mode)
{
    SampleGeom s;
    s.stride = mode == QSA_SAMPLE_STRIDE ? 1 : 0;
    if (n <= kSampleStride * kOneReadSample) {
        // Rows of up to 131,072 blocks: the pages' rate, no division.
        s.period = 1;
        s.ns = s.stride ? (n + kSampleStride - 1) / kSampleStride
                        : (n >> 10) * kSampleStride + min(n & 1023, kSampleStride);
    } else if (s.stride) {
        const int pts = (n + kSampleStride - 1) / kSampleStride;
        s.period = (pts + kOneReadSample - 1) / kOneReadSample;
        const int step = kSampleStride * s.period;
        s.ns = (n + step - 1) / step;
    } else {
        const int groups = (n + 1023) / 1024;
        s.period = (groups + kOneReadSample / kSampleStride - 1) / (kOneReadSample / kSampleStride);
        const int gstep = 1024 * s.period;
        const int used = (n + gstep - 1) / gstep;
        s.ns = (used - 1) * kSampleStride + min(kSampleStride, n - (used - 1) * gstep);
    }
    s.ks = (s.period == 1 ? (2u * (uint32_t)r) / (uint32_t)kSampleStride
                          : 2u * (uint32_t)r / (uint32_t)(kSampleStride * s.period)) + 16u;
    return s;
}

// Block index of sample i (selects, no branch: the loads stay unconditional).
__device__ __forceinline__ int sample_block(const SampleGeom &s, int i)
{
    const int group = s.stride ? i : i / kSampleStride;
    const int within = s.stride ? 0 : i % kSampleStride;
    const int gap = (s.stride ? kSampleStride : 1024) * s.period;
    return group * gap + within;
}

// Sampled lower bound (Strata pull #2093, section Beschreibung, step 1: the
// KS-th largest key of a sample of the row). Here: 2,048 bins of equal value
// width over the sample's [min, max], and the bound is the lower edge of the
// bin that holds the KS-th largest sample value, so at least KS samples lie at
// or above it. Any bound gives the exact ids (the candidates are checked
// afterwards), so this only steers how many blocks are kept. The result
// depends only on the sample's values, so every workgroup that samples the
// same row computes the same bound. Sample u of this thread is index
// threadIdx.x + u*NT, valid below ns. Uses sh.red, sh.fine and sh.coarse
// (zero on entry) and leaves the fine and coarse bins dirty: a caller that
// needs them again clears them after its next barrier.
template <int NT, int SPT>
__device__ __forceinline__ float bound_from_sample(const float (&smp)[SPT], int ns, uint32_t ks, SelectShared &sh)
{
    uint32_t klo = 0xFFFFFFFFu, khi = 0u;
#pragma unroll
    for (int u = 0; u < SPT; ++u) {
        const bool in = (int)threadIdx.x + u * NT < ns;
        const uint32_t k = key_of(smp[u]);
        klo = in ? min(klo, k) : klo;
        khi = in ? max(khi, k) : khi;
    }
    uint32_t mn, mx;
    wg_minmax<NT>(klo, khi, sh, mn, mx);
    const float lo = float_of(mn), hi = float_of(mx);
    // Halved operands keep the width finite for any finite range.
    const float lh = 0.5f * lo, d2 = 0.5f * hi - lh;
    const float inv = (float)kFineBins / d2;
    if (!(d2 > 0.0f) || !(inv < __builtin_inff()))
        return lo;  // every sample equal (or too close to cut): keep what is >= them
#pragma unroll
    for (int u = 0; u < SPT; ++u) {
        if ((int)threadIdx.x + u * NT < ns) {
            const uint32_t fb = value_fine_bin(key_of(smp[u]), lh, inv);
            lds_add(&sh.fine[fb], 1u);
            lds_add(&sh.coarse[fb / kFinePerCoarse], 1u);
        }
    }
    lds_barrier();
    // One wave picks (the others would only repeat its work on the same
    // SIMDs) and hands the bound to the rest.
    if (wave_id() == 0) {
        uint32_t fb, c, h;
        pick_fine<NT>(sh, ks, fb, c, h);
        // The bin's lower edge. Rounding may put a sample of the bin just
        // below it; that only drops that block from the candidates.
        if (lane_id() == 0)
            sh.bcast = __float_as_uint(2.0f * (lh + (float)fb * (d2 * (1.0f / (float)kFineBins))));
    }
    lds_barrier();
    return __uint_as_float(sh.bcast);
}

// The fine bin of a candidate key: the top kFineBits bits of key - kmin over
// a span of kmax - kmin.
__device__ __forceinline__ int cand_fine_shift(uint32_t span)
{
    return span != 0 ? max(0, (32 - __clz(span)) - kFineBits) : 0;
}

// The exact selection over `total` candidate blocks held in LDS in ascending
// block order (keys ck, block indices cb) that contain the query's whole
// selection, every key in [kmin, kmax]: writes the cells, the -1 tail and the
// count. On entry (after the caller's barrier) every candidate is counted in
// sh.fine/coarse with bins of cand_fine_shift(kmax - kmin), sh.small_n is zero
// and qs is already widened for a partial last block. Each thread holds the
// candidates [per*t, per*t + per) in registers from the start (per =
// ceil(total / NT) <= kOneReadCap / NT; slots past per are skipped as a whole):
// the threshold's gather and the emit use them without another pass over the
// LDS, and every wave holds a share.
template <int NT>
__device__ __forceinline__ void select_from_candidates(const uint32_t *ck, const int32_t *cb, int total, uint32_t kmin,
                                                       uint32_t kmax, const QuerySel &qs, const TopkGeom &g, int q,
                                                       SelectShared &sh)
{
    constexpr int NW = NT / kWave;
    static_assert(NW <= 16 && (NW & (NW - 1)) == 0, "wave totals fit one row of lanes");
    constexpr int PER = kOneReadCap / NT;
    const int lane = lane_id(), wid = wave_id();
    const uint32_t span = kmax - kmin;
    const int sF = cand_fine_shift(span);
    const int per = (total + NT - 1) / NT;
    // Slots j >= per (a workgroup-uniform bound) are never read.
    uint32_t k[PER];
    int32_t blk[PER];
    bool v[PER];
    const int c0 = (int)threadIdx.x * per;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        if (j >= per)
            break;
        v[j] = c0 + j < total;
        const int i = v[j] ? c0 + j : 0;
        k[j] = ck[i];
        blk[j] = cb[i];
    }

    // Threshold: the fine bin holding rank r usually holds a handful of keys,
    // which one wave ranks exactly; a crowded one goes on with radix digits
    // over its keys. The tail's time is mostly instruction issue, shared by
    // the four waves of each SIMD, so work that does not depend on a wave's
    // own candidates runs in one wave and is handed on through LDS.
    uint32_t T = kmin, above = 0;
    if (span != 0) {
        if (wid == 0) {
            uint32_t pb, pc, ph;
            pick_fine<NT>(sh, (uint32_t)qs.r, pb, pc, ph);
            if (lane == 0)
                *reinterpret_cast<uint4 *>(sh.pick) = make_uint4(pb, pc, ph, 0u);
        }
        lds_barrier();
        const uint4 pk = *reinterpret_cast<const uint4 *>(sh.pick);
        const uint32_t b = (uint32_t)__builtin_amdgcn_readfirstlane((int)pk.x);
        const uint32_t c = (uint32_t)__builtin_amdgcn_readfirstlane((int)pk.y);
        const uint32_t h = (uint32_t)__builtin_amdgcn_readfirstlane((int)pk.z);
        const uint32_t blo = kmin + (b << sF);
        const uint32_t bspan = sF == 0 ? 0u : min(span - (b << sF), (1u << sF) - 1u);
        const uint32_t r2 = (uint32_t)qs.r - h;
        uint32_t a2 = 0;
        if (bspan == 0) {
            T = blo;
        } else if (c <= (uint32_t)kWave) {
#pragma unroll
            for (int j = 0; j < PER; ++j) {
                if (j < per && v[j] && k[j] - blo <= bspan) {
                    const uint32_t pos =
                        __hip_atomic_fetch_add(&sh.small_n, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
                    if (pos < (uint32_t)kWave)
                        sh.small[pos] = k[j];
                }
            }
            lds_barrier();
            // One wave ranks the bin's keys and hands (T, above) on.
            if (wid == 0) {
                uint32_t t0, a0;
                wave_rank_small(sh.small, c, r2, t0, a0);
                if (lane == 0)
                    *reinterpret_cast<uint2 *>(sh.pick) = make_uint2(t0, a0);
            }
            lds_barrier();
            const uint2 ta = *reinterpret_cast<const uint2 *>(sh.pick);
            T = (uint32_t)__builtin_amdgcn_readfirstlane((int)ta.x);
            a2 = (uint32_t)__builtin_amdgcn_readfirstlane((int)ta.y);
        } else {
            // Digits over the bin's interval (sh.hist; the fine bins stay as they are).
            radix_select_range<NT>(LdsKeys{ck}, total, r2, blo, blo + bspan, sh, T, a2);
        }
        above = h + a2;
    }

    // Emit: one workgroup scan of (blocks above T, blocks equal to T) in block
    // order gives every taken block its output slot: bs cells per taken block,
    // except the last tie taken (rank budget - 1), which takes last_unit cells
    // and moves every later block down.
    const uint32_t budget = (uint32_t)qs.r - above;  // >= 1
    uint32_t gt = 0, tie = 0;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        if (j < per) {  // workgroup-uniform
            gt += v[j] && k[j] > T ? 1u : 0u;
            tie += v[j] && k[j] == T ? 1u : 0u;
        }
    }
    const uint32_t packed = gt | (tie << 16);  // both <= kOneReadCap < 2^16
    const uint32_t incl = wave_incl_sum(packed);
    if (lane == kWave - 1)
        sh.red[0][wid] = incl;
    lds_barrier();
    // The packed totals of the waves before this one: lane w < NW reads
    // wave w's, and one row sum adds them.
    uint32_t before = incl - packed + row0_sum(lane < wid ? sh.red[0][lane & (NW - 1)] : 0u);
    uint32_t ties_before = before >> 16;
    const uint32_t bs = (uint32_t)g.bs;
    const uint32_t shortfall = bs - (uint32_t)qs.last_unit;
    const uint32_t limit = (uint32_t)qs.wq;
    int32_t *out = g.ids + (int64_t)q * g.width;
    uint32_t pos = bs * ((before & 0xFFFFu) + min(ties_before, budget)) - (ties_before >= budget ? shortfall : 0u);
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        if (j >= per)  // workgroup-uniform
            break;
        uint32_t cells = 0;
        if (v[j] && k[j] > T) {
            cells = bs;
        } else if (v[j] && k[j] == T) {
            if (ties_before < budget)
                cells = ties_before == budget - 1u ? (uint32_t)qs.last_unit : bs;
            ++ties_before;
        }
        if (cells != 0u) {
            write_cells(out, pos, cells, blk[j] * (int32_t)bs, limit);
            pos += cells;
        }
    }
#pragma unroll 1
    for (int p = qs.wq + (int)threadIdx.x; p < g.width; p += NT)
        out[p] = -1;
    if (g.counts && threadIdx.x == 0)
        g.counts[q] = qs.wq;
}

// Counts candidate key k into the fine bins of select_from_candidates.
__device__ __forceinline__ void count_candidate(uint32_t k, uint32_t kmin, int sF, SelectShared &sh)
{
    const uint32_t fb = (k - kmin) >> sF;
    lds_add(&sh.fine[fb], 1u);
    lds_add(&sh.coarse[fb / kFinePerCoarse], 1u);
}

// qs widened for a partial last block from per-wave counts of candidates at
// or above its key (sh.red[1], written before the caller's barrier). kmin is
// the candidates' lower bound: the block is a candidate iff its key is >= it,
// and then every block at or above its key is one; if it is not, it is below
// the threshold (the candidates hold the widened selection's cells).
template <int NT>
__device__ __forceinline__ void widen_from_counts(QuerySel &qs, int bs, uint32_t kp, uint32_t kmin,
                                                  const SelectShared &sh)
{
    if (qs.tail == 0)
        return;
    uint32_t n_ge = 0;
#pragma unroll
    for (int w = 0; w < NT / kWave; ++w)
        n_ge += sh.red[1][w];
    widen_for_tail(qs, bs, kp >= kmin ? n_ge : 0xFFFFFFFFu);
}

// Writes a query's selection from n candidate blocks in ascending block order
// that contain it, given T (the r-th largest candidate key) and the number of
// candidates above T: the cells, the -1 tail and the count.
template <int NT, class Src, class BlockAt>
__device__ __forceinline__ void emit_selection(const Src &src, int n, const QuerySel &qs, BlockAt block_at,
                                               const TopkGeom &g, int q, SelectShared &sh, uint32_t T,
                                               uint32_t above)
{
    int32_t *out = g.ids + (int64_t)q * g.width;
    const int bs = g.bs;
    const uint32_t limit = (uint32_t)qs.wq;
    take_ordered<NT>(src, n, T, (uint32_t)qs.r - above, (uint32_t)bs, (uint32_t)qs.last_unit, sh,
                     [&](int i, uint32_t first, uint32_t cnt) {
                         write_cells(out, first, cnt, block_at(i) * bs, limit);
                     });
    for (int p = qs.wq + (int)threadIdx.x; p < g.width; p += NT)
        out[p] = -1;
    if (g.counts && threadIdx.x == 0)
        g.counts[q] = qs.wq;
}

// Final selection over n candidate blocks (n >= qs.r) that contain the
// query's whole selection, in ascending block order: writes the cells, the -1
// tail and the count. Histograms must be zero on entry.
template <int NT, class Src, class BlockAt>
__device__ __forceinline__ void select_cells(const Src &src, int n, const QuerySel &qs, BlockAt block_at,
                                             const TopkGeom &g, int q, SelectShared &sh)
{
    uint32_t T, above;
    radix_select<NT>(src, n, (uint32_t)qs.r, sh, T, above);
    emit_selection<NT>(src, n, qs, block_at, g, q, sh, T, above);
}

// select_cells when the keys' range [mn, mx] is already known.
template <int NT, class Src, class BlockAt>
__device__ __forceinline__ void select_cells_in(const Src &src, int n, uint32_t mn, uint32_t mx, const QuerySel &qs,
                                                BlockAt block_at, const TopkGeom &g, int q, SelectShared &sh)
{
    uint32_t T, above;
    radix_select_in<NT>(src, n, (uint32_t)qs.r, mn, mx, sh, T, above);
    emit_selection<NT>(src, n, qs, block_at, g, q, sh, T, above);
}

// The exact rule over a whole row of n blocks with one read of it, for a
// query whose sampled bound failed: the chunked split's two stages inside one
// workgroup (Strata pull #3987, section Approach). The row passes through LDS
// in chunks of CH blocks (s_chunk, CH words). With r_a = r, or r + 1 when the
// last visible block is partial (widen_for_tail), each chunk appends to the
// candidate list, in block order, its own first r_a blocks in (key desc,
// block asc) order among those at or above the bound lo. A block of the
// selection has fewer than r_a blocks ahead of it in the whole row, hence in
// any part of it, so it is kept. When the list reaches 2*r_a entries, or the
// next chunk could overflow it, the list keeps its own first r_a (the same
// argument) and lo becomes one above the r_a-th key among them: a later block
// with a key at or below that key has those r_a blocks ahead of it. The first
// chunk that keeps r_a blocks into an empty list sets lo the same way. The
// selection is then made over the list, which holds every selected block and
// every block whose key is at or above a partial last block's key kp when
// that block is taken (fewer than r_a blocks are ahead of each of them), so
// its count of such keys decides the widening as the whole row would (if the
// block is not taken, the list holds r_a keys at or above kp either way).
// Needs 2 * r_a <= min(cap, CH); s_ckey and s_cblk hold cap entries; the
// histograms must be zero on entry. VEC: the row may be read in 16-byte
// groups up to n rounded up to a multiple of 4.
template <int NT, int CH, bool VEC>
__device__ __forceinline__ void select_row_chunked(const float *row, int n, QuerySel qs, uint32_t kp,
                                                   uint32_t *s_chunk, uint32_t *s_ckey, int32_t *s_cblk,
                                                   int cap, const TopkGeom &g, int q, SelectShared &sh)
{
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    constexpr int G = CH / (4 * NT);  // 4-key groups per thread and chunk
    static_assert(G >= 1 && G * 4 * NT == CH, "a chunk is whole 4-key groups per thread");
    const uint32_t r_a = (uint32_t)(qs.r + (qs.tail != 0 ? 1 : 0));
    // Loads at or past the resource's end read zero without a memory access.
    const __amdgpu_buffer_rsrc_t rr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float *>(row), (short)0, (VEC ? ((n + 3) & ~3) : n) * 4, kRowBufferWord3);
    uint32_t ncand = 0;  // uniform
    uint32_t lo = 0u;    // keys below lo cannot be selected
#pragma unroll 1
    for (int b0 = 0; b0 < n; b0 += CH) {
        const int nc = min(CH, n - b0);
        // The chunk's keys into LDS, every load issued before any is used,
        // counting the keys at or above lo on the way.
        uint32_t k[G][4];
#pragma unroll
        for (int j = 0; j < G; ++j) {
            const int i = 4 * ((int)threadIdx.x + NT * j);
            if constexpr (VEC) {
                const u32x4 v = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rr, 4 * (b0 + i), 0, 0));
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    k[j][e] = v[e];
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    k[j][e] = __builtin_amdgcn_raw_buffer_load_b32(rr, 4 * (b0 + i + e), 0, 0);
            }
        }
        uint32_t cnt = 0;
#pragma unroll
        for (int j = 0; j < G; ++j) {
            const int i = 4 * ((int)threadIdx.x + NT * j);
            uint32_t kk[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                kk[e] = key_of(__uint_as_float(k[j][e]));
                cnt += (i + e < nc && kk[e] >= lo) ? 1u : 0u;
            }
            if (i + 3 < nc) {
                *reinterpret_cast<uint4 *>(s_chunk + i) = make_uint4(kk[0], kk[1], kk[2], kk[3]);
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (i + e < nc)
                        s_chunk[i + e] = kk[e];
            }
        }
        const uint32_t c_ge = wg_sum<NT>(cnt, sh);  // its barriers order the stores before the reads
        const LdsKeys chunk{s_chunk};
        // Every key at or above lo (the first nc ties at lo are all of them),
        // or the chunk's own first r_a when more pass.
        uint32_t T = lo, budget = (uint32_t)nc, taken = c_ge;
        if (c_ge > r_a) {
            uint32_t above;
            radix_select<NT>(chunk, nc, r_a, sh, T, above);
            budget = r_a - above;
            taken = r_a;
        }
        if (taken != 0) {
            uint32_t *ck = s_ckey + ncand;
            int32_t *cb = s_cblk + ncand;
            ordered_take<NT>(chunk, nc, T, budget, 1u, 1u, sh, [&](int i, uint32_t pos, uint32_t) {
                ck[pos] = s_chunk[i];
                cb[pos] = b0 + i;
            });
        }
        // A list that was empty now holds the first r_a blocks of the row so
        // far: its r_a-th key bounds the rest as a cut-back list's does.
        if (ncand == 0 && c_ge > r_a)
            lo = T != 0xFFFFFFFFu ? T + 1u : T;
        ncand += taken;
        lds_barrier();  // the list is written; the chunk buffer is free
        if (b0 + CH < n && (ncand >= 2 * r_a || ncand + r_a > (uint32_t)cap)) {
            const LdsKeys list{s_ckey};
            uint32_t above;
            radix_select<NT>(list, (int)ncand, r_a, sh, T, above);
            ordered_take<NT>(list, (int)ncand, T, r_a - above, 1u, 1u, sh, [&](int i, uint32_t pos, uint32_t) {
                s_chunk[pos] = s_ckey[i];
                s_chunk[CH / 2 + pos] = (uint32_t)s_cblk[i];
            });
            lds_barrier();
            for (int i = threadIdx.x; i < (int)r_a; i += NT) {
                s_ckey[i] = s_chunk[i];
                s_cblk[i] = (int32_t)s_chunk[CH / 2 + i];
            }
            ncand = r_a;
            lo = T != 0xFFFFFFFFu ? T + 1u : T;
            lds_barrier();
        }
    }
    const LdsKeys list{s_ckey};
    if (qs.tail != 0)
        widen_for_tail(qs, g.bs, count_at_least<NT>(list, (int)ncand, kp, sh));
    uint32_t T, above;
    radix_select<NT>(list, (int)ncand, (uint32_t)qs.r, sh, T, above);
    // The emit of select_cells, with the rolled walk (this runs rarely, and
    // its code shares the instruction cache with the common path's).
    int32_t *out = g.ids + (int64_t)q * g.width;
    const uint32_t limit = (uint32_t)qs.wq;
    ordered_take<NT>(list, (int)ncand, T, (uint32_t)qs.r - above, (uint32_t)g.bs, (uint32_t)qs.last_unit, sh,
                     [&](int i, uint32_t first, uint32_t cnt) { write_cells(out, first, cnt, s_cblk[i] * g.bs, limit); });
    for (int p = qs.wq + (int)threadIdx.x; p < g.width; p += NT)
        out[p] = -1;
    if (g.counts && threadIdx.x == 0)
        g.counts[q] = qs.wq;
}

} // namespace qsa
