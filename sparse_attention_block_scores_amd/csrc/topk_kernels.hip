// topk_kernels.hip - block top-k kernels for gfx950.
//
//  * split_kernel + split_merge_kernel: the exact chunked split (Strata pull
//    #3987, section Approach), two launches. Stage A (split_kernel): one
//    workgroup per (query, chunk) loads the chunk's block keys into LDS once
//    and keeps the chunk's own top-r blocks, in block order, as candidates.
//    Every block of the query's selection is among the candidates of its
//    chunk: if a chunk held a selected block outside its own top r, r blocks
//    of that chunk would precede it in (key desc, block asc) order, and the
//    selection, which has r blocks, would not reach it. Stage B
//    (split_merge_kernel, one workgroup per query, launched after stage A on
//    the same stream so the kernel boundary orders the candidates' stores
//    before their loads) selects over the candidates of all chunks with the
//    same threshold rule and writes the cells. A row that fits one chunk is
//    finished by its single stage-A workgroup. Used for rows that fit one
//    chunk and for rows where a sampled bound would keep a large share of the
//    blocks.
//
//  * oneread_kernel: the prompt path with one read of the scores (Strata
//    pull #2093 "sm_75: the prompt path's top-k with one full read of the
//    scores", section Beschreibung), one workgroup per query. A lower bound LB
//    is the KS-th largest of a sample of the query's block keys
//    (KS = 2*r/32 + 16); one streaming pass keeps the blocks with key >= LB in
//    LDS, in block order. If they hold at least the selection's cells, the
//    threshold is >= LB and the rule over the candidates gives the exact
//    selection. Otherwise (too few cells, or more candidates than the cap) the
//    query takes the exact rule over its whole row in the same workgroup, as
//    the chunked split in one more read of the row (select_row_chunked).
//    Workgroups never talk to each other, so no device-scope fences are
//    needed.
#include <type_traits>

#include "qsa_internal.h"
#include "topk_device.h"
#include "topk_select.h"

namespace qsa {

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));



// Keys of blocks [b0, b0+n) of row q into LDS.
template <int NT>
__device__ __forceinline__ void load_keys_lds(const TopkGeom &g, int q, int b0, int n, uint32_t *s)
{
    const float *row = g.scores + (int64_t)q * g.ld + b0;
    if (g.vec4 && (b0 & 3) == 0) {
        const float4 *r4 = reinterpret_cast<const float4 *>(row);
        const int n4 = (n + 3) >> 2;
        for (int i = threadIdx.x; i < n4; i += NT) {
            const float4 v = r4[i];
            const int b = i << 2;
            if (b + 3 < n) {
                *reinterpret_cast<uint4 *>(s + b) = make_uint4(key_of(v.x), key_of(v.y), key_of(v.z), key_of(v.w));
            } else {
                s[b] = key_of(v.x);
                if (b + 1 < n) s[b + 1] = key_of(v.y);
                if (b + 2 < n) s[b + 2] = key_of(v.z);
            }
        }
    } else {
        for (int i = threadIdx.x; i < n; i += NT)
            s[i] = key_of(row[i]);
    }
}

} // namespace

// ------------------------------------------------------------------ split
template <int NT>
__global__ __launch_bounds__(NT) void split_kernel(SplitArgs a)
{
    extern __shared__ __attribute__((aligned(16))) uint32_t s_keys[];
    __shared__ SelectShared sh;
    const TopkGeom g = a.g;
    const int q = blockIdx.y;
    const int c = blockIdx.x;
    QuerySel qs = query_sel(g, q);
    if (qs.r == 0) {
        if (c == 0)
            write_first_cells<NT>(g, q, 0);
        return;
    }
    const int nchq = (qs.n_vis + a.chunk - 1) / a.chunk;
    if (c >= nchq)
        return;
    const int b0 = c * a.chunk;
    const int nc = min(a.chunk, qs.n_vis - b0);
    clear_hists<NT>(sh);
    load_keys_lds<NT>(g, q, b0, nc, s_keys);
    lds_barrier();
    const LdsKeys lds{s_keys};

    if (nchq == 1) {
        if (qs.tail != 0)
            widen_for_tail(qs, g.bs, count_at_least<NT>(lds, nc, s_keys[nc - 1], sh));
        select_cells<NT>(lds, nc, qs, [&](int i) { return b0 + i; }, g, q, sh);
        return;
    }

    // Stage A: this chunk's top-r_a blocks in block order. A query with a
    // partial last block keeps one block more: its selection may take one
    // more whole block (widen_for_tail), and with r_a = r + 1 the candidates
    // decide exactly whether that block is taken (stage B).
    const int r_a = qs.r + (qs.tail != 0 ? 1 : 0);
    const int cap_q = min(r_a, a.chunk);
    uint32_t *ckey = a.cand_keys + (int64_t)q * a.cand_stride + (int64_t)c * cap_q;
    int32_t *cblk = a.cand_blocks + (int64_t)q * a.cand_stride + (int64_t)c * cap_q;
    uint32_t T = 0, budget = (uint32_t)nc;  // a chunk no larger than r_a is kept whole
    if (nc > r_a) {
        uint32_t above;
        radix_select<NT>(lds, nc, (uint32_t)r_a, sh, T, above);
        budget = (uint32_t)r_a - above;
    }
    take_ordered<NT>(lds, nc, T, budget, 1u, 1u, sh, [&](int i, uint32_t pos, uint32_t) {
        if (pos < (uint32_t)cap_q) {
            ckey[pos] = s_keys[i];
            cblk[pos] = b0 + i;
        }
    });
}

// Stage B, one workgroup per query whose row spans more than one chunk: the
// candidates of all chunks are contiguous and in block order (every chunk but
// the last holds cap_q of them).
template <int NT>
__global__ __launch_bounds__(NT) void split_merge_kernel(SplitArgs a)
{
    extern __shared__ __attribute__((aligned(16))) uint32_t s_keys[];
    __shared__ SelectShared sh;
    const TopkGeom g = a.g;
    const int q = blockIdx.x;
    QuerySel qs = query_sel(g, q);
    const int nchq = (qs.n_vis + a.chunk - 1) / a.chunk;
    if (qs.r == 0 || nchq <= 1)
        return;  // written by stage A
    const int r_a = qs.r + (qs.tail != 0 ? 1 : 0);
    const int cap_q = min(r_a, a.chunk);
    const int last_n = min(r_a, qs.n_vis - (nchq - 1) * a.chunk);
    const int total = (nchq - 1) * cap_q + last_n;
    const uint32_t *gkey = a.cand_keys + (int64_t)q * a.cand_stride;
    const int32_t *gblk = a.cand_blocks + (int64_t)q * a.cand_stride;
    clear_hists<NT>(sh);
    // A partial last block: count the candidates at or above its key. If it is
    // taken, every block with key >= its key is among the top r_a of its chunk,
    // so the count is exact; if it is not, the count still shows that (a chunk
    // that drops such a block holds r_a candidates above it).
    const uint32_t kp = qs.tail != 0 ? key_of(g.scores[(int64_t)q * g.ld + qs.n_vis - 1]) : 0u;
    if (total <= a.blk_words) {
        // Keys and block ids both to LDS: the emit then reads no global memory.
        int32_t *s_blks = reinterpret_cast<int32_t *>(s_keys + a.blk_words);
        const int n4 = total >> 2;  // the candidate arrays start 16-byte aligned
        for (int i = threadIdx.x; i < n4; i += NT) {
            *reinterpret_cast<uint4 *>(s_keys + 4 * i) = reinterpret_cast<const uint4 *>(gkey)[i];
            *reinterpret_cast<int4 *>(s_blks + 4 * i) = reinterpret_cast<const int4 *>(gblk)[i];
        }
        for (int i = (n4 << 2) + (int)threadIdx.x; i < total; i += NT) {
            s_keys[i] = gkey[i];
            s_blks[i] = gblk[i];
        }
        lds_barrier();
        const LdsKeys lds{s_keys};
        if (qs.tail != 0)
            widen_for_tail(qs, g.bs, count_at_least<NT>(lds, total, kp, sh));
        select_cells<NT>(lds, total, qs, [&](int i) { return s_blks[i]; }, g, q, sh);
    } else {
        const GlobalKeys keys{gkey};
        if (qs.tail != 0)
            widen_for_tail(qs, g.bs, count_at_least<NT>(keys, total, kp, sh));
        select_cells<NT>(keys, total, qs, [&](int i) { return gblk[i]; }, g, q, sh);
    }
}

// ------------------------------------------------------------------ one read
// The workgroup streams the row in slices of STEP blocks, F4 float4 loads per
// lane and kOneReadBuffers slices in flight per wave. The first slices are
// dealt out in order; after that a wave claims the next slice from an LDS
// counter as it frees a buffer, so a wave whose loads come back early takes
// more of the row and the waves finish together. Each wave keeps its
// candidates (raw FP32 bits and block index) in its own LDS region and records
// per slice how many it kept and where, so there is no workgroup barrier while
// the row streams; at the end the per-slice counts put them in block order.
template <int NT, int F4, bool VEC>
__global__ __launch_bounds__(NT) void oneread_kernel(OneReadArgs a)
{
    constexpr int NW = NT / kWave;
    constexpr int NBUF = kOneReadBuffers;
    constexpr int STEP = kWave * 4 * F4;                  // blocks per slice
    constexpr int MAXS = kOneReadMaxBatches * NW;         // slices of the longest row taken here
    constexpr int WCAP = kOneReadCap / NW;                // candidates a wave may keep
    constexpr int SPT = kOneReadSample / NT;              // sample keys per thread
    static_assert(kOneReadBatch == NW * STEP || kOneReadShortBatch == NW * STEP, "a batch is one slice per wave");
    __shared__ __attribute__((aligned(16))) uint2 s_wlist[kOneReadCap];    // per-wave candidates: (FP32 bits, block)
    __shared__ __attribute__((aligned(16))) uint32_t s_ckey[kOneReadCap];  // candidates in block order
    __shared__ __attribute__((aligned(16))) int32_t s_cblk[kOneReadCap];
    __shared__ SelectShared sh;
    __shared__ uint32_t s_scnt[MAXS];   // per slice: candidates kept ...
    __shared__ uint32_t s_ssrc[MAXS];   // ... where they start in the list of ...
    __shared__ uint32_t s_swave[MAXS];  // ... this wave
    __shared__ uint32_t s_next;         // next slice to claim
    __shared__ uint4 s_tot;             // candidates, any wave over its cap, largest kept key

    const TopkGeom g = a.g;
    const int q = blockIdx.x;
    QuerySel qs = query_sel(g, q);
    if (qs.r == 0) {
        write_first_cells<NT>(g, q, 0);
        return;
    }
    if (visible_cells(qs, g.bs) <= qs.wq) {
        write_first_cells<NT>(g, q, qs.wq);  // every visible cell
        return;
    }
    const int n = qs.n_vis;
    const float *row = g.scores + (int64_t)q * g.ld;
    const int lane = lane_id(), wid = wave_id();
    // Key of a partial last block (see widen_for_tail), and the cells the
    // candidates must hold in that case: the selection may take it whole.
    const uint32_t kp = qs.tail != 0 ? key_of(row[n - 1]) : 0u;
    const int64_t w_need = (int64_t)qs.wq + (qs.tail != 0 ? g.bs - qs.tail : 0);
    const SampleGeom sg = sample_geom(n, qs.r, a.mode);
    const bool use_bound = !a.force_flag && (uint32_t)sg.ns >= sg.ks;
    const int nslices = (n + STEP - 1) / STEP;  // <= MAXS (the dispatch sees to it)

    // Every load below is unconditional: a load under a branch makes the
    // compiler lose count of the loads in flight and wait for all of them
    // before the next use. 16-byte loads go through a buffer resource over
    // the row's visible blocks, rounded up to whole float4 groups (inside the
    // row: ld is a multiple of 4 here): a slice past the row lies outside it
    // and reads zeros without a memory access, so the loads the last rounds
    // issue past the row cost no memory round trip before the tail. The
    // scalar path re-reads block 0 instead (the row has at least one visible
    // block here); the values are ignored.
    const __amdgpu_buffer_rsrc_t rrow = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float *>(row), (short)0, ((n + 3) & ~3) * 4, kRowBufferWord3);
    auto load_slice = [&](int sl, float4 (&v)[F4]) {
#pragma unroll
        for (int j = 0; j < F4; ++j) {
            const int i0 = sl * STEP + j * 4 * kWave + 4 * lane;
            if constexpr (VEC) {
                // Streamed once: nontemporal loads keep it from displacing cached data.
                const f32x4 t = __builtin_bit_cast(
                    f32x4, __builtin_amdgcn_raw_buffer_load_b128(rrow, 4 * i0, 0, kCachePolicyNontemporal));
                v[j] = make_float4(t[0], t[1], t[2], t[3]);
            } else {
                v[j].x = row[i0 < n ? i0 : 0];
                v[j].y = row[i0 + 1 < n ? i0 + 1 : 0];
                v[j].z = row[i0 + 2 < n ? i0 + 2 : 0];
                v[j].w = row[i0 + 3 < n ? i0 + 3 : 0];
            }
            // Issue order = use order: loads complete in order, so a load
            // the scheduler moved ahead would make the first use wait for it.
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // The sample goes into registers first (SPT per thread) and is waited
    // for before the first slice of every wave is issued: the bound needs
    // every wave's sample, and a sample queued behind the whole chip's first
    // slices arrives later (measured 0.2-0.6 us per call). The second slice
    // follows the bound: a wave stalls while its memory queue is full.
    float smp[SPT];
#pragma unroll
    for (int u = 0; u < SPT; ++u) {
        const int i = (int)threadIdx.x + u * NT;
        smp[u] = row[sample_block(sg, (use_bound && i < sg.ns) ? i : 0)];
    }
    clear_hists<NT>(sh);
    float4 buf[NBUF][F4];
    int cs[NBUF];  // slice in each buffer (wave-uniform)
#pragma unroll
    for (int u = 0; u < NBUF; ++u)
        cs[u] = u * NW + wid;
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the sample is in registers
    load_slice(cs[0], buf[0]);
    if (threadIdx.x == 0) {
        s_next = NBUF * NW;
        s_tot = make_uint4(0u, 0u, 0u, 0u);
    }
    lds_barrier();
    // One read: keep blocks with value >= fbound (every block without a
    // bound), in block order, up to WCAP per wave. The key map preserves order
    // and equates -0.0 with +0.0, exactly as float comparison does, so the
    // kept keys are those >= key_of(fbound).
    const float fbound = use_bound ? bound_from_sample<NT, SPT>(smp, sg.ns, sg.ks, sh) : -__builtin_inff();
    clear_fine<NT>(sh);  // ordered before the selection by the barrier after the stream
#pragma unroll
    for (int u = 1; u < NBUF; ++u)
        load_slice(cs[u], buf[u]);

    uint32_t wcnt = 0;               // wave-uniform
    // Largest value this lane kept (med3 with +inf is max for finite values,
    // without the canonicalising steps fmaxf takes).
    float fmx = -__builtin_inff();
    uint2 *wlist = s_wlist + wid * WCAP;
    auto consume = [&](int sl, const float4 (&v)[F4], auto full_tag) {
        constexpr bool FULL = decltype(full_tag)::value;  // every block of the slice is visible
        const int step0 = sl * STEP;
        const uint32_t start = wcnt;
#pragma unroll
        for (int j = 0; j < F4; ++j) {
            const int i0 = step0 + j * 4 * kWave + 4 * lane;
            const float f[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
            bool keep[4];
            uint64_t m[4];
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                keep[s] = f[s] >= fbound && (FULL || i0 + s < n);
                m[s] = __ballot(keep[s]);
            }
            const uint64_t any = m[0] | m[1] | m[2] | m[3];
            if (any == 0)
                continue;
            const uint64_t two = (m[0] & (m[1] | m[2] | m[3])) | (m[1] & (m[2] | m[3])) | (m[2] & m[3]);
            // A slot past the cap is clamped onto the last one: the wave's
            // count then exceeds the cap and the row takes the exact path.
            if (two == 0) {
                // Common case: no lane keeps more than one of its four keys, so
                // a lane's slot is the number of keeping lanes below it.
                if (keep[0] || keep[1] || keep[2] || keep[3]) {
                    // The kept key's place in the group as two bits (i0 is a
                    // multiple of 4).
                    const bool hi = keep[2] || keep[3], odd = keep[1] || keep[3];
                    const float x = hi ? (odd ? f[3] : f[2]) : (odd ? f[1] : f[0]);
                    const int sel = (hi ? 2 : 0) | (odd ? 1 : 0);
                    const uint32_t pos = min(wcnt + count_below(any), (uint32_t)(WCAP - 1));
                    wlist[pos] = make_uint2(__float_as_uint(x), (uint32_t)(i0 | sel));
                    fmx = __builtin_amdgcn_fmed3f(x, fmx, __builtin_inff());
                }
                wcnt += (uint32_t)__popcll(any);
                continue;
            }
            uint32_t below = 0, step = 0;
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                below += count_below(m[s]);
                step += (uint32_t)__popcll(m[s]);
            }
            uint32_t pos = wcnt + below;
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                if (keep[s]) {
                    const uint32_t p = min(pos, (uint32_t)(WCAP - 1));
                    wlist[p] = make_uint2(__float_as_uint(f[s]), (uint32_t)(i0 + s));
                    fmx = __builtin_amdgcn_fmed3f(f[s], fmx, __builtin_inff());
                    ++pos;
                }
            }
            wcnt += step;
        }
        if (lane == 0) {
            s_scnt[sl] = wcnt - start;
            s_ssrc[sl] = start;
            s_swave[sl] = (uint32_t)wid;
        }
    };
    // Rounds over the buffers until each holds a slice past the row. The next
    // slice is claimed before the buffer is consumed (the claim's latency
    // hides behind it); loads stay unconditional (a slice past the row reads
    // block 0 and is not consumed).
    for (;;) {
        bool done = true;
#pragma unroll
        for (int u = 0; u < NBUF; ++u) {
            uint32_t nxt = 0;
            if (lane == 0)
                nxt = __hip_atomic_fetch_add(&s_next, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            if (cs[u] < nslices) {
                if (cs[u] * STEP + STEP <= n)
                    consume(cs[u], buf[u], std::true_type{});
                else
                    consume(cs[u], buf[u], std::false_type{});
            }
            cs[u] = __builtin_amdgcn_readfirstlane((int)nxt);
            load_slice(cs[u], buf[u]);
            done = done && cs[u] >= nslices;
        }
        if (done)
            break;
    }
    // Totals, overflow and the largest kept key, gathered by LDS atomics
    // (keys are finite, so the largest kept float has the largest key).
    const uint32_t wmax = wave_max(key_of(fmx));
    if (lane == 0) {
        __hip_atomic_fetch_add(&s_tot.x, wcnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        __hip_atomic_fetch_or(&s_tot.y, wcnt > (uint32_t)WCAP ? 1u : 0u, __ATOMIC_RELAXED,
                              __HIP_MEMORY_SCOPE_WORKGROUP);
        __hip_atomic_fetch_max(&s_tot.z, wmax, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
    lds_barrier();
    const uint4 tot = s_tot;
    const uint32_t total = (uint32_t)__builtin_amdgcn_readfirstlane((int)tot.x);
    const bool over = __builtin_amdgcn_readfirstlane((int)tot.y) != 0;
    const uint32_t kmax = (uint32_t)__builtin_amdgcn_readfirstlane((int)tot.z);
    // Every candidate key is >= kbase: the bound's key (the key map keeps
    // order, so value >= bound means key >= key(bound)), or 0 without one.
    const uint32_t kbase = use_bound ? key_of(fbound) : 0u;
    // Every visible block kept and all of one key: ties go to the lowest
    // cells, so the selection is the first cells. With a bound, that is
    // total == n and a largest key equal to the bound's (every key lies in
    // [kbase, kmax]); without one, the exact rule below sees it.
    if (use_bound && total == (uint32_t)n && kmax == kbase) {
        write_first_cells<NT>(g, q, qs.wq);
        return;
    }
    const bool ok = !a.force_flag && !over && (int64_t)total * g.bs >= w_need;
    if (ok) {
        // Slices in order are block order: every wave scans the slice counts
        // itself and leaves, for each of its own slices, how far its run moves
        // from the wave's list to block order in the slice's s_ssrc entry (no
        // other wave touches those); a candidate's slice is its block / STEP.
        {
            uint32_t carry = 0;
#pragma unroll 1
            for (int s0 = 0; s0 < nslices; s0 += kWave) {
                const int sl = s0 + lane;
                const bool in = sl < nslices;
                const uint32_t c = in ? s_scnt[sl] : 0u;
                const uint32_t incl = wave_incl_sum(c);
                if (in && s_swave[sl] == (uint32_t)wid)
                    s_ssrc[sl] = carry + incl - c - s_ssrc[sl];
                carry += (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
        // The copy into block order also counts every candidate into the
        // fine bins over [kbase, kmax] and the candidates at or above a
        // partial last block's key.
        const int sF = cand_fine_shift(kmax - kbase);
        const bool bins = kmax != kbase;
        const uint32_t wtot = wcnt;
        uint32_t gcnt = 0;
        // CPR items per lane per round, all reads issued before any write (a
        // wave keeps about 3r/16 candidates, so one round usually suffices).
        constexpr int CPR = 2;
#pragma unroll 1
        for (uint32_t i0 = (uint32_t)lane; i0 < wtot; i0 += CPR * kWave) {
            int32_t blk[CPR];
            uint32_t raw[CPR], shift[CPR];
#pragma unroll
            for (int u = 0; u < CPR; ++u) {
                const uint32_t i = i0 + u * kWave < wtot ? i0 + u * kWave : 0u;
                const uint2 e = wlist[i];
                raw[u] = e.x;
                blk[u] = (int32_t)e.y;
            }
#pragma unroll
            for (int u = 0; u < CPR; ++u)
                shift[u] = s_ssrc[(uint32_t)blk[u] / STEP];  // blocks are non-negative
#pragma unroll
            for (int u = 0; u < CPR; ++u) {
                if (i0 + u * kWave < wtot) {
                    const uint32_t d = i0 + u * kWave + shift[u];
                    const uint32_t k = key_of(__uint_as_float(raw[u]));
                    s_ckey[d] = k;
                    s_cblk[d] = blk[u];
                    gcnt += k >= kp ? 1u : 0u;
                    if (bins)
                        count_candidate(k, kbase, sF, sh);
                }
            }
        }
        if (qs.tail != 0) {
            gcnt = wave_sum(gcnt);
            if (lane == 0)
                sh.red[1][wid] = gcnt;
        }
        lds_barrier();
        widen_from_counts<NT>(qs, g.bs, kp, kbase, sh);
        select_from_candidates<NT>(s_ckey, s_cblk, (int)total, kbase, kmax, qs, g, q, sh);
        return;
    }
    // Flagged: the exact rule over the whole row with one more read of it, in
    // chunks through the LDS of the per-wave lists (the histograms are zero:
    // no histogram pass ran; the plan keeps 2 * (r + 1) within the cap).
    select_row_chunked<NT, 2 * kOneReadCap, VEC>(row, n, qs, kp, reinterpret_cast<uint32_t *>(s_wlist), s_ckey, s_cblk,
                                                 kOneReadCap, g, q, sh);
}

// ------------------------------------------------------------------- utility
__global__ void zero_kernel(uint32_t *p, size_t n)
{
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
        p[i] = 0u;
}

hipError_t launch_zero(void *p, size_t bytes, hipStream_t s)
{
    const size_t n = bytes / 4;
    if (n == 0)
        return hipSuccess;
    const size_t blocks = (n + 255) / 256;
    const unsigned grid = (unsigned)(blocks < 4096 ? blocks : 4096);
    hipLaunchKernelGGL(zero_kernel, dim3(grid), dim3(256), 0, s, (uint32_t *)p, n);
    return hipGetLastError();
}

hipError_t launch_split(const SplitArgs &a, hipStream_t s)
{
    // Stage B may keep up to 2 * kStageBLdsWords words in dynamic LDS, above
    // the default limit. The attribute belongs to the kernel function, so it
    // is set once per process; the function-local static is initialised by
    // exactly one thread (the C++ guarantee), others wait for its result.
    static const hipError_t lds_limit =
        hipFuncSetAttribute(reinterpret_cast<const void *>(&split_merge_kernel<kSplitMergeThreads>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, 2 * kStageBLdsWords * 4);
    if (lds_limit != hipSuccess)
        return lds_limit;
    const dim3 grid((unsigned)a.n_chunks, (unsigned)a.g.nq);
    hipLaunchKernelGGL(split_kernel<kSplitThreads>, grid, dim3(kSplitThreads), (size_t)a.lds_words * 4, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.n_chunks <= 1)
        return e;
    hipLaunchKernelGGL(split_merge_kernel<kSplitMergeThreads>, dim3((unsigned)a.g.nq), dim3(kSplitMergeThreads),
                       (size_t)(2 * a.blk_words) * 4, s, a);
    return hipGetLastError();
}

hipError_t launch_oneread(const OneReadArgs &a, hipStream_t s)
{
    // A row's slices must fit the kernel's per-slice records (MAXS): the
    // half-size slices serve rows of at most kOneReadShortRow blocks.
    static_assert(kOneReadShortFewRow <= kOneReadShortRow, "the few-query limit is the smaller");
    static_assert((int64_t)kOneReadShortRow <= (int64_t)kOneReadMaxBatches * kOneReadShortBatch,
                  "short rows fit the slice records");
    const dim3 grid((unsigned)a.g.nq);
    const bool shortrow = oneread_short_slices(a.g.nq, a.g.n_blocks);
    if (a.g.vec4) {
        if (shortrow)
            hipLaunchKernelGGL((oneread_kernel<kOneReadThreads, kOneReadShortF4, true>), grid, dim3(kOneReadThreads), 0,
                               s, a);
        else
            hipLaunchKernelGGL((oneread_kernel<kOneReadThreads, kOneReadF4, true>), grid, dim3(kOneReadThreads), 0, s,
                               a);
    } else {
        if (shortrow)
            hipLaunchKernelGGL((oneread_kernel<kOneReadThreads, kOneReadShortF4, false>), grid, dim3(kOneReadThreads),
                               0, s, a);
        else
            hipLaunchKernelGGL((oneread_kernel<kOneReadThreads, kOneReadF4, false>), grid, dim3(kOneReadThreads), 0, s,
                               a);
    }
    return hipGetLastError();
}

} // namespace qsa
