// topk_filter.hip - the block top-k as two launches for gfx950: the sampled
// bound and one read of the scores (Strata pull #2093 "sm_75: the prompt
// path's top-k with one full read of the scores", section Beschreibung)
// spread over many workgroups per query, as the chunked split spreads a row
// (Strata pull #3987, sections Problem and result, Approach).
//
//  * filter_kernel (stage A): one 256-thread workgroup per (query, chunk of
//    1,024-8,192 blocks). It issues the loads of its chunk and of the row's
//    sample together, computes the query's lower bound from the sample (every
//    workgroup of the query computes the same bound from the same values),
//    keeps the chunk's blocks at or above the bound, in block order, in the
//    chunk's slot of the workspace, and writes a header: the count (or an
//    overflow mark), the chunk's smallest and largest key and the bound.
//  * gather_kernel (stage B): one 1,024-thread workgroup per query. The
//    headers give each chunk's place in block order; the candidates of all
//    chunks go to LDS and the exact rule over them gives the ids, provided
//    they hold the selection's cells (then the threshold is at or above the
//    bound, so every block at or above it is a candidate). Otherwise the query
//    takes the exact path over its whole row in the same workgroup; when all
//    visible keys are equal (smallest = largest over the headers) that is
//    simply the first cells.
//
// The kernel boundary orders stage A's writes before stage B's reads; no
// workgroup waits for another.
#include "qsa_internal.h"
#include "topk_device.h"
#include "topk_select.h"

namespace qsa {

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int F4, bool VEC>
__global__ __launch_bounds__(kFilterThreads) void filter_kernel(FilterArgs a)
{
    constexpr int NT = kFilterThreads;
    constexpr int NW = NT / kWave;
    constexpr int CB = NT * 4 * F4;           // blocks per chunk
    constexpr int SPT = kOneReadSample / NT;  // sample keys per thread
    __shared__ SelectShared sh;
    __shared__ uint32_t s_seg[F4 * NW];       // kept blocks per 256-block segment, in block order
    __shared__ uint32_t s_mm[2][NW];

    const TopkGeom g = a.g;
    int q, c;
    if (a.xcd) {
        // Workgroup i runs on XCD i % 8: every chunk of a query on one XCD,
        // so the row's sample is fetched into one L2 only.
        const int y = (int)(blockIdx.x >> 3);
        q = (int)(blockIdx.x & 7u) + 8 * (y / a.n_chunks);
        c = y % a.n_chunks;
    } else {
        q = (int)blockIdx.x / a.n_chunks;
        c = (int)blockIdx.x % a.n_chunks;
    }
    const QuerySel qs = query_sel(g, q);
    const int n = qs.n_vis;
    if (qs.r == 0 || visible_cells(qs, g.bs) <= qs.wq)
        return;  // nothing to choose: stage B writes these queries directly
    if (c * CB >= n)
        return;
    const int tid = (int)threadIdx.x, lane = lane_id(), wid = wave_id();
    const float *row = g.scores + (int64_t)q * g.ld;
    const int b0 = c * CB;
    const int nc = min(CB, n - b0);

    const SampleGeom sg = sample_geom(n, qs.r, a.mode);
    const bool use_bound = !a.force_flag && (uint32_t)sg.ns >= sg.ks;
    // The sample first, then the chunk: every load is issued before the
    // bound is needed, and each is unconditional (an index past its range
    // reads block 0 or the chunk's first block, and the value is ignored).
    float smp[SPT];
#pragma unroll
    for (int u = 0; u < SPT; ++u) {
        const int i = tid + u * NT;
        smp[u] = row[sample_block(sg, (use_bound && i < sg.ns) ? i : 0)];
    }
    const float *crow = row + b0;
    float4 v[F4];
#pragma unroll
    for (int j = 0; j < F4; ++j) {
        const int i0 = j * 4 * NT + 4 * tid;
        if constexpr (VEC) {
            const f32x4 t = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(crow + (i0 < nc ? i0 : 0)));
            v[j] = make_float4(t[0], t[1], t[2], t[3]);
        } else {
            v[j].x = crow[i0 < nc ? i0 : 0];
            v[j].y = crow[i0 + 1 < nc ? i0 + 1 : 0];
            v[j].z = crow[i0 + 2 < nc ? i0 + 2 : 0];
            v[j].w = crow[i0 + 3 < nc ? i0 + 3 : 0];
        }
    }
    clear_fine<NT>(sh);
    lds_barrier();
    // The kept keys are those >= key_of(fbound): the key map preserves order
    // and equates -0.0 with +0.0, exactly as the float comparison does.
    const float fbound = use_bound ? bound_from_sample<NT, SPT>(smp, sg.ns, sg.ks, sh) : -__builtin_inff();
    const bool keep_any = !a.force_flag;

    // Keep flags, the chunk's key range, and per 256-block segment (j, wave)
    // the kept count and each lane's place in it (lane l holds blocks
    // 4l .. 4l+3 of the wave's segment).
    uint32_t kmn = 0xFFFFFFFFu, kmx = 0u, keep = 0u, below[F4];
#pragma unroll
    for (int j = 0; j < F4; ++j) {
        const int i0 = j * 4 * NT + 4 * tid;
        const float f[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
        uint32_t cnt = 0;
        below[j] = 0;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const bool vis = i0 + s < nc;
            const uint32_t k = key_of(f[s]);
            kmn = vis ? min(kmn, k) : kmn;
            kmx = vis ? max(kmx, k) : kmx;
            const bool kp = keep_any && vis && f[s] >= fbound;
            keep |= kp ? 1u << (4 * j + s) : 0u;
            const uint64_t m = __ballot(kp);
            below[j] += count_below(m);
            cnt += (uint32_t)__popcll(m);
        }
        if (lane == 0)
            s_seg[j * NW + wid] = cnt;
    }
    kmn = wave_min(kmn);
    kmx = wave_max(kmx);
    if (lane == 0) {
        s_mm[0][wid] = kmn;
        s_mm[1][wid] = kmx;
    }
    lds_barrier();
    // Segments in block order (j major, wave minor): lane e holds segment
    // e's count, one wave scan gives every segment's place.
    static_assert(F4 * NW <= kWave, "one segment per lane");
    const uint32_t seg = lane < F4 * NW ? s_seg[lane] : 0u;
    const uint32_t seg_incl = wave_incl_sum(seg);
    const uint32_t total = (uint32_t)__builtin_amdgcn_readlane((int)seg_incl, F4 * NW - 1);
    uint32_t pre[F4];
#pragma unroll
    for (int j = 0; j < F4; ++j)
        pre[j] = (uint32_t)__builtin_amdgcn_readlane((int)(seg_incl - seg), j * NW + wid);
    const uint32_t S = (uint32_t)a.slot;
    uint32_t *skey = a.slots + ((int64_t)q * a.n_chunks + c) * 2 * (int64_t)a.slot;
    uint32_t *sblk = skey + a.slot;
#pragma unroll
    for (int j = 0; j < F4; ++j) {
        const int i0 = j * 4 * NT + 4 * tid;
        const float f[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
        uint32_t pos = pre[j] + below[j];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            if ((keep >> (4 * j + s)) & 1u) {
                if (pos < S) {
                    skey[pos] = key_of(f[s]);
                    sblk[pos] = (uint32_t)(b0 + i0 + s);
                }
                ++pos;
            }
        }
    }
    if (tid == 0) {
        uint32_t mn = 0xFFFFFFFFu, mx = 0u;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            mn = min(mn, s_mm[0][w]);
            mx = max(mx, s_mm[1][w]);
        }
        const uint32_t cnt = (!keep_any || total > S) ? kFilterOverflow : total;
        reinterpret_cast<uint4 *>(a.heads)[(int64_t)q * a.n_chunks + c] = make_uint4(cnt, mn, mx, key_of(fbound));
    }
}

template <bool VEC>
__global__ __launch_bounds__(kOneReadThreads) void gather_kernel(FilterArgs a)
{
    constexpr int NT = kOneReadThreads;
    constexpr int NW = NT / kWave;
    constexpr int HPT = kFilterMaxChunks / NT;  // chunk headers per thread, at most
    __shared__ __attribute__((aligned(16))) uint32_t s_ckey[kOneReadCap];
    __shared__ __attribute__((aligned(16))) int32_t s_cblk[kOneReadCap];
    __shared__ SelectShared sh;
    __shared__ uint32_t s_off[kFilterMaxChunks];
    __shared__ uint32_t s_red[6][NW];

    const TopkGeom g = a.g;
    const int q = (int)blockIdx.x;
    QuerySel qs = query_sel(g, q);
    if (qs.r == 0) {
        write_first_cells<NT>(g, q, 0);
        return;
    }
    if (visible_cells(qs, g.bs) <= qs.wq) {
        write_first_cells<NT>(g, q, qs.wq);  // every visible cell
        return;
    }
    const int tid = (int)threadIdx.x, lane = lane_id(), wid = wave_id();
    const int n = qs.n_vis;
    const int nch = (n + a.chunk - 1) / a.chunk;
    const float *row = g.scores + (int64_t)q * g.ld;
    const uint32_t kp = qs.tail != 0 ? key_of(row[n - 1]) : 0u;
    clear_hists<NT>(sh);

    // Headers: thread t takes chunks [t*per, t*per + per); the exclusive
    // prefix of the counts is each chunk's place in block order.
    const int per = (nch + NT - 1) / NT;  // <= HPT
    const int h0 = tid * per;
    const uint4 *heads = reinterpret_cast<const uint4 *>(a.heads) + (int64_t)q * a.n_chunks;
    uint32_t cnt[HPT];
    uint32_t sum = 0, ovf = 0, kmn = 0xFFFFFFFFu, kmx = 0u, blo = 0xFFFFFFFFu, bhi = 0u;
#pragma unroll
    for (int j = 0; j < HPT; ++j) {
        cnt[j] = 0;
        if (j < per && h0 + j < nch) {
            const uint4 h = heads[h0 + j];
            const bool o = h.x == kFilterOverflow;
            ovf |= o ? 1u : 0u;
            cnt[j] = o ? 0u : h.x;
            sum += cnt[j];
            kmn = min(kmn, h.y);
            kmx = max(kmx, h.z);
            blo = min(blo, h.w);
            bhi = max(bhi, h.w);
        }
    }
    const uint32_t incl = wave_incl_sum(sum);
    const uint32_t w_ovf = wave_max(ovf), w_mn = wave_min(kmn), w_mx = wave_max(kmx);
    const uint32_t w_blo = wave_min(blo), w_bhi = wave_max(bhi);
    if (lane == kWave - 1)
        s_red[0][wid] = incl;
    if (lane == 0) {
        s_red[1][wid] = w_ovf;
        s_red[2][wid] = w_mn;
        s_red[3][wid] = w_mx;
        s_red[4][wid] = w_blo;
        s_red[5][wid] = w_bhi;
    }
    lds_barrier();
    uint32_t before = incl - sum, total = 0, any_ovf = 0, mn = 0xFFFFFFFFu, mx = 0u, b_lo = 0xFFFFFFFFu,
             b_hi = 0u;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        before += w < wid ? s_red[0][w] : 0u;
        total += s_red[0][w];
        any_ovf |= s_red[1][w];
        mn = min(mn, s_red[2][w]);
        mx = max(mx, s_red[3][w]);
        b_lo = min(b_lo, s_red[4][w]);
        b_hi = max(b_hi, s_red[5][w]);
    }
#pragma unroll
    for (int j = 0; j < HPT; ++j) {
        if (j < per && h0 + j < nch) {
            s_off[h0 + j] = before;
            before += cnt[j];
        }
    }
    lds_barrier();

    const int64_t w_need = (int64_t)qs.wq + (qs.tail != 0 ? g.bs - qs.tail : 0);
    const bool ok = !a.force_flag && !any_ovf && b_lo == b_hi && total <= (uint32_t)kOneReadCap &&
                    (int64_t)total * g.bs >= w_need;
    if (ok) {
        // Thread t copies candidates [t*cper, t*cper + cper) of the block
        // order: a binary search over the chunk offsets finds the chunk of
        // the first, the rest follow in order, and each batch of loads is
        // issued before any of them is used.
        constexpr int B = 8;
        const int cper = ((int)total + NT - 1) / NT;
        const int i0 = min((int)total, tid * cper), i1 = min((int)total, i0 + cper);
        int c = 0;
        if (i0 < i1) {
            int hi = nch - 1;
#pragma unroll 1
            while (c < hi) {
                const int mid = (c + hi + 1) >> 1;
                if ((int)s_off[mid] <= i0)
                    c = mid;
                else
                    hi = mid - 1;
            }
        }
        int next = c + 1 < nch ? (int)s_off[c + 1] : (int)total;
        const uint32_t *slots_q = a.slots + (int64_t)q * a.n_chunks * 2 * (int64_t)a.slot;
        // The copy also counts every candidate into the fine bins over
        // [bound key, mx] (every candidate key lies there; the row's largest
        // key is a candidate) and those at or above a partial last block's key.
        const int sF = cand_fine_shift(mx - b_lo);
        const bool bins = mx != b_lo;
        uint32_t gcnt = 0;
#pragma unroll 1
        for (int base = i0; base < i1; base += B) {
            uint32_t k[B], b[B];
#pragma unroll
            for (int u = 0; u < B; ++u) {
                const int i = base + u;
                if (i < i1) {
#pragma unroll 1
                    while (i >= next) {
                        ++c;
                        next = c + 1 < nch ? (int)s_off[c + 1] : (int)total;
                    }
                    const uint32_t *sk = slots_q + (int64_t)c * 2 * a.slot + (i - (int)s_off[c]);
                    k[u] = sk[0];
                    b[u] = sk[a.slot];
                }
            }
#pragma unroll
            for (int u = 0; u < B; ++u) {
                if (base + u < i1) {
                    s_ckey[base + u] = k[u];
                    s_cblk[base + u] = (int32_t)b[u];
                    gcnt += k[u] >= kp ? 1u : 0u;
                    if (bins)
                        count_candidate(k[u], b_lo, sF, sh);
                }
            }
        }
        if (qs.tail != 0) {
            gcnt = wave_sum(gcnt);
            if (lane == 0)
                sh.red[1][wid] = gcnt;
        }
        lds_barrier();
        widen_from_counts<NT>(qs, g.bs, kp, b_lo, sh);
        select_from_candidates<NT>(s_ckey, s_cblk, (int)total, b_lo, mx, qs, g, q, sh);
        return;
    }
    if (mn == mx) {
        write_first_cells<NT>(g, q, qs.wq);  // every visible key equal: ties go to the lowest cells
        return;
    }
    // The exact rule over the whole row, with its key range from the headers
    // (a few queries: the row was just read by the first launch, and its
    // passes here mostly hit the caches).
    if (qs.tail != 0)
        widen_for_tail(qs, g.bs, count_at_least<NT>(RowKeys{row, VEC}, n, kp, sh));
    select_cells_in<NT>(RowKeys{row, VEC}, n, mn, mx, qs, [&](int i) { return i; }, g, q, sh);
}

template <int F4>
void launch_filter_f4(const FilterArgs &a, hipStream_t s)
{
    const dim3 grid((unsigned)(a.g.nq * a.n_chunks));
    if (a.g.vec4)
        hipLaunchKernelGGL((filter_kernel<F4, true>), grid, dim3(kFilterThreads), 0, s, a);
    else
        hipLaunchKernelGGL((filter_kernel<F4, false>), grid, dim3(kFilterThreads), 0, s, a);
}

} // namespace

hipError_t launch_filter(const FilterArgs &a, hipStream_t s)
{
    switch (a.chunk) {
    case 1024: launch_filter_f4<1>(a, s); break;
    case 2048: launch_filter_f4<2>(a, s); break;
    case 4096: launch_filter_f4<4>(a, s); break;
    case 8192: launch_filter_f4<8>(a, s); break;
    default: return hipErrorInvalidValue;
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    if (a.g.vec4)
        hipLaunchKernelGGL((gather_kernel<true>), dim3((unsigned)a.g.nq), dim3(kOneReadThreads), 0, s, a);
    else
        hipLaunchKernelGGL((gather_kernel<false>), dim3((unsigned)a.g.nq), dim3(kOneReadThreads), 0, s, a);
    return hipGetLastError();
}

} // namespace qsa
