// attn_kernels.hip - attention of every query head over the cells its query
// selected: the consumer of the block selection (iree-org/wave issue #1257
// "NSA: LDS optimization for block-gather in selection attention", sections
// Problem and Per-block LDS staging). Heads of one group share a key/value
// head; for query q and head h of key/value head g:
//     out[q][h] = sum_c softmax_c(scale * q[q][h] . k[c][g]) * v[c][g]
// over the listed cells c, and lse[q][h] = log sum_c exp(scale * q . k).
//
// Work unit: one query, one key/value head, a block of up to 16 of its query
// heads and a chunk of the query's id list. A workgroup of eight waves (one
// per CU at two waves per SIMD) takes a unit; each wave walks 32-cell steps of
// the chunk with its own running softmax (max, sum, output) and the eight are
// merged in LDS at the end. When a unit's list is split into several chunks,
// each chunk's workgroup leaves its merged partial in the workspace and
// attn_merge_kernel combines them. (A last-arriving-workgroup hand-off in the
// same launch was measured slower on MI355X: its write-through stores, the
// ticket and the device-coherent loads cost more round trips than the kernel
// boundary.)
//
// The gather is software-pipelined: a wave's id loads run two steps ahead and
// its key/value row loads one step ahead (a second register set), so every
// wave keeps a step's rows in flight while it computes the previous one.
// Loads past the wave's range are issued too, masked to cell 0 (cache hits),
// so that no load sits under a branch and the compiler's waits stay exact.
//
// Shared blocks (the same issue, section Shared block deduplication): with
// key/value groups of up to 8 heads, queries 2i and 2i+1 form a pair whose
// two lists attn_union_kernel first merges into one list of distinct cells,
// each entry marked with the queries that listed it (an LDS hash per pair,
// the order that of first occurrence). attn_kernel<true> then walks the
// merged list: its 16 matrix-core columns are the pair's heads (query 2i in
// columns 0-7, query 2i+1 in 8-15), each distinct cell's key and value rows
// are gathered once for both, and a cell's logits in the columns of a query
// that did not list it are -inf (weight 0).
//
// Matrix cores (v_mfma_f32_16x16x32_bf16, FP32 accumulation):
//  * S^T[16 cells x 16 heads] = K[16 cells x 128] . Q^T[128 x 16 heads] in four
//    32-deep steps. The contraction index is permuted: in step s lane group
//    j (lanes 16j..16j+15) supplies dims 32j+8s .. 32j+8s+7, so a lane reads
//    64 contiguous bytes of its cell's key row (keys go straight from memory
//    to registers) and of its head's query row.
//  * S^T comes out with head = lane % 16 and cells 4*(lane/16)+i in register
//    i: a head's softmax is lane-local apart from one max and one sum over the
//    four lane groups.
//  * O^T[128 dims x 16 heads] += V^T[dims x 32 cells] . P^T[32 cells x heads].
//    The cells are the contraction, so the operand is V transposed: the rows
//    go into LDS as they are and come back transposed by gfx950's transpose
//    read (ds_read_b64_tr_b16: within 16 lanes, lane 4a+b receives element b
//    of the 4-element reads of lanes a, 4+a, 8+a, 12+a). P comes straight
//    from the S^T registers: contraction position 8j+i is cell 4j+i of the
//    step's first 16 cells and 8j+4+i is cell 16+4j+i. P is split into a bfloat16 head and tail
//    (hi + lo equals p to about 2^-17 relative) and both are multiplied, so
//    the weighted sum keeps close to FP32 accuracy.
#include <math.h>

#include "qsa_internal.h"
#include "topk_device.h"  // wave scans

namespace qsa {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

constexpr int kThreads = 64 * kAttnWaves;
// V rows in LDS: 128 bfloat16 (64 dwords) + 8 dwords of padding per cell, so
// that the 16 lanes of a transpose read (4 cells x 4 dim quads) fall in
// distinct banks.
constexpr int kVPitch = 72;
constexpr int kVtWords = kAttnStepCells * kVPitch;
constexpr int kOPitch = 132;  // floats per head row of the merge buffer
constexpr float kRescale = 8.f;  // log2 headroom of the running softmax reference

struct AttnMerge {
    float o[kAttnWaves][kAttnHeadBlock][kOPitch];
    float m[kAttnWaves][kAttnHeadBlock];
    float l[kAttnWaves][kAttnHeadBlock];
};

union AttnLds {
    uint32_t vt[kAttnWaves][kVtWords];
    AttnMerge merge;
};

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 x) { return __builtin_bit_cast(bf16x8, x); }

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// The ids of one step: this lane's positions c0+n and c0+16+n (its key and
// value rows in the two 16-cell halves).
struct StepIds {
    int a, b;
    int c0;
};

// One step's gathered rows and the validity of its 32 cells (bit c) and of
// this lane's two cells.
struct StepRows {
    uint4 ka[4], kb[4], v0[4], v1[4];
    uint64_t ma, mb;
    uint64_t pa[2], pb[2];  // shared blocks: the cells each query of the pair listed
    bool va, vb;
};

__device__ __forceinline__ StepIds load_ids(const int32_t *row, int c0, int width, int n)
{
    const int last = width - 1;
    StepIds s;
    s.c0 = c0;
    s.a = row[min(c0 + n, last)];
    s.b = row[min(c0 + 16 + n, last)];
    return s;
}

// Positions at or past `limit` and ids outside [0, n_cells) select nothing;
// their rows are read from cell 0. SHARED: an entry is a merged one, cell id
// in the low kPairIdBits bits and the listing queries of the pair above.
template <bool SHARED>
__device__ __forceinline__ void load_rows(const StepIds &s0, const AttnArgs &a, int limit, int64_t kv_row,
                                          int64_t head_off, int n, StepRows &r)
{
    StepIds s = s0;
    uint32_t qa = 1u, qb = 1u;
    if constexpr (SHARED) {
        constexpr int kIdMask = (1 << kPairIdBits) - 1;
        qa = (uint32_t)s0.a >> kPairIdBits;
        qb = (uint32_t)s0.b >> kPairIdBits;
        s.a = s0.a & kIdMask;
        s.b = s0.b & kIdMask;
    }
    const bool va = s.c0 + n < limit && (unsigned)s.a < (unsigned)a.n_cells;
    const bool vb = s.c0 + 16 + n < limit && (unsigned)s.b < (unsigned)a.n_cells;
    r.ma = __ballot(va);
    r.mb = __ballot(vb);
    if constexpr (SHARED) {
        r.pa[0] = __ballot(va && (qa & 1u));
        r.pa[1] = __ballot(va && (qa & 2u));
        r.pb[0] = __ballot(vb && (qb & 1u));
        r.pb[1] = __ballot(vb && (qb & 2u));
    }
    r.va = va;
    r.vb = vb;
    // Row offsets in elements: a non-negative 31-bit id times the row length.
    const uint64_t len = (uint32_t)kv_row;
    const uint4 *kap = reinterpret_cast<const uint4 *>(a.k + (uint64_t)(uint32_t)(va ? s.a : 0) * len + head_off);
    const uint4 *kbp = reinterpret_cast<const uint4 *>(a.k + (uint64_t)(uint32_t)(vb ? s.b : 0) * len + head_off);
    const uint4 *v0p = reinterpret_cast<const uint4 *>(a.v + (uint64_t)(uint32_t)(va ? s.a : 0) * len + head_off);
    const uint4 *v1p = reinterpret_cast<const uint4 *>(a.v + (uint64_t)(uint32_t)(vb ? s.b : 0) * len + head_off);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        r.ka[i] = kap[i];
        r.kb[i] = kbp[i];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        r.v0[i] = v0p[i];
        r.v1[i] = v1p[i];
    }
}

// One step: logits, the online softmax update, and the weighted value sum.
// SHARED: a column takes the cells its query of the pair listed.
template <bool SHARED>
__device__ __forceinline__ void attend(const StepRows &r, const bf16x8 (&qb)[4], float scale_log2, int n, int lg,
                                       uint32_t *vt, float &m, float &l, f32x4 (&o)[8])
{
    uint64_t ma = r.ma, mb = r.mb;
    if constexpr (SHARED) {
        const bool second = n >= kPairHeads;
        ma = second ? r.pa[1] : r.pa[0];
        mb = second ? r.pb[1] : r.pb[0];
    }
    f32x4 sa = {0.f, 0.f, 0.f, 0.f}, sb = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        sa = mfma(as_bf16x8(r.ka[s]), qb[s], sa);
        sb = mfma(as_bf16x8(r.kb[s]), qb[s], sb);
    }
    float x[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        x[i] = ((ma >> (4 * lg + i)) & 1) ? sa[i] * scale_log2 : -INFINITY;
        x[4 + i] = ((mb >> (4 * lg + i)) & 1) ? sb[i] * scale_log2 : -INFINITY;
    }
    float smax = x[0];
#pragma unroll
    for (int i = 1; i < 8; ++i)
        smax = fmaxf(smax, x[i]);
    smax = fmaxf(smax, __shfl_xor(smax, 16));
    smax = fmaxf(smax, __shfl_xor(smax, 32));
    // The running sums are kept relative to a reference m that moves only when
    // a head's max passes it by more than kRescale (then every lane rebases,
    // a wave-uniform branch): weights stay below 2^kRescale, and any
    // reference gives the same ratios.
    if (__ballot(smax > m + kRescale)) {
        const float mnew = fmaxf(m, smax);
        const float alpha = mnew == m ? 1.f : __builtin_amdgcn_exp2f(m - mnew);
        l *= alpha;
#pragma unroll
        for (int t = 0; t < 8; ++t)
            o[t] *= alpha;
        m = mnew;
    }
    const float mref = m == -INFINITY ? 0.f : m;  // a head with no cell yet has only -inf logits
    float psum = 0.f;
    bf16x8 ph, pl;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float p = __builtin_amdgcn_exp2f(x[i] - mref);
        psum += p;
        const __bf16 hi = (__bf16)p;
        ph[i] = hi;
        pl[i] = (__bf16)(p - (float)hi);
    }
    l += psum;

    // V rows into LDS as they are: this lane holds cells n and 16+n, dims
    // 32lg .. 32lg+31. A masked cell's row (read from cell 0) is zeroed: its
    // weight is exactly 0, and 0 times a non-finite value in a row nobody
    // listed must not reach the sum.
    {
        const uint32_t k0 = r.va ? 0xFFFFFFFFu : 0u, k1 = r.vb ? 0xFFFFFFFFu : 0u;
        uint4 *d0 = reinterpret_cast<uint4 *>(vt + n * kVPitch + 16 * lg);
        uint4 *d1 = reinterpret_cast<uint4 *>(vt + (16 + n) * kVPitch + 16 * lg);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            d0[i] = make_uint4(r.v0[i].x & k0, r.v0[i].y & k0, r.v0[i].z & k0, r.v0[i].w & k0);
            d1[i] = make_uint4(r.v1[i].x & k1, r.v1[i].y & k1, r.v1[i].z & k1, r.v1[i].w & k1);
        }
    }
    // The wave reads what its own lanes wrote (LDS keeps a wave's order).
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // Operand of dim tile t for lane (lg, n): V[4lg + j][16t + n] and
    // V[16 + 4lg + j][16t + n], j = 0..3, by two transpose reads in which lane
    // n of the group reads dims 16t + 4(n%4) .. +3 of cell 4lg + n/4 (16 + ...).
    const int rsel = 4 * lg + (n >> 2), csel = 2 * (n & 3);
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        uint32_t *p0 = vt + rsel * kVPitch + 8 * t + csel;
        uint32_t *p1 = p0 + 16 * kVPitch;
        // vt is LDS: the generic pointer converts to the local address space.
        const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)p0);
        const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)p1);
        const uint2 l2 = __builtin_bit_cast(uint2, lo), h2 = __builtin_bit_cast(uint2, hi);
        const bf16x8 av = as_bf16x8(make_uint4(l2.x, l2.y, h2.x, h2.y));
        o[t] = mfma(av, ph, o[t]);
        o[t] = mfma(av, pl, o[t]);
    }
    __builtin_amdgcn_wave_barrier();
}

// Normalised output (4 dims) and, when asked, the log-sum-exp in natural
// log units; a head with no selected cell gets 0 and -inf.
__device__ __forceinline__ void finish(f32x4 acc, float sum, float ref, float *dst, float *dst_lse)
{
    *reinterpret_cast<float4 *>(dst) = sum > 0.f ? make_float4(acc[0] / sum, acc[1] / sum, acc[2] / sum, acc[3] / sum)
                                                 : make_float4(0.f, 0.f, 0.f, 0.f);
    if (dst_lse)
        *dst_lse = sum > 0.f ? (ref + log2f(sum)) * 0.69314718055994531f : -INFINITY;
}

// Two waves per SIMD: at most 256 VGPRs, room for two steps of rows.
// SHARED: a unit is a pair of queries (iq below is the pair) over its merged
// list.
template <bool SHARED>
__global__ __launch_bounds__(kThreads, 2) void attn_kernel(AttnArgs a)
{
    __shared__ AttnLds sm;
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int n = lane & 15, lg = lane >> 4;

    int u = blockIdx.x;
    const int chunk = u % a.n_chunks;
    const int unit = u / a.n_chunks;
    u = unit;
    const int hb = u % a.hblocks;
    u /= a.hblocks;
    const int g = u % a.kv_heads;
    const int iq = u / a.kv_heads;

    float m = -INFINITY, l = 0.f;
    f32x4 o[8];
#pragma unroll
    for (int t = 0; t < 8; ++t)
        o[t] = f32x4{0.f, 0.f, 0.f, 0.f};

    uint32_t *vt = sm.vt[wv];
    const int32_t *idrow = a.ids + (int64_t)iq * a.ld_ids;
    // Listed positions of the unit's list: the merged list's length, read on
    // the device (wave-uniform), or the callers' width.
    const int wlen = SHARED ? __builtin_amdgcn_readfirstlane(a.union_len[iq]) : a.width;
    const int64_t kv_row = (int64_t)a.kv_heads * 128;
    const int64_t head_off = (int64_t)g * 128 + 32 * lg;
    const int first = (chunk * kAttnWaves + wv) * a.steps_per_wave * kAttnStepCells;
    // Steps of this wave that hold listed positions (wave-uniform).
    const int steps = min(a.steps_per_wave, max(0, (wlen - first + kAttnStepCells - 1) / kAttnStepCells));
    const int limit = min(wlen, first + steps * kAttnStepCells);
    if (steps > 0) {
        // The id loads start the dependent chain; the query rows load beside them.
        StepIds i0 = load_ids(idrow, first, wlen, n);
        // This lane's matrix-core column: query head hb*16 + n of the group,
        // or with SHARED head n % 8 of query 2 iq + n / 8 (a padding column
        // reads head 0 of the group and is zeroed).
        const int qcol = SHARED ? 2 * iq + (n >= kPairHeads ? 1 : 0) : iq;
        const int hcol = SHARED ? (n & (kPairHeads - 1)) : hb * kAttnHeadBlock + n;
        const bool head_ok = hcol < a.group && qcol < a.nq;
        const int head = g * a.group + (head_ok ? hcol : 0);
        const uint32_t keep = head_ok ? 0xFFFFFFFFu : 0u;
        const uint4 *qp = reinterpret_cast<const uint4 *>(
            a.q + ((int64_t)(head_ok ? qcol : iq * (SHARED ? 2 : 1)) * a.n_heads + head) * 128 + 32 * lg);
        bf16x8 qb[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const uint4 x = qp[s];
            qb[s] = as_bf16x8(make_uint4(x.x & keep, x.y & keep, x.z & keep, x.w & keep));
        }
        StepRows r0, r1;
        if (steps == 1) {  // wave-uniform: nothing to overlap (decode calls), no prefetch
            load_rows<SHARED>(i0, a, limit, kv_row, head_off, n, r0);
            attend<SHARED>(r0, qb, a.scale_log2, n, lg, vt, m, l, o);
        } else {
            StepIds i1 = load_ids(idrow, first + kAttnStepCells, wlen, n);
            load_rows<SHARED>(i0, a, limit, kv_row, head_off, n, r0);
            for (int j = 0; j < steps; j += 2) {
                i0 = load_ids(idrow, first + (j + 2) * kAttnStepCells, wlen, n);
                load_rows<SHARED>(i1, a, limit, kv_row, head_off, n, r1);
                attend<SHARED>(r0, qb, a.scale_log2, n, lg, vt, m, l, o);
                if (j + 1 >= steps)
                    break;
                i1 = load_ids(idrow, first + (j + 3) * kAttnStepCells, wlen, n);
                load_rows<SHARED>(i0, a, limit, kv_row, head_off, n, r0);
                attend<SHARED>(r1, qb, a.scale_log2, n, lg, vt, m, l, o);
            }
        }
    }
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);

    // Merge the eight waves.
    __syncthreads();  // every wave is done with its V^T rows
    if (lg == 0) {
        sm.merge.m[wv][n] = m;
        sm.merge.l[wv][n] = l;
    }
#pragma unroll
    for (int t = 0; t < 8; ++t)
        *reinterpret_cast<f32x4 *>(&sm.merge.o[wv][n][16 * t + 4 * lg]) = o[t];
    __syncthreads();

    const int hn = threadIdx.x >> 5, d0 = (threadIdx.x & 31) * 4;
    float mw[kAttnWaves], big = -INFINITY;
#pragma unroll
    for (int w = 0; w < kAttnWaves; ++w) {
        mw[w] = sm.merge.m[w][hn];
        big = fmaxf(big, mw[w]);
    }
    const float ref = big == -INFINITY ? 0.f : big;
    float sum = 0.f;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < kAttnWaves; ++w) {
        const float f = exp2f(mw[w] - ref);
        sum += sm.merge.l[w][hn] * f;
        acc += *reinterpret_cast<const f32x4 *>(&sm.merge.o[w][hn][d0]) * f;
    }
    const int q_out = SHARED ? 2 * iq + (hn >= kPairHeads ? 1 : 0) : iq;
    const int h_out = SHARED ? (hn & (kPairHeads - 1)) : hb * kAttnHeadBlock + hn;
    const bool out_ok = h_out < a.group && q_out < a.nq;
    const int head_out = g * a.group + h_out;
    float *dst = a.out + ((int64_t)q_out * a.n_heads + head_out) * 128 + d0;
    float *dst_lse = a.lse ? a.lse + (int64_t)q_out * a.n_heads + head_out : nullptr;
    if (a.n_chunks == 1) {
        if (out_ok)
            finish(acc, sum, ref, dst, d0 == 0 ? dst_lse : nullptr);
        return;
    }
    // This chunk's partial; attn_merge_kernel combines the chunks.
    const int64_t slot = ((int64_t)unit * a.n_chunks + chunk) * kAttnHeadBlock + hn;
    *reinterpret_cast<f32x4 *>(a.part_o + slot * 128 + d0) = acc;
    if (d0 == 0)
        a.part_ml[slot] = make_float2(big, sum);
}

// One workgroup per (unit, column of the block): merges the unit's chunks.
// Every chunk's partial is loaded before any is used, so the loads overlap.
template <bool SHARED>
__global__ __launch_bounds__(128) void attn_merge_kernel(AttnArgs a)
{
    const int hn = blockIdx.x % kAttnHeadBlock;
    const int unit = blockIdx.x / kAttnHeadBlock;
    int u = unit;
    const int hb = u % a.hblocks;
    u /= a.hblocks;
    const int g = u % a.kv_heads;
    const int iu = u / a.kv_heads;
    const int iq = SHARED ? 2 * iu + (hn >= kPairHeads ? 1 : 0) : iu;
    const int hc = SHARED ? (hn & (kPairHeads - 1)) : hb * kAttnHeadBlock + hn;
    if (hc >= a.group || iq >= a.nq)
        return;
    const int head = g * a.group + hc;
    const int d = threadIdx.x;
    const int64_t slot0 = (int64_t)unit * a.n_chunks * kAttnHeadBlock + hn;
    float2 ml[kAttnMaxChunks];
    float po[kAttnMaxChunks];
#pragma unroll
    for (int c = 0; c < kAttnMaxChunks; ++c) {
        const int64_t sl = slot0 + (int64_t)min(c, a.n_chunks - 1) * kAttnHeadBlock;
        ml[c] = a.part_ml[sl];
        po[c] = a.part_o[sl * 128 + d];
    }
    float big = -INFINITY;
#pragma unroll
    for (int c = 0; c < kAttnMaxChunks; ++c)
        big = c < a.n_chunks ? fmaxf(big, ml[c].x) : big;
    const float ref = big == -INFINITY ? 0.f : big;
    float sum = 0.f, acc = 0.f;
#pragma unroll
    for (int c = 0; c < kAttnMaxChunks; ++c) {
        const float f = c < a.n_chunks ? exp2f(ml[c].x - ref) : 0.f;
        sum += ml[c].y * f;
        acc += po[c] * f;
    }
    a.out[((int64_t)iq * a.n_heads + head) * 128 + d] = sum > 0.f ? acc / sum : 0.f;
    if (a.lse && d == 0)
        a.lse[(int64_t)iq * a.n_heads + head] = sum > 0.f ? (ref + log2f(sum)) * 0.69314718055994531f : -INFINITY;
}

// ------------------------------------------------------------ pair merge
// One workgroup per pair of queries (2p, 2p+1): the pair's listed cells into
// one list of distinct cells (iree-org/wave issue #1257, section Shared block
// deduplication; the dedup index is an LDS hash). Entries are taken in the
// order query 2p's list, then query 2p+1's; each valid id (in [0, n_cells),
// position < width) goes into an open-addressing hash slot, whose counter
// counts the listings of each query. An entry is emitted if it is query 2p's
// or its cell is not in query 2p's list, marked with every query that lists
// the cell; its place in the merged list is the number of emitted entries
// before it, so the list depends only on the input. A query that lists a cell
// more than once must count it that often, so a pair with such a repeat is
// not merged: every valid entry is emitted, marked with its own query only.
constexpr int kUnionThreads = 1024;
constexpr int kUnionSlots = 4 * kPairMaxWidth;                    // twice a pair's entries at the longest width
constexpr uint32_t kUnionEmpty = 0xFFFFFFFFu;

template <int PER>  // entries per thread: 2 * width <= PER * kUnionThreads
__global__ __launch_bounds__(kUnionThreads) void attn_union_kernel(AttnArgs a)
{
    __shared__ uint32_t s_key[kUnionSlots];
    __shared__ uint32_t s_cnt[kUnionSlots];  // listings: query 2p in the low half, query 2p+1 in the high half
    __shared__ uint32_t s_wsum[kUnionThreads / 64];
    __shared__ uint32_t s_dup;
    const int p = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int W = a.src_width, E = 2 * W;
    const int T = 1 << a.slot_bits;
    const int32_t *row0 = a.src_ids + (int64_t)(2 * p) * a.src_ld;
    const bool has1 = 2 * p + 1 < a.nq;

    // Thread tid takes entries [tid * PER, tid * PER + PER) of the pair: query
    // 2p's positions, then 2p+1's. All its ids are loaded before the first
    // probe (a load behind a probing loop would wait for the loop).
    uint32_t id[PER];
    bool valid[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        const int e = tid * PER + j;
        const bool second = e >= W;
        const int pos = min(second ? e - W : e, W - 1);
        const int32_t x = (second && has1 ? row0 + a.src_ld : row0)[pos];
        valid[j] = e < E && (!second || has1) && (unsigned)x < (unsigned)a.n_cells;
        id[j] = (uint32_t)x;
    }
    for (int i = tid; i < T; i += kUnionThreads) {
        s_key[i] = kUnionEmpty;
        s_cnt[i] = 0u;
    }
    if (tid == 0)
        s_dup = 0u;
    __syncthreads();

    uint32_t slot[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        slot[j] = 0u;
        if (!valid[j])
            continue;
        const uint32_t qi = tid * PER + j >= W ? 1u : 0u;
        // Linear probing; the table holds at least twice the entries, so a
        // free or matching slot is always found within T probes.
        uint32_t h = (id[j] * 0x9E3779B1u) >> (32 - a.slot_bits);
        for (int it = 0; it < T; ++it) {
            uint32_t expect = kUnionEmpty;
            __hip_atomic_compare_exchange_strong(&s_key[h], &expect, id[j], __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_WORKGROUP);
            if (expect == kUnionEmpty || expect == id[j])
                break;
            h = (h + 1u) & (uint32_t)(T - 1);
        }
        slot[j] = h;
        const uint32_t old =
            __hip_atomic_fetch_add(&s_cnt[h], qi ? 0x10000u : 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        if (((old >> (16 * qi)) & 0xFFFFu) != 0u)
            __hip_atomic_store(&s_dup, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
    __syncthreads();
    const bool dup = s_dup != 0u;

    uint32_t packed[PER];
    uint32_t mine = 0u;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        const bool second = tid * PER + j >= W;
        const uint32_t c = valid[j] ? s_cnt[slot[j]] : 0u;
        const bool emit = valid[j] && (dup || !second || (c & 0xFFFFu) == 0u);
        const uint32_t mask = dup ? (second ? 2u : 1u) : (second ? 2u : (1u | ((c >> 16) != 0u ? 2u : 0u)));
        packed[j] = emit ? (id[j] | (mask << kPairIdBits)) : kUnionEmpty;
        mine += emit ? 1u : 0u;
    }
    // Places: exclusive prefix of the emitted counts in entry order.
    const uint32_t incl = wave_incl_sum(mine);
    if (lane == 63)
        s_wsum[wv] = incl;
    __syncthreads();
    uint32_t base = incl - mine;
    uint32_t total = 0u;
#pragma unroll
    for (int w = 0; w < kUnionThreads / 64; ++w) {
        const uint32_t c = s_wsum[w];
        base += w < wv ? c : 0u;
        total += c;
    }
    int32_t *dst = a.union_ids + (int64_t)p * a.width;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        if (packed[j] != kUnionEmpty)
            dst[base++] = (int32_t)packed[j];
    }
    if (tid == 0)
        a.union_len[p] = (int32_t)total;
}

} // namespace

bool make_attn_plan(int32_t nq, int32_t n_heads, int32_t kv_heads, int32_t width, AttnPlan &p, bool shared)
{
    p = AttnPlan{};
    if (nq < 0 || n_heads < 1 || kv_heads < 1 || n_heads % kv_heads != 0 || width < 1)
        return false;
    const int32_t group = n_heads / kv_heads;
    int32_t list = width;  // length of the lists the units walk, at most
    if (shared) {
        // A pair's heads fill the 16 columns; its merged list is at most
        // twice the width, hashed into at least twice that many slots.
        if (group > kPairHeads || width > kPairMaxWidth)
            return false;
        p.shared = 1;
        p.pairs = nq / 2 + (nq & 1);
        p.hblocks = 1;
        p.units = (int64_t)p.pairs * kv_heads;
        list = 2 * width;
        int bits = 8;
        while ((1 << bits) < 2 * list)
            ++bits;
        p.slot_bits = bits;
    } else {
        p.hblocks = (group + kAttnHeadBlock - 1) / kAttnHeadBlock;
        p.units = (int64_t)nq * kv_heads * p.hblocks;
    }
    // (64-bit: width may be as large as 2^31 - 1.)
    const int64_t steps = ((int64_t)list + kAttnStepCells - 1) / kAttnStepCells;
    const int64_t max_chunks = (steps + kAttnWaves - 1) / kAttnWaves;
    int64_t chunks = p.units > 0 ? (kAttnTargetGroups + p.units - 1) / p.units : 1;
    chunks = chunks < 1 ? 1 : (chunks > max_chunks ? max_chunks : chunks);
    chunks = chunks > kAttnMaxChunks ? kAttnMaxChunks : chunks;  // the merge loads every partial at once
    p.steps_per_wave = (int32_t)((steps + kAttnWaves * chunks - 1) / (kAttnWaves * chunks));
    p.n_chunks = (int32_t)((steps + (int64_t)kAttnWaves * p.steps_per_wave - 1) /
                           ((int64_t)kAttnWaves * p.steps_per_wave));
    if (p.units * p.n_chunks * kAttnHeadBlock > 0x7fffffffLL)
        return false;
    size_t off = 0;
    if (p.n_chunks > 1) {
        const size_t parts = (size_t)p.units * p.n_chunks * kAttnHeadBlock;
        p.ml_offset = 0;
        p.o_offset = (parts * sizeof(float2) + 255) / 256 * 256;
        off = p.o_offset + parts * 128 * sizeof(float);
    }
    if (shared) {
        const size_t q = (size_t)(p.pairs > 0 ? p.pairs : 1);
        p.union_offset = (off + 255) / 256 * 256;
        p.len_offset = (p.union_offset + q * (size_t)list * 4 + 255) / 256 * 256;
        off = p.len_offset + q * 4;
    }
    p.bytes = off;
    return true;
}

hipError_t launch_attention(const AttnArgs &a, const AttnPlan &p, hipStream_t s)
{
    if (p.shared) {
        const int entries = 2 * a.src_width;  // <= 2 * kPairMaxWidth = 8 * kUnionThreads
        if (entries <= kUnionThreads)
            hipLaunchKernelGGL(attn_union_kernel<1>, dim3((unsigned)p.pairs), dim3(kUnionThreads), 0, s, a);
        else if (entries <= 2 * kUnionThreads)
            hipLaunchKernelGGL(attn_union_kernel<2>, dim3((unsigned)p.pairs), dim3(kUnionThreads), 0, s, a);
        else if (entries <= 4 * kUnionThreads)
            hipLaunchKernelGGL(attn_union_kernel<4>, dim3((unsigned)p.pairs), dim3(kUnionThreads), 0, s, a);
        else
            hipLaunchKernelGGL(attn_union_kernel<8>, dim3((unsigned)p.pairs), dim3(kUnionThreads), 0, s, a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
        hipLaunchKernelGGL(attn_kernel<true>, dim3((unsigned)(p.units * p.n_chunks)), dim3(kThreads), 0, s, a);
        e = hipGetLastError();
        if (e != hipSuccess || p.n_chunks == 1)
            return e;
        hipLaunchKernelGGL(attn_merge_kernel<true>, dim3((unsigned)(p.units * kAttnHeadBlock)), dim3(128), 0, s, a);
        return hipGetLastError();
    }
    hipLaunchKernelGGL(attn_kernel<false>, dim3((unsigned)(p.units * p.n_chunks)), dim3(kThreads), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.n_chunks == 1)
        return e;
    hipLaunchKernelGGL(attn_merge_kernel<false>, dim3((unsigned)(p.units * kAttnHeadBlock)), dim3(128), 0, s, a);
    return hipGetLastError();
}

} // namespace qsa
