// attn_kernels.hip - attention of every query head over the cells its query
// selected: the consumer of the block selection (iree-org/wave issue #1257
// "NSA: LDS optimization for block-gather in selection attention", sections
// Problem and Per-block LDS staging). Heads of one group share a key/value
// head; for query q and head h of key/value head g:
//     out[q][h] = sum_c softmax_c(scale * q[q][h] . k[c][g]) * v[c][g]
// over the listed cells c, and lse[q][h] = log sum_c exp(scale * q . k).
//
// Work unit: one query, one key/value head, a block of up to 16 of its query
// heads and a chunk of the query's id list. A workgroup of four waves takes a
// unit; each wave walks 32-cell steps of the chunk with its own running
// softmax (max, sum, output) and the four are merged in LDS at the end.
// Several chunks per unit are merged by attn_combine_kernel.
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
//    The cells are the contraction, so V is transposed through LDS (cell
//    pairs packed per dword) and P comes straight from the S^T registers:
//    contraction position 8j+i is cell 4j+i of the step's first 16 cells and
//    8j+4+i is cell 16+4j+i. P is split into a bfloat16 head and tail
//    (hi + lo equals p to about 2^-17 relative) and both are multiplied, so
//    the weighted sum keeps close to FP32 accuracy.
#include <math.h>

#include "qsa_internal.h"

namespace qsa {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 64 * kAttnWaves;
// V^T rows: 16 dwords (32 cells as bfloat16 pairs) + 2 of padding, and 16
// more dwords after every 32 rows, so that the four lane groups' packed
// writes and the matrix-core operand reads fall in distinct banks.
constexpr int kVtPitch = 18;
constexpr int kVtWords = 128 * kVtPitch + 4 * 16;
constexpr int kOPitch = 132;  // floats per head row of the merge buffer

__device__ __forceinline__ int vt_index(int row, int pair) { return row * kVtPitch + (row >> 5) * 16 + pair; }

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

// A listed id selects a cell when it lies in [0, n_cells); position p of the
// list counts when p < width.
__device__ __forceinline__ int cell_at(const int32_t *row, int p, int width, int n_cells, bool &ok)
{
    const int id = row[min(p, width - 1)];
    ok = p < width && (unsigned)id < (unsigned)n_cells;
    return ok ? id : 0;
}

__global__ __launch_bounds__(kThreads) void attn_kernel(AttnArgs a)
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

    // This lane's matrix-core column: query head hb*16 + n of the group.
    const bool head_ok = hb * kAttnHeadBlock + n < a.group;
    const int head = g * a.group + (head_ok ? hb * kAttnHeadBlock + n : 0);
    bf16x8 qb[4];
    {
        const uint4 *qp = reinterpret_cast<const uint4 *>(a.q + ((int64_t)iq * a.n_heads + head) * 128 + 32 * lg);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            uint4 x = qp[s];
            if (!head_ok)
                x = make_uint4(0, 0, 0, 0);
            qb[s] = as_bf16x8(x);
        }
    }

    float m = -INFINITY, l = 0.f;
    f32x4 o[8];
#pragma unroll
    for (int t = 0; t < 8; ++t)
        o[t] = f32x4{0.f, 0.f, 0.f, 0.f};

    uint32_t *vt = sm.vt[wv];
    const int32_t *idrow = a.ids + (int64_t)iq * a.ld_ids;
    const int64_t kv_row = (int64_t)a.kv_heads * 128;
    const int step0 = (chunk * kAttnWaves + wv) * a.steps_per_wave;
    for (int j = 0; j < a.steps_per_wave; ++j) {
        const int c0 = (step0 + j) * kAttnStepCells;
        if (c0 >= a.width)
            break;  // wave-uniform
        bool va, vb, v0ok, v1ok;
        const int ida = cell_at(idrow, c0 + n, a.width, a.n_cells, va);
        const int idb = cell_at(idrow, c0 + 16 + n, a.width, a.n_cells, vb);
        const int iv0 = cell_at(idrow, c0 + 2 * n, a.width, a.n_cells, v0ok);
        const int iv1 = cell_at(idrow, c0 + 2 * n + 1, a.width, a.n_cells, v1ok);
        const int64_t head_off = (int64_t)g * 128 + 32 * lg;
        const uint4 *kap = reinterpret_cast<const uint4 *>(a.k + ida * kv_row + head_off);
        const uint4 *kbp = reinterpret_cast<const uint4 *>(a.k + idb * kv_row + head_off);
        const uint4 *v0p = reinterpret_cast<const uint4 *>(a.v + iv0 * kv_row + head_off);
        const uint4 *v1p = reinterpret_cast<const uint4 *>(a.v + iv1 * kv_row + head_off);
        uint4 ka[4], kb[4], v0[4], v1[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            ka[s] = kap[s];
            kb[s] = kbp[s];
        }
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            v0[s] = v0p[s];
            v1[s] = v1p[s];
        }

        f32x4 sa = {0.f, 0.f, 0.f, 0.f}, sb = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            sa = mfma(as_bf16x8(ka[s]), qb[s], sa);
            sb = mfma(as_bf16x8(kb[s]), qb[s], sb);
        }

        // Lanes 0-15 hold cells 0-15 of each half: bit c of the ballot is the
        // validity of cell c.
        const uint64_t ma = __ballot(va), mb = __ballot(vb);
        float x[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[i] = ((ma >> (4 * lg + i)) & 1) ? sa[i] * a.scale_log2 : -INFINITY;
            x[4 + i] = ((mb >> (4 * lg + i)) & 1) ? sb[i] * a.scale_log2 : -INFINITY;
        }
        float smax = x[0];
#pragma unroll
        for (int i = 1; i < 8; ++i)
            smax = fmaxf(smax, x[i]);
        smax = fmaxf(smax, __shfl_xor(smax, 16));
        smax = fmaxf(smax, __shfl_xor(smax, 32));
        const float mnew = fmaxf(m, smax);
        const float mref = mnew == -INFINITY ? 0.f : mnew;
        const float alpha = exp2f(m - mref);
        float psum = 0.f;
        bf16x8 ph, pl;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float p = exp2f(x[i] - mref);
            psum += p;
            const __bf16 hi = (__bf16)p;
            ph[i] = hi;
            pl[i] = (__bf16)(p - (float)hi);
        }
        l = l * alpha + psum;
        m = mnew;
#pragma unroll
        for (int t = 0; t < 8; ++t)
            o[t] *= alpha;

        // V^T into LDS: this lane holds cells 2n and 2n+1, dims 32lg .. 32lg+31.
        {
            const uint32_t *w0 = reinterpret_cast<const uint32_t *>(v0);
            const uint32_t *w1 = reinterpret_cast<const uint32_t *>(v1);
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int row = 32 * lg + 2 * e;
                vt[vt_index(row, n)] = (w0[e] & 0xFFFFu) | (w1[e] << 16);
                vt[vt_index(row + 1, n)] = (w0[e] >> 16) | (w1[e] & 0xFFFF0000u);
            }
        }
        // The wave reads what its own lanes wrote (LDS keeps a wave's order).
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const int row = 16 * t + n;
            const uint2 lo = *reinterpret_cast<const uint2 *>(&vt[vt_index(row, 2 * lg)]);
            const uint2 hi = *reinterpret_cast<const uint2 *>(&vt[vt_index(row, 8 + 2 * lg)]);
            const bf16x8 av = as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
            o[t] = mfma(av, ph, o[t]);
            o[t] = mfma(av, pl, o[t]);
        }
        __builtin_amdgcn_wave_barrier();
    }
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);

    // Merge the four waves.
    __syncthreads();  // every wave is done with its V^T rows
    if (lg == 0) {
        sm.merge.m[wv][n] = m;
        sm.merge.l[wv][n] = l;
    }
#pragma unroll
    for (int t = 0; t < 8; ++t)
        *reinterpret_cast<f32x4 *>(&sm.merge.o[wv][n][16 * t + 4 * lg]) = o[t];
    __syncthreads();

    const int hn = threadIdx.x >> 4, d0 = (threadIdx.x & 15) * 8;
    float mw[kAttnWaves], big = -INFINITY;
#pragma unroll
    for (int w = 0; w < kAttnWaves; ++w) {
        mw[w] = sm.merge.m[w][hn];
        big = fmaxf(big, mw[w]);
    }
    const float ref = big == -INFINITY ? 0.f : big;
    float sum = 0.f, acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e)
        acc[e] = 0.f;
#pragma unroll
    for (int w = 0; w < kAttnWaves; ++w) {
        const float f = exp2f(mw[w] - ref);
        sum += sm.merge.l[w][hn] * f;
#pragma unroll
        for (int e = 0; e < 8; ++e)
            acc[e] += sm.merge.o[w][hn][d0 + e] * f;
    }
    if (hb * kAttnHeadBlock + hn >= a.group)
        return;
    const int head_out = g * a.group + hb * kAttnHeadBlock + hn;
    if (a.n_chunks == 1) {
        float4 *dst = reinterpret_cast<float4 *>(a.out + ((int64_t)iq * a.n_heads + head_out) * 128 + d0);
        if (sum > 0.f) {
            dst[0] = make_float4(acc[0] / sum, acc[1] / sum, acc[2] / sum, acc[3] / sum);
            dst[1] = make_float4(acc[4] / sum, acc[5] / sum, acc[6] / sum, acc[7] / sum);
        } else {
            dst[0] = make_float4(0.f, 0.f, 0.f, 0.f);
            dst[1] = make_float4(0.f, 0.f, 0.f, 0.f);
        }
        if (a.lse && d0 == 0)
            a.lse[(int64_t)iq * a.n_heads + head_out] =
                sum > 0.f ? (ref + log2f(sum)) * 0.69314718055994531f : -INFINITY;
    } else {
        const int64_t slot = ((int64_t)unit * a.n_chunks + chunk) * kAttnHeadBlock + hn;
        float4 *dst = reinterpret_cast<float4 *>(a.part_o + slot * 128 + d0);
        dst[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
        dst[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
        if (d0 == 0)
            a.part_ml[slot] = make_float2(big, sum);
    }
}

// One workgroup per (unit, head of the block): merges the unit's chunks.
__global__ __launch_bounds__(128) void attn_combine_kernel(AttnArgs a)
{
    const int hn = blockIdx.x % kAttnHeadBlock;
    const int unit = blockIdx.x / kAttnHeadBlock;
    int u = unit;
    const int hb = u % a.hblocks;
    u /= a.hblocks;
    const int g = u % a.kv_heads;
    const int iq = u / a.kv_heads;
    if (hb * kAttnHeadBlock + hn >= a.group)
        return;
    const int head = g * a.group + hb * kAttnHeadBlock + hn;
    const int d = threadIdx.x;
    const int64_t slot0 = (int64_t)unit * a.n_chunks * kAttnHeadBlock + hn;
    float big = -INFINITY;
    for (int c = 0; c < a.n_chunks; ++c)
        big = fmaxf(big, a.part_ml[slot0 + (int64_t)c * kAttnHeadBlock].x);
    const float ref = big == -INFINITY ? 0.f : big;
    float sum = 0.f, acc = 0.f;
    for (int c = 0; c < a.n_chunks; ++c) {
        const int64_t slot = slot0 + (int64_t)c * kAttnHeadBlock;
        const float2 ml = a.part_ml[slot];
        const float f = exp2f(ml.x - ref);
        sum += ml.y * f;
        acc += a.part_o[slot * 128 + d] * f;
    }
    a.out[((int64_t)iq * a.n_heads + head) * 128 + d] = sum > 0.f ? acc / sum : 0.f;
    if (a.lse && d == 0)
        a.lse[(int64_t)iq * a.n_heads + head] = sum > 0.f ? (ref + log2f(sum)) * 0.69314718055994531f : -INFINITY;
}

} // namespace

bool make_attn_plan(int32_t nq, int32_t n_heads, int32_t kv_heads, int32_t width, AttnPlan &p)
{
    p = AttnPlan{};
    if (nq < 0 || n_heads < 1 || kv_heads < 1 || n_heads % kv_heads != 0 || width < 1)
        return false;
    const int32_t group = n_heads / kv_heads;
    p.hblocks = (group + kAttnHeadBlock - 1) / kAttnHeadBlock;
    p.units = (int64_t)nq * kv_heads * p.hblocks;
    const int32_t steps = (width + kAttnStepCells - 1) / kAttnStepCells;
    const int32_t max_chunks = (steps + kAttnWaves - 1) / kAttnWaves;
    int64_t chunks = p.units > 0 ? (kAttnTargetGroups + p.units - 1) / p.units : 1;
    chunks = chunks < 1 ? 1 : (chunks > max_chunks ? max_chunks : chunks);
    p.steps_per_wave = (int32_t)((steps + kAttnWaves * chunks - 1) / (kAttnWaves * chunks));
    p.n_chunks = (steps + kAttnWaves * p.steps_per_wave - 1) / (kAttnWaves * p.steps_per_wave);
    if (p.units * p.n_chunks * kAttnHeadBlock > 0x7fffffffLL)
        return false;
    if (p.n_chunks > 1) {
        const size_t parts = (size_t)p.units * p.n_chunks * kAttnHeadBlock;
        p.ml_offset = 0;
        p.o_offset = (parts * sizeof(float2) + 255) / 256 * 256;
        p.bytes = p.o_offset + parts * 128 * sizeof(float);
    }
    return true;
}

hipError_t launch_attention(const AttnArgs &a, const AttnPlan &p, hipStream_t s)
{
    const int64_t groups = p.units * p.n_chunks;
    hipLaunchKernelGGL(attn_kernel, dim3((unsigned)groups), dim3(kThreads), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.n_chunks == 1)
        return e;
    hipLaunchKernelGGL(attn_combine_kernel, dim3((unsigned)(p.units * kAttnHeadBlock)), dim3(128), 0, s, a);
    return hipGetLastError();
}

} // namespace qsa
