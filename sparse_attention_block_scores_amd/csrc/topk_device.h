// topk_device.h - workgroup-level building blocks of the block top-k on gfx950.
//
// The selection rule (Strata pull #3987, section Approach; Strata pull #2093
// "sm_75: the prompt path's top-k with one full read of the scores", section
// Beschreibung): with r the number of blocks a selection touches, T is the
// r-th largest block key; blocks above T are taken, then blocks equal to T in
// ascending block order until r blocks are taken; the last block taken in
// that order may contribute only part of its cells. Everything below works on
// 32-bit order-preserving block keys, so "largest" is plain unsigned order.
//
// Radix select. Each digit is a 256-bin LDS histogram of the keys still in
// play, and a scan of the bins from the top picks the bin holding the target
// rank (the pages pick every digit with a parallel scan of 256 bins, Strata
// pull #3987, section Approach). Digits are taken over the keys' actual range
// [min, max] rather than at fixed bit positions: the first digit splits the
// range into 256 equal bins, the next splits the chosen bin, and so on, so a
// narrow range needs fewer passes and equal keys need none.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qsa {

constexpr int kWave = 64;

// Order-preserving image of an FP32 key in uint32 (-0.0 folded onto +0.0).
__device__ __forceinline__ uint32_t key_of(float f)
{
    uint32_t b = __float_as_uint(f);
    b = (b == 0x80000000u) ? 0u : b;
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// The float with that image (inverse of key_of; -0.0 comes back as +0.0).
__device__ __forceinline__ float float_of(uint32_t key)
{
    return __uint_as_float((key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key);
}

__device__ __forceinline__ int lane_id() { return (int)__lane_id(); }
// Wave index in the workgroup, as a wave-uniform (scalar) value.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave)); }

__device__ __forceinline__ uint64_t lanes_below()
{
    const int l = lane_id();
    return l == 0 ? 0ull : (~0ull >> (64 - l));
}

// Set bits of a wave mask in the lanes below this one (v_mbcnt).
__device__ __forceinline__ uint32_t count_below(uint64_t mask)
{
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// ------------------------------------------------------------ wave scans
// Row shifts within rows of 16 lanes, then the row broadcasts join rows
// (0,1) and (2,3), then the two halves. Lanes a shift does not reach add 0.
__device__ __forceinline__ uint32_t wave_incl_sum(uint32_t x)
{
    x += __builtin_amdgcn_update_dpp(0u, x, 0x111, 0xF, 0xF, false);  // row_shr:1
    x += __builtin_amdgcn_update_dpp(0u, x, 0x112, 0xF, 0xF, false);  // row_shr:2
    x += __builtin_amdgcn_update_dpp(0u, x, 0x114, 0xF, 0xF, false);  // row_shr:4
    x += __builtin_amdgcn_update_dpp(0u, x, 0x118, 0xF, 0xF, false);  // row_shr:8
    x += __builtin_amdgcn_update_dpp(0u, x, 0x142, 0xA, 0xF, false);  // row_bcast:15
    x += __builtin_amdgcn_update_dpp(0u, x, 0x143, 0xC, 0xF, false);  // row_bcast:31
    return x;
}

__device__ __forceinline__ uint32_t wave_incl_max(uint32_t x)
{
    x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0u, x, 0x111, 0xF, 0xF, false));
    x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0u, x, 0x112, 0xF, 0xF, false));
    x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0u, x, 0x114, 0xF, 0xF, false));
    x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0u, x, 0x118, 0xF, 0xF, false));
    x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0u, x, 0x142, 0xA, 0xF, false));
    x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0u, x, 0x143, 0xC, 0xF, false));
    return x;
}

// Sum of x over lanes 0-15 (the first row), in every lane.
__device__ __forceinline__ uint32_t row0_sum(uint32_t x)
{
    x += __builtin_amdgcn_update_dpp(0u, x, 0x111, 0xF, 0xF, false);  // row_shr:1
    x += __builtin_amdgcn_update_dpp(0u, x, 0x112, 0xF, 0xF, false);  // row_shr:2
    x += __builtin_amdgcn_update_dpp(0u, x, 0x114, 0xF, 0xF, false);  // row_shr:4
    x += __builtin_amdgcn_update_dpp(0u, x, 0x118, 0xF, 0xF, false);  // row_shr:8
    return (uint32_t)__builtin_amdgcn_readlane((int)x, 15);
}

// Largest x over lanes 0-15, in every lane.
__device__ __forceinline__ uint32_t row0_max(uint32_t x)
{
    x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0u, x, 0x111, 0xF, 0xF, false));
    x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0u, x, 0x112, 0xF, 0xF, false));
    x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0u, x, 0x114, 0xF, 0xF, false));
    x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0u, x, 0x118, 0xF, 0xF, false));
    return (uint32_t)__builtin_amdgcn_readlane((int)x, 15);
}

__device__ __forceinline__ uint32_t wave_sum(uint32_t x)
{
    return (uint32_t)__builtin_amdgcn_readlane((int)wave_incl_sum(x), 63);
}

__device__ __forceinline__ uint32_t wave_max(uint32_t x)
{
    return (uint32_t)__builtin_amdgcn_readlane((int)wave_incl_max(x), 63);
}

// min(a) == ~max(~a)
__device__ __forceinline__ uint32_t wave_min(uint32_t x) { return ~wave_max(~x); }

// Workgroup barrier that orders LDS only: global loads stay in flight across
// it (a full __syncthreads() would first wait for every outstanding load).
__device__ __forceinline__ void lds_barrier()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ __forceinline__ void lds_add(uint32_t *p, uint32_t v)
{
    __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// Count digit d in an LDS histogram. Digits are taken over the keys' own range
// (see radix_select_range), so even skewed keys spread over many bins; equal
// keys never reach a histogram at all.
__device__ __forceinline__ void hist_add(uint32_t *hist, uint32_t d) { lds_add(&hist[d], 1u); }

// ------------------------------------------------------------ key sources
// Keys in LDS (16-byte aligned array).
// Fourth word of a raw buffer resource on gfx9-family GPUs (32-bit data
// format, no swizzle); with stride 0 a load at or past num_records bytes reads
// zero without a memory access.
constexpr int kRowBufferWord3 = 0x00020000;
// Cache-policy operand of a buffer load: nontemporal (the hint a
// __builtin_nontemporal_load gives a global load).
constexpr int kCachePolicyNontemporal = 2;

struct LdsKeys {
    const uint32_t *p;
    static constexpr bool vec = true;
    __device__ __forceinline__ uint4 load4(int i) const { return *reinterpret_cast<const uint4 *>(p + i); }
    __device__ __forceinline__ uint32_t load1(int i) const { return p[i]; }
};

// Keys already mapped, in global memory (16-byte aligned array).
struct GlobalKeys {
    const uint32_t *p;
    static constexpr bool vec = true;
    __device__ __forceinline__ uint4 load4(int i) const { return *reinterpret_cast<const uint4 *>(p + i); }
    __device__ __forceinline__ uint32_t load1(int i) const { return p[i]; }
};

// FP32 block scores in global memory, mapped on load. `aligned` means p is
// 16-byte aligned, so float4 loads are allowed at multiples of 4.
struct RowKeys {
    const float *p;
    bool aligned;
    static constexpr bool vec = false;  // decided at run time through `aligned`
    __device__ __forceinline__ uint4 load4(int i) const
    {
        const float4 f = *reinterpret_cast<const float4 *>(p + i);
        return make_uint4(key_of(f.x), key_of(f.y), key_of(f.z), key_of(f.w));
    }
    __device__ __forceinline__ uint32_t load1(int i) const { return key_of(p[i]); }
};

template <class Src>
__device__ __forceinline__ bool vector_ok(const Src &s)
{
    if constexpr (Src::vec)
        return true;
    else
        return s.aligned;
}

// f(key) for every key 0..n-1, in no particular order; vector loads, four
// in flight per thread.
template <int NT, class Src, class F>
__device__ __forceinline__ void for_each_key(const Src &src, int n, F f)
{
    if (vector_ok(src)) {
        const int n4 = n >> 2;
        int i = threadIdx.x;
        for (; i + 3 * NT < n4; i += 4 * NT) {
            const uint4 a = src.load4(4 * i), b = src.load4(4 * (i + NT));
            const uint4 c = src.load4(4 * (i + 2 * NT)), d = src.load4(4 * (i + 3 * NT));
            f(a.x); f(a.y); f(a.z); f(a.w);
            f(b.x); f(b.y); f(b.z); f(b.w);
            f(c.x); f(c.y); f(c.z); f(c.w);
            f(d.x); f(d.y); f(d.z); f(d.w);
        }
        for (; i < n4; i += NT) {
            const uint4 a = src.load4(4 * i);
            f(a.x); f(a.y); f(a.z); f(a.w);
        }
        for (int j = (n4 << 2) + (int)threadIdx.x; j < n; j += NT)
            f(src.load1(j));
    } else {
        int j = threadIdx.x;
        for (; j + 3 * NT < n; j += 4 * NT) {
            const uint32_t a = src.load1(j), b = src.load1(j + NT), c = src.load1(j + 2 * NT),
                           d = src.load1(j + 3 * NT);
            f(a); f(b); f(c); f(d);
        }
        for (; j < n; j += NT)
            f(src.load1(j));
    }
}

// ------------------------------------------------------------ shared state
constexpr int kDigitBits = 8;
constexpr int kBins = 1 << kDigitBits;
constexpr int kFineBits = 11;                        // fine bins: 2,048 ...
constexpr int kFineBins = 1 << kFineBits;
constexpr int kFinePerCoarse = kFineBins / kBins;    // ... in 256 coarse bins of 8

// LDS state of a selection, sized for workgroups of up to 16 waves.
struct SelectShared {
    static constexpr int NW = 16;
    alignas(16) uint32_t hist[3][kBins];  // rotating: fill one, pick from it, clear the one before
    alignas(16) uint32_t fine[kFineBins];
    alignas(16) uint32_t coarse[kBins];
    uint32_t small[kWave];                // keys of one fine bin
    uint32_t small_n;
    uint32_t bcast;                       // one value from one wave to all
    alignas(16) uint32_t pick[4];         // a pick from one wave to all
    uint32_t red[2][NW];
    uint32_t wave_ties[NW];
    uint32_t wave_gts[NW];
};

template <int NT>
__device__ __forceinline__ void clear_fine(SelectShared &sh)
{
    uint4 *f = reinterpret_cast<uint4 *>(sh.fine);
    for (int i = threadIdx.x; i < kFineBins / 4; i += NT)
        f[i] = make_uint4(0u, 0u, 0u, 0u);
    uint4 *c = reinterpret_cast<uint4 *>(sh.coarse);
    for (int i = threadIdx.x; i < kBins / 4; i += NT)
        c[i] = make_uint4(0u, 0u, 0u, 0u);
}

// Every histogram and counter of sh to zero (a barrier must follow).
template <int NT>
__device__ __forceinline__ void clear_hists(SelectShared &sh)
{
    uint4 *h = reinterpret_cast<uint4 *>(&sh.hist[0][0]);
    for (int i = threadIdx.x; i < 3 * kBins / 4; i += NT)
        h[i] = make_uint4(0u, 0u, 0u, 0u);
    clear_fine<NT>(sh);
    if (threadIdx.x == 0)
        sh.small_n = 0;
}

template <int NT>
__device__ __forceinline__ void clear_hist(SelectShared &sh, int which)
{
    uint4 *h = reinterpret_cast<uint4 *>(&sh.hist[which][0]);
    for (int i = threadIdx.x; i < kBins / 4; i += NT)
        h[i] = make_uint4(0u, 0u, 0u, 0u);
}

// Workgroup min and max of a per-thread pair (all threads call).
template <int NT>
__device__ __forceinline__ void wg_minmax(uint32_t lo, uint32_t hi, SelectShared &sh, uint32_t &mn,
                                          uint32_t &mx)
{
    constexpr int NW = NT / kWave;
    lo = wave_min(lo);
    hi = wave_max(hi);
    if (lane_id() == 0) {
        sh.red[0][wave_id()] = lo;
        sh.red[1][wave_id()] = hi;
    }
    lds_barrier();
    // Lane w < NW reads wave w's; one row reduction each (max(~x) = ~min).
    static_assert(NW <= 16, "wave results fit one row of lanes");
    const int l = lane_id();
    const bool in = l < NW;
    mn = ~row0_max(in ? ~sh.red[0][l & 15] : 0u);
    mx = row0_max(in ? sh.red[1][l & 15] : 0u);
    lds_barrier();
}

// The bin of a histogram of BINS bins (highest bin first) that holds rank r,
// and the count of everything in higher bins. Every wave computes it on its
// own: lane l owns the BINS/64 bins just below the (BINS/64)*l highest.
template <int BINS = kBins>
__device__ __forceinline__ void wave_pick(const uint32_t *hist, uint32_t r, uint32_t &bin, uint32_t &higher)
{
    constexpr int PL = BINS / kWave;
    static_assert(PL % 4 == 0, "16-byte reads of each lane's bins");
    const int lane = lane_id();
    const int lo_bin = BINS - PL * (lane + 1);
    uint32_t c[PL];
#pragma unroll
    for (int i = 0; i < PL / 4; ++i) {
        const uint4 v = *reinterpret_cast<const uint4 *>(hist + lo_bin + 4 * i);
        c[4 * i] = v.x; c[4 * i + 1] = v.y; c[4 * i + 2] = v.z; c[4 * i + 3] = v.w;
    }
    uint32_t mine = 0;
#pragma unroll
    for (int i = 0; i < PL; ++i)
        mine += c[i];
    const uint32_t before = wave_incl_sum(mine) - mine;
    const uint64_t hit = __ballot(before < r && r <= before + mine);
    const int L = hit ? (int)__ffsll((unsigned long long)hit) - 1 : 0;
    // In the lane that holds rank r, walk its bins from the highest down.
    uint32_t cum = before, my_bin = 0, my_higher = 0;
#pragma unroll
    for (int i = PL - 1; i >= 0; --i) {
        if (cum < r && r <= cum + c[i]) {
            my_bin = (uint32_t)(lo_bin + i);
            my_higher = cum;
        }
        cum += c[i];
    }
    bin = (uint32_t)__builtin_amdgcn_readlane((int)my_bin, L);
    higher = (uint32_t)__builtin_amdgcn_readlane((int)my_higher, L);
}

// The fine bin holding rank r (1-based) by way of the coarse bins (fine bin f
// lies in coarse bin f / kFinePerCoarse): its index, its count, and the count
// of everything in higher fine bins. Every wave computes it on its own.
template <int NT>
__device__ __forceinline__ void pick_fine(const SelectShared &sh, uint32_t r, uint32_t &fb, uint32_t &c,
                                          uint32_t &above)
{
    uint32_t cb, h;
    wave_pick(sh.coarse, r, cb, h);
    uint32_t f[kFinePerCoarse];
#pragma unroll
    for (int i = 0; i < kFinePerCoarse / 4; ++i) {
        const uint4 v = *reinterpret_cast<const uint4 *>(sh.fine + cb * kFinePerCoarse + 4 * i);
        f[4 * i] = v.x; f[4 * i + 1] = v.y; f[4 * i + 2] = v.z; f[4 * i + 3] = v.w;
    }
    fb = cb * kFinePerCoarse;
    c = 0;
    above = h;
    uint32_t cum = h;
    bool found = false;
#pragma unroll
    for (int i = kFinePerCoarse - 1; i >= 0; --i) {
        const bool here = !found && cum + f[i] >= r;
        fb = here ? cb * kFinePerCoarse + i : fb;
        c = here ? f[i] : c;
        above = here ? cum : above;
        found = found || here;
        cum += f[i];
    }
}

// Within one wave: the rank-th largest (1-based, 1 <= rank <= c) of the c <= 64
// keys in keys[0..c), and how many of them are strictly larger. Every lane
// counts the keys above and at its own key against all c keys in turn.
__device__ __forceinline__ void wave_rank_small(const uint32_t *keys, uint32_t c, uint32_t rank, uint32_t &T,
                                                uint32_t &n_above)
{
    const int lane = lane_id();
    const bool valid = lane < (int)c;
    const uint32_t x = valid ? keys[lane] : 0u;
    uint32_t gt = 0, ge = 0;
    for (uint32_t j = 0; j < c; ++j) {
        const uint32_t y = (uint32_t)__builtin_amdgcn_readlane((int)x, (int)j);
        gt += y > x ? 1u : 0u;
        ge += y >= x ? 1u : 0u;
    }
    const uint64_t hit = __ballot(valid && gt < rank && rank <= ge);
    const int L = hit ? (int)__ffsll((unsigned long long)hit) - 1 : 0;
    T = (uint32_t)__builtin_amdgcn_readlane((int)x, L);
    n_above = (uint32_t)__builtin_amdgcn_readlane((int)gt, L);
}

// The rank-th largest (1 <= rank <= c) of the c <= 64 keys of src for which
// member(k) holds, and how many of them lie above it: the members are gathered
// into sh.small in any order and one wave ranks them (every wave does, which
// saves a barrier). sh.small_n is zero on entry and again after the call's
// barrier.
template <int NT, class Src, class Member>
__device__ __forceinline__ void rank_members(const Src &src, int n, Member member, uint32_t c, uint32_t rank,
                                             SelectShared &sh, uint32_t &T, uint32_t &n_above)
{
    for_each_key<NT>(src, n, [&](uint32_t k) {
        if (member(k)) {
            const uint32_t pos = __hip_atomic_fetch_add(&sh.small_n, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            if (pos < (uint32_t)kWave)
                sh.small[pos] = k;
        }
    });
    lds_barrier();
    if (threadIdx.x == 0)
        sh.small_n = 0;
    wave_rank_small(sh.small, c, rank, T, n_above);
}

// Shift of the first digit over a key range of the given span (span > 0).
__device__ __forceinline__ int first_digit_shift(uint32_t span)
{
    const int bits = 32 - __clz(span);
    return bits > kDigitBits ? bits - kDigitBits : 0;
}

// Rank-th largest key (1-based, 1 <= rank <= n) among keys 0..n-1 of src, and
// the number of keys strictly above it. [kmin, kmax] must bound the keys.
// All threads call. The histograms must be zero on entry and a barrier must
// separate this call from any earlier one; they are zero again on return.
// Each pass costs one barrier: every wave picks the digit itself, and the
// histogram filled two passes earlier is cleared while the next one fills.
template <int NT, class Src>
__device__ __forceinline__ void radix_select_range(const Src &src, int n, uint32_t rank, uint32_t kmin,
                                                   uint32_t kmax, SelectShared &sh, uint32_t &T,
                                                   uint32_t &n_above)
{
    uint32_t lo = kmin, span = kmax - kmin, r = rank, above = 0;
    int p = 0;
    while (span != 0) {
        const int s = first_digit_shift(span);
        uint32_t *hist = sh.hist[p % 3];
        for_each_key<NT>(src, n, [&](uint32_t k) {
            const uint32_t sub = k - lo;
            if (sub <= span)
                hist_add(hist, sub >> s);
        });
        lds_barrier();
        uint32_t d, h;
        wave_pick(hist, r, d, h);
        clear_hist<NT>(sh, (p + 2) % 3);  // filled two passes ago; every wave has read it
        r -= h;
        above += h;
        lo += d << s;
        span = (s == 0) ? 0u : min(span - (d << s), (1u << s) - 1u);
        ++p;
    }
    if (p > 0) {
        lds_barrier();  // every wave is done reading the last histogram
        clear_hist<NT>(sh, (p - 1) % 3);
    }
    T = lo;
    n_above = above;
}

// Sum over the workgroup of one value per thread (all threads call).
template <int NT>
__device__ __forceinline__ uint32_t wg_sum(uint32_t v, SelectShared &sh)
{
    constexpr int NW = NT / kWave;
    v = wave_sum(v);
    if (lane_id() == 0)
        sh.red[0][wave_id()] = v;
    lds_barrier();
    uint32_t t = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w)
        t += sh.red[0][w];
    lds_barrier();
    return t;
}

// Number of keys of src[0..n) that are >= kp (all threads call).
template <int NT, class Src>
__device__ __forceinline__ uint32_t count_at_least(const Src &src, int n, uint32_t kp, SelectShared &sh)
{
    uint32_t c = 0;
    for_each_key<NT>(src, n, [&](uint32_t k) { c += k >= kp ? 1u : 0u; });
    return wg_sum<NT>(c, sh);
}

// Min and max key of src[0..n).
template <int NT, class Src>
__device__ __forceinline__ void key_range(const Src &src, int n, SelectShared &sh, uint32_t &mn, uint32_t &mx)
{
    uint32_t lo = 0xFFFFFFFFu, hi = 0u;
    for_each_key<NT>(src, n, [&](uint32_t k) {
        lo = min(lo, k);
        hi = max(hi, k);
    });
    wg_minmax<NT>(lo, hi, sh, mn, mx);
}

// Fine bin of a key among kFineBins bins of equal value width over
// [lo, lo + 2*d2] (lh = lo/2, inv = kFineBins/d2; halved operands keep the
// width finite for any finite range). Each step rounds monotonically, so the
// bin never decreases as the key grows: a bin's keys form an interval of
// keys. The explicit roundings keep every evaluation bit-identical.
__device__ __forceinline__ uint32_t value_fine_bin(uint32_t k, float lh, float inv)
{
    const float t = __fmul_rn(__fsub_rn(__fmul_rn(0.5f, float_of(k)), lh), inv);
    return (uint32_t)min(kFineBins - 1, max(0, (int)t));
}

// Rank-th largest key of src (see radix_select_range) among keys in [mn, mx].
// Ranges of more than 2^16 keys take one pass of 2,048 fine bins (in 256
// coarse ones) instead of 8-bit digits. Up to 2^27 keys (a few binades) the
// fine bins are the top bits of (key - min); wider ranges, such as signed
// normal-like keys spanning most binades, take bins of equal value width, as
// key bits would put a large share of the keys into a few bins. The fine bin
// that holds the rank usually holds a handful of keys, which one wave ranks
// exactly; a crowded one is an interval of keys, which radix digits finish.
template <int NT, class Src>
__device__ __forceinline__ void radix_select_in(const Src &src, int n, uint32_t rank, uint32_t mn, uint32_t mx,
                                                SelectShared &sh, uint32_t &T, uint32_t &n_above)
{
    const uint32_t span = mx - mn;
    const float lo = float_of(mn), hi = float_of(mx);
    const float lh = 0.5f * lo, d2 = 0.5f * hi - lh;
    const float inv = (float)kFineBins / d2;
    const bool by_value = span >= (1u << 27) && d2 > 0.0f && inv < __builtin_inff();
    if (span < (1u << 16) || (span >= (1u << 27) && !by_value)) {
        radix_select_range<NT>(src, n, rank, mn, mx, sh, T, n_above);
        return;
    }
    const int sF = (32 - __clz(span)) - kFineBits;  // >= 6 here
    auto fine_bin = [&](uint32_t k) { return by_value ? value_fine_bin(k, lh, inv) : (k - mn) >> sF; };
    for_each_key<NT>(src, n, [&](uint32_t k) {
        const uint32_t fb = fine_bin(k);
        lds_add(&sh.fine[fb], 1u);
        lds_add(&sh.coarse[fb / kFinePerCoarse], 1u);
    });
    lds_barrier();
    uint32_t fb, c, h;
    pick_fine<NT>(sh, rank, fb, c, h);
    uint32_t a2;
    if (c <= (uint32_t)kWave) {
        rank_members<NT>(src, n, [&](uint32_t k) { return fine_bin(k) == fb; }, c, rank - h, sh, T, a2);
        clear_fine<NT>(sh);  // after rank_members' barrier: every wave has picked
    } else {
        // The bin's keys: an interval, exact from the bits or from a min/max pass.
        uint32_t kmin_b = mn + (fb << sF), kmax_b = min(mx, kmin_b + ((1u << sF) - 1u));
        if (by_value) {
            uint32_t blo = 0xFFFFFFFFu, bhi = 0u;
            for_each_key<NT>(src, n, [&](uint32_t k) {
                const bool in = fine_bin(k) == fb;
                blo = in ? min(blo, k) : blo;
                bhi = in ? max(bhi, k) : bhi;
            });
            wg_minmax<NT>(blo, bhi, sh, kmin_b, kmax_b);
        } else {
            lds_barrier();  // every wave has picked before the bins are cleared
        }
        clear_fine<NT>(sh);
        radix_select_range<NT>(src, n, rank - h, kmin_b, kmax_b, sh, T, a2);
    }
    n_above = h + a2;
}

// radix_select_in over the keys' own range, found with one pass.
template <int NT, class Src>
__device__ __forceinline__ void radix_select(const Src &src, int n, uint32_t rank, SelectShared &sh,
                                             uint32_t &T, uint32_t &n_above)
{
    uint32_t mn, mx;
    key_range<NT>(src, n, sh, mn, mx);
    radix_select_in<NT>(src, n, rank, mn, mx, sh, T, n_above);
}

// Walk items 0..n-1 in order and take every item with key > T plus the first
// `tie_budget` items with key == T (tie_budget >= 1). Taken item i gets the
// output slot `first` (a running sum of weights: `unit` per taken item, except
// the last taken tie, which weighs `last_unit`), and emit(i, first, weight) is
// called for it. Waves own contiguous ranges of items, walked 256 at a time
// (four per lane); the only workgroup exchange is one round of per-wave counts.
template <int NT, class Src, class Emit>
__device__ __forceinline__ void ordered_take(const Src &src, int n, uint32_t T, uint32_t tie_budget, uint32_t unit,
                             uint32_t last_unit, SelectShared &sh, Emit emit)
{
    constexpr int NW = NT / kWave;
    constexpr int STEP = 4 * kWave;
    const int lane = lane_id(), wid = wave_id();
    const int per_wave = ((n + NW - 1) / NW + STEP - 1) / STEP * STEP;
    const int lo = wid * per_wave;
    const int hi = min(n, lo + per_wave);
    const bool vec = vector_ok(src);

    auto load = [&](int base, uint32_t k[4], bool ok[4]) {
        const int i0 = base + 4 * lane;
        if (vec && i0 + 3 < hi) {
            const uint4 v = src.load4(i0);
            k[0] = v.x; k[1] = v.y; k[2] = v.z; k[3] = v.w;
            ok[0] = ok[1] = ok[2] = ok[3] = true;
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                ok[j] = i0 + j < hi;
                k[j] = ok[j] ? src.load1(i0 + j) : 0u;
            }
        }
    };

    uint32_t ties = 0, gts = 0;
    for (int base = lo; base < hi; base += STEP) {
        uint32_t k[4];
        bool ok[4];
        load(base, k, ok);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            ties += (uint32_t)__popcll(__ballot(ok[j] && k[j] == T));
            gts += (uint32_t)__popcll(__ballot(ok[j] && k[j] > T));
        }
    }
    if (lane == 0) {
        sh.wave_ties[wid] = ties;
        sh.wave_gts[wid] = gts;
    }
    lds_barrier();
    uint32_t ties_before = 0, taken_before = 0;
#pragma unroll
    for (int v = 0; v < NW; ++v) {
        const uint32_t t = v < wid ? sh.wave_ties[v] : 0u;
        const uint32_t left = tie_budget > ties_before ? tie_budget - ties_before : 0u;
        taken_before += (v < wid ? sh.wave_gts[v] : 0u) + (t < left ? t : left);
        ties_before += t;
    }
    lds_barrier();
    if (gts == 0 && ties_before >= tie_budget)
        return;  // nothing of this wave's range is taken

    const uint32_t shortfall = unit - last_unit;
    bool short_seen = ties_before >= tie_budget;
    for (int base = lo; base < hi; base += STEP) {
        uint32_t k[4];
        bool ok[4];
        load(base, k, ok);
        bool tie[4], take[4], shrt[4];
        uint32_t own_ties = 0, own_take = 0;
        uint32_t tie_rank[4], take_rank[4];
        bool own_short_before[4];
        bool any_short_before = false;
        uint64_t tie_m[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            tie[j] = ok[j] && k[j] == T;
            tie_m[j] = __ballot(tie[j]);
        }
        uint32_t lanes_ties = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            lanes_ties += count_below(tie_m[j]);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            tie_rank[j] = ties_before + lanes_ties + own_ties;
            own_ties += tie[j] ? 1u : 0u;
            take[j] = ok[j] && (k[j] > T || (tie[j] && tie_rank[j] < tie_budget));
            shrt[j] = tie[j] && tie_rank[j] == tie_budget - 1;
        }
        uint64_t take_m[4], short_m = 0;
        uint32_t lanes_take = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            take_m[j] = __ballot(take[j]);
            lanes_take += count_below(take_m[j]);
            short_m |= __ballot(shrt[j]);
        }
        const bool short_in_lower_lanes = (short_m & lanes_below()) != 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            take_rank[j] = taken_before + lanes_take + own_take;
            own_take += take[j] ? 1u : 0u;
            own_short_before[j] = any_short_before;
            any_short_before = any_short_before || shrt[j];
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (take[j]) {
                const bool after = short_seen || short_in_lower_lanes || own_short_before[j];
                emit(base + 4 * lane + j, unit * take_rank[j] - (after ? shortfall : 0u),
                     shrt[j] ? last_unit : unit);
            }
        }
        uint32_t step_take = 0, step_ties = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            step_take += (uint32_t)__popcll(take_m[j]);
            step_ties += (uint32_t)__popcll(tie_m[j]);
        }
        taken_before += step_take;
        ties_before += step_ties;
        short_seen = short_seen || short_m != 0;
    }
}

// ordered_take for n <= PER * NT items, with one workgroup exchange: thread
// t holds items [PER*t, PER*t + PER) in registers, and one scan of (items
// above T, items equal to T) over the workgroup gives every taken item its
// slot. Same contract as ordered_take. Uses sh.red[0] until the caller's next
// barrier.
template <int NT, int PER, class Src, class Emit>
__device__ __forceinline__ void take_in_order(const Src &src, int n, uint32_t T, uint32_t tie_budget,
                                              uint32_t unit, uint32_t last_unit, SelectShared &sh, Emit emit)
{
    static_assert(PER % 4 == 0, "16-byte loads of each thread's items");
    constexpr int NW = NT / kWave;
    const int lane = lane_id(), wid = wave_id();
    const int c0 = (int)threadIdx.x * PER;
    const bool vec = vector_ok(src);
    uint32_t k[PER];
    bool v[PER];
#pragma unroll
    for (int u = 0; u < PER / 4; ++u) {
        const int i = c0 + 4 * u;
        if (vec && i + 3 < n) {
            const uint4 x = src.load4(i);
            k[4 * u] = x.x; k[4 * u + 1] = x.y; k[4 * u + 2] = x.z; k[4 * u + 3] = x.w;
            v[4 * u] = v[4 * u + 1] = v[4 * u + 2] = v[4 * u + 3] = true;
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                v[4 * u + j] = i + j < n;
                k[4 * u + j] = v[4 * u + j] ? src.load1(i + j) : 0u;
            }
        }
    }
    uint32_t gt = 0, tie = 0;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        gt += v[j] && k[j] > T ? 1u : 0u;
        tie += v[j] && k[j] == T ? 1u : 0u;
    }
    const uint32_t packed = gt | (tie << 16);  // both < 2^16 (n <= PER * NT)
    const uint32_t incl = wave_incl_sum(packed);
    if (lane == kWave - 1)
        sh.red[0][wid] = incl;
    lds_barrier();
    uint32_t before = incl - packed;
#pragma unroll
    for (int w = 0; w < NW; ++w)
        before += w < wid ? sh.red[0][w] : 0u;
    uint32_t ties_before = before >> 16;
    const uint32_t shortfall = unit - last_unit;
    uint32_t first = unit * ((before & 0xFFFFu) + min(ties_before, tie_budget)) -
                     (ties_before >= tie_budget ? shortfall : 0u);
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        uint32_t w = 0;
        if (v[j] && k[j] > T) {
            w = unit;
        } else if (v[j] && k[j] == T) {
            if (ties_before < tie_budget)
                w = ties_before == tie_budget - 1u ? last_unit : unit;
            ++ties_before;
        }
        if (w != 0u) {
            emit(c0 + j, first, w);
            first += w;
        }
    }
}

// The ordered take for any n: in registers up to 16 items per thread, else
// walked in ranges (ordered_take).
template <int NT, class Src, class Emit>
__device__ __forceinline__ void take_ordered(const Src &src, int n, uint32_t T, uint32_t tie_budget, uint32_t unit,
                                             uint32_t last_unit, SelectShared &sh, Emit emit)
{
    if (n <= 8 * NT)
        take_in_order<NT, 8>(src, n, T, tie_budget, unit, last_unit, sh, emit);
    else if (n <= 16 * NT)
        take_in_order<NT, 16>(src, n, T, tie_budget, unit, last_unit, sh, emit);
    else
        ordered_take<NT>(src, n, T, tie_budget, unit, last_unit, sh, emit);
}

// Cells of one taken block: `cnt` consecutive ids from cell0 at out[first],
// none at or past `limit`.
__device__ __forceinline__ void write_cells(int32_t *out, uint32_t first, uint32_t cnt, int32_t cell0,
                                            uint32_t limit)
{
    if (cnt == 4 && (first & 3u) == 0 && first + 4 <= limit) {
        *reinterpret_cast<int4 *>(out + first) = make_int4(cell0, cell0 + 1, cell0 + 2, cell0 + 3);
        return;
    }
    for (uint32_t j = 0; j < cnt; ++j)
        if (first + j < limit)
            out[first + j] = cell0 + (int32_t)j;
}

} // namespace qsa
