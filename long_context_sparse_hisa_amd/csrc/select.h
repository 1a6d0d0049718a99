// Workgroup-level top-n selection on register-held ranking keys.
//
// A workgroup of NT threads holds ITEMS keys per thread; key[it] of thread
// tid belongs to slot it*NT + tid.  Key 0 means "no candidate".  The n
// largest keys are selected, equal keys going to the lower slot, and handed
// to a callback with their rank in ascending slot order, so the output of a
// selection is ordered by slot without a sort.  Everything here is
// force-inlined so the key arrays stay in registers.
#pragma once

#include "common.h"

#define HISA_INLINE __device__ __attribute__((always_inline)) inline

namespace hisa {

// ---- workgroup scans for NT threads ------------------------------------------

template <int NT>
HISA_INLINE int wg_incl_scan(int v, int* scratch)
{
    constexpr int NW = NT / 64;
    int s = wave_incl_scan(v);
    if (lane_id() == 63) scratch[wave_id()] = s;
    __syncthreads();
    int add = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) add += w < wave_id() ? scratch[w] : 0;
    __syncthreads();
    return s + add;
}

template <int NT>
HISA_INLINE int wg_sum(int v, int* scratch)
{
    constexpr int NW = NT / 64;
    int s = wave_sum(v);
    if (lane_id() == 0) scratch[wave_id()] = s;
    __syncthreads();
    int tot = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) tot += scratch[w];
    __syncthreads();
    return tot;
}

// ---- radix select --------------------------------------------------------------

template <int NT, int ITEMS>
struct SelectSmem {
    static constexpr int NW = NT / 64;
    int hist[256];
    int cnt[2 * ITEMS * NW];
    int scratch[NW];
    int pick[2];
};

struct Threshold {
    uint32_t T;      // the n-th largest key (0 when every candidate is taken)
    int need_eq;     // how many keys equal to T are taken, lowest slots first
    bool all;        // n >= number of candidates: take every nonzero key
};

// 8 bits per pass from the top: after four passes the exact n-th largest
// key is known together with how many of its copies to take.
template <int NT, int ITEMS>
HISA_INLINE Threshold wg_radix_select(const uint32_t (&key)[ITEMS], int n, SelectSmem<NT, ITEMS>& sm)
{
    static_assert(NT >= 256, "one digit per thread");
    Threshold th;
    if (n <= 0) {
        th.T = 0xffffffffu;
        th.need_eq = 0;
        th.all = false;
        return th;
    }
    int nvalid = 0;
#pragma unroll
    for (int it = 0; it < ITEMS; ++it) nvalid += key[it] != 0u;
    nvalid = wg_sum<NT>(nvalid, sm.scratch);
    if (nvalid <= n) {
        th.T = 0u;
        th.need_eq = 0;
        th.all = true;
        return th;
    }
    uint32_t prefix = 0u, mask = 0u;
    int rem = n;
    for (int pass = 0; pass < 4; ++pass) {
        const int shift = 24 - 8 * pass;
        if (threadIdx.x < 256) sm.hist[threadIdx.x] = 0;
        __syncthreads();
#pragma unroll
        for (int it = 0; it < ITEMS; ++it) {
            const uint32_t kk = key[it];
            if (kk != 0u && (kk & mask) == prefix) atomicAdd(&sm.hist[(kk >> shift) & 255u], 1);
        }
        __syncthreads();
        // thread t < 256 looks at digit 255 - t; the scan counts keys whose
        // digit is >= that one
        const int h = threadIdx.x < 256 ? sm.hist[255 - threadIdx.x] : 0;
        const int cum = wg_incl_scan<NT>(h, sm.scratch);
        if (threadIdx.x < 256 && cum >= rem && cum - h < rem) {
            sm.pick[0] = 255 - (int)threadIdx.x;
            sm.pick[1] = cum - h;
        }
        __syncthreads();
        prefix |= (uint32_t)sm.pick[0] << shift;
        mask |= 0xffu << shift;
        rem -= sm.pick[1];
        __syncthreads();
    }
    th.T = prefix;
    th.need_eq = rem;
    th.all = false;
    return th;
}

// Hand every selected key to emit(slot, key, rank), rank = its position in
// ascending slot order among the selected.  Returns how many were selected.
template <int NT, int ITEMS, class Emit>
HISA_INLINE int wg_emit_selected(const uint32_t (&key)[ITEMS], const Threshold& th, SelectSmem<NT, ITEMS>& sm,
                                 Emit emit)
{
    constexpr int NW = NT / 64;
    constexpr int kEntries = ITEMS * NW;
    static_assert(kEntries <= NT, "one count entry per thread");
    const int w = wave_id();
#pragma unroll
    for (int it = 0; it < ITEMS; ++it) {
        const bool gt = key[it] > th.T;
        const bool eq = !th.all && key[it] == th.T;
        const uint64_t bg = __ballot(gt);
        const uint64_t be = __ballot(eq);
        if (lane_id() == 0) {
            sm.cnt[2 * (it * NW + w) + 0] = __popcll(bg);
            sm.cnt[2 * (it * NW + w) + 1] = __popcll(be);
        }
    }
    __syncthreads();
    // one scan over both counts, packed 16 + 16 bits (each total < 65536)
    const int e = threadIdx.x;
    const int g = e < kEntries ? sm.cnt[2 * e + 0] : 0;
    const int q = e < kEntries ? sm.cnt[2 * e + 1] : 0;
    const int packed = g | (q << 16);
    const int pi = wg_incl_scan<NT>(packed, sm.scratch);
    const int gi = pi & 0xffff, qi = (int)((uint32_t)pi >> 16);
    if (e < kEntries) {
        sm.cnt[2 * e + 0] = gi - g;
        sm.cnt[2 * e + 1] = qi - q;
    }
    if (e == NT - 1) {
        sm.pick[0] = gi;
        sm.pick[1] = qi;
    }
    __syncthreads();
    const int total = sm.pick[0] + min(sm.pick[1], th.need_eq);
#pragma unroll
    for (int it = 0; it < ITEMS; ++it) {
        const bool gt = key[it] > th.T;
        const bool eq = !th.all && key[it] == th.T;
        const uint64_t bg = __ballot(gt);
        const uint64_t be = __ballot(eq);
        const int pg = sm.cnt[2 * (it * NW + w) + 0] + __popcll(bg & lanemask_lt());
        const int pe = sm.cnt[2 * (it * NW + w) + 1] + __popcll(be & lanemask_lt());
        const int slot = it * NT + threadIdx.x;
        if (gt) emit(slot, key[it], pg + min(pe, th.need_eq));
        else if (eq && pe < th.need_eq) emit(slot, key[it], pg + pe);
    }
    __syncthreads();
    return total;
}

// ---- bucket select ---------------------------------------------------------------
// The same contract as wg_radix_select, in fewer passes for ordinary data:
// the candidate scores are spread over kBins equal-width bins between their
// minimum and maximum (a monotone map, so every key in a higher bin is
// larger than every key in a lower one and equal keys share a bin), one
// histogram finds the bin holding the n-th largest key, and only that bin's
// members are ranked exactly.  When the bin holds more than kListCap keys
// (heavy ties) the radix select finishes the job on that bin alone.

constexpr int kBins = 1024;
constexpr int kListCap = 512;

template <int NT, int ITEMS>
struct BucketSmem {
    static constexpr int NW = NT / 64;
    int hist[kBins];
    uint32_t list_key[kListCap];
    int list_slot[kListCap];
    uint32_t red[3][NW];
    int misc[8];
    SelectSmem<NT, ITEMS> radix;
};

struct Binning {
    float lo;
    float scale;
    HISA_INLINE int operator()(uint32_t key) const
    {
        const float x = (key_score(key) - lo) * scale;
        return x >= (float)(kBins - 1) ? kBins - 1 : (int)x;
    }
};

template <int NT, int ITEMS>
HISA_INLINE Threshold wg_bucket_select(const uint32_t (&key)[ITEMS], int n, BucketSmem<NT, ITEMS>& sm)
{
    constexpr int NW = NT / 64;
    static_assert(kBins % NT == 0, "whole bins per thread");
    Threshold th;
    if (n <= 0) {
        th.T = 0xffffffffu;
        th.need_eq = 0;
        th.all = false;
        return th;
    }
    // count, smallest and largest candidate key; clear the histogram
    uint32_t cnt = 0, kmin = 0xffffffffu, kmax = 0u;
#pragma unroll
    for (int it = 0; it < ITEMS; ++it) {
        const uint32_t kk = key[it];
        cnt += kk != 0u;
        kmin = kk ? min(kmin, kk) : kmin;
        kmax = max(kmax, kk);
    }
    cnt = (uint32_t)wave_sum((int)cnt);
    kmin = wave_min_u32(kmin);
    kmax = wave_max_u32(kmax);
    if (lane_id() == 0) {
        sm.red[0][wave_id()] = cnt;
        sm.red[1][wave_id()] = kmin;
        sm.red[2][wave_id()] = kmax;
    }
    for (int b = threadIdx.x; b < kBins; b += NT) sm.hist[b] = 0;
    if (threadIdx.x == 0) sm.misc[2] = 0;
    __syncthreads();
    int nvalid = 0;
    kmin = 0xffffffffu;
    kmax = 0u;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        nvalid += (int)sm.red[0][w];
        kmin = min(kmin, sm.red[1][w]);
        kmax = max(kmax, sm.red[2][w]);
    }
    if (nvalid <= n) {
        th.T = 0u;
        th.need_eq = 0;
        th.all = true;
        return th;
    }
    if (kmin == kmax) {                       // every candidate has the same key
        th.T = kmin;
        th.need_eq = n;
        th.all = false;
        return th;
    }
    const float smin = key_score(kmin), smax = key_score(kmax);
    const float range = smax - smin;
    if (!(range > 0.f) || !__builtin_isfinite(range))
        return wg_radix_select<NT, ITEMS>(key, n, sm.radix);   // non-finite scores: exact radix path
    const Binning bin{smin, (float)kBins / range};
#pragma unroll
    for (int it = 0; it < ITEMS; ++it)
        if (key[it]) atomicAdd(&sm.hist[bin(key[it])], 1);
    __syncthreads();
    // thread t owns kPer bins counted down from the top
    constexpr int kPer = kBins / NT;
    int own = 0;
#pragma unroll
    for (int j = 0; j < kPer; ++j) own += sm.hist[kBins - 1 - kPer * threadIdx.x - j];
    const int cum = wg_incl_scan<NT>(own, sm.radix.scratch);
    if (cum >= n && cum - own < n) {
        int above = cum - own;
        int b = kBins - 1 - kPer * threadIdx.x;
        for (int j = 0; j < kPer; ++j, --b) {
            const int h = sm.hist[b];
            if (above + h >= n) break;
            above += h;
        }
        sm.misc[0] = b;
        sm.misc[1] = above;
    }
    __syncthreads();
    const int bstar = sm.misc[0];
    const int need = n - sm.misc[1];          // >= 1 keys still to take from bin bstar
    const int c = sm.hist[bstar];
    if (c > kListCap) {
        // heavy ties: exact radix select on the members of bin bstar
        uint32_t sub[ITEMS];
#pragma unroll
        for (int it = 0; it < ITEMS; ++it) sub[it] = (key[it] && bin(key[it]) == bstar) ? key[it] : 0u;
        return wg_radix_select<NT, ITEMS>(sub, need, sm.radix);
    }
#pragma unroll
    for (int it = 0; it < ITEMS; ++it) {
        if (key[it] && bin(key[it]) == bstar) {
            const int p = atomicAdd(&sm.misc[2], 1);
            sm.list_key[p] = key[it];
            sm.list_slot[p] = it * NT + threadIdx.x;
        }
    }
    __syncthreads();
    // rank of member j in (key desc, slot asc) order; the member of rank
    // need-1 is the threshold key
    for (int j = threadIdx.x; j < c; j += NT) {
        const uint32_t kj = sm.list_key[j];
        const int sj = sm.list_slot[j];
        int r = 0;
        for (int i = 0; i < c; ++i) {
            const uint32_t ki = sm.list_key[i];
            r += (ki > kj) || (ki == kj && sm.list_slot[i] < sj);
        }
        if (r == need - 1) sm.misc[3] = (int)kj;
    }
    __syncthreads();
    const uint32_t T = (uint32_t)sm.misc[3];
    int gt = 0;
    for (int j = threadIdx.x; j < c; j += NT) gt += sm.list_key[j] > T;
    gt = wg_sum<NT>(gt, sm.radix.scratch);
    th.T = T;
    th.need_eq = need - gt;
    th.all = false;
    return th;
}

}  // namespace hisa
