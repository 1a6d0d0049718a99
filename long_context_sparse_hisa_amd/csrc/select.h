// Workgroup-level top-n selection on register-held ranking keys.
//
// A workgroup of NT threads holds ITEMS keys per thread.  Wave w owns the
// contiguous slots [w*ITEMS*64, (w+1)*ITEMS*64): key[it] of lane l belongs
// to slot (w*ITEMS + it)*64 + l (see slot_of).  Key 0 means "no
// candidate".  The n largest keys are selected, equal keys going to the
// lower slot, and handed to a callback with their rank in ascending slot
// order, so the output of a selection is ordered by slot without a sort.
// Everything here is force-inlined so the key arrays stay in registers.
#pragma once

#include "common.h"

#define HISA_INLINE __device__ __attribute__((always_inline)) inline

namespace hisa {

template <int ITEMS>
HISA_INLINE int slot_of(int it)
{
    return ((wave_id() * ITEMS + it) << 6) | lane_id();
}

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

struct Threshold {
    uint32_t T;      // the n-th largest key (0 when every candidate is taken)
    int need_eq;     // how many keys equal to T are taken, lowest slots first
    bool all;        // n >= number of candidates: take every nonzero key
};

// ---- radix select (exact fallback) ----------------------------------------------

template <int NT>
struct RadixSmem {
    int hist[256];
    int scratch[NT / 64];
    int pick[2];
};

// 8 bits per pass from the top: after four passes the exact n-th largest
// key is known together with how many of its copies to take.  Used when
// the bucket select meets heavy ties or non-finite scores.  may_take_all:
// when at most n keys are nonzero, answer "take every nonzero key"; a
// caller that passes a subset of the keys it will emit from must say false
// (the threshold then stays exact, 1 <= n <= number of nonzero keys).
template <int NT, int ITEMS>
HISA_INLINE Threshold wg_radix_select(const uint32_t (&key)[ITEMS], int n, RadixSmem<NT>& sm, bool may_take_all)
{
    static_assert(NT >= 256, "one digit per thread");
    Threshold th;
    int nvalid = 0;
#pragma unroll
    for (int it = 0; it < ITEMS; ++it) nvalid += key[it] != 0u;
    nvalid = wg_sum<NT>(nvalid, sm.scratch);
    if (may_take_all && nvalid <= n) {
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

// ---- bucket select ---------------------------------------------------------------
// The candidate scores are spread over kBins equal-width bins between their
// minimum and maximum.  That map is monotone, so every key in a higher bin
// is larger than every key in a lower one and equal keys share a bin.  One
// histogram finds the bin holding the n-th largest key, and only that bin's
// members are ranked exactly.  When the bin holds more than kListCap keys
// (heavy ties), or scores are not finite, the radix select takes over.

constexpr int kBins = 1024;
constexpr int kListCap = 512;

template <int NT>
struct BucketSmem {
    static constexpr int NW = NT / 64;
    int hist[kBins + 1];                      // the extra bin counts the empty slots
    uint32_t list_key[kListCap];
    int list_slot[kListCap];
    uint32_t red[3][NW];
    int wave_tot[2][NW];
    int misc[8];
    RadixSmem<NT> radix;
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
HISA_INLINE Threshold wg_bucket_select(const uint32_t (&key)[ITEMS], int n, BucketSmem<NT>& sm)
{
    constexpr int NW = NT / 64;
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
    for (int b = threadIdx.x; b <= kBins; b += NT) sm.hist[b] = 0;
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
        return wg_radix_select<NT, ITEMS>(key, n, sm.radix, true);   // non-finite scores: exact radix path
    const Binning bin{smin, (float)kBins / range};
#pragma unroll
    for (int it = 0; it < ITEMS; ++it) atomicAdd(&sm.hist[key[it] ? bin(key[it]) : kBins], 1);   // no branch
    __syncthreads();
    // one wave finds the bin of the n-th largest key: lane l owns the 16
    // bins counted down from kBins-1-16l
    if (wave_id() == 0) {
        constexpr int kPer = kBins / 64;
        int own = 0;
#pragma unroll
        for (int j = 0; j < kPer; ++j) own += sm.hist[kBins - 1 - kPer * lane_id() - j];
        const int cum = wave_incl_scan(own);
        if (cum >= n && cum - own < n) {
            int above = cum - own;
            int b = kBins - 1 - kPer * lane_id();
            for (int j = 0; j < kPer; ++j, --b) {
                const int h = sm.hist[b];
                if (above + h >= n) break;
                above += h;
            }
            sm.misc[0] = b;
            sm.misc[1] = above;
        }
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
        return wg_radix_select<NT, ITEMS>(sub, need, sm.radix, false);
    }
#pragma unroll
    for (int it = 0; it < ITEMS; ++it) {
        if (key[it] && bin(key[it]) == bstar) {
            const int p = atomicAdd(&sm.misc[2], 1);
            sm.list_key[p] = key[it];
            sm.list_slot[p] = slot_of<ITEMS>(it);
        }
    }
    __syncthreads();
    // rank of member j in (key desc, slot asc) order; the member of rank
    // need-1 is the threshold key, and the equal keys before it plus itself
    // are the copies of it to take
    for (int j = threadIdx.x; j < c; j += NT) {
        const uint32_t kj = sm.list_key[j];
        const int sj = sm.list_slot[j];
        int r = 0, eq_before = 0;
        for (int i = 0; i < c; ++i) {
            const uint32_t ki = sm.list_key[i];
            const bool before = ki == kj && sm.list_slot[i] < sj;
            r += (ki > kj) || before;
            eq_before += before;
        }
        if (r == need - 1) {
            sm.misc[3] = (int)kj;
            sm.misc[4] = eq_before + 1;
        }
    }
    __syncthreads();
    th.T = (uint32_t)sm.misc[3];
    th.need_eq = sm.misc[4];
    th.all = false;
    return th;
}

// Hand every selected key to emit(slot, key, rank), rank = its position in
// ascending slot order among the selected, for ranks below `limit` (a
// guard: a consistent threshold never selects more than the n asked for).
// Returns how many were selected, at most limit.
// One barrier: each wave knows the counts of its own slots from ballots and
// only needs the totals of the waves before it.  No barrier at the end:
// synchronise before reusing the shared memory.
template <int NT, int ITEMS, class Emit>
HISA_INLINE int wg_emit_selected(const uint32_t (&key)[ITEMS], const Threshold& th, BucketSmem<NT>& sm, int limit,
                                 Emit emit)
{
    constexpr int NW = NT / 64;
    const int w = wave_id();
    int wg = 0, we = 0;
#pragma unroll
    for (int it = 0; it < ITEMS; ++it) {
        wg += __popcll(__ballot(key[it] > th.T));
        we += __popcll(__ballot(!th.all && key[it] == th.T));
    }
    if (lane_id() == 0) {
        sm.wave_tot[0][w] = wg;
        sm.wave_tot[1][w] = we;
    }
    __syncthreads();
    int rg = 0, re = 0, tg = 0, te = 0;
#pragma unroll
    for (int v = 0; v < NW; ++v) {
        const int g = sm.wave_tot[0][v], q = sm.wave_tot[1][v];
        rg += v < w ? g : 0;
        re += v < w ? q : 0;
        tg += g;
        te += q;
    }
    const uint64_t lt = lanemask_lt();
    if (th.all || te <= th.need_eq) {
        // every key equal to the threshold is taken: selected = key >= T
        // (or every nonzero key), ranked by one ballot per item
        const uint32_t lo = th.all ? 1u : th.T;
        int r = rg + re;
#pragma unroll
        for (int it = 0; it < ITEMS; ++it) {
            const bool take = key[it] >= lo;
            const uint64_t b = __ballot(take);
            const int rank = r + __popcll(b & lt);
            if (take && rank < limit) emit(slot_of<ITEMS>(it), key[it], rank);
            r += __popcll(b);
        }
        return min(limit, tg + te);
    }
#pragma unroll
    for (int it = 0; it < ITEMS; ++it) {
        const bool gt = key[it] > th.T;
        const bool eq = key[it] == th.T;
        const uint64_t bg = __ballot(gt);
        const uint64_t be = __ballot(eq);
        const int pg = rg + __popcll(bg & lt);
        const int pe = re + __popcll(be & lt);
        const int rank = gt ? pg + min(pe, th.need_eq) : pg + pe;
        if ((gt || (eq && pe < th.need_eq)) && rank < limit) emit(slot_of<ITEMS>(it), key[it], rank);
        rg += __popcll(bg);
        re += __popcll(be);
    }
    return min(limit, tg + min(te, th.need_eq));
}

}  // namespace hisa
