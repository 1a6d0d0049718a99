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

// Makes the compiler treat the keys as new values (no instruction): lane
// masks computed from them before this point are not kept live across it
// in scalar registers.
template <int ITEMS>
HISA_INLINE void opaque_keys(uint32_t (&key)[ITEMS])
{
#pragma unroll
    for (int it = 0; it < ITEMS; ++it) asm volatile("" : "+v"(key[it]));
}

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
    bool eq_all = false;   // known: every key equal to T is taken (the selection is key >= T)
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
    alignas(16) uint32_t list_key[kListCap];  // 16-byte aligned: read four at a time
    alignas(16) int list_slot[kListCap];
    uint32_t red[3][NW];
    int wave_tot[2][NW];
    int misc[9];
    RadixSmem<NT> radix;
};

// Inclusive prefix sum within each row of 16 lanes.
HISA_INLINE int row_incl_scan(int v)
{
    uint32_t x = (uint32_t)v;
    x += dpp_u32<0x111>(x);
    x += dpp_u32<0x112>(x);
    x += dpp_u32<0x114>(x);
    x += dpp_u32<0x118>(x);
    return (int)x;
}

// Orders one wave's LDS accesses around it (a compiler fence: the LDS
// operations of one wave complete in order).
HISA_INLINE void wave_lds_fence()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// The bin of a key in [kmin, kmax]: x = score * scale + off, clamped to
// [0, kBins-1] and truncated.  Monotone in the key (equal keys share a
// bin); keys below kmin (the empty key 0) fall in bin 0.
struct Binning {
    uint32_t kmin;
    float scale;
    float off;
    HISA_INLINE int operator()(uint32_t key) const
    {
        const float x = fmaf(key_score(max(key, kmin)), scale, off);
        return (int)__builtin_amdgcn_fmed3f(x, 0.f, (float)(kBins - 1));
    }
};

// Smallest key in [lo, hi] whose bin is >= b, given that hi's is.  One
// wave: first a window of 64 keys around the bin edge computed from the
// scale, then, if the edge is not in it, rounds that each test 64 evenly
// spaced keys (six rounds cover 32 bits).  Uniform over the wave.
HISA_INLINE uint32_t first_key_of_bin(uint32_t lo, uint32_t hi, int b, const Binning& bin)
{
    const int lane = lane_id();
    {
        const float edge = (b - bin.off) / bin.scale;
        const uint32_t g = score_key(edge);
        const uint32_t g0 = min(g < lo + 32u ? lo : g - 32u, hi);
        const uint32_t k = min(g0 + (uint32_t)lane, hi);
        const uint64_t bal = __ballot(bin(k) >= b);
        // the edge lies in the window when the window starts below it and
        // reaches it
        if (bal != 0 && (g0 == lo || !(bal & 1ull))) return (uint32_t)__builtin_amdgcn_readlane((int)k, (int)__builtin_ctzll(bal));
        if (bal == 0) lo = (uint32_t)__builtin_amdgcn_readlane((int)k, 63) + 1u;
        else hi = g0;
    }
    while (lo < hi) {
        const uint32_t w = hi - lo;
        const uint32_t k = lo + min((w / 64u + 1u) * (uint32_t)lane, w);
        const uint64_t bal = __ballot(bin(k) >= b);
        if (bal == 0) {
            lo = (uint32_t)__builtin_amdgcn_readlane((int)k, 63) + 1u;
        } else {
            const int f = (int)__builtin_ctzll(bal);
            if (f == 0) return lo;
            hi = (uint32_t)__builtin_amdgcn_readlane((int)k, f);
            lo = (uint32_t)__builtin_amdgcn_readlane((int)k, f - 1) + 1u;
        }
    }
    return lo;
}

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
    int nz = 0;
    uint32_t kmax = 0u, kmin1 = 0xffffffffu;
#pragma unroll
    for (int it = 0; it < ITEMS; ++it) {
        kmax = max(kmax, key[it]);
        kmin1 = min(kmin1, key[it] - 1u);     // an empty slot wraps to the top
        nz += __popcll(__ballot(key[it] != 0u));
    }
    kmax = wave_max_u32(kmax);
    kmin1 = wave_min_u32(kmin1);
    if (lane_id() == 0) {
        sm.red[0][wave_id()] = (uint32_t)nz;
        sm.red[1][wave_id()] = kmin1;
        sm.red[2][wave_id()] = kmax;
    }
    for (int b = threadIdx.x; b < kBins; b += NT) sm.hist[b] = 0;
    if (threadIdx.x == 0) sm.misc[2] = 0;
    __syncthreads();
    int nvalid = 0;
    kmin1 = 0xffffffffu;
    kmax = 0u;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        nvalid += (int)sm.red[0][w];
        kmin1 = min(kmin1, sm.red[1][w]);
        kmax = max(kmax, sm.red[2][w]);
    }
    const uint32_t kmin = kmin1 + 1u;
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
    const float scale = (float)kBins / range;
    const float off = -smin * scale;
    if (!(range > 0.f) || !__builtin_isfinite(range) || !__builtin_isfinite(scale) || !__builtin_isfinite(off))
        return wg_radix_select<NT, ITEMS>(key, n, sm.radix, true);   // non-finite or unbinnable scores
    const Binning bin{kmin, scale, off};
    // empty slots land in bin 0 and are taken off it below
#pragma unroll
    for (int it = 0; it < ITEMS; ++it) atomicAdd(&sm.hist[bin(key[it])], 1);
    __syncthreads();
    // one wave finds the bin of the n-th largest key (lane l owns the 16
    // bins counted down from kBins-1-16l) and the range of keys in it
    if (wave_id() == 0) {
        constexpr int kPer = kBins / 64;
        const int nzero = NT * ITEMS - nvalid;
        if (threadIdx.x == 0) sm.hist[0] -= nzero;
        wave_lds_fence();
        int own = 0;
#pragma unroll
        for (int j = 0; j < kPer; ++j) own += sm.hist[kBins - 1 - kPer * lane_id() - j];
        const int cum = wave_incl_scan(own);
        const int L = (int)__builtin_ctzll(__ballot(cum >= n && cum - own < n));
        // lanes 0..15 take the 16 bins of lane L, a row scan finds the bin
        const int h = lane_id() < kPer ? sm.hist[kBins - 1 - kPer * L - lane_id()] : 0;
        const int rc = row_incl_scan(h);
        const int aboveL = __builtin_amdgcn_readlane(cum - own, L);
        const int J = (int)__builtin_ctzll(__ballot(lane_id() < kPer && aboveL + rc >= n));
        const int bstar = kBins - 1 - kPer * L - J;
        const int c = __builtin_amdgcn_readlane(h, J);
        const int above = aboveL + __builtin_amdgcn_readlane(rc, J) - c;
        uint32_t klo = kmin, khi1 = kmax + 1u;
        if (n - above < c) {                  // the bin is split: its key range
            if (bstar > 0) klo = first_key_of_bin(kmin, kmax, bstar, bin);
            if (bstar < kBins - 1) khi1 = first_key_of_bin(klo, kmax, bstar + 1, bin);
        } else if (bstar > 0) {
            klo = first_key_of_bin(kmin, kmax, bstar, bin);
        }
        if (lane_id() == 0) {
            sm.misc[0] = bstar;
            sm.misc[1] = above;
            sm.misc[3] = c;
            sm.misc[4] = (int)klo;
            sm.misc[5] = (int)khi1;
        }
    }
    __syncthreads();
    const int need = n - sm.misc[1];          // 1 <= need <= c keys still to take from the bin
    const int c = sm.misc[3];
    const uint32_t klo = (uint32_t)sm.misc[4], khi1 = (uint32_t)sm.misc[5];
    if (need == c) {
        // the whole bin is taken: everything from its smallest key up
        th.T = klo;
        th.need_eq = c;
        th.all = false;
        th.eq_all = true;
        return th;
    }
    const uint32_t span = khi1 - klo;
    if (c > kListCap) {
        // heavy ties: exact radix select on the members of the bin
        uint32_t sub[ITEMS];
#pragma unroll
        for (int it = 0; it < ITEMS; ++it) sub[it] = key[it] - klo < span ? key[it] : 0u;
        return wg_radix_select<NT, ITEMS>(sub, need, sm.radix, false);
    }
#pragma unroll
    for (int it = 0; it < ITEMS; ++it) {
        if (key[it] - klo < span) {
            const int p = atomicAdd(&sm.misc[2], 1);
            sm.list_key[p] = key[it];
            sm.list_slot[p] = slot_of<ITEMS>(it);
        }
    }
    __syncthreads();
    // rank of member j in (key desc, slot asc) order; the member of rank
    // need-1 is the threshold key, and the equal keys before it plus itself
    // are the copies of it to take.  Thread j ranks member j against all c
    // members, read four at a time as broadcast 16-byte LDS loads (several
    // in flight); up to 64 members this is wave 0 alone.
    for (int j = threadIdx.x; j < c; j += NT) {
        const uint32_t kj = sm.list_key[j];
        const int sj = sm.list_slot[j];
        int r = 0, eq_before = 0, eq_n = 0;
        auto step = [&](uint32_t ki, int si) {
            const bool before = ki == kj && si < sj;
            r += (ki > kj) || before;
            eq_before += before;
            eq_n += ki == kj;
        };
        int i = 0;
#pragma unroll 4
        for (; i + 4 <= c; i += 4) {
            const uint4 kv = *reinterpret_cast<const uint4*>(sm.list_key + i);
            const int4 sv = *reinterpret_cast<const int4*>(sm.list_slot + i);
            step(kv.x, sv.x);
            step(kv.y, sv.y);
            step(kv.z, sv.z);
            step(kv.w, sv.w);
        }
        for (; i < c; ++i) step(sm.list_key[i], sm.list_slot[i]);
        if (r == need - 1) {
            sm.misc[6] = (int)kj;
            sm.misc[7] = eq_before + 1;
            sm.misc[8] = eq_n;
        }
    }
    __syncthreads();
    th.T = (uint32_t)sm.misc[6];
    th.need_eq = sm.misc[7];
    th.all = false;
    th.eq_all = sm.misc[8] == sm.misc[7];   // no copy of T after the last one taken
    return th;
}

// Hand every selected key to emit(it, key, rank) (item it of this thread,
// slot slot_of<ITEMS>(it)), rank = its position in ascending slot order
// among the selected, for ranks below `limit` (a guard: a consistent
// threshold never selects more than the n asked for).  Returns how many
// were selected, at most limit.
// One barrier: each wave knows the counts of its own slots from ballots and
// only needs the totals of the waves before it.  No barrier at the end:
// synchronise before reusing the shared memory.
template <int NT, int ITEMS, class Emit>
HISA_INLINE int wg_emit_selected_items(const uint32_t (&key_in)[ITEMS], const Threshold& th, BucketSmem<NT>& sm,
                                       int limit, Emit emit)
{
    constexpr int NW = NT / 64;
    uint32_t key[ITEMS];
#pragma unroll
    for (int it = 0; it < ITEMS; ++it) key[it] = key_in[it];
    const int w = wave_id();
    if (th.all || th.eq_all) {
        // the selection is key >= lo: one count per item, and each wave
        // only needs the totals of the waves before it
        const uint32_t lo = th.all ? 1u : th.T;
        int wg = 0;
#pragma unroll
        for (int it = 0; it < ITEMS; ++it) wg += __popcll(__ballot(key[it] >= lo));
        if (lane_id() == 0) sm.wave_tot[0][w] = wg;
        __syncthreads();
        opaque_keys(key);
        int r = 0, tg = 0;
#pragma unroll
        for (int v = 0; v < NW; ++v) {
            const int g = sm.wave_tot[0][v];
            r += v < w ? g : 0;
            tg += g;
        }
        r = __builtin_amdgcn_readfirstlane(r);
#pragma unroll
        for (int it = 0; it < ITEMS; ++it) {
            const bool take = key[it] >= lo;
            const uint64_t b = __ballot(take);
            const int rank = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(b >> 32),
                                                            __builtin_amdgcn_mbcnt_lo((uint32_t)b, (uint32_t)r));
            if (take && rank < limit) emit(it, key[it], rank);
            r += __popcll(b);
        }
        return min(limit, tg);
    }
    int wg = 0, we = 0;
#pragma unroll
    for (int it = 0; it < ITEMS; ++it) {
        wg += __popcll(__ballot(key[it] > th.T));
        we += __popcll(__ballot(key[it] == th.T));
    }
    if (lane_id() == 0) {
        sm.wave_tot[0][w] = wg;
        sm.wave_tot[1][w] = we;
    }
    __syncthreads();
    opaque_keys(key);
    int rg = 0, re = 0, tg = 0, te = 0;
#pragma unroll
    for (int v = 0; v < NW; ++v) {
        const int g = sm.wave_tot[0][v], q = sm.wave_tot[1][v];
        rg += v < w ? g : 0;
        re += v < w ? q : 0;
        tg += g;
        te += q;
    }
    rg = __builtin_amdgcn_readfirstlane(rg);
    re = __builtin_amdgcn_readfirstlane(re);
    if (te <= th.need_eq) {
        // every key equal to the threshold is taken: selected = key >= T,
        // ranked by one ballot per item
        int r = rg + re;
#pragma unroll
        for (int it = 0; it < ITEMS; ++it) {
            const bool take = key[it] >= th.T;
            const uint64_t b = __ballot(take);
            const int rank = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(b >> 32),
                                                            __builtin_amdgcn_mbcnt_lo((uint32_t)b, (uint32_t)r));
            if (take && rank < limit) emit(it, key[it], rank);
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
        const int pg = rg + count_below(bg);
        const int pe = re + count_below(be);
        const int rank = gt ? pg + min(pe, th.need_eq) : pg + pe;
        if ((gt || (eq && pe < th.need_eq)) && rank < limit) emit(it, key[it], rank);
        rg += __popcll(bg);
        re += __popcll(be);
    }
    return min(limit, tg + min(te, th.need_eq));
}

// The same with emit(slot, key, rank).
template <int NT, int ITEMS, class Emit>
HISA_INLINE int wg_emit_selected(const uint32_t (&key)[ITEMS], const Threshold& th, BucketSmem<NT>& sm, int limit,
                                 Emit emit)
{
    return wg_emit_selected_items<NT, ITEMS>(key, th, sm, limit,
                                             [&](int it, uint32_t kk, int rank) { emit(slot_of<ITEMS>(it), kk, rank); });
}

// ---- wave-level select -------------------------------------------------------------
// One wave selects alone, with no workgroup barrier: key[it] of lane l is
// slot it*64 + l.  The same bucket idea on kWaveBins bins: count, range,
// histogram in the wave's own LDS, the threshold bin found by a wave scan,
// its members ranked exactly; more than 64 members (heavy ties) or
// non-finite scores go to an 8-bit radix select.  LDS traffic of one wave
// is ordered, so only compiler ordering fences separate the phases.

constexpr int kWaveBins = 256;

struct WaveSmem {
    int hist[kWaveBins];
    alignas(16) uint32_t list_key[64];        // 16-byte aligned: read four at a time
    alignas(16) int list_slot[64];
};

// Exact n-th largest nonzero key by four 8-bit passes (n <= count of
// nonzero keys), and how many of its copies to take.
template <int ITEMS>
HISA_INLINE Threshold wave_radix_select(const uint32_t (&key)[ITEMS], int n, WaveSmem& ws)
{
    const int lane = lane_id();
    uint32_t prefix = 0u, mask = 0u;
    int rem = n;
    for (int pass = 0; pass < 4; ++pass) {
        const int shift = 24 - 8 * pass;
#pragma unroll
        for (int j = 0; j < kWaveBins / 64; ++j) ws.hist[lane + 64 * j] = 0;
        wave_lds_fence();
#pragma unroll
        for (int it = 0; it < ITEMS; ++it) {
            const uint32_t kk = key[it];
            if (kk != 0u && (kk & mask) == prefix) atomicAdd(&ws.hist[(kk >> shift) & 255u], 1);
        }
        wave_lds_fence();
        // lane l owns digits 255-4l .. 252-4l (descending)
        int h[4], own = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            h[j] = ws.hist[255 - 4 * lane - j];
            own += h[j];
        }
        const int cum = wave_incl_scan(own);
        const int L = (int)__builtin_ctzll(__ballot(cum >= rem && cum - own < rem));
        int above = __builtin_amdgcn_readlane(cum - own, L);
        int digit = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int hj = __builtin_amdgcn_readlane(h[j], L);
            if (digit == 0 && above + hj >= rem) digit = 255 - 4 * L - j + 1;   // +1: 0 means not found yet
            else if (digit == 0) above += hj;
        }
        prefix |= (uint32_t)(digit - 1) << shift;
        mask |= 0xffu << shift;
        rem -= above;
        wave_lds_fence();
    }
    Threshold th;
    th.T = prefix;
    th.need_eq = rem;
    th.all = false;
    return th;
}

// Select the n largest nonzero keys of the wave (equal keys: lower slot
// first) and hand each to emit(slot, key, rank), rank in ascending slot
// order.  Returns the number selected, min(n, number of nonzero keys).
template <int ITEMS, class Emit>
HISA_INLINE int wave_select(const uint32_t (&key)[ITEMS], int n, WaveSmem& ws, Emit emit)
{
    const int lane = lane_id();
    if (n <= 0) return 0;
    int nvalid = 0;
    uint32_t kmax = 0u, kmin1 = 0xffffffffu;
#pragma unroll
    for (int it = 0; it < ITEMS; ++it) {
        nvalid += __popcll(__ballot(key[it] != 0u));
        kmax = max(kmax, key[it]);
        kmin1 = min(kmin1, key[it] - 1u);     // an empty slot wraps to the top
    }
    kmax = wave_max_u32(kmax);
    const uint32_t kmin = wave_min_u32(kmin1) + 1u;
    Threshold th;
    th.all = false;
    if (nvalid <= n || kmin == kmax) {
        // every nonzero key, or the first n of all-equal keys
        th.T = nvalid <= n ? 0u : kmin;
        th.need_eq = nvalid <= n ? 0 : n;
        th.all = nvalid <= n;
    } else {
        const float smin = key_score(kmin), smax = key_score(kmax);
        const float range = smax - smin;
        const float scale = (float)kWaveBins / range;
        if (!(range > 0.f) || !__builtin_isfinite(range) || !__builtin_isfinite(scale)) {
            th = wave_radix_select<ITEMS>(key, n, ws);
        } else {
            auto bin = [&](uint32_t kk) {
                const float x = (key_score(max(kk, kmin)) - smin) * scale;   // >= 0, finite
                return (int)min((uint32_t)x, (uint32_t)(kWaveBins - 1));
            };
#pragma unroll
            for (int j = 0; j < kWaveBins / 64; ++j) ws.hist[lane + 64 * j] = 0;
            wave_lds_fence();
#pragma unroll
            for (int it = 0; it < ITEMS; ++it)
                if (key[it]) atomicAdd(&ws.hist[bin(key[it])], 1);
            wave_lds_fence();
            int h[4], own = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                h[j] = ws.hist[kWaveBins - 1 - 4 * lane - j];
                own += h[j];
            }
            const int cum = wave_incl_scan(own);
            const int L = (int)__builtin_ctzll(__ballot(cum >= n && cum - own < n));
            int above = __builtin_amdgcn_readlane(cum - own, L);
            int bstar = -1, c = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int hj = __builtin_amdgcn_readlane(h[j], L);
                if (bstar < 0 && above + hj >= n) {
                    bstar = kWaveBins - 1 - 4 * L - j;
                    c = hj;
                } else if (bstar < 0) {
                    above += hj;
                }
            }
            const int need = n - above;        // 1 <= need <= c
            if (c > 64) {
                uint32_t sub[ITEMS];
#pragma unroll
                for (int it = 0; it < ITEMS; ++it) sub[it] = (key[it] && bin(key[it]) == bstar) ? key[it] : 0u;
                th = wave_radix_select<ITEMS>(sub, need, ws);
            } else {
                // list the bin's members, then rank them in (key desc, slot asc) order
                int base = 0;
#pragma unroll
                for (int it = 0; it < ITEMS; ++it) {
                    const bool mem = key[it] && bin(key[it]) == bstar;
                    const uint64_t b = __ballot(mem);
                    if (mem) {
                        const int p = base + count_below(b);
                        ws.list_key[p] = key[it];
                        ws.list_slot[p] = it * 64 + lane;
                    }
                    base += __popcll(b);
                }
                wave_lds_fence();
                const uint32_t kj = lane < c ? ws.list_key[lane] : 0u;
                const int sj = lane < c ? ws.list_slot[lane] : 0;
                int r = 0, eq_before = 0;
                auto step = [&](uint32_t ki, int si) {
                    const bool before = ki == kj && si < sj;
                    r += (ki > kj) || before;
                    eq_before += before;
                };
                int i = 0;
#pragma unroll 4
                for (; i + 4 <= c; i += 4) {   // broadcast 16-byte LDS loads, several in flight
                    const uint4 kv = *reinterpret_cast<const uint4*>(ws.list_key + i);
                    const int4 sv = *reinterpret_cast<const int4*>(ws.list_slot + i);
                    step(kv.x, sv.x);
                    step(kv.y, sv.y);
                    step(kv.z, sv.z);
                    step(kv.w, sv.w);
                }
                for (; i < c; ++i) step(ws.list_key[i], ws.list_slot[i]);
                const int J = (int)__builtin_ctzll(__ballot(lane < c && r == need - 1));
                th.T = (uint32_t)__builtin_amdgcn_readlane((int)kj, J);
                th.need_eq = __builtin_amdgcn_readlane(eq_before, J) + 1;
                wave_lds_fence();
            }
        }
    }
    // emit in slot order: keys above T, then the first need_eq copies of T
    const uint32_t lo = th.all ? 1u : th.T;
    int rank = 0, eq = 0;
#pragma unroll
    for (int it = 0; it < ITEMS; ++it) {
        const bool gt = th.all ? key[it] >= lo : key[it] > th.T;
        const bool is_eq = !th.all && key[it] == th.T;
        const uint64_t bg = __ballot(gt), be = __ballot(is_eq);
        const int pe = eq + count_below(be);
        const bool take = gt || (is_eq && pe < th.need_eq);
        const uint64_t bt = __ballot(take);
        if (take) emit(it * 64 + lane, key[it], rank + count_below(bt));
        rank += __popcll(bt);
        eq += __popcll(be);
        (void)bg;
    }
    return rank;
}

}  // namespace hisa
