// Workgroup-level top-n selection on register-held ranking keys.
//
// A workgroup of 256 threads holds ITEMS keys per thread; key[it] of thread
// tid belongs to slot it*256 + tid.  Key 0 means "no candidate".  The n
// largest keys are selected, equal keys going to the lower slot, and handed
// to a callback with their rank in ascending slot order, so the output of a
// selection is ordered by slot without a sort.
#pragma once

#include "common.h"

namespace hisa {

// Shared memory a selection needs (ints).
template <int ITEMS>
struct SelectSmem {
    int hist[256];
    int cnt[2 * ITEMS * kWaves];
    int scratch[kWaves];
    int pick[2];
};

struct Threshold {
    uint32_t T;      // the n-th largest key (0 when every candidate is taken)
    int need_eq;     // how many keys equal to T are taken, lowest slots first
    bool all;        // n >= number of candidates: take every nonzero key
};

// Radix select, 8 bits per pass from the top: after four passes the exact
// n-th largest key is known together with how many of its copies to take.
template <int ITEMS>
__device__ Threshold wg_radix_select(const uint32_t (&key)[ITEMS], int n, SelectSmem<ITEMS>& sm)
{
    Threshold th;
    if (n <= 0) {                 // nothing to take
        th.T = 0xffffffffu;
        th.need_eq = 0;
        th.all = false;
        return th;
    }
    int nvalid = 0;
#pragma unroll
    for (int it = 0; it < ITEMS; ++it) nvalid += key[it] != 0u;
    nvalid = block_sum(nvalid, sm.scratch);
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
        sm.hist[threadIdx.x] = 0;
        __syncthreads();
#pragma unroll
        for (int it = 0; it < ITEMS; ++it) {
            uint32_t kk = key[it];
            if (kk != 0u && (kk & mask) == prefix) atomicAdd(&sm.hist[(kk >> shift) & 255u], 1);
        }
        __syncthreads();
        // thread tid looks at digit 255 - tid: the scan counts keys whose
        // digit is >= that one
        const int h = sm.hist[255 - threadIdx.x];
        const int cum = block_incl_scan(h, sm.scratch);
        if (cum >= rem && cum - h < rem) {
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
template <int ITEMS, class Emit>
__device__ int wg_emit_selected(const uint32_t (&key)[ITEMS], const Threshold& th, SelectSmem<ITEMS>& sm,
                                Emit emit)
{
    const int w = wave_id();
#pragma unroll
    for (int it = 0; it < ITEMS; ++it) {
        const bool gt = key[it] > th.T;
        const bool eq = !th.all && key[it] == th.T;
        const uint64_t bg = __ballot(gt);
        const uint64_t be = __ballot(eq);
        if (lane_id() == 0) {
            sm.cnt[2 * (it * kWaves + w) + 0] = __popcll(bg);
            sm.cnt[2 * (it * kWaves + w) + 1] = __popcll(be);
        }
    }
    __syncthreads();
    constexpr int kEntries = ITEMS * kWaves;   // <= 256
    const int e = threadIdx.x;
    const int g = e < kEntries ? sm.cnt[2 * e + 0] : 0;
    const int q = e < kEntries ? sm.cnt[2 * e + 1] : 0;
    const int gi = block_incl_scan(g, sm.scratch);
    const int qi = block_incl_scan(q, sm.scratch);
    if (e < kEntries) {
        sm.cnt[2 * e + 0] = gi - g;
        sm.cnt[2 * e + 1] = qi - q;
    }
    if (e == kThreads - 1) {
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
        const int pg = sm.cnt[2 * (it * kWaves + w) + 0] + __popcll(bg & lanemask_lt());
        const int pe = sm.cnt[2 * (it * kWaves + w) + 1] + __popcll(be & lanemask_lt());
        const int slot = it * kThreads + threadIdx.x;
        if (gt) emit(slot, key[it], pg + min(pe, th.need_eq));
        else if (eq && pe < th.need_eq) emit(slot, key[it], pg + pe);
    }
    __syncthreads();
    return total;
}

}  // namespace hisa
