// LSA-Flat: semantic buckets over the index keys and the flat search over
// their centroids (the latent sparse attention digest, section on how LSA
// works, steps 1-4, and Fig. 2 Flat; footnote 3 for the fill to k).
//
// Build: one workgroup per complete block of 512 keys.  The keys are
// L2-normalised and summed four at a time into 128 pool keys (fp64), which
// start as buckets; rounds of mutually cheapest pairs under Ward's
// criterion merge them, at most 16 keys (4 pool keys) per bucket, until 64
// remain.  A bucket's centroid is its normalised sum, stored as bf16.
//
// Ward costs decide integers, and neighbouring costs of random keys differ
// by as little as 1e-5 relative, so they are fp64.  A bucket's cost to b is
// nA nB / (nA + nB) * (|mA|^2 + |mB|^2 - 2 mA.mB) with the means m: each
// lane keeps one bucket's mean in registers and streams the other means
// from LDS as wave-wide broadcasts; the expression is symmetric, so the
// lanes of A and B compute bit-identical costs for the pair.
//
// Query: a small kernel maps each query to its last visible bucket, the
// flat indexer's kernels score and select the top p buckets (centroids in
// place of keys), and the fill kernel ranks those buckets, cuts at k keys
// and writes the positions in ascending order from a bitmap of pool keys.
#include "../../include/hisa.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>

#include "common.h"
#include "kernels.h"
#include "select.h"

namespace hisa {

namespace {

constexpr int kLsaBlock = 512;
constexpr int kLsaPool = 4;
constexpr int kLsaPoints = kLsaBlock / kLsaPool;   // 128 pool keys per block
constexpr int kLsaBuckets = 64;
constexpr int kLsaCap = 4;                         // pool keys per bucket (16 keys)
constexpr int kLsaThreads = 256;

static_assert(kLsaPoints == 2 * 64 && kLsaThreads == 4 * 64, "two waves of rows, two halves of partners");

struct LsaBuildSmem {
    double sum[kLsaPoints][kDim];     // bucket sums, by root point
    double mean[kLsaPoints][kDim];    // bucket means; pool keys again at the end
    double sq[kLsaPoints];            // |mean|^2
    double half_cost[2][kLsaPoints];
    double pair_cost[kLsaPoints / 2];
    int cnt[kLsaPoints];              // pool keys in the bucket rooted here, 0 once absorbed
    int parent[kLsaPoints];
    int half_best[2][kLsaPoints];
    int best[kLsaPoints];
    int pair_a[kLsaPoints / 2], pair_b[kLsaPoints / 2];
    int merge[kLsaPoints / 2];        // the pair merges this round
    int id[kLsaPoints];               // bucket id of each root
    int start[kLsaBuckets + 1];
    uint8_t memb[kLsaPoints];
    int npairs, count;
};

// Normalised pool keys of a block into p[128][64]: thread t sums pool key
// t / 2, dimensions 32 * (t % 2) .. + 32, over its four keys in order.
__device__ __forceinline__ void lsa_pool_keys(const uint16_t* kb, double (*p)[kDim])
{
    const int pk = threadIdx.x >> 1, h = threadIdx.x & 1;
    double acc[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) acc[i] = 0.0;
#pragma unroll
    for (int r = 0; r < kLsaPool; ++r) {
        const uint4* row = reinterpret_cast<const uint4*>(kb + (size_t)(pk * kLsaPool + r) * kDim + h * 32);
        uint32_t w[16];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const uint4 x = row[v];
            w[4 * v] = x.x;
            w[4 * v + 1] = x.y;
            w[4 * v + 2] = x.z;
            w[4 * v + 3] = x.w;
        }
        double ss = 0.0;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const double lo = bf16_lo(w[i]), hi = bf16_hi(w[i]);
            ss += lo * lo;
            ss += hi * hi;
        }
        // both lanes of the pair add the halves in the same order
        const double other = __shfl_xor(ss, 1);
        const double total = h == 0 ? ss + other : other + ss;
        const double norm = sqrt(total);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            acc[2 * i] += norm > 0.0 ? (double)bf16_lo(w[i]) / norm : 0.0;
            acc[2 * i + 1] += norm > 0.0 ? (double)bf16_hi(w[i]) / norm : 0.0;
        }
    }
#pragma unroll
    for (int i = 0; i < 32; ++i) p[pk][h * 32 + i] = acc[i];
}

__global__ __launch_bounds__(kLsaThreads) void lsa_build_kernel(const uint16_t* keys, int64_t b0, uint16_t* centroids,
                                                                uint8_t* members, uint8_t* offs)
{
    __shared__ LsaBuildSmem sm;
    const int t = threadIdx.x;
    const int64_t blk = b0 + blockIdx.x;
    const uint16_t* kb = keys + blk * kLsaBlock * kDim;
    lsa_pool_keys(kb, sm.mean);
    __syncthreads();
    for (int e = t; e < kLsaPoints * kDim; e += kLsaThreads) (&sm.sum[0][0])[e] = (&sm.mean[0][0])[e];
    if (t < kLsaPoints) {
        sm.cnt[t] = 1;
        sm.parent[t] = t;
        double s = 0.0;
        for (int c = 0; c < kDim; ++c) s += sm.mean[t][c] * sm.mean[t][c];
        sm.sq[t] = s;
    }
    if (t == 0) sm.count = kLsaPoints;
    const int lane = lane_id(), w = wave_id();
    const int a = (w & 1) * 64 + lane;        // this lane's bucket
    const int hb = w >> 1;                    // which half of the partners
    for (;;) {
        __syncthreads();
        const int count = sm.count;
        if (count <= kLsaBuckets) break;
        // each bucket's cheapest admissible partner within this half
        const int na = sm.cnt[a];
        double ma[kDim];
#pragma unroll
        for (int c = 0; c < kDim; ++c) ma[c] = sm.mean[a][c];
        const double sqa = sm.sq[a];
        double c1 = INFINITY;
        int b1 = -1;
        for (int bb = 0; bb < 64; ++bb) {
            const int b = hb * 64 + bb;
            const int nb = sm.cnt[b];
            if (nb == 0) continue;                 // absorbed: the same for the whole wave
            double d0 = 0.0, d1 = 0.0, d2 = 0.0, d3 = 0.0;
#pragma unroll
            for (int c = 0; c < kDim; c += 4) {
                d0 = fma(ma[c], sm.mean[b][c], d0);
                d1 = fma(ma[c + 1], sm.mean[b][c + 1], d1);
                d2 = fma(ma[c + 2], sm.mean[b][c + 2], d2);
                d3 = fma(ma[c + 3], sm.mean[b][c + 3], d3);
            }
            const double dot = (d0 + d1) + (d2 + d3);
            const double cost = (double)(na * nb) / (double)(na + nb) * ((sqa + sm.sq[b]) - 2.0 * dot);
            if (b != a && na > 0 && na + nb <= kLsaCap && cost < c1) {
                c1 = cost;
                b1 = b;
            }
        }
        sm.half_best[hb][a] = b1;
        sm.half_cost[hb][a] = c1;
        if (t == 0) sm.npairs = 0;
        __syncthreads();
        // the lower half holds the lower partner ids: it wins ties
        if (t < kLsaPoints) {
            const bool hi = sm.half_cost[1][t] < sm.half_cost[0][t];
            sm.best[t] = sm.half_best[hi][t];
            sm.half_cost[0][t] = sm.half_cost[hi][t];
        }
        __syncthreads();
        if (t < kLsaPoints) {
            const int b = sm.best[t];
            if (b > t && sm.best[b] == t) {
                const int i = atomicAdd(&sm.npairs, 1);
                sm.pair_a[i] = t;
                sm.pair_b[i] = b;
                sm.pair_cost[i] = sm.half_cost[0][t];
            }
        }
        __syncthreads();
        const int np = sm.npairs;
        // some admissible pair is always mutual (the cheapest one, lowest
        // indices first) while more than 64 buckets remain; none exists
        // only when costs are not finite (non-finite keys)
        if (np == 0) break;
        const int take = min(np, count - kLsaBuckets);
        // the cheapest `take` pairs merge (ties: lower first bucket); the
        // larger bucket index joins the smaller, which stays the root
        if (t < np) {
            const double ci = sm.pair_cost[t];
            const int ai = sm.pair_a[t];
            int rank = 0;
            for (int j = 0; j < np; ++j) {
                const double cj = sm.pair_cost[j];
                rank += (cj < ci || (cj == ci && sm.pair_a[j] < ai)) ? 1 : 0;
            }
            sm.merge[t] = rank < take;
        }
        __syncthreads();
        for (int e = t; e < np * kDim; e += kLsaThreads) {
            const int i = e / kDim, c = e % kDim;
            if (sm.merge[i]) sm.sum[sm.pair_a[i]][c] += sm.sum[sm.pair_b[i]][c];
        }
        __syncthreads();
        if (t < np && sm.merge[t]) {
            const int pa = sm.pair_a[t], pb = sm.pair_b[t];
            sm.cnt[pa] += sm.cnt[pb];
            sm.cnt[pb] = 0;
            sm.parent[pb] = pa;
        }
        __syncthreads();
        for (int e = t; e < np * kDim; e += kLsaThreads) {
            const int i = e / kDim, c = e % kDim;
            const int pa = sm.pair_a[i];
            if (sm.merge[i]) sm.mean[pa][c] = sm.sum[pa][c] / (double)sm.cnt[pa];
        }
        __syncthreads();
        if (t < np && sm.merge[t]) {
            const int pa = sm.pair_a[t];
            double s = 0.0;
            for (int c = 0; c < kDim; ++c) s += sm.mean[pa][c] * sm.mean[pa][c];
            sm.sq[pa] = s;
        }
        if (t == 0) sm.count = count - take;
    }
    uint8_t* mb = members + blk * kLsaPoints;
    uint8_t* ob = offs + blk * (kLsaBuckets + 1);
    uint16_t* cb = centroids + (size_t)blk * kLsaBuckets * kDim;
    __syncthreads();
    if (sm.count != kLsaBuckets) {
        // non-finite keys: every bucket empty, zero centroids
        if (t < kLsaPoints) mb[t] = (uint8_t)t;
        if (t <= kLsaBuckets) ob[t] = 0;
        for (int e = t; e < kLsaBuckets * kDim; e += kLsaThreads) cb[e] = 0;
        return;
    }
    // bucket ids in order of their root (the smallest pool key), starts by
    // a scan of the sizes; every point's slot is the number of smaller
    // points of its bucket
    if (t == 0) {
        int n = 0, s = 0;
        for (int r = 0; r < kLsaPoints; ++r) {
            if (sm.cnt[r] == 0) continue;
            sm.id[r] = n;
            sm.start[n] = s;
            s += sm.cnt[r];
            ++n;
        }
        sm.start[kLsaBuckets] = s;
    }
    __syncthreads();
    if (t < kLsaPoints) {
        int r = t;
        while (sm.parent[r] != r) r = sm.parent[r];
        sm.half_best[0][t] = r;                   // the point's root
    }
    __syncthreads();
    if (t < kLsaPoints) {
        const int r = sm.half_best[0][t];
        int slot = 0;
        for (int j = 0; j < t; ++j) slot += sm.half_best[0][j] == r ? 1 : 0;
        sm.memb[sm.start[sm.id[r]] + slot] = (uint8_t)t;
    }
    if (t <= kLsaBuckets) ob[t] = (uint8_t)sm.start[t];
    __syncthreads();
    if (t < kLsaPoints) mb[t] = sm.memb[t];
    // centroids: the pool keys again, summed in ascending member order,
    // normalised, rounded to bf16; four threads per bucket, 16 dims each
    lsa_pool_keys(kb, sm.mean);
    __syncthreads();
    {
        const int bkt = t >> 2, q4 = t & 3;
        const int s0 = sm.start[bkt], s1 = sm.start[bkt + 1];
        double v[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) v[i] = 0.0;
        for (int j = s0; j < s1; ++j) {
            const int pt = sm.memb[j];
#pragma unroll
            for (int i = 0; i < 16; ++i) v[i] += sm.mean[pt][q4 * 16 + i];
        }
        double ss = 0.0;
#pragma unroll
        for (int i = 0; i < 16; ++i) ss += v[i] * v[i];
        const double s01 = ss + __shfl_xor(ss, 1);       // the same sums in all four lanes,
        const double o01 = __shfl_xor(s01, 2);           // added in one fixed order
        const double nn = (q4 & 2) ? o01 + s01 : s01 + o01;
        const double norm = sqrt(nn);
        uint16_t* cr = cb + (size_t)bkt * kDim + q4 * 16;
#pragma unroll
        for (int i = 0; i < 16; ++i) cr[i] = f64_to_bf16_rne(norm > 0.0 ? v[i] / norm : 0.0);
    }
}

// ---- flat search -------------------------------------------------------------

constexpr int kLsaFillThreads = 512;
constexpr int kLsaMaxP = HISA_LSA_MAX_P;
constexpr int kLsaMaxWords = (int)(HISA_LSA_MAX_LEN / kLsaBlock * kLsaPoints / 32);   // pool-key bitmap

// Per query: the last visible bucket of its sequence, or -1 (invalid query
// or no complete block before it).  Per sequence: bucket offset and count,
// in the form the flat indexer takes (keys -> centroids).
__global__ void lsa_meta_kernel(const int64_t* q_pos, const int32_t* q_seq, int64_t nq, const int64_t* seq_blk_off,
                                const int64_t* seq_nblk, const int64_t* seq_len, int nseq, int64_t max_blocks,
                                int64_t* q_bucket, int64_t* q_blk_off, int64_t* seq_boff, int64_t* seq_blen)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < nq) {
        const int s = q_seq ? q_seq[i] : 0;
        int64_t last = -1, bo = 0;
        if (s >= 0 && s < nseq) {
            bo = seq_blk_off[s];
            const int64_t t = q_pos[i];
            if (t >= 0 && t < seq_len[s]) {
                // never more blocks than the host bound the fill kernel's
                // bitmap is sized for
                const int64_t vis = min(min((t + 1) / kLsaBlock, seq_nblk[s]), max_blocks);
                last = vis * kLsaBuckets - 1;
            }
        }
        q_bucket[i] = last;
        q_blk_off[i] = bo;
    }
    if (i < nseq) {
        seq_boff[i] = seq_blk_off[i] * kLsaBuckets;
        seq_blen[i] = max<int64_t>(min(seq_nblk[i], max_blocks) * kLsaBuckets, 1);
    }
}

// One workgroup per query.  Every selected bucket's id, score, offsets and
// members are loaded up front (three dependent round trips, all entries at
// once) into a 64-bit payload; the buckets are ranked (score descending,
// lower id first: the selection lists them by ascending id, so the entry
// index breaks ties) by counting for up to kLsaCountRank entries, by a
// bitonic sort beyond; their sizes are scanned in rank order, the pool keys
// of the buckets that fit (the last one cut to the keys left) are marked
// in a bitmap, and the positions are written in ascending order.
constexpr int kLsaCountRank = 512;

__host__ __device__ constexpr size_t lsa_rank_bytes(int P2)
{
    return (size_t)P2 * 16 > (size_t)kLsaFillThreads * 4 ? (size_t)P2 * 16 : (size_t)kLsaFillThreads * 4;
}

// payload: bucket id (bits 0-31), pool-key count (32-34), up to four
// member pool keys (7 bits each from bit 35)
__device__ __forceinline__ uint64_t lsa_payload(uint32_t id, int n, const int (&m)[kLsaCap])
{
    uint64_t v = (uint64_t)id | ((uint64_t)n << 32);
#pragma unroll
    for (int j = 0; j < kLsaCap; ++j) v |= (uint64_t)(m[j] & 127) << (35 + 7 * j);
    return v;
}

__global__ __launch_bounds__(kLsaFillThreads) void lsa_fill_kernel(const int32_t* sel, const float* score, int p,
                                                                   int P2, const int64_t* q_bucket,
                                                                   const int64_t* q_blk_off, const uint8_t* members,
                                                                   const uint8_t* offs, int k, int32_t* out_idx,
                                                                   int32_t* out_buckets)
{
    extern __shared__ uint64_t s_dyn[];
    uint64_t* skey = s_dyn;                                     // [P2] rank keys, then sorted
    uint64_t* pay = skey + P2;                                  // [P2] payload by entry
    // [visible words], after the rank arrays (at least one int per thread:
    // they hold the owners' first slots at the end)
    uint32_t* bits = reinterpret_cast<uint32_t*>(reinterpret_cast<char*>(s_dyn) + lsa_rank_bytes(P2));
    __shared__ int s_scan[kLsaFillThreads / 64];
    __shared__ int s_part_g, s_part_n;
    constexpr int kPer = kLsaMaxP / kLsaFillThreads;            // entries per thread
    const int t = threadIdx.x;
    const int64_t row = blockIdx.x;
    int32_t* orow = out_idx + row * (int64_t)k;
    int32_t* brow = out_buckets ? out_buckets + row * (int64_t)p : nullptr;
    // one round trip for the query's meta data and its selected buckets
    // (rows of an invalid query hold -1 entries), then the offsets, then
    // the members
    const int64_t last = q_bucket[row];
    const int64_t boff = q_blk_off[row];
    int32_t id[kPer];
    uint32_t sk[kPer];
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        const int i = t + j * kLsaFillThreads;
        id[j] = i < p ? sel[row * p + i] : -1;
        sk[j] = i < p ? score_key(score[row * p + i]) : 0u;
    }
    if (last < 0) {
        for (int e = t; e < k; e += kLsaFillThreads) orow[e] = -1;
        if (brow)
            for (int e = t; e < p; e += kLsaFillThreads) brow[e] = -1;
        return;
    }
    const int words = (int)((last + 1) / kLsaBuckets) * (kLsaPoints / 32);
    int o0[kPer], o1[kPer];
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        o0[j] = o1[j] = 0;
        if (id[j] >= 0) {
            const int64_t base = (boff + id[j] / kLsaBuckets) * (kLsaBuckets + 1) + id[j] % kLsaBuckets;
            // offsets clamped to the block row: a damaged cache cannot send
            // the reads past it
            o1[j] = min((int)offs[base + 1], kLsaPoints);
            o0[j] = min((int)offs[base], o1[j]);
            o1[j] = min(o1[j], o0[j] + kLsaCap);
        }
    }
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        const int i = t + j * kLsaFillThreads;
        if (i >= P2) continue;
        int m[kLsaCap];
        const uint8_t* mrow = members + (boff + max(id[j], 0) / kLsaBuckets) * kLsaPoints;
#pragma unroll
        for (int c = 0; c < kLsaCap; ++c) m[c] = o0[j] + c < o1[j] ? mrow[o0[j] + c] : 0;
        pay[i] = lsa_payload((uint32_t)id[j], o1[j] - o0[j], m);
        skey[i] = id[j] >= 0 ? ((uint64_t)sk[j] << 32) | (uint32_t)~(uint32_t)i : 0ull;
    }
    for (int i = t; i < words; i += kLsaFillThreads) bits[i] = 0u;
    if (t == 0) {
        s_part_g = -1;
        s_part_n = 0;
    }
    __syncthreads();
    if (P2 <= kLsaCountRank) {
        // rank = number of larger keys (keys are distinct); then place
        uint64_t mine[kLsaCountRank / kLsaFillThreads];
        int rank[kLsaCountRank / kLsaFillThreads];
#pragma unroll
        for (int j = 0; j < kLsaCountRank / kLsaFillThreads; ++j) {
            const int i = t + j * kLsaFillThreads;
            mine[j] = i < P2 ? skey[i] : 0ull;
            int r = 0;
            for (int x = 0; x < P2; ++x) r += skey[x] > mine[j] ? 1 : 0;
            rank[j] = r;
        }
        __syncthreads();
        // clear, then place the keys of real buckets (the empty ones rank
        // last and stay zero)
#pragma unroll
        for (int j = 0; j < kLsaCountRank / kLsaFillThreads; ++j) {
            const int i = t + j * kLsaFillThreads;
            if (i < P2) skey[i] = 0ull;
        }
        __syncthreads();
#pragma unroll
        for (int j = 0; j < kLsaCountRank / kLsaFillThreads; ++j) {
            const int i = t + j * kLsaFillThreads;
            if (i < P2 && mine[j] != 0ull) skey[rank[j]] = mine[j];
        }
    } else {
        for (int size = 2; size <= P2; size <<= 1) {
            for (int stride = size >> 1; stride > 0; stride >>= 1) {
                for (int i = t; i < (P2 >> 1); i += kLsaFillThreads) {
                    const int lo = 2 * i - (i & (stride - 1));
                    const int hi = lo + stride;
                    const bool desc = (lo & size) == 0;
                    const uint64_t x = skey[lo], y = skey[hi];
                    if ((x < y) == desc) {
                        skey[lo] = y;
                        skey[hi] = x;
                    }
                }
                __syncthreads();
            }
        }
    }
    __syncthreads();
    // sizes in rank order: thread t owns ranks [t * per, (t + 1) * per)
    const int per = (P2 + kLsaFillThreads - 1) / kLsaFillThreads;
    int mine_keys = 0;
    for (int j = 0; j < per; ++j) {
        const int r = t * per + j;
        if (r < p && skey[r] != 0ull)
            mine_keys += kLsaPool * (int)((pay[~(uint32_t)skey[r]] >> 32) & 7u);
    }
    int excl = wg_incl_scan<kLsaFillThreads>(mine_keys, s_scan) - mine_keys;
    for (int j = 0; j < per; ++j) {
        const int r = t * per + j;
        if (r >= p) break;
        int32_t used = -1;
        if (skey[r] != 0ull && excl < k) {
            const uint64_t v = pay[~(uint32_t)skey[r]];
            const uint32_t bid = (uint32_t)v;
            const int n = (int)((v >> 32) & 7u);
            const int take = min(kLsaPool * n, k - excl);
            for (int c = 0; c < n; ++c) {
                const int got = take - kLsaPool * c;
                if (got <= 0) break;
                const int g = (int)(bid / kLsaBuckets) * kLsaPoints + (int)((v >> (35 + 7 * c)) & 127u);
                atomicOr(&bits[g >> 5], 1u << (g & 31));
                if (got < kLsaPool) {
                    s_part_g = g;
                    s_part_n = got;
                }
            }
            excl += kLsaPool * n;
            used = (int32_t)bid;
        }
        if (brow) brow[r] = used;
    }
    __syncthreads();
    // emit: thread t owns words [t * wper, (t + 1) * wper); after a scan of
    // their set-bit counts it lists their pool keys, ascending, in LDS (over
    // the rank arrays, which are free now: at most 4 pool keys per bucket,
    // so at most 4 * P2 of them); then every output slot e (strided over
    // the threads, so the stores coalesce) reads its pool key from the list,
    // the slots past the partial pool key shifted by the keys it lacks
    const int wper = (words + kLsaFillThreads - 1) / kLsaFillThreads;
    const int pg = s_part_g, pn = s_part_n;
    int cnt = 0;
    for (int j = 0; j < wper; ++j) {
        const int wi = t * wper + j;
        if (wi < words) cnt += __popc(bits[wi]);
    }
    const int incl = wg_incl_scan<kLsaFillThreads>(cnt, s_scan);
    int* list = reinterpret_cast<int*>(skey);
    int o = incl - cnt;
    for (int j = 0; j < wper; ++j) {
        const int wi = t * wper + j;
        if (wi >= words) break;
        uint32_t b = bits[wi];
        while (b) {
            const int g = wi * 32 + __builtin_ctz(b);
            b &= b - 1u;
            if (o < 4 * P2) list[o] = g;
            if (g == pg) s_part_g = o;       // the partial pool key's ordinal
            ++o;
        }
    }
    if (t == kLsaFillThreads - 1) s_scan[0] = incl;
    __syncthreads();
    const int ip = pg >= 0 ? s_part_g : -1;
    const int nkeys = min(s_scan[0], 4 * P2);
    const int total = min(kLsaPool * nkeys - (ip >= 0 ? kLsaPool - pn : 0), k);
    for (int e = t; e < total; e += kLsaFillThreads) {
        int x = e;
        if (ip >= 0 && e >= kLsaPool * ip + pn) x += kLsaPool - pn;
        orow[e] = kLsaPool * list[x / kLsaPool] + x % kLsaPool;
    }
    for (int e = total + t; e < k; e += kLsaFillThreads) orow[e] = -1;
}

}  // namespace

hipError_t launch_lsa_build(const uint16_t* keys, int64_t b0, int64_t nblk, uint16_t* centroids, uint8_t* members,
                            uint8_t* offs, hipStream_t stream)
{
    if (nblk <= 0) return hipSuccess;
    hipLaunchKernelGGL(lsa_build_kernel, dim3((unsigned)nblk), dim3(kLsaThreads), 0, stream, keys, b0, centroids,
                       members, offs);
    return hipGetLastError();
}

}  // namespace hisa

// ---- C ABI --------------------------------------------------------------------

namespace {

using namespace hisa;

size_t align_256(size_t x) { return (x + 255) / 256 * 256; }

int lsa_validate(const hisa_lsa_args* a)
{
    if (!a) return HISA_ERR_INVALID_ARG;
    if (a->nq < 0 || a->nseq < 1 || a->p < 1 || a->k < 1 || a->max_len < 1) return HISA_ERR_INVALID_ARG;
    if (a->d != kDim || a->p > HISA_LSA_MAX_P || a->k > HISA_MAX_K || a->max_len > HISA_LSA_MAX_LEN)
        return HISA_ERR_UNSUPPORTED;
    if (a->nq == 0) return HISA_OK;
    if (!a->queries || !a->q_pos || !a->centroids || !a->members || !a->offs || !a->seq_blk_off || !a->seq_nblk ||
        !a->seq_len || !a->out_idx)
        return HISA_ERR_INVALID_ARG;
    return HISA_OK;
}

// The bucket-level flat call: centroids as keys, the last visible bucket
// as each query's position.
hisa_index_args bucket_args(const hisa_lsa_args* a, int64_t* q_bucket, int64_t* seq_boff, int64_t* seq_blen,
                            int32_t* sel, float* score, void* ws, size_t ws_bytes)
{
    hisa_index_args b;
    memset(&b, 0, sizeof b);
    b.queries = a->queries;
    b.q_pos = q_bucket;
    b.q_seq = a->q_seq;
    b.nq = a->nq;
    b.keys = a->centroids;
    b.seq_key_off = seq_boff;
    b.seq_len = seq_blen;
    b.nseq = a->nseq;
    b.max_len = std::max<int64_t>(a->max_len / kLsaBlock * kLsaBuckets, 1);
    b.d = a->d;
    b.k = a->p;
    b.out_idx = sel;
    b.out_scores = score;
    b.workspace = ws;
    b.workspace_bytes = ws_bytes;
    return b;
}

struct LsaLayout {
    size_t q_bucket, q_blk_off, seq_boff, seq_blen, sel, score, flat, total;
};

LsaLayout lsa_layout(const hisa_lsa_args* a, size_t flat_bytes)
{
    LsaLayout L;
    size_t off = 0;
    L.q_bucket = off;
    off += align_256((size_t)std::max<int64_t>(a->nq, 1) * 8);
    L.q_blk_off = off;
    off += align_256((size_t)std::max<int64_t>(a->nq, 1) * 8);
    L.seq_boff = off;
    off += align_256((size_t)a->nseq * 8);
    L.seq_blen = off;
    off += align_256((size_t)a->nseq * 8);
    L.sel = off;
    off += align_256((size_t)std::max<int64_t>(a->nq, 1) * a->p * 4);
    L.score = off;
    off += align_256((size_t)std::max<int64_t>(a->nq, 1) * a->p * 4);
    L.flat = off;
    L.total = off + flat_bytes;
    return L;
}

int next_pow2(int x)
{
    int p = 1;
    while (p < x) p <<= 1;
    return p;
}

}  // namespace

extern "C" {

int hisa_lsa_build(const uint16_t* keys, int64_t len, int64_t first_block, int d, uint16_t* centroids,
                   uint8_t* members, uint8_t* offs, void* stream)
{
    if (len < 0 || first_block < 0) return HISA_ERR_INVALID_ARG;
    if (d != kDim) return HISA_ERR_UNSUPPORTED;
    if (len > HISA_LSA_MAX_LEN) return HISA_ERR_UNSUPPORTED;
    const int64_t nblk = len / kLsaBlock - first_block;
    if (nblk <= 0) return HISA_OK;
    if (!keys || !centroids || !members || !offs) return HISA_ERR_INVALID_ARG;
    if (reinterpret_cast<uintptr_t>(keys) & 15) return HISA_ERR_UNSUPPORTED;
    return launch_lsa_build(keys, first_block, nblk, centroids, members, offs, static_cast<hipStream_t>(stream)) ==
                   hipSuccess
               ? HISA_OK
               : HISA_ERR_HIP;
}

int hisa_lsa_workspace_bytes(const hisa_lsa_args* a, size_t* bytes)
{
    if (!bytes) return HISA_ERR_INVALID_ARG;
    const int rc = lsa_validate(a);
    if (rc != HISA_OK) return rc;
    if (a->nq == 0) {
        *bytes = 0;
        return HISA_OK;
    }
    hisa_index_args b = bucket_args(a, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 0);
    // sizing only: the flat validation wants non-null pointers
    b.q_pos = reinterpret_cast<const int64_t*>(16);
    b.seq_key_off = reinterpret_cast<const int64_t*>(16);
    b.seq_len = reinterpret_cast<const int64_t*>(16);
    b.out_idx = reinterpret_cast<int32_t*>(16);
    size_t want = 0, least = 0, all = 0;
    const int frc = hisa_workspace_bytes(&b, 1, &want, &least, &all);
    if (frc != HISA_OK) return frc;
    *bytes = lsa_layout(a, want).total;
    return HISA_OK;
}

int hisa_lsa_index(const hisa_lsa_args* a, void* stream_)
{
    const int rc = lsa_validate(a);
    if (rc != HISA_OK) return rc;
    if (a->nq == 0) return HISA_OK;
    if (!a->workspace) return HISA_ERR_WORKSPACE;
    const LsaLayout L = lsa_layout(a, 0);
    if (a->workspace_bytes <= L.total) return HISA_ERR_WORKSPACE;
    hipStream_t stream = static_cast<hipStream_t>(stream_);
    char* ws = static_cast<char*>(a->workspace);
    int64_t* q_bucket = reinterpret_cast<int64_t*>(ws + L.q_bucket);
    int64_t* q_blk_off = reinterpret_cast<int64_t*>(ws + L.q_blk_off);
    int64_t* seq_boff = reinterpret_cast<int64_t*>(ws + L.seq_boff);
    int64_t* seq_blen = reinterpret_cast<int64_t*>(ws + L.seq_blen);
    int32_t* sel = reinterpret_cast<int32_t*>(ws + L.sel);
    float* score = reinterpret_cast<float*>(ws + L.score);
    const int64_t nthreads = std::max<int64_t>(a->nq, a->nseq);
    hipLaunchKernelGGL(lsa_meta_kernel, dim3((unsigned)((nthreads + 255) / 256)), dim3(256), 0, stream, a->q_pos,
                       a->q_seq, a->nq, a->seq_blk_off, a->seq_nblk, a->seq_len, (int)a->nseq,
                       (int64_t)(a->max_len / kLsaBlock), q_bucket, q_blk_off, seq_boff, seq_blen);
    if (hipGetLastError() != hipSuccess) return HISA_ERR_HIP;
    hisa_index_args b = bucket_args(a, q_bucket, seq_boff, seq_blen, sel, score, ws + L.flat,
                                    a->workspace_bytes - L.flat);
    const int frc = hisa_flat_index(&b, stream_);
    if (frc != HISA_OK) return frc;
    const int P2 = next_pow2(a->p);
    const int words = (int)(a->max_len / kLsaBlock * kLsaPoints / 32);
    const size_t lds = lsa_rank_bytes(P2) + (size_t)std::max(words, 1) * 4;
    hipLaunchKernelGGL(lsa_fill_kernel, dim3((unsigned)a->nq), dim3(kLsaFillThreads), lds, stream,
                       static_cast<const int32_t*>(sel), static_cast<const float*>(score), (int)a->p, P2,
                       static_cast<const int64_t*>(q_bucket), static_cast<const int64_t*>(q_blk_off), a->members,
                       a->offs, (int)a->k, a->out_idx, a->out_buckets);
    if (hipGetLastError() != hipSuccess) return HISA_ERR_HIP;
    return HISA_OK;
}

}  // extern "C"
