// libhisa kernels for gfx950: mean pooling / append, HISA stage 1 (block
// scores, causal + forced top-m), HISA stage 2 (token scores in the kept
// blocks), the flat indexer's scores, and top-k selection.
//
// What each kernel computes follows "HISA: Efficient Hierarchical Indexing
// for Fine-Grained Sparse Attention" (aitrends.kr summary): structure
// paragraph (blocks of B, mean-pooled representatives), stage-1 paragraph
// (inner-product block scores, causal mask, first and last two blocks
// forced, top-m), stage-2 paragraph (token scores only inside the kept
// blocks, top-k out), maintenance paragraph (representatives updated at
// append); and the "DSA" section of "Why long-context LLMs slow down and
// how sparse attention fixes it" (idea.jsleekr.com) for the flat indexer.
#include "kernels.h"

#include <hip/hip_ext.h>
#include <math.h>

#include <algorithm>

#include "common.h"
#include "select.h"

namespace hisa {

template <class T>
struct exact {
    using type = T;
};

// Launch `kernel` with arguments converted to its exact parameter types,
// recording the optional start / stop events from the dispatch itself.
template <typename... P>
static hipError_t launch_k(void (*kernel)(P...), dim3 grid, dim3 block, hipStream_t stream, hipEvent_t ev0,
                           hipEvent_t ev1, typename exact<P>::type... args)
{
    hipExtLaunchKernelGGL(kernel, grid, block, 0, stream, ev0, ev1, 0, args...);
    return hipGetLastError();
}

// The same with `lds` bytes of dynamic shared memory.
template <typename... P>
static hipError_t launch_kl(void (*kernel)(P...), dim3 grid, dim3 block, size_t lds, hipStream_t stream,
                            hipEvent_t ev0, hipEvent_t ev1, typename exact<P>::type... args)
{
    hipExtLaunchKernelGGL(kernel, grid, block, lds, stream, ev0, ev1, 0, args...);
    return hipGetLastError();
}

__global__ __launch_bounds__(kThreads) void fill_u32_kernel(uint32_t* p, int64_t n, uint32_t v)
{
    const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (i < n) p[i] = v;
}

// ---- pooling and append ---------------------------------------------------
// One workgroup per block: 8 threads cover one 128-byte key row (16 bytes,
// 8 dims each), 32 rows in flight per step, so every load is a fully used
// 16-byte vector.  The sum is taken in fp64, where adding bf16 values is
// exact (see the precondition in hisa.h), so the partial-sum order does not
// change the result.

struct PoolJobs {
    PoolJob j[kPoolJobsPerLaunch];
};

struct DecodeJobs {
    PoolJob j[kDecodeJobs];
};

// Block `bx` of one job: load every row of the block (old rows from the
// cache, new rows from new_keys), write the new rows, write the block's
// representative.
HISA_INLINE void pool_block(uint16_t* keys, uint16_t* reps, const uint16_t* new_keys, int B, const PoolJob& job,
                            int64_t bx)
{
    const int64_t blk = job.blk_first + bx;
    const int64_t start = blk * B;
    const int count = (int)min((int64_t)B, job.len_new - start);
    const int col = threadIdx.x & 7;
    const int grp = threadIdx.x >> 3;

    // every row of the block is loaded before any is used, so one block
    // costs one memory round trip; new rows are then written to the cache
    constexpr int kPasses = kMaxB / (kThreads / 8);
    uint4 v[kPasses];
#pragma unroll
    for (int p = 0; p < kPasses; ++p) {
        const int r = grp + p * (kThreads / 8);
        const int64_t j = start + r;
        v[p] = make_uint4(0u, 0u, 0u, 0u);
        if (r < count)
            v[p] = j < job.len_old
                       ? reinterpret_cast<const uint4*>(keys + (job.key_off + j) * kDim)[col]
                       : reinterpret_cast<const uint4*>(new_keys + (job.new_row + (j - job.len_old)) * kDim)[col];
    }
#pragma unroll
    for (int p = 0; p < kPasses; ++p) {
        const int r = grp + p * (kThreads / 8);
        const int64_t j = start + r;
        if (r < count && j >= job.len_old) reinterpret_cast<uint4*>(keys + (job.key_off + j) * kDim)[col] = v[p];
    }
    double acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.0;
#pragma unroll
    for (int p = 0; p < kPasses; ++p) {
        const uint32_t w[4] = {v[p].x, v[p].y, v[p].z, v[p].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            acc[2 * e + 0] += (double)bf16_lo(w[e]);
            acc[2 * e + 1] += (double)bf16_hi(w[e]);
        }
    }
    __shared__ double part[32][kDim];
#pragma unroll
    for (int e = 0; e < 8; ++e) part[grp][col * 8 + e] = acc[e];
    __syncthreads();
    if (threadIdx.x < kDim) {
        double s = 0.0;
        for (int g = 0; g < 32; ++g) s += part[g][threadIdx.x];
        const double mean = s / (double)count;
        reps[(job.rep_off + blk) * kDim + threadIdx.x] = f64_to_bf16_rne(mean);
    }
}

__global__ __launch_bounds__(kThreads) void pool_kernel(uint16_t* keys, uint16_t* reps, const uint16_t* new_keys,
                                                        int B, PoolJobs jobs)
{
    const PoolJob& job = jobs.j[blockIdx.y];
    if ((int64_t)blockIdx.x >= job.nblk) return;
    pool_block(keys, reps, new_keys, B, job, blockIdx.x);
}

hipError_t launch_pool(uint16_t* keys, uint16_t* reps, const uint16_t* new_keys, int B, const PoolJob* jobs,
                       int njobs, hipStream_t stream)
{
    for (int base = 0; base < njobs; base += kPoolJobsPerLaunch) {
        const int n = std::min(kPoolJobsPerLaunch, njobs - base);
        PoolJobs pj;
        int64_t maxblk = 0;
        for (int i = 0; i < kPoolJobsPerLaunch; ++i) {
            pj.j[i] = i < n ? jobs[base + i] : PoolJob{0, 0, 0, 0, 0, 0, 0, 0};
            if (i < n) maxblk = std::max<int64_t>(maxblk, pj.j[i].nblk);
        }
        if (maxblk == 0) continue;
        const hipError_t err = launch_k(pool_kernel, dim3((unsigned)maxblk, (unsigned)n), dim3(kThreads), stream,
                                        nullptr, nullptr, keys, reps, new_keys, B, pj);
        if (err != hipSuccess) return err;
    }
    return hipSuccess;
}

// ---- HISA stage 1: block scores ----------------------------------------------
// One thread per (query, causal block): a 128-byte representative row
// against the query held in registers.  Used when a query has too many
// blocks for one workgroup to score (long contexts).

__global__ __launch_bounds__(kThreads) void block_score_kernel(QueryMeta qm, const uint16_t* reps, int64_t q0,
                                                               int lb, int64_t Mmax, float* sigma)
{
    const int64_t row = blockIdx.y;
    const int64_t i = q0 + row;
    const QueryInfo qi =
        query_info(i, qm.q_pos, qm.q_seq, qm.seq_key_off, qm.seq_rep_off, qm.seq_len, qm.nseq, qm.max_len);
    if (!qi.valid) return;
    const int64_t c = qi.t >> lb;
    const int64_t b = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (b < 1 || b > c - 2) return;               // the selection reads only the free candidates
    uint32_t q[32];
    load_query(qm.queries + i * kDim, q);
    const uint4* rp = reinterpret_cast<const uint4*>(reps + (qi.rep_off + b) * kDim);
    sigma[row * Mmax + b] = dot64_packed(q, rp);
}

// The same with a decode step's append folded in: rows y < njobs run the
// append jobs (job y, block x), rows y >= njobs score query y - njobs.  The
// blocks the append re-pools are the queries' forced last two, which are
// not scored; the token stage runs after this launch.
__global__ __launch_bounds__(kThreads) void block_score_append_kernel(QueryMeta qm, uint16_t* reps, uint16_t* keys,
                                                                      const uint16_t* new_keys, int B,
                                                                      DecodeJobs jobs, int njobs, int64_t q0, int lb,
                                                                      int64_t Mmax, float* sigma)
{
    if ((int)blockIdx.y < njobs) {
        const PoolJob& job = jobs.j[blockIdx.y];
        if ((int64_t)blockIdx.x < job.nblk) pool_block(keys, reps, new_keys, B, job, blockIdx.x);
        return;
    }
    const int64_t row = blockIdx.y - njobs;
    const int64_t i = q0 + row;
    const QueryInfo qi =
        query_info(i, qm.q_pos, qm.q_seq, qm.seq_key_off, qm.seq_rep_off, qm.seq_len, qm.nseq, qm.max_len);
    if (!qi.valid) return;
    const int64_t c = qi.t >> lb;
    const int64_t b = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (b < 1 || b > c - 2) return;
    uint32_t q[32];
    load_query(qm.queries + i * kDim, q);
    const uint4* rp = reinterpret_cast<const uint4*>(reps + (qi.rep_off + b) * kDim);
    sigma[row * Mmax + b] = dot64_packed(q, rp);
}

// ---- HISA stage 1: causal + forced top-m -----------------------------------
// One workgroup per query.  Block b sits in slot b; the free candidates are
// blocks 1 .. c-2, from which m-3 are chosen; blocks 0, c-1, c are added and
// the kept list comes out ascending.  FUSED: the workgroup scores the
// representatives itself; otherwise it reads the scores from sigma.

template <int NT, int ITEMS, bool FUSED>
__global__ __launch_bounds__(NT) void stage1_select_kernel(QueryMeta qm, const uint16_t* reps, int64_t q0, int lb,
                                                           int m, int64_t Mmax, const float* sigma, int32_t* sel,
                                                           RowInfo* rinfo, int32_t* out_blocks)
{
    __shared__ BucketSmem<NT> sm;
    const int64_t row = blockIdx.x;
    const int64_t i = q0 + row;
    const QueryInfo qi =
        query_info(i, qm.q_pos, qm.q_seq, qm.seq_key_off, qm.seq_rep_off, qm.seq_len, qm.nseq, qm.max_len);
    if (threadIdx.x == 0) rinfo[row] = RowInfo{qi.key_off, qi.valid ? qi.t : -1};
    int32_t* srow = sel + row * m;
    int32_t* orow = out_blocks ? out_blocks + i * m : nullptr;
    if (!qi.valid) {
        for (int r = threadIdx.x; r < m; r += NT) {
            srow[r] = -1;
            if (orow) orow[r] = -1;
        }
        return;
    }
    const int64_t c = qi.t >> lb;
    if (c + 1 <= m) {
        for (int r = threadIdx.x; r < m; r += NT) {
            const int32_t v = r <= c ? r : -1;
            srow[r] = v;
            if (orow) orow[r] = v;
        }
        return;
    }
    uint32_t key[ITEMS];
    if (FUSED) {
        uint32_t q[32];
        load_query(qm.queries + i * kDim, q);
#pragma unroll
        for (int it = 0; it < ITEMS; ++it) {
            const int64_t b = slot_of<ITEMS>(it);
            key[it] = (b >= 1 && b <= c - 2)
                          ? score_key(dot64_packed(q, reinterpret_cast<const uint4*>(reps + (qi.rep_off + b) * kDim)))
                          : 0u;
        }
    } else {
        const float* sg = sigma + row * Mmax;
#pragma unroll
        for (int it = 0; it < ITEMS; ++it) {
            const int64_t b = slot_of<ITEMS>(it);
            key[it] = (b >= 1 && b <= c - 2) ? score_key(sg[b]) : 0u;
        }
    }
    const Threshold th = wg_bucket_select<NT, ITEMS>(key, m - 3, sm);
    wg_emit_selected<NT, ITEMS>(key, th, sm, m - 3, [&](int slot, uint32_t, int rank) {
        srow[1 + rank] = slot;
        if (orow) orow[1 + rank] = slot;
    });
    if (threadIdx.x == 0) {
        srow[0] = 0;
        srow[m - 2] = (int32_t)(c - 1);
        srow[m - 1] = (int32_t)c;
        if (orow) {
            orow[0] = 0;
            orow[m - 2] = (int32_t)(c - 1);
            orow[m - 1] = (int32_t)c;
        }
    }
}

template <int NT, int ITEMS, bool FUSED>
static hipError_t launch_stage1_items(const QueryMeta& qm, const uint16_t* reps, int64_t q0, int64_t nq, int lb,
                                      int m, int64_t Mmax, const float* sigma, int32_t* sel, RowInfo* rinfo,
                                      int32_t* out_blocks, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1)
{
    return launch_k(stage1_select_kernel<NT, ITEMS, FUSED>, dim3((unsigned)nq), dim3(NT), stream, ev0, ev1, qm, reps,
                    q0, lb, m, Mmax, sigma, sel, rinfo, out_blocks);
}

// Many queries (prefill): 16 consecutive query rows form a tile, one
// workgroup of WT waves per tile.  The waves score the tile's rows against
// the representatives on the bf16 MFMA together (the 16-block tiles dealt
// round-robin, 16 blocks x 16 rows per pair of v_mfma_f32_16x16x32_bf16)
// into the workgroup's LDS, so a representative is read once per query
// tile; then wave w selects the top-m of rows w, w+WT, ... with the
// barrier-free wave select.  WT grows when tiles are few, so the selects
// still fill the chip.  Rows of a tile in different sequences are handled
// one sequence at a time.  ITEMS = 64-slot groups per row: block b is slot b.

constexpr int kS1TileMaxBlocks = 1024;
constexpr int64_t kS1TargetWaves = 8192;   // measured: 32K prefill stage 1 34 -> 28 us against 4096
constexpr int kS1MaxWaves = 16;

__host__ __device__ constexpr int s1_row_stride(int items) { return 64 * items + 16; }   // floats; +16 spreads banks
__host__ __device__ constexpr size_t s1_tile_lds(int items, int wt)
{
    return (size_t)16 * s1_row_stride(items) * sizeof(float) + (size_t)wt * sizeof(WaveSmem);
}

template <int ITEMS>
__global__ __launch_bounds__(64 * kS1MaxWaves) void stage1_tile_kernel(QueryMeta qm, const uint16_t* reps, int64_t q0,
                                                                       int64_t nq, int lb, int m, int32_t* sel,
                                                                       RowInfo* rinfo, int32_t* out_blocks)
{
    extern __shared__ __align__(16) float s_dyn[];
    constexpr int RS = s1_row_stride(ITEMS);
    const int WT = (int)(blockDim.x >> 6);
    const int w = wave_id(), lane = lane_id();
    float* sc = s_dyn;                                   // [16][RS]: the tile's block scores
    WaveSmem& ws = reinterpret_cast<WaveSmem*>(s_dyn + 16 * RS)[w];
    const int64_t row0 = (int64_t)blockIdx.x * 16;
    const int nrows = (int)min<int64_t>(16, nq - row0);
    const int r = lane & 15;
    QueryInfo qi;
    qi.valid = false;
    qi.seq = -1;
    qi.t = -1;
    qi.key_off = 0;
    qi.rep_off = 0;
    if (lane < 16 && r < nrows) {
        qi = query_info(q0 + row0 + r, qm.q_pos, qm.q_seq, qm.seq_key_off, qm.seq_rep_off, qm.seq_len, qm.nseq,
                        qm.max_len);
        if (w == 0) rinfo[row0 + r] = RowInfo{qi.key_off, qi.valid ? qi.t : -1};
    }
    // invalid rows keep no block
    for (uint64_t iv = __ballot(lane < 16 && r < nrows && r % WT == w && !qi.valid); iv; iv &= iv - 1) {
        const int rr = (int)__builtin_ctzll(iv);
        for (int i = lane; i < m; i += 64) {
            sel[(row0 + rr) * m + i] = -1;
            if (out_blocks) out_blocks[(q0 + row0 + rr) * m + i] = -1;
        }
    }
    const int col = lane & 15, kg = lane >> 4;
    bf16x8_t a0 = {}, a1 = {};
    if (col < nrows) {
        const uint16_t* qrow = qm.queries + (q0 + row0 + col) * kDim + 8 * kg;
        a0 = *reinterpret_cast<const bf16x8_t*>(qrow);
        a1 = *reinterpret_cast<const bf16x8_t*>(qrow + 32);
    }
    const int c_own = qi.valid ? (int)(qi.t >> lb) : -1;
    // every wave computes the same row infos, so the loop below is uniform
    // over the workgroup
    const bool act = lane < 16 && r < nrows && qi.valid;
    uint64_t pending = __ballot(act);
    while (pending) {
        const int lead = (int)__builtin_ctzll(pending);
        const int s = __builtin_amdgcn_readlane(qi.seq, lead);
        const bool mine = act && qi.seq == s;
        const uint64_t mine_rows = __ballot(mine);
        pending &= ~mine_rows;
        const int64_t rep_off = ((int64_t)__builtin_amdgcn_readlane((int)(qi.rep_off >> 32), lead) << 32) |
                                (uint32_t)__builtin_amdgcn_readlane((int)qi.rep_off, lead);
        const int cmax = (int)wave_max_u32(mine ? (uint32_t)c_own : 0u);
        // scores of blocks 0 .. cmax: the representatives are the A
        // operand, so lane l receives blocks 4*(l/16)..+4 of the 16-block
        // tile for query row l%16 and stores them as one 16-byte vector
        for (int bt = w; bt * 16 <= cmax; bt += WT) {
            const int b = bt * 16 + col;
            bf16x8_t b0 = {}, b1 = {};
            if (b <= cmax) {
                const uint16_t* rp = reps + (rep_off + b) * kDim + 8 * kg;
                b0 = *reinterpret_cast<const bf16x8_t*>(rp);
                b1 = *reinterpret_cast<const bf16x8_t*>(rp + 32);
            }
            f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b0, a0, acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b1, a1, acc, 0, 0, 0);
            *reinterpret_cast<f32x4_t*>(sc + col * RS + bt * 16 + 4 * kg) = acc;
        }
        __syncthreads();
        for (int rr = w; rr < 16; rr += WT) {
            if (!((mine_rows >> rr) & 1ull)) continue;
            const int cr = __builtin_amdgcn_readlane(c_own, rr);
            int32_t* srow = sel + (row0 + rr) * m;
            int32_t* orow = out_blocks ? out_blocks + (q0 + row0 + rr) * m : nullptr;
            if (cr + 1 <= m) {
                for (int j = lane; j < m; j += 64) {
                    const int32_t v = j <= cr ? j : -1;
                    srow[j] = v;
                    if (orow) orow[j] = v;
                }
                continue;
            }
            uint32_t key[ITEMS];
#pragma unroll
            for (int it = 0; it < ITEMS; ++it) {
                const int b = it * 64 + lane;
                key[it] = (b >= 1 && b <= cr - 2) ? score_key(sc[rr * RS + b]) : 0u;
            }
            wave_select<ITEMS>(key, m - 3, ws, [&](int slot, uint32_t, int rank) {
                srow[1 + rank] = slot;
                if (orow) orow[1 + rank] = slot;
            });
            if (lane == 0) {
                srow[0] = 0;
                srow[m - 2] = cr - 1;
                srow[m - 1] = cr;
                if (orow) {
                    orow[0] = 0;
                    orow[m - 2] = cr - 1;
                    orow[m - 1] = cr;
                }
            }
        }
        __syncthreads();
    }
}

template <int ITEMS>
static hipError_t launch_stage1_tile_items(const QueryMeta& qm, const uint16_t* reps, int64_t q0, int64_t nq, int lb,
                                           int m, int32_t* sel, RowInfo* rinfo, int32_t* out_blocks,
                                           hipStream_t stream, Timing t)
{
    const int64_t tiles = (nq + 15) / 16;
    int WT = 1;
    while (WT < kS1MaxWaves && tiles * WT < kS1TargetWaves) WT *= 2;
    return launch_kl(stage1_tile_kernel<ITEMS>, dim3((unsigned)tiles), dim3(64 * WT), s1_tile_lds(ITEMS, WT), stream,
                     t.start, t.stop, qm, reps, q0, nq, lb, m, sel, rinfo, out_blocks);
}

hipError_t launch_block_scores(const QueryMeta& qm, const uint16_t* reps, int64_t q0, int64_t nq, int lb,
                               int64_t Mmax, float* sigma, hipStream_t stream, Timing t, const StepAppend* app)
{
    if (app) {
        DecodeJobs dj;
        int rows = 1;
        for (int i = 0; i < kDecodeJobs; ++i) {
            dj.j[i] = i < app->njobs ? app->jobs[i] : PoolJob{0, 0, 0, 0, 0, 0, 0, 0};
            if (i < app->njobs) rows = std::max<int>(rows, app->jobs[i].nblk);
        }
        dim3 grid((unsigned)std::max<int64_t>((Mmax + kThreads - 1) / kThreads, rows), (unsigned)(nq + app->njobs));
        return launch_k(block_score_append_kernel, grid, dim3(kThreads), stream, t.start, t.stop, qm,
                        const_cast<uint16_t*>(reps), app->keys, app->new_keys, app->B, dj, app->njobs, q0, lb, Mmax,
                        sigma);
    }
    dim3 grid((unsigned)((Mmax + kThreads - 1) / kThreads), (unsigned)nq);
    return launch_k(block_score_kernel, grid, dim3(kThreads), stream, t.start, t.stop, qm, reps, q0, lb, Mmax, sigma);
}

hipError_t launch_stage1(const QueryMeta& qm, const uint16_t* reps, int64_t q0, int64_t nq, int lb, int m,
                         int64_t Mmax, float* sigma, int32_t* sel, RowInfo* rinfo, int32_t* out_blocks,
                         hipStream_t stream, Timing t)
{
    if (nq >= kManyRows && Mmax <= kS1TileMaxBlocks) {
        // many queries: MFMA block scores, wave-level top-m
        const int64_t per = (Mmax + 63) / 64;
#define HISA_S1T(N) \
    if (per <= N) return launch_stage1_tile_items<N>(qm, reps, q0, nq, lb, m, sel, rinfo, out_blocks, stream, t)
        HISA_S1T(1);
        HISA_S1T(2);
        HISA_S1T(4);
        HISA_S1T(8);
        HISA_S1T(16);
#undef HISA_S1T
    }
    if (Mmax <= kStage1FusedMax) {
        // 256 threads score up to 2048 representatives, 8 per thread
        const int64_t per = (Mmax + 255) / 256;
#define HISA_S1F(N) \
    if (per <= N) return launch_stage1_items<256, N, true>(qm, reps, q0, nq, lb, m, Mmax, nullptr, sel, rinfo, out_blocks, stream, t.start, t.stop)
        HISA_S1F(1);
        HISA_S1F(2);
        HISA_S1F(4);
        HISA_S1F(8);
#undef HISA_S1F
        return hipErrorInvalidValue;
    }
    const hipError_t err = launch_block_scores(qm, reps, q0, nq, lb, Mmax, sigma, stream, Timing{t.start, nullptr});
    if (err != hipSuccess) return err;
    // 1024 threads select among up to 16384 scores, 16 per thread
    const int64_t per = (Mmax + 1023) / 1024;
#define HISA_S1S(N) \
    if (per <= N) return launch_stage1_items<1024, N, false>(qm, reps, q0, nq, lb, m, Mmax, sigma, sel, rinfo, out_blocks, stream, nullptr, t.stop)
    HISA_S1S(2);
    HISA_S1S(4);
    HISA_S1S(8);
    HISA_S1S(16);
#undef HISA_S1S
    return hipErrorInvalidValue;
}

// ---- HISA stage 2: token scores in the kept blocks and top-k ---------------
// Candidate slot s of a query is row s % B of kept block s / B; slots of
// padding blocks and keys after the query get key 0.

// Few queries: kStage2SlotsPerWg slots of one query per workgroup, scored
// into ukeys so that few queries still fill the chip.  Slot s is row s % B
// of kept block s / B; slots of -1 blocks and keys after the query get
// key 0.  Eight lanes share a candidate row, each reading 16 of its 128
// bytes, so every wave load is 1 KiB of whole rows; the eight partial dots
// are summed across the lanes with DPP.  The top-k follows in
// topk_rows_kernel.
// The slots of this workgroup (NT threads): kept(i) gives entry i of the
// row's kept list.  Two round trips when the list is in memory, no
// branches: every pass's list entry, then every pass's key part (row 0 of
// the sequence stands in for a masked slot).
template <int NT = kThreads, class Kept, class Row>
HISA_INLINE void score_slots(const uint16_t* qrow, Row row_of, int64_t t, int lb, int N, Kept kept, uint32_t* urow,
                             int chunk)
{
    constexpr int kScoreRowsPerPass = NT / 8;
    constexpr int kScorePasses = kStage2SlotsPerWg / kScoreRowsPerPass;
    const int sub = threadIdx.x & 7;              // which 16 bytes of a row
    const int grp = threadIdx.x >> 3;             // which row of a pass
    const int beg = chunk * kStage2SlotsPerWg + grp;
    const uint4 qv = reinterpret_cast<const uint4*>(qrow)[sub];
    int32_t blk[kScorePasses];
#pragma unroll
    for (int p = 0; p < kScorePasses; ++p) blk[p] = kept(min(beg + p * kScoreRowsPerPass, N - 1) >> lb);
    uint4 v[kScorePasses];
    bool ok[kScorePasses];
#pragma unroll
    for (int p = 0; p < kScorePasses; ++p) {
        const int s = beg + p * kScoreRowsPerPass;
        const int64_t j = ((int64_t)blk[p] << lb) + (s & ((1 << lb) - 1));
        ok[p] = s < N && blk[p] >= 0 && j <= t;
        v[p] = reinterpret_cast<const uint4*>(row_of(ok[p] ? j : 0))[sub];
    }
#pragma unroll
    for (int p = 0; p < kScorePasses; ++p) {
        if (!ok[p]) v[p] = make_uint4(0u, 0u, 0u, 0u);
        float acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(qv.x), as_bf16x2(v[p].x), 0.f, false);
        acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(qv.y), as_bf16x2(v[p].y), acc, false);
        acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(qv.z), as_bf16x2(v[p].z), acc, false);
        acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(qv.w), as_bf16x2(v[p].w), acc, false);
        // sum over the 8 lanes of the row: xor 1 and 2 inside quads (DPP
        // quad_perm), then xor 4; every lane of the row holds the total
        acc += __uint_as_float(dpp_u32<0xb1>(__float_as_uint(acc)));
        acc += __uint_as_float(dpp_u32<0x4e>(__float_as_uint(acc)));
        acc += __shfl_xor(acc, 4);
        const int s = beg + p * kScoreRowsPerPass;
        if (sub == 0 && s < N) urow[s] = ok[p] ? score_key(acc) : 0u;
    }
}

// Few queries with more than kStage1FusedMax blocks: the representative
// scores come from block_score_kernel (sigma); this launch does the rest of
// stage 1 and the token scores.  Every workgroup of a query (1024 threads)
// selects the kept blocks from the query's scores itself - the same
// selection in each, a few KiB of L2 reads - then scores its own
// kStage2SlotsPerWg slots; workgroup 0 of the query also writes the kept
// list, the row info and out_blocks.
template <int ITEMS>
__global__ __launch_bounds__(1024) void select_score_kernel(QueryMeta qm, const uint16_t* keys, int64_t q0, int lb,
                                                            int m, int64_t Mmax, const float* sigma, int32_t* sel,
                                                            RowInfo* rinfo, int32_t* out_blocks, uint32_t* ukeys)
{
    constexpr int NT = 1024;
    __shared__ BucketSmem<NT> sm;
    __shared__ int32_t s_kept[kMaxKept];
    const int64_t row = blockIdx.x;
    const int64_t i = q0 + row;
    const QueryInfo qi =
        query_info(i, qm.q_pos, qm.q_seq, qm.seq_key_off, qm.seq_rep_off, qm.seq_len, qm.nseq, qm.max_len);
    const int64_t c = qi.valid ? qi.t >> lb : -1;
    if (!qi.valid || c + 1 <= m) {
        for (int r = threadIdx.x; r < m; r += NT) s_kept[r] = r <= c ? r : -1;
    } else {
        const float* sg = sigma + row * Mmax;
        uint32_t key[ITEMS];
#pragma unroll
        for (int it = 0; it < ITEMS; ++it) {
            const int64_t b = slot_of<ITEMS>(it);
            key[it] = (b >= 1 && b <= c - 2) ? score_key(sg[b]) : 0u;
        }
        const Threshold th = wg_bucket_select<NT, ITEMS>(key, m - 3, sm);
        wg_emit_selected<NT, ITEMS>(key, th, sm, m - 3, [&](int slot, uint32_t, int rank) { s_kept[1 + rank] = slot; });
        if (threadIdx.x == 0) {
            s_kept[0] = 0;
            s_kept[m - 2] = (int32_t)(c - 1);
            s_kept[m - 1] = (int32_t)c;
        }
    }
    __syncthreads();
    if (blockIdx.y == 0) {
        if (threadIdx.x == 0) rinfo[row] = RowInfo{qi.key_off, qi.valid ? qi.t : -1};
        for (int r = threadIdx.x; r < m; r += NT) {
            sel[row * m + r] = s_kept[r];
            if (out_blocks) out_blocks[i * m + r] = s_kept[r];
        }
    }
    const int N = m << lb;
    score_slots<NT>(qm.queries + i * kDim, [&](int64_t j) { return keys + (qi.key_off + j) * kDim; },
                    qi.valid ? qi.t : -1, lb, N, [&](int e) { return s_kept[e]; }, ukeys + row * N, blockIdx.y);
}

hipError_t launch_select_scores(const QueryMeta& qm, const uint16_t* keys, int64_t q0, int64_t nq, int lb, int m,
                                int64_t Mmax, const float* sigma, int32_t* sel, RowInfo* rinfo, int32_t* out_blocks,
                                uint32_t* ukeys, hipStream_t stream, Timing t)
{
    const int N = m << lb;
    const dim3 grid((unsigned)nq, (unsigned)((N + kStage2SlotsPerWg - 1) / kStage2SlotsPerWg));
    const int64_t per = (Mmax + 1023) / 1024;
#define HISA_SS(N_) \
    if (per <= N_) return launch_k(select_score_kernel<N_>, grid, dim3(1024), stream, t.start, t.stop, qm, keys, q0, lb, m, Mmax, sigma, sel, rinfo, out_blocks, ukeys)
    HISA_SS(2);
    HISA_SS(4);
    HISA_SS(8);
    HISA_SS(16);
#undef HISA_SS
    return hipErrorInvalidValue;
}

// Few queries with at most kStage1FusedMax blocks: stage 1 and the token
// scores in one launch.  Every workgroup of a query scores the causal
// representatives (v_dot2 GEMV) and selects the kept blocks itself - the
// same selection in each, a few KiB of L2 reads - then scores its own
// slots from the list in LDS.  Workgroup 0 of the query also writes the
// kept list, the row info and out_blocks.
// The body of a fused workgroup; source(qi) gives the key-row functor of
// the query's sequence.
template <int ITEMS, class Source>
HISA_INLINE void decode_fused_body(const QueryMeta& qm, const uint16_t* reps, int64_t q0, int64_t row, int lb, int m,
                                   int groups, int32_t* sel, RowInfo* rinfo, int32_t* out_blocks, uint32_t* ukeys,
                                   Source source)
{
    __shared__ BucketSmem<kThreads> sm;
    __shared__ int32_t s_kept[kMaxKept];
    const int64_t i = q0 + row;
    const QueryInfo qi =
        query_info(i, qm.q_pos, qm.q_seq, qm.seq_key_off, qm.seq_rep_off, qm.seq_len, qm.nseq, qm.max_len);
    const int64_t c = qi.valid ? qi.t >> lb : -1;
    if (!qi.valid || c + 1 <= m) {
        for (int r = threadIdx.x; r < m; r += kThreads) s_kept[r] = r <= c ? r : -1;
    } else {
        uint32_t q[32];
        load_query(qm.queries + i * kDim, q);
        uint32_t key[ITEMS];
#pragma unroll
        for (int it = 0; it < ITEMS; ++it) {
            const int64_t b = slot_of<ITEMS>(it);
            key[it] = (b >= 1 && b <= c - 2)
                          ? score_key(dot64_packed(q, reinterpret_cast<const uint4*>(reps + (qi.rep_off + b) * kDim)))
                          : 0u;
        }
        const Threshold th = wg_bucket_select<kThreads, ITEMS>(key, m - 3, sm);
        wg_emit_selected<kThreads, ITEMS>(key, th, sm, m - 3, [&](int slot, uint32_t, int rank) { s_kept[1 + rank] = slot; });
        if (threadIdx.x == 0) {
            s_kept[0] = 0;
            s_kept[m - 2] = (int32_t)(c - 1);
            s_kept[m - 1] = (int32_t)c;
        }
    }
    __syncthreads();
    if (blockIdx.y == 0) {
        if (threadIdx.x == 0) rinfo[row] = RowInfo{qi.key_off, qi.valid ? qi.t : -1};
        for (int r = threadIdx.x; r < m; r += kThreads) {
            sel[row * m + r] = s_kept[r];
            if (out_blocks) out_blocks[i * m + r] = s_kept[r];
        }
    }
    // the workgroup's `groups` chunks of kStage2SlotsPerWg slots, one after
    // the other (more than one when queries are many: fewer redundant
    // selections)
    const int N = m << lb;
    for (int g = 0; g < groups; ++g) {
        const int chunk = (int)blockIdx.y * groups + g;
        if (chunk * kStage2SlotsPerWg >= N) break;
        score_slots(qm.queries + i * kDim, source(qi), qi.valid ? qi.t : -1, lb, N, [&](int e) { return s_kept[e]; },
                    ukeys + row * N, chunk);
    }
}

template <int ITEMS>
__global__ __launch_bounds__(kThreads) void decode_fused_kernel(QueryMeta qm, const uint16_t* reps,
                                                                const uint16_t* keys, int64_t q0, int lb, int m,
                                                                int groups, int32_t* sel, RowInfo* rinfo,
                                                                int32_t* out_blocks, uint32_t* ukeys)
{
    decode_fused_body<ITEMS>(qm, reps, q0, blockIdx.x, lb, m, groups, sel, rinfo, out_blocks, ukeys,
                             [&](const QueryInfo& qi) {
        return [=](int64_t j) { return keys + (qi.key_off + j) * kDim; };
    });
}

// A decode step in one launch: workgroups x < njobs run the append jobs
// (job x, block y; first in the grid so they are dispatched early),
// workgroups x >= njobs index query x - njobs as decode_fused_kernel does.  An index workgroup reads a key at or past its
// sequence's old length from new_keys, not from the cache the append
// workgroups are writing.  The blocks the append re-pools are the query's
// own block and the one before (the new keys span at most two blocks and
// no query lies past them), which are forced and never scored, so no
// index workgroup reads a representative being rewritten.
template <int ITEMS>
__global__ __launch_bounds__(kThreads) void decode_step_kernel(QueryMeta qm, uint16_t* reps, uint16_t* keys,
                                                               const uint16_t* new_keys, int B, DecodeJobs jobs,
                                                               int njobs, int splits, int groups, int lb, int m,
                                                               int32_t* sel, RowInfo* rinfo, int32_t* out_blocks,
                                                               uint32_t* ukeys)
{
    if ((int)blockIdx.x < njobs) {
        const PoolJob& job = jobs.j[blockIdx.x];
        if ((int64_t)blockIdx.y < job.nblk) pool_block(keys, reps, new_keys, B, job, blockIdx.y);
        return;
    }
    if ((int)blockIdx.y >= splits) return;       // rows of the grid kept for two-block appends
    decode_fused_body<ITEMS>(qm, reps, 0, blockIdx.x - njobs, lb, m, groups, sel, rinfo, out_blocks, ukeys,
                             [&](const QueryInfo& qi) {
        // an invalid query reads no key; job 0 (or a zero padding job)
        // keeps its row functor in bounds
        const PoolJob& job = jobs.j[(qi.seq >= 0 && qi.seq < kDecodeJobs) ? qi.seq : 0];
        const int64_t len_old = job.len_old, len_new = job.len_new;
        const uint16_t* nk = new_keys + (int64_t)job.new_row * kDim;
        const uint16_t* ck = keys + qi.key_off * kDim;
        // rows past the appended ones (only for lengths inconsistent with
        // the append) stay in the cache, inside the sequence's capacity
        return [=](int64_t j) { return (j >= len_old && j < len_new) ? nk + (j - len_old) * kDim : ck + j * kDim; };
    });
}

// Slot chunks per workgroup in the fused decode launches: one (every
// workgroup selects the query's blocks itself and scores 512 slots) until
// the launch has work for four workgroups per CU, then more, so that large
// batches repeat the selection less.
inline int decode_groups(int64_t nq, int chunks)
{
    int g = 1;
    while (g < chunks && nq * chunks / (2 * g) >= 1024) g *= 2;
    return g;
}

template <int ITEMS>
static hipError_t launch_decode_fused_items(const QueryMeta& qm, const uint16_t* reps, const uint16_t* keys,
                                            int64_t q0, int64_t nq, int lb, int m, int32_t* sel, RowInfo* rinfo,
                                            int32_t* out_blocks, uint32_t* ukeys, hipStream_t stream, Timing t)
{
    const int N = m << lb;
    const int chunks = (N + kStage2SlotsPerWg - 1) / kStage2SlotsPerWg;
    const int groups = decode_groups(nq, chunks);
    const dim3 grid((unsigned)nq, (unsigned)((chunks + groups - 1) / groups));
    return launch_k(decode_fused_kernel<ITEMS>, grid, dim3(kThreads), stream, t.start, t.stop, qm, reps, keys, q0, lb,
                    m, groups, sel, rinfo, out_blocks, ukeys);
}

hipError_t launch_decode_step(const QueryMeta& qm, uint16_t* reps, uint16_t* keys, const uint16_t* new_keys, int B,
                              const PoolJob* jobs, int njobs, int64_t nq, int lb, int m, int64_t Mmax, int32_t* sel,
                              RowInfo* rinfo, int32_t* out_blocks, uint32_t* ukeys, hipStream_t stream, Timing t)
{
    DecodeJobs dj;
    for (int i = 0; i < kDecodeJobs; ++i) dj.j[i] = i < njobs ? jobs[i] : PoolJob{0, 0, 0, 0, 0, 0, 0, 0};
    const int N = m << lb;
    const int chunks = (N + kStage2SlotsPerWg - 1) / kStage2SlotsPerWg;
    const int groups = decode_groups(nq, chunks);
    const int splits = (chunks + groups - 1) / groups;
    int rows = splits;                                // an append touches at most two blocks
    for (int i = 0; i < njobs; ++i) rows = std::max<int>(rows, jobs[i].nblk);
    const dim3 grid((unsigned)(nq + njobs), (unsigned)rows);
    const int64_t per = (Mmax + kThreads - 1) / kThreads;
#define HISA_DS(N_)                                                                                             \
    if (per <= N_)                                                                                              \
    return launch_k(decode_step_kernel<N_>, grid, dim3(kThreads), stream, t.start, t.stop, qm, reps, keys, new_keys, \
                    B, dj, njobs, splits, groups, lb, m, sel, rinfo, out_blocks, ukeys)
    HISA_DS(1);
    HISA_DS(2);
    HISA_DS(4);
    HISA_DS(8);
#undef HISA_DS
    return hipErrorInvalidValue;
}

hipError_t launch_decode_fused(const QueryMeta& qm, const uint16_t* reps, const uint16_t* keys, int64_t q0,
                               int64_t nq, int lb, int m, int64_t Mmax, int32_t* sel, RowInfo* rinfo,
                               int32_t* out_blocks, uint32_t* ukeys, hipStream_t stream, Timing t)
{
    const int64_t per = (Mmax + kThreads - 1) / kThreads;
#define HISA_DF(N_) \
    if (per <= N_) return launch_decode_fused_items<N_>(qm, reps, keys, q0, nq, lb, m, sel, rinfo, out_blocks, ukeys, stream, t)
    HISA_DF(1);
    HISA_DF(2);
    HISA_DF(4);
    HISA_DF(8);
#undef HISA_DF
    return hipErrorInvalidValue;
}

// Many queries: tiles of 16 consecutive query rows on the bf16 MFMA
// (v_mfma_f32_16x16x32_bf16, two per 16 keys since d = 64).  Workgroup
// (tile, g) has four waves; wave w takes the blocks [b0, b0 + range) with
// b0 = (4g + w) * range and walks the union of the 16 rows' kept blocks
// inside them in ascending order: lane r (r < 16) holds a cursor into row
// r's list, and the next block is the smallest one under the 16 cursors.
// Each union block is scored for all 16 rows at once, so a key row is read
// once per 16 queries rather than once per query.  A row that kept the
// block at list position p writes the scores to its slots [p*B, (p+1)*B),
// key 0 for tokens after the query; slots of -1 entries are never written
// (the top-k stops at the kept blocks).  Rows of a tile in different
// sequences are walked one sequence at a time.  MFMA lanes: lane l feeds
// key l%16 (A operand) and query row l%16 (B operand) with dims
// 8*(l/16)..+8 of each half of d, and receives the scores of keys
// 4*(l/16)..+4 for query row l%16, which it stores as one 16-byte vector.

constexpr int kTileQueries = 16;
constexpr int kTileWaves = 4;
constexpr int kTileEnd = 0x7fffffff;     // cursor past the end of a list
// Waves to aim for (the blocks of each tile are split into ranges until
// there are this many): dense lists want many short ranges; sparse ones,
// walked in pieces, do better with fewer, longer ranges (measured: 128K
// chunk 172 -> 159 us at 4096, the 32K prefill best at 16384).
constexpr int64_t kTileTargetWaves = 16384;
constexpr int64_t kTileTargetWavesSparse = 4096;
// LDS budget of one tile's kept-block lists: two workgroups per CU (the
// kernel's occupancy) fit in the 160 KB of LDS
constexpr size_t kTileListBytes = 80 * 1024;

template <int LB, int SUB, int P>
__global__ __launch_bounds__(64 * kTileWaves) void stage2_tile_kernel(const uint16_t* queries, const uint16_t* keys,
                                                                      int64_t q0, int64_t nq, int m, int range,
                                                                      const RowInfo* rinfo, const int32_t* sel,
                                                                      uint32_t* ukeys)
{
    // SUB sub-tiles of 16 query rows per wave: every key block loaded from
    // L2 feeds SUB MFMA tiles, so the union walk reads each block once per
    // 16 * SUB queries.  A block is taken in P pieces of KT/P key tiles,
    // and the next piece (of this block or the next one) is loaded while
    // the current one is on the MFMA.
    constexpr int TQ = kTileQueries * SUB;
    extern __shared__ int32_t s_sel[];            // [TQ][m] kept-block lists of the tile's rows
    constexpr int B = 1 << LB;
    constexpr int KT = B / 16;
    const int lane = lane_id();
    const int64_t row0 = (int64_t)blockIdx.x * TQ;
    const int nrows = (int)min<int64_t>(TQ, nq - row0);
    const int N = m << LB;
    for (int e = threadIdx.x; e < TQ * m; e += 64 * kTileWaves)
        s_sel[e] = e < nrows * m ? sel[row0 * m + e] : -1;
    __syncthreads();
    const int blo = ((int)blockIdx.y * kTileWaves + wave_id()) * range;
    const int bhi = blo + range;
    // lanes 0..TQ-1: one row each; rows whose keys start at the same row of
    // the cache are walked together
    const int r = lane % TQ;
    const int32_t* lst = s_sel + r * m;
    RowInfo ri{0, -1};
    if (lane < TQ && r < nrows) ri = rinfo[row0 + r];
    const bool valid = ri.t >= 0;
    // this row's first list entry at or after blo (the list ascends, then -1s)
    int first = m;
    if (valid) {
        int lo = 0, hi = m;
        while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            const int v = lst[mid];
            if (v >= 0 && v < blo)
                lo = mid + 1;
            else
                hi = mid;
        }
        first = lo;
    }
    const bool active = valid && first < m && lst[first] >= 0 && lst[first] < bhi;
    const int t32 = valid ? (int)ri.t : -1;
    uint64_t pending = __ballot(active);
    if (!pending) return;
    // A operands: the queries of each sub-tile
    const int col = lane & 15, kg = lane >> 4;
    bf16x8_t a0[SUB], a1[SUB];
#pragma unroll
    for (int sb = 0; sb < SUB; ++sb) {
        a0[sb] = bf16x8_t{};
        a1[sb] = bf16x8_t{};
        if (16 * sb + col < nrows) {
            const uint16_t* qrow = queries + (q0 + row0 + 16 * sb + col) * kDim + 8 * kg;
            a0[sb] = *reinterpret_cast<const bf16x8_t*>(qrow);
            a1[sb] = *reinterpret_cast<const bf16x8_t*>(qrow + 32);
        }
    }
    constexpr int KP = KT / P;                    // key tiles per piece
    while (pending) {
        const int lead = (int)__builtin_ctzll(pending);
        const int64_t koff = ((int64_t)__builtin_amdgcn_readlane((int)(ri.key_off >> 32), lead) << 32) |
                             (uint32_t)__builtin_amdgcn_readlane((int)ri.key_off, lead);
        const bool mine = active && ri.key_off == koff;
        pending &= ~__ballot(mine);
        const int tmax = (int)wave_max_u32(mine ? (uint32_t)t32 : 0u);
        const int tmin = (int)wave_min_u32(mine ? (uint32_t)t32 : 0xffffffffu);
        const int tm = mine ? t32 : -1;
        int cur = first;
        int nxt = mine ? lst[first] : kTileEnd;
        // this lane's output row in sub-tile sb is row 16 * sb + col of the
        // tile (position -1 when that row is not walked now)
        int tq[SUB];
#pragma unroll
        for (int sb = 0; sb < SUB; ++sb) tq[sb] = __shfl(tm, 16 * sb + col);
        // piece p of block b: key tiles p*KP .. p*KP+KP-1 (keys past the
        // walked rows' last position read as zero)
        auto load_piece = [&](int b, int p, bf16x8_t (&k0)[KP], bf16x8_t (&k1)[KP]) {
            const uint16_t* kb = keys + (koff + ((int64_t)b << LB)) * kDim + 8 * kg;
            if (((b + 1) << LB) - 1 <= tmax) {           // every key of the block exists
#pragma unroll
                for (int kt = 0; kt < KP; ++kt) {
                    const int jj = (p * KP + kt) * 16 + col;
                    k0[kt] = *reinterpret_cast<const bf16x8_t*>(kb + jj * kDim);
                    k1[kt] = *reinterpret_cast<const bf16x8_t*>(kb + jj * kDim + 32);
                }
            } else {
#pragma unroll
                for (int kt = 0; kt < KP; ++kt) {
                    const int jj = (p * KP + kt) * 16 + col;
                    k0[kt] = bf16x8_t{};
                    k1[kt] = bf16x8_t{};
                    if ((b << LB) + jj <= tmax) {
                        k0[kt] = *reinterpret_cast<const bf16x8_t*>(kb + jj * kDim);
                        k1[kt] = *reinterpret_cast<const bf16x8_t*>(kb + jj * kDim + 32);
                    }
                }
            }
        };
        // per block: advance the cursors of the rows that kept it; pq[sb]
        // is the list position for this lane's row of sub-tile sb (-1 unless
        // that row kept b)
        int b = (int)wave_min_u32((uint32_t)nxt), bn = kTileEnd;
        int pq[SUB];
        bool seen = true;
        auto enter_block = [&]() {
            const bool hit = nxt == b;
            const int pos = hit ? cur : -1;
            if (hit) {
                ++cur;
                const int v = cur < m ? lst[cur] : -1;
                nxt = v >= 0 && v < bhi ? v : kTileEnd;
            }
#pragma unroll
            for (int sb = 0; sb < SUB; ++sb) pq[sb] = __shfl(pos, 16 * sb + col);
            bn = (int)wave_min_u32((uint32_t)nxt);
            seen = ((b + 1) << LB) - 1 <= tmin;           // no walked row masks a token of b
        };
        // keys as the A operand: lane l receives keys 4*(l/16)..+4 of each
        // 16-key tile for query row l%16 of the sub-tile; the tiles are
        // independent accumulations, issued back to back
        auto score_piece = [&](int p, const bf16x8_t (&k0)[KP], const bf16x8_t (&k1)[KP]) {
#pragma unroll
            for (int sb = 0; sb < SUB; ++sb) {
                f32x4_t c[KP];
#pragma unroll
                for (int kt = 0; kt < KP; ++kt)
                    c[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0[kt], a0[sb], f32x4_t{0.f, 0.f, 0.f, 0.f}, 0,
                                                                    0, 0);
#pragma unroll
                for (int kt = 0; kt < KP; ++kt)
                    c[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1[kt], a1[sb], c[kt], 0, 0, 0);
                if (pq[sb] >= 0) {
                    uint32_t* urow = ukeys + (row0 + 16 * sb + col) * N + ((int64_t)pq[sb] << LB) + 4 * kg;
#pragma unroll
                    for (int kt = 0; kt < KP; ++kt) {
                        uint4 o = make_uint4(score_key(c[kt][0]), score_key(c[kt][1]), score_key(c[kt][2]),
                                             score_key(c[kt][3]));
                        if (!seen) {
                            const int j = (b << LB) + (p * KP + kt) * 16 + 4 * kg;
                            o.x = j + 0 <= tq[sb] ? o.x : 0u;
                            o.y = j + 1 <= tq[sb] ? o.y : 0u;
                            o.z = j + 2 <= tq[sb] ? o.z : 0u;
                            o.w = j + 3 <= tq[sb] ? o.w : 0u;
                        }
                        *reinterpret_cast<uint4*>(urow + (p * KP + kt) * 16) = o;
                    }
                }
            }
        };
        if (b == kTileEnd) continue;
        if constexpr (P == 1) {
            // whole blocks, one at a time
            while (b != kTileEnd) {
                enter_block();
                bf16x8_t k0[KP], k1[KP];
                load_piece(b, 0, k0, k1);
                score_piece(0, k0, k1);
                b = bn;
            }
            continue;
        }
        enter_block();
        bf16x8_t x0[KP], x1[KP], y0[KP], y1[KP];
        load_piece(b, 0, x0, x1);
        int p = 0;
        // one work item: score piece p of block b from (c0, c1) while the
        // next item's keys load into (n0, n1); false when the walk ends
        auto item = [&](const bf16x8_t (&c0)[KP], const bf16x8_t (&c1)[KP], bf16x8_t (&n0)[KP],
                        bf16x8_t (&n1)[KP]) {
            const bool last_piece = p + 1 == P;
            const int b2 = last_piece ? bn : b;
            const int p2 = last_piece ? 0 : p + 1;
            if (b2 != kTileEnd) load_piece(b2, p2, n0, n1);
            score_piece(p, c0, c1);
            if (last_piece) {
                b = bn;
                if (b == kTileEnd) return false;
                enter_block();
            }
            p = p2;
            return true;
        };
        while (item(x0, x1, y0, y1) && item(y0, y1, x0, x1)) {
        }
    }
}

// Pieces per key block in the tile walk: a piece of KT/P key tiles loads
// while the previous one is scored.  Kept-block lists that are sparse in
// the block range (a tile's rows share few blocks, so the walk visits many
// blocks for few stores each) are bound by the load latency of each block
// and walk in pieces of one key tile; dense ones are bound by the stores and
// walk whole blocks (measured: 128K chunk 185 -> 167 us, 32K prefill 311
// against 411 us in pieces).
template <int LB, int SPARSE>
constexpr int kTilePieces = SPARSE ? (1 << LB) / 16 : 1;

template <int SUB>
hipError_t launch_tile_sub(const QueryMeta& qm, const uint16_t* keys, int64_t q0, int64_t nq, int lb, int m,
                           int64_t Mmax, const RowInfo* rinfo, const int32_t* sel, uint32_t* ukeys,
                           hipStream_t stream, Timing t)
{
    // enough waves to fill the chip: split each tile's blocks into ranges
    const bool sparse = Mmax >= 8 * (int64_t)m;
    const int64_t target = sparse ? kTileTargetWavesSparse : kTileTargetWaves;
    const int64_t ntiles = (nq + kTileQueries * SUB - 1) / (kTileQueries * SUB);
    const int64_t want = std::max<int64_t>(1, (target + ntiles - 1) / ntiles);
    const int64_t range = std::max<int64_t>(1, (Mmax + want - 1) / want);
    const int64_t nranges = (Mmax + range - 1) / range;
    const dim3 grid((unsigned)ntiles, (unsigned)((nranges + kTileWaves - 1) / kTileWaves));
    const dim3 block(64 * kTileWaves);
    const size_t lds = (size_t)kTileQueries * SUB * m * sizeof(int32_t);
#define HISA_T2(LB_) \
    if (lb == LB_) return sparse ? launch_kl(stage2_tile_kernel<LB_, SUB, kTilePieces<LB_, 1>>, grid, block, lds, stream, t.start, t.stop, qm.queries, keys, q0, nq, m, (int)range, rinfo, sel, ukeys) \
                                 : launch_kl(stage2_tile_kernel<LB_, SUB, kTilePieces<LB_, 0>>, grid, block, lds, stream, t.start, t.stop, qm.queries, keys, q0, nq, m, (int)range, rinfo, sel, ukeys)
    HISA_T2(4);
    HISA_T2(5);
    HISA_T2(6);
    HISA_T2(7);
    HISA_T2(8);
#undef HISA_T2
    return hipErrorInvalidValue;
}

hipError_t launch_stage2_tile_scores(const QueryMeta& qm, const uint16_t* keys, int64_t q0, int64_t nq, int lb, int m,
                                     int64_t Mmax, const RowInfo* rinfo, const int32_t* sel, uint32_t* ukeys,
                                     hipStream_t stream, Timing t)
{
    // as many 16-query sub-tiles per wave (up to 4, all 64 lanes) as the
    // lists of kept blocks leave room for in LDS
    const size_t per16 = (size_t)kTileQueries * m * sizeof(int32_t);
    if (4 * per16 <= kTileListBytes)
        return launch_tile_sub<4>(qm, keys, q0, nq, lb, m, Mmax, rinfo, sel, ukeys, stream, t);
    if (2 * per16 <= kTileListBytes)
        return launch_tile_sub<2>(qm, keys, q0, nq, lb, m, Mmax, rinfo, sel, ukeys, stream, t);
    return launch_tile_sub<1>(qm, keys, q0, nq, lb, m, Mmax, rinfo, sel, ukeys, stream, t);
}

// Top-k of rows of N ranking keys, one workgroup per row; out rows start at
// out_idx / out_scores (the caller offsets them).  sel: slot -> token map.
// WAVE_BLK (sel given, B >= 64, so N and the row's candidate count are
// multiples of 64): the 64 slots of one item lie in one kept block, so an
// item's token is a wave-uniform base plus the lane, the wave reads its
// kept blocks once (lane j holds the j-th block of its slot range) instead
// of one LDS lookup per emitted key, and the bounds of an item are scalar
// tests.  SCORES: out_scores is written.
template <int NT>
constexpr bool kTopkBufferIo = NT < 1024;    // see the WAVE_BLK loads below

template <int NT, int ITEMS, bool WAVE_BLK, bool SCORES>
__global__ __launch_bounds__(NT) void topk_rows_kernel(const uint32_t* ukeys, int N, int k, const int32_t* sel, int m,
                                                       int lb, int32_t* out_idx, float* out_scores)
{
    __shared__ BucketSmem<NT> sm;
    __shared__ int32_t s_list[kMaxKept];                   // the row's kept blocks
    const int64_t row = blockIdx.x;
    const uint32_t* src = ukeys + row * N;
    const int lane = lane_id();
    const int g0 = __builtin_amdgcn_readfirstlane(wave_id()) * ITEMS;   // the wave's first item (scalar)
    int32_t* orow = out_idx + row * k;
    float* scrow = SCORES ? out_scores + row * k : nullptr;
    int total;
    if constexpr (WAVE_BLK) {
        const int sh = lb - 6;                             // item -> kept block: (wave item) >> sh
        const int j0 = g0 >> sh;
        const int mask = (1 << lb) - 1;
        // Every item loads (items past the row re-read its last 64 slots)
        // and is masked after by a scalar: slots of -1 list entries (a
        // suffix of the list) and past N hold no candidate.  The many-rows
        // shapes, bound by instruction issue, load and store through buffer
        // resources (the lane is the vector offset, the item's slot a
        // scalar one: no vector address arithmetic); the 1024-thread shape
        // for few rows keeps plain loads, measured slightly faster there.
        uint32_t key[ITEMS];
        if constexpr (kTopkBufferIo<NT>) {
            const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(src, (uint32_t)N * 4u);
#pragma unroll
            for (int it = 0; it < ITEMS; ++it)
                key[it] = __builtin_amdgcn_raw_buffer_load_b32(rs, lane * 4, min((g0 + it) << 6, N - 64) * 4, 0);
        } else {
#pragma unroll
            for (int it = 0; it < ITEMS; ++it) key[it] = src[min((g0 + it) << 6, N - 64) + lane];
        }
        const int myblk = j0 + lane < m ? sel[row * m + j0 + lane] : 0;
        int cnt = 0;
        for (int i = lane; i < m; i += 64) cnt += sel[row * m + i] >= 0;
        const int n = min(N, wave_sum(cnt) << lb);
#pragma unroll
        for (int it = 0; it < ITEMS; ++it) key[it] &= ((g0 + it) << 6) < n ? 0xffffffffu : 0u;
        const Threshold th = wg_bucket_select<NT, ITEMS>(key, k, sm);
        const __amdgpu_buffer_rsrc_t ro = buffer_rsrc(orow, (uint32_t)k * 4u);
        total = wg_emit_selected_items<NT, ITEMS>(key, th, sm, k, [&](int it, uint32_t kk, int rank) {
            const int g = g0 + it;
            const int base = (__builtin_amdgcn_readlane(myblk, (g >> sh) - j0) << lb) + ((g << 6) & mask);
            if constexpr (kTopkBufferIo<NT>)
                __builtin_amdgcn_raw_buffer_store_b32(base + lane, ro, rank * 4, 0, 0);
            else
                orow[(uint32_t)rank] = base + lane;
            if constexpr (SCORES) scrow[(uint32_t)rank] = key_score(kk);
        });
    } else {
        // the keys and the kept-block list load together; slots of -1 list
        // entries (a suffix of the list) hold no candidate and are masked after
        uint32_t key[ITEMS];
#pragma unroll
        for (int it = 0; it < ITEMS; ++it) {
            const int s = slot_of<ITEMS>(it);
            key[it] = s < N ? src[s] : 0u;
        }
        if (sel) {
            int cnt = 0;
            for (int i = lane; i < m; i += 64) {
                const int32_t v = sel[row * m + i];
                cnt += v >= 0;
                if (wave_id() == 0) s_list[i] = v;
            }
            const int n = min(N, wave_sum(cnt) << lb);
#pragma unroll
            for (int it = 0; it < ITEMS; ++it)
                if (slot_of<ITEMS>(it) >= n) key[it] = 0u;
        }
        // the select's barriers publish s_list before anything is emitted
        const Threshold th = wg_bucket_select<NT, ITEMS>(key, k, sm);
        total = wg_emit_selected<NT, ITEMS>(key, th, sm, k, [&](int slot, uint32_t kk, int rank) {
            orow[rank] = sel ? (s_list[slot >> lb] << lb) + (slot & ((1 << lb) - 1)) : slot;
            if constexpr (SCORES) scrow[rank] = key_score(kk);
        });
    }
    for (int r = total + threadIdx.x; r < k; r += NT) {
        orow[r] = -1;
        if constexpr (SCORES) scrow[r] = __builtin_nanf("");
    }
}

template <int NT, int ITEMS>
static hipError_t launch_topk_rows_items(const uint32_t* ukeys, int64_t nrows, int N, int k, const int32_t* sel,
                                         int m, int lb, int32_t* out_idx, float* out_scores, hipStream_t stream,
                                         Timing t)
{
#define HISA_TR(W_, S_) \
    return launch_k(topk_rows_kernel<NT, ITEMS, W_, S_>, dim3((unsigned)nrows), dim3(NT), stream, t.start, t.stop, \
                    ukeys, N, k, sel, m, lb, out_idx, out_scores)
    const bool wave_blk = sel && lb >= 6;
    if (wave_blk && out_scores) HISA_TR(true, true);
    if (wave_blk) HISA_TR(true, false);
    if (out_scores) HISA_TR(false, true);
    HISA_TR(false, false);
#undef HISA_TR
}

// ---- block-only selection: the kept blocks expanded -------------------------
// Entry e of a row is row e % B of kept block e / B.  The kept list is
// ascending and only its last block (the query's own) can hold keys past
// t, so the visible entries form a prefix of the row and the rest is -1.
// Each workgroup writes kExpandPerWg entries of one row, VEC per store.
constexpr int kExpandPerWg = 2048;

template <int VEC>
__global__ __launch_bounds__(kThreads) void expand_blocks_kernel(const int32_t* sel, const RowInfo* rinfo, int m,
                                                                 int lb, int32_t* out_idx)
{
    __shared__ int32_t s_blk[kMaxKept];
    const int64_t row = blockIdx.x;
    const int N = m << lb;
    const int e0 = blockIdx.y * kExpandPerWg;
    const int r0 = e0 >> lb;
    const int nr = min(kExpandPerWg >> lb, m - r0) + 1;
    for (int r = threadIdx.x; r < nr; r += kThreads) s_blk[r] = r0 + r < m ? sel[row * m + r0 + r] : -1;
    const int64_t t = rinfo[row].t;
    __syncthreads();
    int32_t* o = out_idx + row * (int64_t)N;
    const int e1 = min(N, e0 + kExpandPerWg);
    const int mask = (1 << lb) - 1;
    for (int e = e0 + threadIdx.x * VEC; e < e1; e += kThreads * VEC) {
        int v[VEC];
#pragma unroll
        for (int i = 0; i < VEC; ++i) {
            const int32_t b = s_blk[((e + i) >> lb) - r0];
            const int64_t tok = ((int64_t)b << lb) + ((e + i) & mask);
            v[i] = (b >= 0 && tok <= t) ? (int32_t)tok : -1;
        }
        if constexpr (VEC == 4)
            *reinterpret_cast<int4*>(o + e) = make_int4(v[0], v[1], v[2], v[3]);
        else
            o[e] = v[0];
    }
}

hipError_t launch_expand_blocks(const int32_t* sel, const RowInfo* rinfo, int64_t nq, int m, int lb,
                                int32_t* out_idx, hipStream_t stream, Timing t)
{
    const int N = m << lb;
    dim3 grid((unsigned)nq, (unsigned)((N + kExpandPerWg - 1) / kExpandPerWg));
    // rows of m*B >= 48 entries (a multiple of 16): 16-byte stores when the
    // output is 16-byte aligned
    if ((reinterpret_cast<uintptr_t>(out_idx) & 15) == 0)
        return launch_k(expand_blocks_kernel<4>, grid, dim3(kThreads), stream, t.start, t.stop, sel, rinfo, m, lb,
                        out_idx);
    return launch_k(expand_blocks_kernel<1>, grid, dim3(kThreads), stream, t.start, t.stop, sel, rinfo, m, lb,
                    out_idx);
}

hipError_t launch_topk_small(const uint32_t* ukeys, int64_t nrows, int N, int k, const int32_t* sel, int m, int lb,
                             int32_t* out_idx, float* out_scores, hipStream_t stream, Timing t)
{
    // rows up to 4096 keys: 256 threads.  Longer rows: 1024 threads when
    // there are few of them (one row's latency is the cost), otherwise 32
    // keys per thread in 256- or 512-thread workgroups, several per CU
    // hiding each other's barriers.
    if (N <= 4096) {
        const int per = (N + 255) / 256;
#define HISA_TK(N_) \
    if (per <= N_) return launch_topk_rows_items<256, N_>(ukeys, nrows, N, k, sel, m, lb, out_idx, out_scores, stream, t)
        HISA_TK(1);
        HISA_TK(2);
        HISA_TK(4);
        HISA_TK(8);
        HISA_TK(16);
#undef HISA_TK
    }
    if (nrows >= kManyRows) {
        if (N <= 8192) return launch_topk_rows_items<256, 32>(ukeys, nrows, N, k, sel, m, lb, out_idx, out_scores, stream, t);
        return launch_topk_rows_items<512, 32>(ukeys, nrows, N, k, sel, m, lb, out_idx, out_scores, stream, t);
    }
    const int per = (N + 1023) / 1024;
#define HISA_TK(N_) \
    if (per <= N_) return launch_topk_rows_items<1024, N_>(ukeys, nrows, N, k, sel, m, lb, out_idx, out_scores, stream, t)
    HISA_TK(8);
    HISA_TK(16);
#undef HISA_TK
    return hipErrorInvalidValue;
}

// ---- flat indexer: every key ------------------------------------------------

// One thread per (query, key); masked keys get key 0 so that whole rows can
// be read (few queries, and the radix path).
__global__ __launch_bounds__(kThreads) void flat_score_kernel(QueryMeta qm, const uint16_t* keys, int64_t q0,
                                                              int64_t Lmax, uint32_t* ukeys)
{
    const int64_t row = blockIdx.y;
    const int64_t i = q0 + row;
    const int64_t j = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (j >= Lmax) return;
    uint32_t* out = ukeys + row * Lmax + j;
    const QueryInfo qi =
        query_info(i, qm.q_pos, qm.q_seq, qm.seq_key_off, qm.seq_rep_off, qm.seq_len, qm.nseq, qm.max_len);
    if (!qi.valid || j > qi.t) {
        *out = 0u;
        return;
    }
    uint32_t q[32];
    load_query(qm.queries + i * kDim, q);
    *out = score_key(dot64_packed(q, reinterpret_cast<const uint4*>(keys + (qi.key_off + j) * kDim)));
}

// Many queries: 16 query rows x 256 keys per workgroup on the bf16 MFMA
// (v_mfma_f32_16x16x32_bf16, two per 16x16 tile since d = 64), so every
// key row is loaded once per 16 queries.  Lane l feeds key l%16 (A
// operand) and query row l%16 (B operand) with dims 8*(l/16)..+8 of each
// half of d, and receives the scores of keys 4*(l/16)..+4 for query row
// l%16, written as one 16-byte vector.  Visible keys (j <= t)
// get their score; the rest of the row is left alone (rows are read back
// up to t) or, with zero_masked, gets key 0.  A tile whose queries sit in
// different sequences falls back to one thread per key.

constexpr int kTileRows = 16;
constexpr int kTileKeys = 256;

__global__ __launch_bounds__(kThreads) void flat_score_mfma_kernel(QueryMeta qm, const uint16_t* keys, int64_t q0,
                                                                   int64_t nq, int64_t Lmax, bool zero_masked,
                                                                   uint32_t* ukeys)
{
    __shared__ int64_t s_t[kTileRows];
    __shared__ int64_t s_koff[kTileRows];
    __shared__ int s_seq[kTileRows];
    const int64_t row0 = (int64_t)blockIdx.y * kTileRows;
    const int64_t kt0 = (int64_t)blockIdx.x * kTileKeys;
    if (threadIdx.x < kTileRows) {
        const int64_t row = row0 + threadIdx.x;
        QueryInfo qi;
        qi.valid = false;
        qi.key_off = 0;
        if (row < nq)
            qi = query_info(q0 + row, qm.q_pos, qm.q_seq, qm.seq_key_off, qm.seq_rep_off, qm.seq_len, qm.nseq,
                            qm.max_len);
        s_t[threadIdx.x] = qi.valid ? qi.t : -1;
        s_koff[threadIdx.x] = qi.key_off;
        s_seq[threadIdx.x] = qi.valid ? qi.seq : -1;
    }
    __syncthreads();
    int64_t tmax = -1, koff = 0;
    int seq0 = -1;
    bool uniform = true;
    for (int r = 0; r < kTileRows; ++r) {
        if (s_t[r] < 0) continue;
        if (seq0 < 0) {
            seq0 = s_seq[r];
            koff = s_koff[r];
        } else if (s_seq[r] != seq0) {
            uniform = false;
        }
        tmax = max(tmax, s_t[r]);
    }
    if (kt0 > tmax) {                          // no row sees any key of this tile
        if (zero_masked)
            for (int r = 0; r < kTileRows; ++r) {
                const int64_t j = kt0 + threadIdx.x;
                if (row0 + r < nq && j < Lmax) ukeys[(row0 + r) * Lmax + j] = 0u;
            }
        return;
    }
    const int lane = lane_id();
    const bool vec_rows = (Lmax & 3) == 0;         // rows start 16-byte aligned
    if (uniform) {
        const int col = lane & 15, kg = lane >> 4;
        bf16x8_t a0 = {}, a1 = {};
        if (s_t[col] >= 0) {
            const uint16_t* qrow = qm.queries + (q0 + row0 + col) * kDim + 8 * kg;
            a0 = *reinterpret_cast<const bf16x8_t*>(qrow);
            a1 = *reinterpret_cast<const bf16x8_t*>(qrow + 32);
        }
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            const int64_t j = kt0 + 64 * wave_id() + 16 * st + col;
            bf16x8_t b0 = {}, b1 = {};
            if (j <= tmax) {
                const uint16_t* krow = keys + (koff + j) * kDim + 8 * kg;
                b0 = *reinterpret_cast<const bf16x8_t*>(krow);
                b1 = *reinterpret_cast<const bf16x8_t*>(krow + 32);
            }
            // keys as the A operand: lane l receives keys j0..j0+3 for
            // query row l%16
            f32x4_t c = {0.f, 0.f, 0.f, 0.f};
            c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b0, a0, c, 0, 0, 0);
            c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b1, a1, c, 0, 0, 0);
            const int64_t j0 = kt0 + 64 * wave_id() + 16 * st + 4 * kg;
            const int64_t t = s_t[col];
            if (row0 + col < nq && j0 <= (zero_masked ? Lmax - 1 : t)) {
                uint32_t o[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) o[e] = j0 + e <= t ? score_key(c[e]) : 0u;
                uint32_t* dst = ukeys + (row0 + col) * Lmax + j0;
                if (vec_rows && j0 + 3 < Lmax) {
                    *reinterpret_cast<uint4*>(dst) = make_uint4(o[0], o[1], o[2], o[3]);
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (j0 + e < Lmax) dst[e] = o[e];
                }
            }
        }
    } else {
        const int64_t j = kt0 + threadIdx.x;
        for (int r = 0; r < kTileRows; ++r) {
            if (j > s_t[r]) {
                if (zero_masked && row0 + r < nq && j < Lmax) ukeys[(row0 + r) * Lmax + j] = 0u;
                continue;
            }
            uint32_t q[32];
            load_query(qm.queries + (q0 + row0 + r) * kDim, q);
            ukeys[(row0 + r) * Lmax + j] =
                score_key(dot64_packed(q, reinterpret_cast<const uint4*>(keys + (s_koff[r] + j) * kDim)));
        }
    }
}

hipError_t launch_flat_scores(const QueryMeta& qm, const uint16_t* keys, int64_t q0, int64_t nq, int64_t Lmax,
                              uint32_t* ukeys, bool mfma, bool zero_masked, hipStream_t stream, Timing t)
{
    if (mfma) {
        dim3 grid((unsigned)((Lmax + kTileKeys - 1) / kTileKeys), (unsigned)((nq + kTileRows - 1) / kTileRows));
        return launch_k(flat_score_mfma_kernel, grid, dim3(kThreads), stream, t.start, t.stop, qm, keys, q0, nq, Lmax,
                        zero_masked, ukeys);
    }
    dim3 grid((unsigned)((Lmax + kThreads - 1) / kThreads), (unsigned)nq);
    return launch_k(flat_score_kernel, grid, dim3(kThreads), stream, t.start, t.stop, qm, keys, q0, Lmax, ukeys);
}

// ---- flat top-k in levels -----------------------------------------------------
// Level 1: workgroup (row, g) selects the top min(k, SL) of slice g of the
// row's visible keys (slots [g*SL, (g+1)*SL) of [0, t]).  With one slice
// that is the answer; otherwise each slice leaves K1 candidates (key,
// token; key 0 pads), in ascending token order, and further levels merge
// groups of G slices' candidates until one group remains.  Slices and
// candidates stay in token order, so every output is ascending.

template <int NT, int ITEMS, bool TO_CAND>
__global__ __launch_bounds__(NT) void flat_select_kernel(QueryMeta qm, int64_t q0, const uint32_t* ukeys,
                                                         int64_t Lmax, int SL, int k, int K1, uint32_t* cand_key,
                                                         int32_t* cand_tok, int32_t* out_idx, float* out_scores)
{
    __shared__ BucketSmem<NT> sm;
    const int64_t row = blockIdx.x;
    const int g = blockIdx.y;
    const QueryInfo qi =
        query_info(q0 + row, qm.q_pos, qm.q_seq, qm.seq_key_off, qm.seq_rep_off, qm.seq_len, qm.nseq, qm.max_len);
    const int64_t n_row = qi.valid ? qi.t + 1 : 0;
    const int64_t beg = (int64_t)g * SL;
    const int64_t n = max<int64_t>(0, min<int64_t>(SL, n_row - beg));
    const uint32_t* src = ukeys + row * Lmax + beg;
    uint32_t key[ITEMS];
#pragma unroll
    for (int it = 0; it < ITEMS; ++it) {
        const int s = slot_of<ITEMS>(it);
        key[it] = s < n ? src[s] : 0u;
    }
    const int want = TO_CAND ? K1 : k;
    const Threshold th = wg_bucket_select<NT, ITEMS>(key, want, sm);
    if (TO_CAND) {
        uint32_t* ck = cand_key + (row * gridDim.y + g) * K1;
        int32_t* ct = cand_tok + (row * gridDim.y + g) * K1;
        const int total = wg_emit_selected<NT, ITEMS>(key, th, sm, K1, [&](int slot, uint32_t kk, int rank) {
            ck[rank] = kk;
            ct[rank] = (int32_t)(beg + slot);
        });
        for (int r = total + threadIdx.x; r < K1; r += NT) {
            ck[r] = 0u;
            ct[r] = -1;
        }
    } else {
        int32_t* orow = out_idx + (q0 + row) * k;
        float* srow = out_scores ? out_scores + (q0 + row) * k : nullptr;
        const int total = wg_emit_selected<NT, ITEMS>(key, th, sm, k, [&](int slot, uint32_t kk, int rank) {
            orow[rank] = (int32_t)(beg + slot);
            if (srow) srow[rank] = key_score(kk);
        });
        for (int r = total + threadIdx.x; r < k; r += NT) {
            orow[r] = -1;
            if (srow) srow[r] = __builtin_nanf("");
        }
    }
}

// Merge level: workgroup (row, g) takes the candidates of slices
// [g*G, (g+1)*G) of S_in (G*K1 keys) and keeps the top K1 (TO_CAND) or
// writes the final top-k.
template <int NT, int ITEMS, bool TO_CAND>
__global__ __launch_bounds__(NT) void cand_select_kernel(int64_t q0, const uint32_t* in_key, const int32_t* in_tok,
                                                         int S_in, int G, int k, int K1, uint32_t* out_key,
                                                         int32_t* out_tok, int32_t* out_idx, float* out_scores)
{
    __shared__ BucketSmem<NT> sm;
    const int64_t row = blockIdx.x;
    const int g = blockIdx.y;
    const int s0 = g * G;
    const int n = max(0, min(G, S_in - s0)) * K1;
    const uint32_t* kin = in_key + ((int64_t)row * S_in + s0) * K1;
    const int32_t* tin = in_tok + ((int64_t)row * S_in + s0) * K1;
    uint32_t key[ITEMS];
#pragma unroll
    for (int it = 0; it < ITEMS; ++it) {
        const int s = slot_of<ITEMS>(it);
        key[it] = s < n ? kin[s] : 0u;
    }
    const Threshold th = wg_bucket_select<NT, ITEMS>(key, TO_CAND ? K1 : k, sm);
    if (TO_CAND) {
        uint32_t* ok = out_key + (row * gridDim.y + g) * K1;
        int32_t* ot = out_tok + (row * gridDim.y + g) * K1;
        const int total = wg_emit_selected<NT, ITEMS>(key, th, sm, K1, [&](int slot, uint32_t kk, int rank) {
            ok[rank] = kk;
            ot[rank] = tin[slot];
        });
        for (int r = total + threadIdx.x; r < K1; r += NT) {
            ok[r] = 0u;
            ot[r] = -1;
        }
    } else {
        int32_t* orow = out_idx + (q0 + row) * k;
        float* srow = out_scores ? out_scores + (q0 + row) * k : nullptr;
        const int total = wg_emit_selected<NT, ITEMS>(key, th, sm, k, [&](int slot, uint32_t kk, int rank) {
            orow[rank] = tin[slot];
            if (srow) srow[rank] = key_score(kk);
        });
        for (int r = total + threadIdx.x; r < k; r += NT) {
            orow[r] = -1;
            if (srow) srow[r] = __builtin_nanf("");
        }
    }
}

template <int NT, int ITEMS>
static hipError_t launch_flat_level(const QueryMeta& qm, int64_t q0, int64_t nq, const uint32_t* ukeys, int64_t Lmax,
                                    int SL, int S, int k, int K1, uint32_t* ck, int32_t* ct, int32_t* out_idx,
                                    float* out_scores, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1)
{
    if (S > 1)
        return launch_k(flat_select_kernel<NT, ITEMS, true>, dim3((unsigned)nq, (unsigned)S), dim3(NT), stream, ev0,
                        ev1, qm, q0, ukeys, Lmax, SL, k, K1, ck, ct, out_idx, out_scores);
    return launch_k(flat_select_kernel<NT, ITEMS, false>, dim3((unsigned)nq, 1u), dim3(NT), stream, ev0, ev1, qm, q0,
                    ukeys, Lmax, SL, k, K1, ck, ct, out_idx, out_scores);
}

template <int NT, int ITEMS>
static hipError_t launch_cand_level(int64_t q0, int64_t nq, const uint32_t* ik, const int32_t* itok, int S_in, int G,
                                    int S_out, int k, int K1, uint32_t* ok, int32_t* otok, int32_t* out_idx,
                                    float* out_scores, hipStream_t stream, hipEvent_t ev1)
{
    if (S_out > 1)
        return launch_k(cand_select_kernel<NT, ITEMS, true>, dim3((unsigned)nq, (unsigned)S_out), dim3(NT), stream,
                        nullptr, ev1, q0, ik, itok, S_in, G, k, K1, ok, otok, out_idx, out_scores);
    return launch_k(cand_select_kernel<NT, ITEMS, false>, dim3((unsigned)nq, 1u), dim3(NT), stream, nullptr, ev1, q0,
                    ik, itok, S_in, G, k, K1, ok, otok, out_idx, out_scores);
}

FlatPlan flat_plan(int64_t nq, int64_t Lmax, int k)
{
    FlatPlan p;
    p.SL = nq < 256 ? 8192 : 16384;
    p.S = (int)((Lmax + p.SL - 1) / p.SL);
    p.K1 = std::min<int64_t>(k, p.SL);
    p.levels = 1;
    p.radix = false;
    if (p.S > 1) {
        if (p.K1 > kFlatMergeWidth / 4) {
            p.radix = true;                    // too few candidates merge per group
            return p;
        }
        p.G = kFlatMergeWidth / p.K1;
        int S = p.S;
        while (S > 1) {
            S = (S + p.G - 1) / p.G;
            ++p.levels;
        }
        // few long rows: each level is one latency-bound launch, and the
        // multi-workgroup radix select needs fewer steps than three levels
        if (nq < 256 && p.levels >= 3) p.radix = true;
    }
    return p;
}

hipError_t launch_flat_topk(const FlatPlan& p, const QueryMeta& qm, int64_t q0, int64_t nq, const uint32_t* ukeys,
                            int64_t Lmax, int k, uint32_t* cand_key[2], int32_t* cand_tok[2], int32_t* out_idx,
                            float* out_scores, hipStream_t stream, Timing t)
{
    hipEvent_t first_stop = p.S > 1 ? nullptr : t.stop;
    hipError_t err;
    // few rows: 1024 threads (latency); many rows: 512 threads, two
    // workgroups per CU (throughput)
    if (p.SL == 8192)
        err = launch_flat_level<1024, 8>(qm, q0, nq, ukeys, Lmax, p.SL, p.S, k, p.K1, cand_key[0], cand_tok[0],
                                         out_idx, out_scores, stream, t.start, first_stop);
    else
        err = launch_flat_level<512, 32>(qm, q0, nq, ukeys, Lmax, p.SL, p.S, k, p.K1, cand_key[0], cand_tok[0],
                                         out_idx, out_scores, stream, t.start, first_stop);
    int S = p.S, cur = 0;
    while (err == hipSuccess && S > 1) {
        const int S_out = (S + p.G - 1) / p.G;
        hipEvent_t stop = S_out > 1 ? nullptr : t.stop;
        if (p.SL == 8192)
            err = launch_cand_level<1024, 16>(q0, nq, cand_key[cur], cand_tok[cur], S, p.G, S_out, k, p.K1,
                                              cand_key[cur ^ 1], cand_tok[cur ^ 1], out_idx, out_scores, stream, stop);
        else
            err = launch_cand_level<512, 32>(q0, nq, cand_key[cur], cand_tok[cur], S, p.G, S_out, k, p.K1,
                                             cand_key[cur ^ 1], cand_tok[cur ^ 1], out_idx, out_scores, stream, stop);
        S = S_out;
        cur ^= 1;
    }
    return err;
}

// ---- top-k of long rows: S workgroups per row --------------------------------
// Four histogram passes of 8 bits (partial histograms merged with global
// atomics, one small kernel per pass picking the digit), then a count pass
// and an emit pass that writes each slice's selection at the offset given by
// the counts of the slices before it, so rows come out in ascending order.
// state[row] = {prefix, mask, remaining, all}.

constexpr int64_t kSliceMin = 4096;
constexpr int64_t kRadixTargetWgs = 1024;

size_t radix_slices(int64_t nrows, int64_t N)
{
    const int64_t max_s = (N + kSliceMin - 1) / kSliceMin;
    int64_t want = (kRadixTargetWgs + nrows - 1) / std::max<int64_t>(nrows, 1);
    if (want < 1) want = 1;
    return (size_t)std::min(want, std::max<int64_t>(max_s, 1));
}

static int64_t slice_len_of(int64_t N, int64_t S)
{
    const int64_t per = (N + S - 1) / S;
    return (per + kThreads - 1) / kThreads * kThreads;
}

__global__ __launch_bounds__(kThreads) void radix_hist_kernel(const uint32_t* ukeys, int64_t N, int64_t slice_len,
                                                              int pass, int* hist, const uint32_t* state)
{
    __shared__ int h[256];
    const int64_t row = blockIdx.y;
    uint32_t prefix = 0u, mask = 0u;
    if (pass > 0) {
        const uint32_t* st = state + row * 4;
        if (st[3]) return;
        prefix = st[0];
        mask = st[1];
    }
    h[threadIdx.x] = 0;
    __syncthreads();
    const int shift = 24 - 8 * pass;
    const int64_t beg = (int64_t)blockIdx.x * slice_len;
    const int64_t end = min(N, beg + slice_len);
    const uint32_t* src = ukeys + row * N;
    for (int64_t e = beg + threadIdx.x; e < end; e += kThreads) {
        const uint32_t kk = src[e];
        if (kk != 0u && (kk & mask) == prefix) atomicAdd(&h[(kk >> shift) & 255u], 1);
    }
    __syncthreads();
    const int v = h[threadIdx.x];
    if (v) atomicAdd(&hist[row * 256 + threadIdx.x], v);
}

__global__ __launch_bounds__(kThreads) void radix_digit_kernel(int* hist, uint32_t* state, int k, int pass)
{
    __shared__ int scratch[kWaves];
    __shared__ int pick[2];
    const int64_t row = blockIdx.x;
    uint32_t* st = state + row * 4;
    if (pass > 0 && st[3]) return;
    int* hr = hist + row * 256;
    const int h = hr[255 - threadIdx.x];
    hr[255 - threadIdx.x] = 0;   // ready for the next pass
    const uint32_t prefix = pass ? st[0] : 0u;
    const uint32_t mask = pass ? st[1] : 0u;
    const int rem = pass ? (int)st[2] : k;
    if (pass == 0) {
        const int total = block_sum(h, scratch);
        if (total <= k) {
            if (threadIdx.x == 0) {
                st[0] = 0u;
                st[1] = 0u;
                st[2] = 0u;
                st[3] = 1u;
            }
            return;
        }
    }
    const int cum = block_incl_scan(h, scratch);
    if (cum >= rem && cum - h < rem) {
        pick[0] = 255 - (int)threadIdx.x;
        pick[1] = cum - h;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        const int shift = 24 - 8 * pass;
        st[0] = prefix | ((uint32_t)pick[0] << shift);
        st[1] = mask | (0xffu << shift);
        st[2] = (uint32_t)(rem - pick[1]);
        st[3] = 0u;
    }
}

__global__ __launch_bounds__(kThreads) void radix_count_kernel(const uint32_t* ukeys, int64_t N, int64_t slice_len,
                                                               const uint32_t* state, int* counts, int64_t S)
{
    __shared__ int scratch[kWaves];
    const int64_t row = blockIdx.y;
    const uint32_t* st = state + row * 4;
    const bool all = st[3] != 0u;
    const uint32_t T = all ? 0u : st[0];
    const int64_t beg = (int64_t)blockIdx.x * slice_len;
    const int64_t end = min(N, beg + slice_len);
    const uint32_t* src = ukeys + row * N;
    int g = 0, q = 0;
    for (int64_t e = beg + threadIdx.x; e < end; e += kThreads) {
        const uint32_t kk = src[e];
        g += kk > T;
        q += !all && kk == T;
    }
    g = block_sum(g, scratch);
    q = block_sum(q, scratch);
    if (threadIdx.x == 0) {
        counts[(row * S + blockIdx.x) * 2 + 0] = g;
        counts[(row * S + blockIdx.x) * 2 + 1] = q;
    }
}

__global__ __launch_bounds__(kThreads) void radix_emit_kernel(const uint32_t* ukeys, int64_t N, int64_t slice_len,
                                                              const uint32_t* state, const int* counts, int64_t S,
                                                              int k, int32_t* out_idx, float* out_scores)
{
    __shared__ int scratch[kWaves];
    __shared__ int wc[2][kWaves];
    const int64_t row = blockIdx.y;
    const int64_t slice = blockIdx.x;
    const uint32_t* st = state + row * 4;
    const bool all = st[3] != 0u;
    const uint32_t T = all ? 0u : st[0];
    const int need_eq = all ? 0 : (int)st[2];
    int bg = 0, be = 0, tg = 0, te = 0;
    for (int64_t s = threadIdx.x; s < S; s += kThreads) {
        const int g = counts[(row * S + s) * 2 + 0];
        const int q = counts[(row * S + s) * 2 + 1];
        if (s < slice) {
            bg += g;
            be += q;
        }
        tg += g;
        te += q;
    }
    bg = block_sum(bg, scratch);
    be = block_sum(be, scratch);
    tg = block_sum(tg, scratch);
    te = block_sum(te, scratch);
    int32_t* orow = out_idx + row * k;
    float* srow = out_scores ? out_scores + row * k : nullptr;
    if (slice == 0) {
        const int total = tg + min(te, need_eq);
        for (int r = total + threadIdx.x; r < k; r += kThreads) {
            orow[r] = -1;
            if (srow) srow[r] = __builtin_nanf("");
        }
    }
    const int64_t beg = slice * slice_len;
    const int64_t end = min(N, beg + slice_len);
    const uint32_t* src = ukeys + row * N;
    const int w = wave_id();
    for (int64_t base = beg; base < end; base += kThreads) {
        const int64_t e = base + threadIdx.x;
        const uint32_t kk = e < end ? src[e] : 0u;
        const bool gt = kk > T;
        const bool eq = !all && e < end && kk == T;
        const uint64_t mg = __ballot(gt);
        const uint64_t me = __ballot(eq);
        if (lane_id() == 0) {
            wc[0][w] = __popcll(mg);
            wc[1][w] = __popcll(me);
        }
        __syncthreads();
        int og = bg, oe = be, sg = 0, se = 0;
        for (int v = 0; v < kWaves; ++v) {
            if (v < w) {
                og += wc[0][v];
                oe += wc[1][v];
            }
            sg += wc[0][v];
            se += wc[1][v];
        }
        const int pg = og + count_below(mg);
        const int pe = oe + count_below(me);
        int pos = -1;
        if (gt) pos = pg + min(pe, need_eq);
        else if (eq && pe < need_eq) pos = pg + pe;
        if (pos >= 0) {
            orow[pos] = (int32_t)e;
            if (srow) srow[pos] = key_score(kk);
        }
        bg += sg;
        be += se;
        __syncthreads();
    }
}

hipError_t launch_topk_radix(const uint32_t* ukeys, int64_t nrows, int64_t N, int k, const RadixWorkspace& ws,
                             int32_t* out_idx, float* out_scores, hipStream_t stream, Timing t)
{
    const int64_t S = (int64_t)radix_slices(nrows, N);
    const int64_t slice_len = slice_len_of(N, S);
    const int64_t nh = nrows * 256;
    hipError_t err = launch_k(fill_u32_kernel, dim3((unsigned)((nh + kThreads - 1) / kThreads)), dim3(kThreads), stream,
                              t.start, nullptr, reinterpret_cast<uint32_t*>(ws.hist), nh, 0u);
    if (err != hipSuccess) return err;
    const dim3 grid((unsigned)S, (unsigned)nrows);
    for (int pass = 0; pass < 4; ++pass) {
        err = launch_k(radix_hist_kernel, grid, dim3(kThreads), stream, nullptr, nullptr, ukeys, N, slice_len, pass,
                       ws.hist, ws.state);
        if (err == hipSuccess)
            err = launch_k(radix_digit_kernel, dim3((unsigned)nrows), dim3(kThreads), stream, nullptr, nullptr, ws.hist,
                           ws.state, k, pass);
        if (err != hipSuccess) return err;
    }
    err = launch_k(radix_count_kernel, grid, dim3(kThreads), stream, nullptr, nullptr, ukeys, N, slice_len, ws.state,
                   ws.counts, S);
    if (err != hipSuccess) return err;
    return launch_k(radix_emit_kernel, grid, dim3(kThreads), stream, nullptr, t.stop, ukeys, N, slice_len, ws.state,
                    ws.counts, S, k, out_idx, out_scores);
}

}  // namespace hisa
