// libhisa kernels for gfx950: mean pooling / append, HISA stage 1 (block
// scores, causal + forced top-m), HISA stage 2 (token scores in the kept
// blocks), top-k selection and the block-only expansion (the flat
// indexer's kernels are in flat.hip).
//
// What each kernel computes follows "HISA: Efficient Hierarchical Indexing
// for Fine-Grained Sparse Attention" (aitrends.kr summary): structure
// paragraph (blocks of B, mean-pooled representatives), stage-1 paragraph
// (inner-product block scores, causal mask, first and last two blocks
// forced, top-m), stage-2 paragraph (token scores only inside the kept
// blocks, top-k out), maintenance paragraph (representatives updated at
// append).
#include "kernels.h"

#include <math.h>

#include <algorithm>

#include "common.h"
#include "launch.h"
#include "select.h"

namespace hisa {

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
    // slot 0 (block 0 is forced, never a free candidate) marks the query as
    // one to index (select_score_kernel reads it)
    if (b == 0) sigma[row * Mmax] = 1.0f;
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
    // a position at or past the sequence's length after the append (lengths
    // inconsistent with it) is not scored: its causal blocks could include
    // one the append workgroups are rewriting.  Slot 0 of the score row
    // (block 0 is forced, never a free candidate) tells select_score_kernel
    // whether to index the query (1) or give it a -1 row (0).
    const bool ok = !(qi.seq < njobs && qi.t >= jobs.j[qi.seq].len_new);
    const int64_t c = qi.t >> lb;
    const int64_t b = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (b == 0) sigma[row * Mmax] = ok ? 1.0f : 0.0f;
    if (!ok || b < 1 || b > c - 2) return;
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
HISA_INLINE void stage1_select_body(const QueryMeta& qm, const uint16_t* reps, int64_t q0, int64_t row, int lb,
                                    int m, int64_t Mmax, const float* sigma, int32_t* sel, RowInfo* rinfo,
                                    int32_t* out_blocks)
{
    __shared__ BucketSmem<NT> sm;
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
        // every item scores a representative (outside 1 .. c-2 the nearest
        // free one; c >= m >= 3 here), masked after: no branch around loads
#pragma unroll
        for (int it = 0; it < ITEMS; ++it) {
            const int64_t b = slot_of<ITEMS>(it);
            const int64_t bc = min<int64_t>(max<int64_t>(b, 1), c - 2);
            const uint32_t kk =
                score_key(dot64_packed(q, reinterpret_cast<const uint4*>(reps + (qi.rep_off + bc) * kDim)));
            key[it] = (b >= 1 && b <= c - 2) ? kk : 0u;
        }
    } else {
        // every item loads (through a buffer resource: the lane is the
        // vector offset, the item a scalar one, and slots past the row read
        // as zero), then the slots outside 1 .. c-2 are masked
        const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(sigma + row * Mmax, (uint32_t)Mmax * 4u);
        const int w0 = __builtin_amdgcn_readfirstlane(wave_id()) * ITEMS;
        const int lane = lane_id();
        const int hi = (int)(c - 2);
#pragma unroll
        for (int it = 0; it < ITEMS; ++it) {
            const int b = ((w0 + it) << 6) + lane;            // slot_of<ITEMS>(it)
            const float v = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, lane * 4, (w0 + it) * 256, 0));
            key[it] = (b >= 1 && b <= hi) ? score_key(v) : 0u;
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
__global__ __launch_bounds__(NT) void stage1_select_kernel(QueryMeta qm, const uint16_t* reps, int64_t q0, int lb,
                                                           int m, int64_t Mmax, const float* sigma, int32_t* sel,
                                                           RowInfo* rinfo, int32_t* out_blocks)
{
    stage1_select_body<NT, ITEMS, FUSED>(qm, reps, q0, blockIdx.x, lb, m, Mmax, sigma, sel, rinfo, out_blocks);
}

// The select from sigma for many rows of 32 scores per thread, held to six
// waves per SIMD like the many-row token top-k (148 VGPRs otherwise: three
// rows per CU instead of six).
template <int NT, int ITEMS, bool FUSED>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(6, 8))) void stage1_select_many_kernel(
    QueryMeta qm, const uint16_t* reps, int64_t q0, int lb, int m, int64_t Mmax, const float* sigma, int32_t* sel,
    RowInfo* rinfo, int32_t* out_blocks)
{
    stage1_select_body<NT, ITEMS, FUSED>(qm, reps, q0, blockIdx.x, lb, m, Mmax, sigma, sel, rinfo, out_blocks);
}

template <int NT, int ITEMS, bool FUSED, bool MANY = false>
static hipError_t launch_stage1_items(const QueryMeta& qm, const uint16_t* reps, int64_t q0, int64_t nq, int lb,
                                      int m, int64_t Mmax, const float* sigma, int32_t* sel, RowInfo* rinfo,
                                      int32_t* out_blocks, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1)
{
    if constexpr (MANY)
        return launch_k(stage1_select_many_kernel<NT, ITEMS, FUSED>, dim3((unsigned)nq), dim3(NT), stream, ev0, ev1,
                        qm, reps, q0, lb, m, Mmax, sigma, sel, rinfo, out_blocks);
    else
        return launch_k(stage1_select_kernel<NT, ITEMS, FUSED>, dim3((unsigned)nq), dim3(NT), stream, ev0, ev1, qm,
                        reps, q0, lb, m, Mmax, sigma, sel, rinfo, out_blocks);
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
            // every item reads its score (b < 64 * ITEMS lies inside the LDS
            // row) and is masked after: no branch around the reads
            uint32_t key[ITEMS];
#pragma unroll
            for (int it = 0; it < ITEMS; ++it) {
                const int b = it * 64 + lane;
                const uint32_t kk = score_key(sc[rr * RS + b]);
                key[it] = (b >= 1 && b <= cr - 2) ? kk : 0u;
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

// Many queries with more blocks than stage1_tile_kernel holds in LDS: the
// representative scores on the bf16 MFMA into sigma [nq, Mmax], for the
// stage-1 select (or select_score_kernel) to select from.  A wave takes 64
// consecutive query rows (four 16-row sub-tiles, the B operands, loaded
// once) and a range of 16-block tiles; each representative tile it loads
// (the A operand) feeds the two v_mfma_f32_16x16x32_bf16 of every sub-tile
// (d = 64).  Lane l receives blocks 4*(l/16)..+4 of the tile for query row
// l%16 of a sub-tile and stores them as one 16-byte vector.  Tiles past the
// largest causal block of the walked rows are not scored; rows of several
// sequences are walked one sequence at a time.  Slot 0 of a valid row holds
// 1 instead of block 0's score (block 0 is forced, never a free candidate;
// select_score_kernel reads the flag).
constexpr int kBsRows = 64;
constexpr int kBsWaves = 4;
constexpr int64_t kBsTargetWaves = 8192;

__global__ __launch_bounds__(64 * kBsWaves) void block_score_tile_kernel(QueryMeta qm, const uint16_t* reps,
                                                                         int64_t q0, int64_t nq, int lb, int64_t Mmax,
                                                                         int range, float* sigma)
{
    const int lane = lane_id();
    const int64_t row0 = (int64_t)blockIdx.x * kBsRows;
    const int nrows = (int)min<int64_t>(kBsRows, nq - row0);
    const int ntile = (int)((Mmax + 15) / 16);
    const int bt0 = ((int)blockIdx.y * kBsWaves + wave_id()) * range;
    if (bt0 >= ntile) return;
    const int bt1 = min(bt0 + range, ntile);
    QueryInfo qi;
    qi.valid = false;
    qi.seq = -1;
    qi.t = -1;
    qi.key_off = 0;
    qi.rep_off = 0;
    if (lane < nrows)
        qi = query_info(q0 + row0 + lane, qm.q_pos, qm.q_seq, qm.seq_key_off, qm.seq_rep_off, qm.seq_len, qm.nseq,
                        qm.max_len);
    const int c_own = qi.valid ? (int)(qi.t >> lb) : 0;
    const int col = lane & 15, kg = lane >> 4;
    bf16x8_t a0[4], a1[4];
#pragma unroll
    for (int sb = 0; sb < 4; ++sb) {
        a0[sb] = bf16x8_t{};
        a1[sb] = bf16x8_t{};
        if (16 * sb + col < nrows) {
            const uint16_t* qrow = qm.queries + (q0 + row0 + 16 * sb + col) * kDim + 8 * kg;
            a0[sb] = *reinterpret_cast<const bf16x8_t*>(qrow);
            a1[sb] = *reinterpret_cast<const bf16x8_t*>(qrow + 32);
        }
    }
    const bool vec = (Mmax & 3) == 0;                  // 16-byte aligned score rows
    uint64_t pending = __ballot(qi.valid);
    while (pending) {
        const int lead = (int)__builtin_ctzll(pending);
        const int s = __builtin_amdgcn_readlane(qi.seq, lead);
        const bool mine = qi.valid && qi.seq == s;
        const uint64_t mrows = __ballot(mine);
        pending &= ~mrows;
        const int64_t rep_off = ((int64_t)__builtin_amdgcn_readlane((int)(qi.rep_off >> 32), lead) << 32) |
                                (uint32_t)__builtin_amdgcn_readlane((int)qi.rep_off, lead);
        const int cmax = (int)wave_max_u32(mine ? (uint32_t)c_own : 0u);
        const int tend = min(bt1, cmax / 16 + 1);
        for (int bt = bt0; bt < tend; ++bt) {
            const int b = bt * 16 + col;
            bf16x8_t r0 = {}, r1 = {};
            if (b <= cmax) {
                const uint16_t* rp = reps + (rep_off + b) * kDim + 8 * kg;
                r0 = *reinterpret_cast<const bf16x8_t*>(rp);
                r1 = *reinterpret_cast<const bf16x8_t*>(rp + 32);
            }
#pragma unroll
            for (int sb = 0; sb < 4; ++sb) {
                if (((mrows >> (16 * sb)) & 0xffffull) == 0) continue;      // uniform: no walked row here
                f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(r0, a0[sb], acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(r1, a1[sb], acc, 0, 0, 0);
                if (!((mrows >> (16 * sb + col)) & 1ull)) continue;
                const int j = bt * 16 + 4 * kg;
                if (j == 0) acc[0] = 1.0f;
                float* dst = sigma + (row0 + 16 * sb + col) * Mmax + j;
                if (vec && j + 3 < Mmax) {
                    *reinterpret_cast<f32x4_t*>(dst) = acc;
                } else {
#pragma unroll
                    for (int v = 0; v < 4; ++v)
                        if (j + v < Mmax) dst[v] = acc[v];
                }
            }
        }
    }
}

static hipError_t launch_block_scores_tile(const QueryMeta& qm, const uint16_t* reps, int64_t q0, int64_t nq, int lb,
                                           int64_t Mmax, float* sigma, hipStream_t stream, Timing t)
{
    const int64_t qtiles = (nq + kBsRows - 1) / kBsRows;
    const int64_t ntile = (Mmax + 15) / 16;
    const int64_t want = std::max<int64_t>(1, (kBsTargetWaves + qtiles - 1) / qtiles);
    const int64_t range = std::max<int64_t>(1, (ntile + want - 1) / want);
    const int64_t nranges = (ntile + range - 1) / range;
    const dim3 grid((unsigned)qtiles, (unsigned)((nranges + kBsWaves - 1) / kBsWaves));
    return launch_k(block_score_tile_kernel, grid, dim3(64 * kBsWaves), stream, t.start, t.stop, qm, reps, q0, nq, lb,
                    Mmax, (int)range, sigma);
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
    // many queries: the scores on the matrix cores; few: one thread per score
    if (nq >= kManyRows) return launch_block_scores_tile(qm, reps, q0, nq, lb, Mmax, sigma, stream, t);
    dim3 grid((unsigned)((Mmax + kThreads - 1) / kThreads), (unsigned)nq);
    return launch_k(block_score_kernel, grid, dim3(kThreads), stream, t.start, t.stop, qm, reps, q0, lb, Mmax, sigma);
}

// ---- many queries, many blocks: block scores and top-m, no score row -------
// Rows with more blocks than stage1_tile_kernel holds, when m - 3 is at most
// kBfMaxFree.  The representative scores are never written: a workgroup of
// kBfWaves waves takes kBfRows consecutive query rows (four 16-row MFMA
// sub-tiles; queries are the A operand, representatives the B operand, so
// lane l receives rows 4*(l/16)+v, v = 0..3, of each sub-tile against block
// 16*bt + l%16), and wave w walks the 16-block tiles w, w+kBfWaves, ...
// (representatives through a buffer resource, the next tile loading while
// one is scored; tiles inside every walked row's free range unmasked, tile 0
// and the last ones masked) twice:
//  1. every lane keeps, for each row it holds, the kBfTrack largest scores of
//     the free blocks in its column (kBfTrack medians of three per score).
//     The four waves' lists are merged per (row, column) through LDS, and
//     theta_r is the (m-3)-th largest of the row's 16*kBfTrack merged
//     values (found bit by bit over their ranking keys), so at least m-3
//     free blocks score >= theta_r when those values are real scores.
//  2. the scores again; every free block with !(score < theta_r) is listed
//     (score, block) in this wave's kBfSeg-entry segment of the row's LDS
//     list, its place given by the ballot of the row's 16 lanes.
// A row whose list holds at least m-3 blocks, no segment overflowing and
// none scoring NaN, then holds every block of its top m-3: a block left out
// scores below theta_r, below every listed one, and m-3 are listed (this
// holds whatever theta_r is, so the first walk only has to make it tight).
// So the exact top
// m-3 of the list (ties to the lower block) is the row's selection, found by
// the wave select over the list in ascending block order (a bitmap of the
// listed blocks gives each its place).  Any other row is marked by
// sel[row][0] = -2 and selected again from scratch by stage1_fixup_kernel.
constexpr int kBfRows = 64;
constexpr int kBfWaves = 4;
constexpr int kBfTrack = 6;
constexpr int kBfSeg = 32;                   // list entries of one row from one wave
constexpr int kBfCap = kBfWaves * kBfSeg;
constexpr int kBfMaxFree = 64;
constexpr int kBfMaxBlocks = 16384;
constexpr int kBfWords = kBfMaxBlocks / 32;

struct BfWave {
    alignas(16) uint32_t bm[kBfWords];   // the listed blocks of one row as bits
    int pre[kBfWords];                   // listed blocks before each word
    uint32_t skey[kBfCap];               // the list in ascending block order
    int32_t sblk[kBfCap];
    WaveSmem ws;
};

struct BfSmem {
    union {
        float xch[kBfWaves][4][kBfTrack][64];   // walk-1 lists on their way to the wave that merges them
        struct {
            float score[kBfWaves][kBfRows][kBfSeg];   // the blocks a wave lists for a row
            int16_t blk[kBfWaves][kBfRows][kBfSeg];
        } lst;
    } u;
    float theta[kBfRows];
    int cnt[kBfWaves][kBfRows];         // blocks each wave listed for a row (more than kBfSeg: overflow)
    int hi[kBfRows];          // last free block of each walked row (-1: not walked now)
    BfWave pw[kBfWaves];
};

// The T largest of t and x, descending (t is descending): T medians of
// three, the first against the largest finite float (a median against +inf
// would be compiled as a maximum with its operands canonicalised, three
// instructions).  An infinite score may enter as that float; the lists only
// set a threshold, and a row the threshold does not certify is reselected.
template <int T>
HISA_INLINE void track_insert(float (&t)[T], float x)
{
#pragma unroll
    for (int i = T - 1; i >= 1; --i) t[i] = __builtin_amdgcn_fmed3f(t[i - 1], t[i], x);
    t[0] = __builtin_amdgcn_fmed3f(t[0], x, 3.40282347e38f);
}

// Sum over the 16 lanes of each row of the wave (DPP row rotations).
HISA_INLINE int row_sum16(int v)
{
    uint32_t x = (uint32_t)v;
    x += dpp_u32<0x128>(x);          // row_ror:8
    x += dpp_u32<0x124>(x);          // row_ror:4
    x += dpp_u32<0x122>(x);          // row_ror:2
    x += dpp_u32<0x121>(x);          // row_ror:1
    return (int)x;
}

HISA_INLINE bool nan_key(uint32_t k) { return k > 0xff800000u || k < 0x007fffffu; }

__global__ __launch_bounds__(64 * kBfWaves) __attribute__((amdgpu_waves_per_eu(2, 2))) void block_select_tile_kernel(QueryMeta qm, const uint16_t* reps,
                                                                          int64_t q0, int64_t nq, int lb, int m,
                                                                          int32_t* sel, RowInfo* rinfo,
                                                                          int32_t* out_blocks)
{
    extern __shared__ __align__(16) unsigned char s_raw[];
    BfSmem& S = *reinterpret_cast<BfSmem*>(s_raw);
    const int w = wave_id(), lane = lane_id();
    const int col = lane & 15, kg = lane >> 4;
    const int64_t row0 = (int64_t)blockIdx.x * kBfRows;
    const int nrows = (int)min<int64_t>(kBfRows, nq - row0);
    const int mf = m - 3;
    // lane r holds the info of row r (every wave the same, so the loops
    // below are uniform over the workgroup)
    QueryInfo qi;
    qi.valid = false;
    qi.seq = -1;
    qi.t = -1;
    qi.key_off = 0;
    qi.rep_off = 0;
    if (lane < nrows) {
        qi = query_info(q0 + row0 + lane, qm.q_pos, qm.q_seq, qm.seq_key_off, qm.seq_rep_off, qm.seq_len, qm.nseq,
                        qm.max_len);
        if (w == 0) rinfo[row0 + lane] = RowInfo{qi.key_off, qi.valid ? qi.t : -1};
    }
    const int c_own = qi.valid ? (int)(qi.t >> lb) : -1;
    // invalid rows keep no block, rows with c + 1 <= m every causal block
    for (uint64_t sv = __ballot(lane < nrows && c_own + 1 <= m && (lane & 3) == w); sv; sv &= sv - 1) {
        const int rr = (int)__builtin_ctzll(sv);
        const int cr = __builtin_amdgcn_readlane(c_own, rr);
        for (int j = lane; j < m; j += 64) {
            const int32_t v = j <= cr ? j : -1;
            sel[(row0 + rr) * m + j] = v;
            if (out_blocks) out_blocks[(q0 + row0 + rr) * m + j] = v;
        }
    }
    bf16x8_t a0[4], a1[4];
#pragma unroll
    for (int sb = 0; sb < 4; ++sb) {
        a0[sb] = bf16x8_t{};
        a1[sb] = bf16x8_t{};
        if (16 * sb + col < nrows) {
            const uint16_t* qrow = qm.queries + (q0 + row0 + 16 * sb + col) * kDim + 8 * kg;
            a0[sb] = *reinterpret_cast<const bf16x8_t*>(qrow);
            a1[sb] = *reinterpret_cast<const bf16x8_t*>(qrow + 32);
        }
    }
    const bool act = lane < nrows && c_own + 1 > m;
    uint64_t pending = __ballot(act);
    while (pending) {
        // the rows of one sequence at a time
        const int lead = (int)__builtin_ctzll(pending);
        const int s = __builtin_amdgcn_readlane(qi.seq, lead);
        const bool mine = act && qi.seq == s;
        const uint64_t mrows = __ballot(mine);
        pending &= ~mrows;
        const int64_t rep_off = ((int64_t)__builtin_amdgcn_readlane((int)(qi.rep_off >> 32), lead) << 32) |
                                (uint32_t)__builtin_amdgcn_readlane((int)qi.rep_off, lead);
        // free blocks of a row: 1 .. hi (hi = -1: not walked now)
        const int hi_own = mine ? c_own - 2 : -1;
        if (w == 0) S.hi[lane] = hi_own;          // read by the tiles that need a mask
        __syncthreads();
        const int hmax = (int)wave_max_u32(mine ? (uint32_t)hi_own : 0u);
        // tiles 1 .. tint lie inside every walked row's free blocks: scored
        // without a mask (rows not walked now are scored too and ignored:
        // their theta is +inf); tile 0 and tiles past tint are masked
        const int hmin = (int)wave_min_u32(mine ? (uint32_t)hi_own : 0x7fffffffu);
        const int tint = (hmin + 1) / 16 - 1;
        const int ntile = hmax / 16 + 1;
        // representative rows 0 .. hmax through a buffer resource: every
        // load is issued unconditionally (rows past hmax read as zero and are
        // masked like any block outside a row's free range), so the next
        // tile's loads stay in flight while the current one is scored
        const __amdgpu_buffer_rsrc_t rrs = buffer_rsrc(reps + rep_off * kDim, (uint32_t)(hmax + 1) * 128u);
        auto load_rep = [&](int bt, bf16x8_t& r0, bf16x8_t& r1) {
            const uint32_t off = (uint32_t)(bt * 16 + col) * 128u + 16u * (uint32_t)kg;
            r0 = __builtin_bit_cast(bf16x8_t, __builtin_amdgcn_raw_buffer_load_b128(rrs, off, 0, 0));
            r1 = __builtin_bit_cast(bf16x8_t, __builtin_amdgcn_raw_buffer_load_b128(rrs, off + 64u, 0, 0));
        };

        // the scores of tile bt for the four sub-tiles
        auto tile_scores = [&](const bf16x8_t& r0, const bf16x8_t& r1, f32x4_t (&acc)[4]) {
#pragma unroll
            for (int sb = 0; sb < 4; ++sb) {
                acc[sb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
                acc[sb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0[sb], r0, acc[sb], 0, 0, 0);
                acc[sb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1[sb], r1, acc[sb], 0, 0, 0);
            }
        };
        // this wave's tiles: bt = w (mod kBfWaves); interior ones first,
        // then the masked ones (tile 0 and those past tint)
        const int ib = w == 0 ? kBfWaves : w;          // first interior tile of the wave
        const int eb = tint < w ? w : w + ((tint - w) / kBfWaves + 1) * kBfWaves;   // first tile past tint
        auto edge_tile = [&](int i) {                  // i-th masked tile of the wave, or -1
            if (w == 0) {
                if (i == 0) return 0;
                --i;
            }
            const int bt = max(eb, w == 0 ? kBfWaves : w) + i * kBfWaves;
            return bt < ntile ? bt : -1;
        };

        // walk 1: the kBfTrack largest free scores per (row, column)
        float tr[4][4][kBfTrack];
#pragma unroll
        for (int sb = 0; sb < 4; ++sb)
#pragma unroll
            for (int v = 0; v < 4; ++v)
#pragma unroll
                for (int t = 0; t < kBfTrack; ++t) tr[sb][v][t] = -__builtin_inff();
        {
            bf16x8_t n0, n1;
            load_rep(ib, n0, n1);
            for (int bt = ib; bt <= tint; bt += kBfWaves) {
                const bf16x8_t r0 = n0, r1 = n1;
                load_rep(bt + kBfWaves, n0, n1);
                f32x4_t acc[4];
                tile_scores(r0, r1, acc);
#pragma unroll
                for (int sb = 0; sb < 4; ++sb)
#pragma unroll
                    for (int v = 0; v < 4; ++v) track_insert(tr[sb][v], acc[sb][v]);
            }
            for (int i = 0;; ++i) {
                const int bt = edge_tile(i);
                if (bt < 0) break;
                bf16x8_t r0, r1;
                load_rep(bt, r0, r1);
                f32x4_t acc[4];
                tile_scores(r0, r1, acc);
                const int b = bt * 16 + col;
#pragma unroll
                for (int sb = 0; sb < 4; ++sb)
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        const int h = S.hi[16 * sb + 4 * kg + v];
                        track_insert(tr[sb][v], (b >= 1 && b <= h) ? acc[sb][v] : -__builtin_inff());
                    }
            }
        }
        // merge: in round r wave w sends its lists of sub-tile (w + r) % 4
        // and merges those of sub-tile w from wave (w - r) % 4
#pragma unroll
        for (int r = 1; r < kBfWaves; ++r) {
            const int out_sb = (w + r) & 3;
#pragma unroll
            for (int sb = 0; sb < 4; ++sb) {
                if (sb != out_sb) continue;
#pragma unroll
                for (int v = 0; v < 4; ++v)
#pragma unroll
                    for (int t = 0; t < kBfTrack; ++t) S.u.xch[w][v][t][lane] = tr[sb][v][t];
            }
            __syncthreads();
            const int from = (w - r) & 3;
#pragma unroll
            for (int sb = 0; sb < 4; ++sb) {
                if (sb != w) continue;
#pragma unroll
                for (int v = 0; v < 4; ++v)
#pragma unroll
                    for (int t = 0; t < kBfTrack; ++t) track_insert(tr[sb][v], S.u.xch[from][v][t][lane]);
            }
            __syncthreads();
        }
        // theta of the rows of sub-tile w: the mf-th largest ranking key of
        // the 16 lanes' merged lists, bit by bit from the top
        uint32_t kk[4][kBfTrack];
#pragma unroll
        for (int sb = 0; sb < 4; ++sb) {
            if (sb != w) continue;
#pragma unroll
            for (int v = 0; v < 4; ++v)
#pragma unroll
                for (int t = 0; t < kBfTrack; ++t) kk[v][t] = score_key(tr[sb][v][t]);
        }
        uint32_t p[4] = {0u, 0u, 0u, 0u};
        for (int bit = 31; bit >= 0; --bit) {
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const uint32_t cand = p[v] | (1u << bit);
                int cnt = 0;
#pragma unroll
                for (int t = 0; t < kBfTrack; ++t) cnt += kk[v][t] >= cand;
                if (row_sum16(cnt) >= mf) p[v] = cand;
            }
        }
        if (col == 0) {
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int r = 16 * w + 4 * kg + v;
                S.theta[r] = ((mrows >> r) & 1ull) ? key_score(p[v]) : __builtin_inff();
            }
        }
        __syncthreads();

        // walk 2: list every free block scoring at least theta, in this
        // wave's segment of the row's list; a lane's place comes from the
        // ballot of its 16-lane group (the lanes of one row), no atomics
        float th[4][4];
        int cnt[4][4];
#pragma unroll
        for (int sb = 0; sb < 4; ++sb)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                th[sb][v] = S.theta[16 * sb + 4 * kg + v];
                cnt[sb][v] = 0;
            }
        const uint32_t gm_lo = kg == 0 ? 0x0000ffffu : (kg == 1 ? 0xffff0000u : 0u);
        const uint32_t gm_hi = kg == 2 ? 0x0000ffffu : (kg == 3 ? 0xffff0000u : 0u);
        auto list_tile = [&](const f32x4_t (&acc)[4], int b, bool masked) {
#pragma unroll
            for (int sb = 0; sb < 4; ++sb)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const float x = acc[sb][v];
                    bool take = !(x < th[sb][v]);
                    if (masked) take = take && b >= 1 && b <= S.hi[16 * sb + 4 * kg + v];
                    const uint64_t M = __ballot(take);
                    if (M == 0) continue;
                    const uint32_t lo = (uint32_t)M & gm_lo, hi = (uint32_t)(M >> 32) & gm_hi;
                    const int pos = cnt[sb][v] + (int)__builtin_amdgcn_mbcnt_hi(hi, __builtin_amdgcn_mbcnt_lo(lo, 0u));
                    if (take && pos < kBfSeg) {
                        const int r = 16 * sb + 4 * kg + v;
                        S.u.lst.score[w][r][pos] = x;
                        S.u.lst.blk[w][r][pos] = (int16_t)b;
                    }
                    cnt[sb][v] += __popc(lo) + __popc(hi);
                }
        };
        {
            bf16x8_t n0, n1;
            load_rep(ib, n0, n1);
            for (int bt = ib; bt <= tint; bt += kBfWaves) {
                const bf16x8_t r0 = n0, r1 = n1;
                load_rep(bt + kBfWaves, n0, n1);
                f32x4_t acc[4];
                tile_scores(r0, r1, acc);
                list_tile(acc, bt * 16 + col, false);
            }
            for (int i = 0;; ++i) {
                const int bt = edge_tile(i);
                if (bt < 0) break;
                bf16x8_t r0, r1;
                load_rep(bt, r0, r1);
                f32x4_t acc[4];
                tile_scores(r0, r1, acc);
                list_tile(acc, bt * 16 + col, true);
            }
        }
        if (col == 0) {
#pragma unroll
            for (int sb = 0; sb < 4; ++sb)
#pragma unroll
                for (int v = 0; v < 4; ++v) S.cnt[w][16 * sb + 4 * kg + v] = cnt[sb][v];
        }
        __syncthreads();

        // each listed row: wave w takes rows w, w + 4, ...
        BfWave& P = S.pw[w];
        for (uint64_t mv = mrows & (0x1111111111111111ull << w); mv; mv &= mv - 1) {
            const int r = (int)__builtin_ctzll(mv);
            int nw[kBfWaves], n = 0, nmax = 0;
#pragma unroll
            for (int v = 0; v < kBfWaves; ++v) {
                nw[v] = __builtin_amdgcn_readfirstlane(S.cnt[v][r]);
                n += nw[v];
                nmax = max(nmax, nw[v]);
            }
            const int cr = __builtin_amdgcn_readlane(c_own, r);
            int32_t* srow = sel + (row0 + r) * m;
            int32_t* orow = out_blocks ? out_blocks + (q0 + row0 + r) * m : nullptr;
            bool ok = n >= mf && nmax <= kBfSeg;
            uint32_t k0 = 0u, k1 = 0u;
            int b0 = 0, b1 = 0;
            if (ok) {
                // entry e: the segments one after the other
                const int p1 = nw[0], p2 = p1 + nw[1], p3 = p2 + nw[2];
                auto load_entry = [&](int e, uint32_t& kk, int& bb) {
                    const int v = (e >= p1) + (e >= p2) + (e >= p3);
                    const int base = v == 0 ? 0 : (v == 1 ? p1 : (v == 2 ? p2 : p3));
                    kk = score_key(S.u.lst.score[v][r][e - base]);
                    bb = S.u.lst.blk[v][r][e - base];
                };
                if (lane < n) load_entry(lane, k0, b0);
                if (lane + 64 < n) load_entry(lane + 64, k1, b1);
                ok = __ballot((lane < n && nan_key(k0)) || (lane + 64 < n && nan_key(k1))) == 0;
            }
            if (!ok) {
                if (lane == 0) srow[0] = -2;
                continue;
            }
            // place of each listed block in ascending block order
#pragma unroll
            for (int i = 0; i < kBfWords / 64; ++i) P.bm[lane + 64 * i] = 0u;
            wave_lds_fence();
            if (lane < n) atomicOr(&P.bm[b0 >> 5], 1u << (b0 & 31));
            if (lane + 64 < n) atomicOr(&P.bm[b1 >> 5], 1u << (b1 & 31));
            wave_lds_fence();
            constexpr int kPer = kBfWords / 64;   // words of lane l: kPer*l ..
            int pc[kPer];
            int tot = 0;
#pragma unroll
            for (int j = 0; j < kPer; ++j) {
                pc[j] = tot;
                tot += __popc(P.bm[kPer * lane + j]);
            }
            const int ex = wave_incl_scan(tot) - tot;
#pragma unroll
            for (int j = 0; j < kPer; ++j) P.pre[kPer * lane + j] = ex + pc[j];
            wave_lds_fence();
            if (lane < n) {
                const int sl = P.pre[b0 >> 5] + __popc(P.bm[b0 >> 5] & ((1u << (b0 & 31)) - 1u));
                P.skey[sl] = k0;
                P.sblk[sl] = b0;
            }
            if (lane + 64 < n) {
                const int sl = P.pre[b1 >> 5] + __popc(P.bm[b1 >> 5] & ((1u << (b1 & 31)) - 1u));
                P.skey[sl] = k1;
                P.sblk[sl] = b1;
            }
            wave_lds_fence();
            uint32_t key2[2];
            key2[0] = lane < n ? P.skey[lane] : 0u;
            key2[1] = lane + 64 < n ? P.skey[lane + 64] : 0u;
            wave_select<2>(key2, mf, P.ws, [&](int slot, uint32_t, int rank) {
                const int32_t blk = P.sblk[slot];
                srow[1 + rank] = blk;
                if (orow) orow[1 + rank] = blk;
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
            wave_lds_fence();
        }
        __syncthreads();
    }
}

// Rows block_select_tile_kernel marked (sel[row][0] = -2): selected from
// scratch, one row at a time by the workgroup of the row's tile (1024
// threads score the representatives and run the workgroup select).
template <int ITEMS>
__global__ __launch_bounds__(1024) void stage1_fixup_kernel(QueryMeta qm, const uint16_t* reps, int64_t q0,
                                                            int64_t nq, int lb, int m, int32_t* sel, RowInfo* rinfo,
                                                            int32_t* out_blocks)
{
    const int64_t row0 = (int64_t)blockIdx.x * kBfRows;
    const int64_t r = row0 + lane_id();
    uint64_t fl = __ballot(r < nq && sel[r * m] == -2);
    __syncthreads();                  // every wave has read the marks before any row is rewritten
    while (fl) {
        const int rr = (int)__builtin_ctzll(fl);
        fl &= fl - 1;
        stage1_select_body<1024, ITEMS, true>(qm, reps, q0, row0 + rr, lb, m, 0, nullptr, sel, rinfo, out_blocks);
        __syncthreads();
    }
}

static hipError_t launch_block_select(const QueryMeta& qm, const uint16_t* reps, int64_t q0, int64_t nq, int lb,
                                      int m, int64_t Mmax, int32_t* sel, RowInfo* rinfo, int32_t* out_blocks,
                                      hipStream_t stream, Timing t)
{
    const int64_t tiles = (nq + kBfRows - 1) / kBfRows;
    hipError_t err = launch_kl(block_select_tile_kernel, dim3((unsigned)tiles), dim3(64 * kBfWaves), sizeof(BfSmem),
                               stream, t.start, nullptr, qm, reps, q0, nq, lb, m, sel, rinfo, out_blocks);
    if (err != hipSuccess) return err;
    const int64_t per = (Mmax + 1023) / 1024;
#define HISA_FX(N_)                                                                                              \
    if (per <= N_)                                                                                               \
    return launch_k(stage1_fixup_kernel<N_>, dim3((unsigned)tiles), dim3(1024), stream, nullptr, t.stop, qm, reps, \
                    q0, nq, lb, m, sel, rinfo, out_blocks)
    HISA_FX(2);
    HISA_FX(4);
    HISA_FX(8);
    HISA_FX(16);
#undef HISA_FX
    return hipErrorInvalidValue;
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
    if (nq >= kManyRows && Mmax <= kBfMaxBlocks && m - 3 >= 1 && m - 3 <= kBfMaxFree)
        // many queries, many blocks: MFMA walks, no score row in memory
        return launch_block_select(qm, reps, q0, nq, lb, m, Mmax, sel, rinfo, out_blocks, stream, t);
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
    if (nq >= kManyRows) {
        // many rows: 32 scores per thread in 256- or 512-thread workgroups,
        // several per CU hiding each other's barriers
        if (Mmax <= 4096)
            return launch_stage1_items<256, 16, false>(qm, reps, q0, nq, lb, m, Mmax, sigma, sel, rinfo, out_blocks,
                                                       stream, nullptr, t.stop);
        if (Mmax <= 8192)
            return launch_stage1_items<256, 32, false, true>(qm, reps, q0, nq, lb, m, Mmax, sigma, sel, rinfo,
                                                             out_blocks, stream, nullptr, t.stop);
        return launch_stage1_items<512, 32, false>(qm, reps, q0, nq, lb, m, Mmax, sigma, sel, rinfo, out_blocks,
                                                   stream, nullptr, t.stop);
    }
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
    QueryInfo qi =
        query_info(i, qm.q_pos, qm.q_seq, qm.seq_key_off, qm.seq_rep_off, qm.seq_len, qm.nseq, qm.max_len);
    // the block-score launch marks in slot 0 the valid queries it scored
    if (qi.valid && sigma[row * Mmax] == 0.0f) qi.valid = false;
    const int64_t c = qi.valid ? qi.t >> lb : -1;
    if (!qi.valid || c + 1 <= m) {
        for (int r = threadIdx.x; r < m; r += NT) s_kept[r] = r <= c ? r : -1;
    } else {
        // every item loads (buffer resource over the row: the lane is the
        // vector offset, the item a scalar one), then slots outside 1 .. c-2
        // are masked
        const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(sigma + row * Mmax, (uint32_t)Mmax * 4u);
        const int w0 = __builtin_amdgcn_readfirstlane(wave_id()) * ITEMS;
        const int hi = (int)(c - 2);
        uint32_t key[ITEMS];
#pragma unroll
        for (int it = 0; it < ITEMS; ++it) {
            const int b = ((w0 + it) << 6) + lane_id();
            const float v = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, lane_id() * 4, (w0 + it) * 256, 0));
            key[it] = (b >= 1 && b <= hi) ? score_key(v) : 0u;
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
// No cap on the positions a fused workgroup treats as valid.
struct NoCap {
    HISA_INLINE int64_t operator()(const QueryInfo&) const { return INT64_MAX; }
};

template <int ITEMS, class Source, class Cap = NoCap>
HISA_INLINE void decode_fused_body(const QueryMeta& qm, const uint16_t* reps, int64_t q0, int64_t row, int lb, int m,
                                   int groups, int32_t* sel, RowInfo* rinfo, int32_t* out_blocks, uint32_t* ukeys,
                                   Source source, Cap cap = Cap{})
{
    __shared__ BucketSmem<kThreads> sm;
    __shared__ int32_t s_kept[kMaxKept];
    const int64_t i = q0 + row;
    QueryInfo qi =
        query_info(i, qm.q_pos, qm.q_seq, qm.seq_key_off, qm.seq_rep_off, qm.seq_len, qm.nseq, qm.max_len);
    if (qi.valid && qi.t >= cap(qi)) qi.valid = false;
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
        return [=](int64_t j) { return (j >= len_old && j < len_new) ? nk + (j - len_old) * kDim : ck + j * kDim; };
    }, [&](const QueryInfo& qi) -> int64_t {
        // positions at or past the sequence's length after the append
        // (lengths inconsistent with it) are invalid here: their causal
        // blocks could include one the append workgroups are rewriting
        return qi.seq < njobs ? (int64_t)jobs.j[qi.seq].len_new : INT64_MAX;
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
        // piece p of block b: key tiles p*KP .. p*KP+KP-1, through a buffer
        // resource over the sequence's keys 0 .. tmax (keys past the walked
        // rows' last position read as zero): every load is issued
        // unconditionally, so a prefetched piece stays in flight while the
        // current one is on the MFMA
        const __amdgpu_buffer_rsrc_t krs = buffer_rsrc(keys + koff * kDim, (uint32_t)(tmax + 1) * 128u);
        auto load_piece = [&](int b, int p, bf16x8_t (&k0)[KP], bf16x8_t (&k1)[KP]) {
#pragma unroll
            for (int kt = 0; kt < KP; ++kt) {
                const uint32_t off = (uint32_t)((b << LB) + (p * KP + kt) * 16 + col) * 128u + 16u * (uint32_t)kg;
                k0[kt] = __builtin_bit_cast(bf16x8_t, __builtin_amdgcn_raw_buffer_load_b128(krs, off, 0, 0));
                k1[kt] = __builtin_bit_cast(bf16x8_t, __builtin_amdgcn_raw_buffer_load_b128(krs, off + 64u, 0, 0));
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
            load_piece(b2 != kTileEnd ? b2 : b, p2, n0, n1);   // past the walk's end: a harmless reload
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

// ---- token scores of sparse kept lists, block-major ------------------------
// Many queries of one sequence whose kept lists are sparse in the block range
// (8m <= Mmax <= 128m: a 64-row tile of the union walk would score most of
// the blocks it walks for only a few of its rows; measured 152 -> 66 us at
// Mmax = 16m, 2.90 -> 1.75 ms at 128m, where a tile's block has about two
// keepers).  Workgroup (x, y) takes
// the kGatherRows query rows of tile x and the BR blocks of range y.  Every
// row's list (ascending, m <= kGatherMaxM entries, loaded by one thread as
// 16-byte vectors) gives the (row, list position) pairs whose block lies in
// the range; they are grouped by block in LDS (a count, a scan, a scatter).
// Each wave then takes blocks of the range: the block's keys are the A
// operand (lane l: key l%16 of each 16-key tile, dims 8*(l/16)..+8 of each
// half of d, through a buffer resource over the sequence's keys up to the
// tile's last position: keys past it read as zero), its keepers the B
// operand, 16 at a time, two v_mfma_f32_16x16x32_bf16 per 16-key tile as in
// the union walk; lane l receives keys 4*(l/16)..+4 of each tile for keeper
// l%16 and stores them as one 16-byte vector into the keeper's slots, key 0
// for tokens after its position.  Every kept (row, block) pair is scored
// once, and each slot is written by one workgroup.
constexpr int kGatherRows = 256;
constexpr int kGatherMaxM = 64;

__host__ __device__ constexpr size_t gather_lds(int BR, int m)
{
    return sizeof(int32_t) * ((size_t)(BR + 1) + BR + (size_t)kGatherRows * (m < BR ? m : BR) + kGatherRows + 8);
}

template <int LB>
__global__ __launch_bounds__(kGatherRows) void stage2_gather_kernel(const uint16_t* queries, const uint16_t* keys,
                                                                    int64_t q0, int64_t nq, int m, int BR,
                                                                    const RowInfo* rinfo, const int32_t* sel,
                                                                    uint32_t* ukeys)
{
    constexpr int B = 1 << LB;
    constexpr int KT = B / 16;
    extern __shared__ __align__(16) int32_t s_g[];
    int* off = s_g;                                   // [BR + 1]: keepers per block, then their offsets
    int* cur = off + (BR + 1);                        // [BR]: scatter cursors
    int32_t* ent = cur + BR;                          // keepers grouped by block: (row << 10) | list position
    int* trow = ent + kGatherRows * min(m, BR);       // [kGatherRows]: each row's position (-1: none)
    int* misc = trow + kGatherRows;                   // [0]: largest position, [1..2]: key offset
    const int tid = threadIdx.x, lane = lane_id(), w = wave_id();
    const int64_t row0 = (int64_t)blockIdx.x * kGatherRows;
    const int nrows = (int)min<int64_t>(kGatherRows, nq - row0);
    const int blo = (int)blockIdx.y * BR, bhi = blo + BR;
    const int N = m << LB;
    for (int i = tid; i <= BR; i += kGatherRows) off[i] = 0;
    // thread tid: row tid of the tile, its list in registers
    RowInfo ri{0, -1};
    if (tid < nrows) ri = rinfo[row0 + tid];
    const bool valid = ri.t >= 0;
    trow[tid] = valid ? (int)ri.t : -1;
    int4 lst[kGatherMaxM / 4];
#pragma unroll
    for (int i = 0; i < kGatherMaxM / 4; ++i) {
        lst[i] = make_int4(-1, -1, -1, -1);
        if (valid && 4 * i < m) lst[i] = reinterpret_cast<const int4*>(sel + (row0 + tid) * m)[i];
    }
    const uint32_t tmax = wave_max_u32(valid ? (uint32_t)ri.t : 0u);
    if (lane == 0) misc[4 + w] = (int)tmax;
    if (valid) {
        misc[1] = (int)(ri.key_off & 0xffffffff);     // every valid row of the call has the same key offset
        misc[2] = (int)(ri.key_off >> 32);
    }
    __syncthreads();
    auto in_range = [&](int v) { return v >= blo && v < bhi; };
#pragma unroll
    for (int i = 0; i < kGatherMaxM / 4; ++i) {
        const int v[4] = {lst[i].x, lst[i].y, lst[i].z, lst[i].w};
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (in_range(v[e])) atomicAdd(&off[v[e] - blo], 1);
    }
    __syncthreads();
    if (w == 0) {
        // exclusive scan of the counts (BR <= 64: one wave)
        const int c = lane < BR ? off[lane] : 0;
        const int incl = wave_incl_scan(c);
        if (lane < BR) {
            off[lane] = incl - c;
            cur[lane] = incl - c;
        }
        if (lane == 63) off[BR] = incl;
        if (lane == 0) misc[0] = (int)max(max((uint32_t)misc[4], (uint32_t)misc[5]), max((uint32_t)misc[6], (uint32_t)misc[7]));
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kGatherMaxM / 4; ++i) {
        const int v[4] = {lst[i].x, lst[i].y, lst[i].z, lst[i].w};
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (in_range(v[e])) ent[atomicAdd(&cur[v[e] - blo], 1)] = (tid << 10) | (4 * i + e);
    }
    __syncthreads();
    if (off[BR] == 0) return;                         // uniform: no kept block in this range
    const int64_t koff = ((int64_t)misc[2] << 32) | (uint32_t)misc[1];
    const int tlast = misc[0];
    const int col = lane & 15, kg = lane >> 4;
    const __amdgpu_buffer_rsrc_t krs = buffer_rsrc(keys + koff * kDim, (uint32_t)(tlast + 1) * 128u);
    for (int j = w; j < BR; j += kWaves) {
        const int e0 = off[j], nk = off[j + 1] - e0;
        if (nk == 0) continue;
        const int b = blo + j;
        bf16x8_t k0[KT], k1[KT];
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) {
            const uint32_t o = (uint32_t)((b << LB) + kt * 16 + col) * 128u + 16u * (uint32_t)kg;
            k0[kt] = __builtin_bit_cast(bf16x8_t, __builtin_amdgcn_raw_buffer_load_b128(krs, o, 0, 0));
            k1[kt] = __builtin_bit_cast(bf16x8_t, __builtin_amdgcn_raw_buffer_load_b128(krs, o + 64u, 0, 0));
        }
        for (int g = 0; g < nk; g += 16) {
            // keeper g + col of the block (a clamped one past the last loads
            // a valid row and stores nothing)
            const bool have = g + col < nk;
            const int e = ent[e0 + min(g + col, nk - 1)];
            const int rl = e >> 10, p = e & 1023;
            const uint16_t* qrow = queries + (q0 + row0 + rl) * kDim + 8 * kg;
            const bf16x8_t a0 = *reinterpret_cast<const bf16x8_t*>(qrow);
            const bf16x8_t a1 = *reinterpret_cast<const bf16x8_t*>(qrow + 32);
            f32x4_t c[KT];
#pragma unroll
            for (int kt = 0; kt < KT; ++kt)
                c[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0[kt], a0, f32x4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
            for (int kt = 0; kt < KT; ++kt) c[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1[kt], a1, c[kt], 0, 0, 0);
            if (have) {
                const int t = trow[rl];
                uint32_t* urow = ukeys + (row0 + rl) * N + ((int64_t)p << LB) + 4 * kg;
#pragma unroll
                for (int kt = 0; kt < KT; ++kt) {
                    const int jj = (b << LB) + kt * 16 + 4 * kg;
                    uint4 o = make_uint4(score_key(c[kt][0]), score_key(c[kt][1]), score_key(c[kt][2]),
                                         score_key(c[kt][3]));
                    o.x = jj + 0 <= t ? o.x : 0u;
                    o.y = jj + 1 <= t ? o.y : 0u;
                    o.z = jj + 2 <= t ? o.z : 0u;
                    o.w = jj + 3 <= t ? o.w : 0u;
                    *reinterpret_cast<uint4*>(urow + kt * 16) = o;
                }
            }
        }
    }
}

static hipError_t launch_stage2_gather(const QueryMeta& qm, const uint16_t* keys, int64_t q0, int64_t nq, int lb,
                                       int m, int64_t Mmax, const RowInfo* rinfo, const int32_t* sel, uint32_t* ukeys,
                                       hipStream_t stream, Timing t)
{
    // about 512 workgroups, ranges of BR blocks (a power of two, 4 .. 64):
    // measured on the 128K chunk (4,096 rows, 1,024 blocks) 66 us at 512,
    // 73 at 256, 85 at 1024, 101 at 2048 (each workgroup reads its rows'
    // whole lists, so more workgroups repeat that more)
    const int64_t tiles = (nq + kGatherRows - 1) / kGatherRows;
    int BR = 4;
    while (BR < 64 && tiles * ((Mmax + BR - 1) / BR) > 512) BR *= 2;
    const dim3 grid((unsigned)tiles, (unsigned)((Mmax + BR - 1) / BR));
    const size_t lds = gather_lds(BR, m);
#define HISA_G2(LB_) \
    if (lb == LB_) return launch_kl(stage2_gather_kernel<LB_>, grid, dim3(kGatherRows), lds, stream, t.start, t.stop, qm.queries, keys, q0, nq, m, BR, rinfo, sel, ukeys)
    HISA_G2(4);
    HISA_G2(5);
    HISA_G2(6);
    HISA_G2(7);
    HISA_G2(8);
#undef HISA_G2
    return hipErrorInvalidValue;
}

hipError_t launch_stage2_tile_scores(const QueryMeta& qm, const uint16_t* keys, int64_t q0, int64_t nq, int lb, int m,
                                     int64_t Mmax, const RowInfo* rinfo, const int32_t* sel, uint32_t* ukeys,
                                     hipStream_t stream, Timing t)
{
    // sparse lists of one sequence: block-major, every kept pair scored once
    if (qm.nseq == 1 && nq >= kManyRows && m <= kGatherMaxM && m % 4 == 0 && Mmax >= 8 * (int64_t)m &&
        Mmax <= 128 * (int64_t)m)
        return launch_stage2_gather(qm, keys, q0, nq, lb, m, Mmax, rinfo, sel, ukeys, stream, t);
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
HISA_INLINE void topk_rows_body(const uint32_t* ukeys, int N, int k, const int32_t* sel, int m, int lb,
                                int32_t* out_idx, float* out_scores)
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
        // every item loads through a buffer resource of the row's N keys
        // (the lane is the vector offset, the item a scalar one; slots past
        // N read 0)
        const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(src, (uint32_t)N * 4u);
        uint32_t key[ITEMS];
#pragma unroll
        for (int it = 0; it < ITEMS; ++it) key[it] = __builtin_amdgcn_raw_buffer_load_b32(rs, lane * 4, (g0 + it) * 256, 0);
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

template <int NT, int ITEMS, bool WAVE_BLK, bool SCORES>
__global__ __launch_bounds__(NT) void topk_rows_kernel(const uint32_t* ukeys, int N, int k, const int32_t* sel, int m,
                                                       int lb, int32_t* out_idx, float* out_scores)
{
    topk_rows_body<NT, ITEMS, WAVE_BLK, SCORES>(ukeys, N, k, sel, m, lb, out_idx, out_scores);
}

// The same for many rows of up to 8192 keys (256 threads x 32 keys): the
// compiler is held to 80 VGPRs (six waves per SIMD, some values kept in
// scratch), so six rows share a CU instead of four and hide more of each
// other's barrier and LDS latency (measured at 32K: 469 -> 407 us; five
// waves per SIMD 422 us, seven 418, eight 430).
template <int NT, int ITEMS, bool WAVE_BLK, bool SCORES>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(6, 8))) void topk_rows_many_kernel(
    const uint32_t* ukeys, int N, int k, const int32_t* sel, int m, int lb, int32_t* out_idx, float* out_scores)
{
    topk_rows_body<NT, ITEMS, WAVE_BLK, SCORES>(ukeys, N, k, sel, m, lb, out_idx, out_scores);
}

template <int NT, int ITEMS, bool MANY = false>
static hipError_t launch_topk_rows_items(const uint32_t* ukeys, int64_t nrows, int N, int k, const int32_t* sel,
                                         int m, int lb, int32_t* out_idx, float* out_scores, hipStream_t stream,
                                         Timing t)
{
#define HISA_TR(W_, S_)                                                                                       \
    if constexpr (MANY)                                                                                       \
        return launch_k(topk_rows_many_kernel<NT, ITEMS, W_, S_>, dim3((unsigned)nrows), dim3(NT), stream,      \
                        t.start, t.stop, ukeys, N, k, sel, m, lb, out_idx, out_scores);                        \
    else                                                                                                      \
        return launch_k(topk_rows_kernel<NT, ITEMS, W_, S_>, dim3((unsigned)nrows), dim3(NT), stream, t.start,  \
                        t.stop, ukeys, N, k, sel, m, lb, out_idx, out_scores)
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
        if (N <= 8192)
            return launch_topk_rows_items<256, 32, true>(ukeys, nrows, N, k, sel, m, lb, out_idx, out_scores, stream, t);
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

}  // namespace hisa
