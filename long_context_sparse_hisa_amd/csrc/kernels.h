// Host-side launchers of the libhisa kernels (internal; the public C ABI is
// include/hisa.h).  Every launcher only enqueues on `stream` and returns the
// launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace hisa {

// Optional kernel timing: when set, the first kernel of a launcher records
// `start` when it begins and the last records `stop` when it ends (the
// dispatch packet's own timestamps, as a profiler sees them).
struct Timing {
    hipEvent_t start = nullptr;
    hipEvent_t stop = nullptr;
};

// What stage 1 learns about a query row, kept for the stage-2 kernels so
// they start with one round trip instead of the query -> sequence chain.
struct RowInfo {
    int64_t key_off;  // first key row of its sequence
    int64_t t;        // position in its sequence, -1 for an invalid query
};

// One sequence's part of a pool / append launch.
struct PoolJob {
    int64_t key_off;    // first key row of the sequence
    int64_t rep_off;    // first representative row
    int32_t len_old;    // keys already in the cache
    int32_t len_new;    // keys after the append (== len_old for plain pooling)
    int32_t new_row;    // row of this sequence's first key in new_keys
    int32_t blk_first;  // first block to (re)compute
    int32_t nblk;       // blocks to (re)compute
    int32_t pad;
};

// Jobs travel in the kernel arguments (96 x 40 bytes, inside the 4 KiB
// argument limit), so a decode step of up to 96 sequences is one launch.
constexpr int kPoolJobsPerLaunch = 96;

hipError_t launch_pool(uint16_t* keys, uint16_t* reps, const uint16_t* new_keys, int B, const PoolJob* jobs,
                       int njobs, hipStream_t stream);

// Query metadata as passed through the C ABI (device pointers).
struct QueryMeta {
    const uint16_t* queries;
    const int64_t* q_pos;
    const int32_t* q_seq;
    const int64_t* seq_key_off;
    const int64_t* seq_rep_off;
    const int64_t* seq_len;
    int32_t nseq;
    int64_t max_len;
};

// HISA stage 1: block scores, causal + forced top-m.  sel [nq, m] (the
// chunk's rows) and rinfo [nq]; out_blocks (nullable) gets the same rows at query offset
// q0.  Many queries (>= kManyRows) are scored on the matrix cores: up to
// 1024 blocks into LDS tiles, more blocks (m - 3 <= 64) by two walks that
// keep no score row; otherwise queries with at most kStage1FusedMax blocks
// are scored by the selecting workgroup and longer ones go through sigma
// [nq, Mmax].  lb = log2(B).
constexpr int64_t kStage1FusedMax = 2048;
// A decode step's append, folded into the first launch of the path for
// more than 2048 blocks (the block scores, launch_block_scores): one job
// per sequence, at most kDecodeJobs.
struct StepAppend {
    uint16_t* keys;
    const uint16_t* new_keys;
    int B;
    const PoolJob* jobs;
    int njobs;
};

hipError_t launch_stage1(const QueryMeta& qm, const uint16_t* reps, int64_t q0, int64_t nq, int lb, int m,
                         int64_t Mmax, float* sigma, int32_t* sel, RowInfo* rinfo, int32_t* out_blocks,
                         hipStream_t stream, Timing t = {});

// The representative scores alone into sigma [nq, Mmax] (at least the free
// candidates 1 .. c-2 of each query; slot 0 flags the query as one to
// index), with a decode step's append folded in when app is given;
// launch_select_scores or the stage-1 select then selects.  Many queries
// are scored on the matrix cores, few one thread per score.
hipError_t launch_block_scores(const QueryMeta& qm, const uint16_t* reps, int64_t q0, int64_t nq, int lb,
                               int64_t Mmax, float* sigma, hipStream_t stream, Timing t = {},
                               const struct StepAppend* app = nullptr);

// Few queries with more than kStage1FusedMax blocks: the selection from
// sigma and the token scores in one launch (every workgroup of a query
// selects the kept blocks itself); writes sel, rinfo, out_blocks and ukeys.
hipError_t launch_select_scores(const QueryMeta& qm, const uint16_t* keys, int64_t q0, int64_t nq, int lb, int m,
                                int64_t Mmax, const float* sigma, int32_t* sel, RowInfo* rinfo, int32_t* out_blocks,
                                uint32_t* ukeys, hipStream_t stream, Timing t = {});

// HISA stage 2 for many queries: 16 query rows per wave scored on the
// MFMA against the union of their kept blocks, into ukeys [nq, m*B] (only
// the kept blocks' slots are written); launch_topk_small then selects.
hipError_t launch_stage2_tile_scores(const QueryMeta& qm, const uint16_t* keys, int64_t q0, int64_t nq, int lb, int m,
                                     int64_t Mmax, const RowInfo* rinfo, const int32_t* sel, uint32_t* ukeys,
                                     hipStream_t stream, Timing t = {});

// Few queries with at most kStage1FusedMax blocks: stage 1 and the token
// scores of stage 2 in one launch (every workgroup of a query selects the
// kept blocks itself); writes sel, rinfo, out_blocks and ukeys.
hipError_t launch_decode_fused(const QueryMeta& qm, const uint16_t* reps, const uint16_t* keys, int64_t q0,
                               int64_t nq, int lb, int m, int64_t Mmax, int32_t* sel, RowInfo* rinfo,
                               int32_t* out_blocks, uint32_t* ukeys, hipStream_t stream, Timing t = {});

// The same launch with the decode step's append folded in: one job per
// sequence (at most kDecodeJobs, new keys spanning at most two blocks);
// jobs travel in the kernel arguments.
constexpr int kDecodeJobs = 64;
hipError_t launch_decode_step(const QueryMeta& qm, uint16_t* reps, uint16_t* keys, const uint16_t* new_keys, int B,
                              const PoolJob* jobs, int njobs, int64_t nq, int lb, int m, int64_t Mmax, int32_t* sel,
                              RowInfo* rinfo, int32_t* out_blocks, uint32_t* ukeys, hipStream_t stream, Timing t = {});

// HISA stage 2 for few queries: kStage2SlotsPerWg candidate slots per
// workgroup scored into ukeys [nq, m*B] (inside the fused decode and
// select-and-score launches); launch_topk_small then selects.
constexpr int kStage2SlotsPerWg = 512;

// Flat: ranking keys of the visible keys into ukeys [nq, Lmax].  mfma: 16
// query rows per tile on the matrix cores, otherwise one thread per
// (query, key).  zero_masked: keys after the query get key 0 (what the
// radix top-k needs; the levelled top-k reads rows only up to t).  The
// one-thread path always zeroes them.
hipError_t launch_flat_scores(const QueryMeta& qm, const uint16_t* keys, int64_t q0, int64_t nq,
                              int64_t Lmax, uint32_t* ukeys, bool mfma, bool zero_masked, hipStream_t stream,
                              Timing t = {});

// Flat top-k in levels: slices of SL keys keep their top K1 = min(k, SL),
// then groups of G = kFlatMergeWidth / K1 slices are merged until one is
// left.  radix: K1 too large to merge, use launch_topk_radix instead.
constexpr int kFlatMergeWidth = 16384;
struct FlatPlan {
    int SL, S, K1, G, levels;
    bool radix;
};
FlatPlan flat_plan(int64_t nq, int64_t Lmax, int k);
// p: the plan of the whole call (its workspace was laid out for it).
hipError_t launch_flat_topk(const FlatPlan& p, const QueryMeta& qm, int64_t q0, int64_t nq, const uint32_t* ukeys,
                            int64_t Lmax, int k, uint32_t* cand_key[2], int32_t* cand_tok[2], int32_t* out_idx,
                            float* out_scores, hipStream_t stream, Timing t = {});

// Block sizes are powers of two in [kMinB, kMaxB]; m*B is at most 16384
// candidates, so a query keeps at most kMaxKept blocks.
constexpr int kMinB = 16;
constexpr int kMaxB = 256;
constexpr int kMaxKept = 16384 / kMinB;

// Rows per launch from which a select is sized for throughput, not latency.
constexpr int64_t kManyRows = 256;

// Top-k of rows of N ranking keys held by one workgroup (N <= 16384).
// sel == NULL: slot s is token s; otherwise slot s is token
// sel[row*m + s/B]*B + s%B (lb = log2(B)).  Output row r starts at
// out_idx + r*k.
hipError_t launch_topk_small(const uint32_t* ukeys, int64_t nrows, int N, int k, const int32_t* sel, int m,
                             int lb, int32_t* out_idx, float* out_scores, hipStream_t stream, Timing t = {});

// Block-only rows [nq, m*B]: every visible token of each query's kept
// blocks (sel, ascending with -1 padding), ascending, then -1.
hipError_t launch_expand_blocks(const int32_t* sel, const RowInfo* rinfo, int64_t nq, int m, int lb,
                                int32_t* out_idx, hipStream_t stream, Timing t = {});

// Top-k of long rows (slot s is token s) with several workgroups per row.
struct RadixWorkspace {
    int* hist;        // [nrows, 256]
    uint32_t* state;  // [nrows, 4]
    int* counts;      // [nrows, S, 2]
};
size_t radix_slices(int64_t nrows, int64_t N);
hipError_t launch_topk_radix(const uint32_t* ukeys, int64_t nrows, int64_t N, int k, const RadixWorkspace& ws,
                             int32_t* out_idx, float* out_scores, hipStream_t stream, Timing t = {});

}  // namespace hisa
