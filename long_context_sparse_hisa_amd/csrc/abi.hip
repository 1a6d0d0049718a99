// C ABI of libhisa: host-side validation, workspace layout, query chunking
// and kernel launches.  The contract of every entry point is documented in
// include/hisa.h.
#include "../../include/hisa.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <mutex>

#include "kernels.h"

using namespace hisa;

// Device scratch of hisa_index_static: one copy per GPU the library runs
// on, held until the process ends.  Host code never uses this name as an
// address: static_scratch() looks the array up once per device and every
// launch takes that address.
static __device__ __align__(256) unsigned char scratch[HISA_STATIC_SCRATCH_BYTES];

namespace {

constexpr size_t kRecommendedBytes = size_t(1) << 30;   // the recommended workspace: up to 1 GiB of chunk
constexpr int64_t kChunkMax = 65535;      // grid.y limit
constexpr size_t kAlign = 256;

inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// The kernels read and write workspace regions as 16-byte vectors.
inline bool ws_aligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

static_assert(kMaxKept * kMinB == HISA_MAX_CANDIDATES, "kept-block bound of the kernels");
inline bool valid_B(int B) { return B >= kMinB && B <= kMaxB && (B & (B - 1)) == 0; }

int status_of(hipError_t e) { return e == hipSuccess ? HISA_OK : HISA_ERR_HIP; }

// Validation shared by both index calls.  flat selects which rules apply.
int validate_index(const hisa_index_args* a, int flat)
{
    if (!a) return HISA_ERR_INVALID_ARG;
    if (a->nq < 0 || a->nseq < 1 || a->k < 1 || a->max_len < 1) return HISA_ERR_INVALID_ARG;
    if (a->d != 64) return HISA_ERR_UNSUPPORTED;
    if (a->max_len > HISA_MAX_LEN || a->k > HISA_MAX_K) return HISA_ERR_UNSUPPORTED;
    if (a->nseq > 1 && (!a->seq_key_off || !a->seq_len)) return HISA_ERR_INVALID_ARG;
    if (!flat) {
        if (a->m < 3) return HISA_ERR_INVALID_ARG;
        if (!valid_B(a->B)) return HISA_ERR_UNSUPPORTED;
        if ((int64_t)a->m * a->B < a->k) return HISA_ERR_INVALID_ARG;
        if ((int64_t)a->m * a->B > HISA_MAX_CANDIDATES) return HISA_ERR_UNSUPPORTED;
        if ((a->max_len + a->B - 1) / a->B > HISA_MAX_CANDIDATES) return HISA_ERR_UNSUPPORTED;
        if (a->nseq > 1 && !a->seq_rep_off) return HISA_ERR_INVALID_ARG;
    }
    if (a->nq == 0) return HISA_OK;
    if (!a->queries || !a->q_pos || !a->keys || !a->out_idx) return HISA_ERR_INVALID_ARG;
    if (!flat && !a->reps) return HISA_ERR_INVALID_ARG;
    return HISA_OK;
}

// Workspace regions of one chunk of `chunk` queries.
struct Layout {
    // HISA
    size_t sigma = 0, sel = 0, rinfo = 0, ukeys = 0;
    // flat
    size_t hist = 0, state = 0, counts = 0, cand_key[2] = {0, 0}, cand_tok[2] = {0, 0};
    size_t total = 0;
};

int64_t hisa_Mmax(const hisa_index_args* a) { return (a->max_len + a->B - 1) / a->B; }

// Below this many queries the token stage splits every query over several
// workgroups (decode); above it one workgroup per query fills the chip.
constexpr int64_t kSplitBelow = 512;

bool hisa_split(const hisa_index_args* a) { return a->nq < kSplitBelow; }

int log2_of(int B)
{
    int lb = 0;
    while ((1 << lb) < B) ++lb;
    return lb;
}

FlatPlan flat_plan_of(const hisa_index_args* a) { return flat_plan(a->nq, a->max_len, a->k); }

// Flat scores on the matrix cores once a call has enough queries to fill
// 16-row tiles.
bool flat_mfma(const hisa_index_args* a) { return a->nq >= 32; }

Layout layout_for(const hisa_index_args* a, int flat, int64_t chunk)
{
    Layout L;
    size_t off = 0;
    if (!flat) {
        const int64_t Mmax = hisa_Mmax(a);
        L.sel = off;
        off += align_up((size_t)chunk * a->m * sizeof(int32_t));
        L.rinfo = off;
        off += align_up((size_t)chunk * sizeof(RowInfo));
        if (Mmax > kStage1FusedMax) {
            L.sigma = off;
            off += align_up((size_t)chunk * Mmax * sizeof(float));
        }
        L.ukeys = off;                          // candidate ranking keys [chunk, m*B]
        off += align_up((size_t)chunk * a->m * a->B * sizeof(uint32_t));
    } else {
        L.ukeys = off;
        off += align_up((size_t)chunk * a->max_len * sizeof(uint32_t));
        const FlatPlan p = flat_plan_of(a);
        if (!p.radix && p.S > 1) {
            for (int b = 0; b < 2; ++b) {
                L.cand_key[b] = off;
                off += align_up((size_t)chunk * p.S * p.K1 * sizeof(uint32_t));
                L.cand_tok[b] = off;
                off += align_up((size_t)chunk * p.S * p.K1 * sizeof(int32_t));
            }
        }
        if (p.radix) {
            const size_t S = radix_slices(1, a->max_len);   // the largest slice count any chunk uses
            L.hist = off;
            off += align_up((size_t)chunk * 256 * sizeof(int));
            L.state = off;
            off += align_up((size_t)chunk * 4 * sizeof(uint32_t));
            L.counts = off;
            off += align_up((size_t)chunk * S * 2 * sizeof(int));
        }
    }
    L.total = off;
    return L;
}

// Largest chunk whose layout fits in the given workspace (0 if none).
int64_t chunk_for(const hisa_index_args* a, int flat, size_t bytes)
{
    const int64_t cap = std::min<int64_t>(std::max<int64_t>(a->nq, 1), kChunkMax);
    if (layout_for(a, flat, 1).total > bytes) return 0;
    int64_t lo = 1, hi = cap;
    while (lo < hi) {
        const int64_t mid = (lo + hi + 1) / 2;
        if (layout_for(a, flat, mid).total <= bytes) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

QueryMeta meta_of(const hisa_index_args* a)
{
    QueryMeta qm;
    qm.queries = a->queries;
    qm.q_pos = a->q_pos;
    qm.q_seq = a->q_seq;
    qm.seq_key_off = a->seq_key_off;
    qm.seq_rep_off = a->seq_rep_off;
    qm.seq_len = a->seq_len;
    qm.nseq = a->nseq;
    qm.max_len = a->max_len;
    return qm;
}

template <class T>
T* at(void* base, size_t off) { return reinterpret_cast<T*>(static_cast<char*>(base) + off); }

// Start / stop events of stage s for the last query chunk, if asked for.
Timing stage_timing(const hisa_index_args* a, bool last_chunk, int s)
{
    Timing t;
    if (a->stage_events && last_chunk) {
        t.start = static_cast<hipEvent_t>(a->stage_events[2 * s]);
        t.stop = static_cast<hipEvent_t>(a->stage_events[2 * s + 1]);
    }
    return t;
}

// Address of the current device's copy of `scratch` (looked up on the
// first call on that device, with the device current); nullptr on error.
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

int static_scratch(void** out)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return HISA_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return HISA_ERR_UNSUPPORTED;
    void* p = g_scratch[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch[dev].load(std::memory_order_relaxed);
        if (!p) {
            if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return HISA_ERR_HIP;
            g_scratch[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return HISA_OK;
}

}  // namespace

extern "C" {

int hisa_abi_version(void) { return HISA_ABI_VERSION; }

const char* hisa_status_str(int status)
{
    switch (status) {
        case HISA_OK: return "ok";
        case HISA_ERR_INVALID_ARG: return "invalid argument";
        case HISA_ERR_UNSUPPORTED: return "unsupported size or shape";
        case HISA_ERR_WORKSPACE: return "workspace too small";
        case HISA_ERR_HIP: return "HIP runtime error";
        default: return "unknown status";
    }
}

int hisa_pool_blocks(const uint16_t* keys, int64_t L, int d, int B, uint16_t* reps, void* stream)
{
    if (L < 0 || L > HISA_MAX_LEN) return HISA_ERR_INVALID_ARG;
    if (d != 64 || !valid_B(B)) return HISA_ERR_UNSUPPORTED;
    if (L == 0) return HISA_OK;
    if (!keys || !reps) return HISA_ERR_INVALID_ARG;
    PoolJob job{0, 0, (int32_t)L, (int32_t)L, 0, 0, (int32_t)((L + B - 1) / B), 0};
    return status_of(launch_pool(const_cast<uint16_t*>(keys), reps, nullptr, B, &job, 1,
                                 static_cast<hipStream_t>(stream)));
}

int hisa_append_keys(uint16_t* keys, uint16_t* reps, const hisa_seq* seqs, int nseq, const uint16_t* new_keys,
                     int64_t n_new, int d, int B, void* stream)
{
    if (nseq < 0 || n_new < 0) return HISA_ERR_INVALID_ARG;
    if (d != 64 || !valid_B(B)) return HISA_ERR_UNSUPPORTED;
    if (nseq == 0 || n_new == 0) return HISA_OK;
    if (!keys || !reps || !seqs || !new_keys) return HISA_ERR_INVALID_ARG;
    if (n_new > HISA_MAX_LEN || (int64_t)nseq * n_new > INT32_MAX) return HISA_ERR_INVALID_ARG;
    for (int s = 0; s < nseq; ++s) {
        const hisa_seq& q = seqs[s];
        if (q.key_off < 0 || q.rep_off < 0 || q.len < 0 || q.capacity > HISA_MAX_LEN) return HISA_ERR_INVALID_ARG;
        if (q.len + n_new > q.capacity) return HISA_ERR_INVALID_ARG;
    }
    PoolJob jobs[kPoolJobsPerLaunch];
    for (int base = 0; base < nseq; base += kPoolJobsPerLaunch) {
        const int n = std::min(kPoolJobsPerLaunch, nseq - base);
        for (int i = 0; i < n; ++i) {
            const hisa_seq& q = seqs[base + i];
            const int64_t first = q.len / B;
            const int64_t last = (q.len + n_new - 1) / B;
            jobs[i] = PoolJob{q.key_off, q.rep_off, (int32_t)q.len, (int32_t)(q.len + n_new),
                              (int32_t)((int64_t)(base + i) * n_new), (int32_t)first, (int32_t)(last - first + 1), 0};
        }
        const hipError_t err = launch_pool(keys, reps, new_keys, B, jobs, n, static_cast<hipStream_t>(stream));
        if (err != hipSuccess) return HISA_ERR_HIP;
    }
    return HISA_OK;
}

int hisa_workspace_bytes(const hisa_index_args* a, int flat, size_t* bytes, size_t* min_bytes, size_t* all_bytes)
{
    if (!bytes) return HISA_ERR_INVALID_ARG;
    const int rc = validate_index(a, flat);
    if (rc != HISA_OK) return rc;
    const int64_t chunk = std::max<int64_t>(1, chunk_for(a, flat, kRecommendedBytes));
    *bytes = layout_for(a, flat, chunk).total;
    if (min_bytes) *min_bytes = layout_for(a, flat, 1).total;
    if (all_bytes) *all_bytes = layout_for(a, flat, std::max<int64_t>(1, std::min<int64_t>(a->nq, kChunkMax))).total;
    return HISA_OK;
}

int hisa_index(const hisa_index_args* a, void* stream_)
{
    const int rc = validate_index(a, 0);
    if (rc != HISA_OK) return rc;
    if (a->nq == 0) return HISA_OK;
    if (!a->workspace) return HISA_ERR_WORKSPACE;
    if (!ws_aligned(a->workspace)) return HISA_ERR_INVALID_ARG;
    const int64_t chunk = chunk_for(a, 0, a->workspace_bytes);
    if (chunk < 1) return HISA_ERR_WORKSPACE;
    const Layout L = layout_for(a, 0, chunk);
    hipStream_t stream = static_cast<hipStream_t>(stream_);
    const QueryMeta qm = meta_of(a);
    const int64_t Mmax = hisa_Mmax(a);
    const int lb = log2_of(a->B);
    const bool split = hisa_split(a);
    float* sigma = Mmax > kStage1FusedMax ? at<float>(a->workspace, L.sigma) : nullptr;
    int32_t* sel = at<int32_t>(a->workspace, L.sel);
    RowInfo* rinfo = at<RowInfo>(a->workspace, L.rinfo);
    uint32_t* ukeys = at<uint32_t>(a->workspace, L.ukeys);
    for (int64_t q0 = 0; q0 < a->nq; q0 += chunk) {
        const int64_t nc = std::min(chunk, a->nq - q0);
        const bool last = q0 + nc >= a->nq;
        hipError_t err;
        if (split && Mmax <= kStage1FusedMax) {
            // few queries, few blocks: stage 1 and the token scores in one
            // launch (recorded as stage 1)
            err = launch_decode_fused(qm, a->reps, a->keys, q0, nc, lb, a->m, Mmax, sel, rinfo, a->out_blocks, ukeys,
                                      stream, stage_timing(a, last, 1));
        } else if (split) {
            // few queries, many blocks: the representative scores over many
            // workgroups, then the selection and the token scores in one
            // launch (the selection recorded with the token scores)
            err = launch_block_scores(qm, a->reps, q0, nc, lb, Mmax, sigma, stream, stage_timing(a, last, 0));
            if (err == hipSuccess)
                err = launch_select_scores(qm, a->keys, q0, nc, lb, a->m, Mmax, sigma, sel, rinfo, a->out_blocks,
                                           ukeys, stream, stage_timing(a, last, 1));
        } else {
            err = launch_stage1(qm, a->reps, q0, nc, lb, a->m, Mmax, sigma, sel, rinfo, a->out_blocks, stream,
                                stage_timing(a, last, 0));
            // token scores into ukeys: many queries share key loads up to 64
            // at a time on the MFMA
            if (err == hipSuccess)
                err = launch_stage2_tile_scores(qm, a->keys, q0, nc, lb, a->m, Mmax, rinfo, sel, ukeys, stream,
                                                stage_timing(a, last, 1));
        }
        if (err == hipSuccess)
            err = launch_topk_small(ukeys, nc, a->m << lb, a->k, sel, a->m, lb, a->out_idx + q0 * a->k,
                                    a->out_scores ? a->out_scores + q0 * a->k : nullptr, stream,
                                    stage_timing(a, last, 2));
        if (err != hipSuccess) return HISA_ERR_HIP;
    }
    return HISA_OK;
}

int hisa_index_static(const hisa_index_args* a, void* stream)
{
    const int rc = validate_index(a, 0);
    if (rc != HISA_OK) return rc;
    if (a->nq == 0) return HISA_OK;
    // one query's regions must fit; more queries than fit at once run in
    // chunks, as hisa_index does with a small workspace
    if (layout_for(a, 0, 1).total > HISA_STATIC_SCRATCH_BYTES) return HISA_ERR_WORKSPACE;
    void* ws = nullptr;
    const int src = static_scratch(&ws);
    if (src != HISA_OK) return src;
    hisa_index_args b = *a;
    b.workspace = ws;
    b.workspace_bytes = HISA_STATIC_SCRATCH_BYTES;
    return hisa_index(&b, stream);
}

int hisa_decode_step(const hisa_index_args* a, const hisa_seq* seqs, const uint16_t* new_keys, int64_t n_new,
                     void* stream_)
{
    const int rc = validate_index(a, 0);
    if (rc != HISA_OK) return rc;
    if (n_new < 0) return HISA_ERR_INVALID_ARG;
    if (n_new > 0 && (!seqs || !new_keys)) return HISA_ERR_INVALID_ARG;
    for (int s = 0; s < a->nseq && n_new > 0; ++s) {
        const hisa_seq& q = seqs[s];
        if (q.key_off < 0 || q.rep_off < 0 || q.len < 0 || q.capacity > HISA_MAX_LEN || q.len + n_new > q.capacity)
            return HISA_ERR_INVALID_ARG;
        if (q.len + n_new > a->max_len) return HISA_ERR_INVALID_ARG;
    }
    if (n_new > 0 && (int64_t)a->nseq * n_new > INT32_MAX) return HISA_ERR_INVALID_ARG;
    if (a->nq > 0 && !a->workspace) return HISA_ERR_WORKSPACE;
    if (a->nq > 0 && !ws_aligned(a->workspace)) return HISA_ERR_INVALID_ARG;
    const int64_t chunk = a->nq > 0 ? chunk_for(a, 0, a->workspace_bytes) : 1;
    if (chunk < 1) return HISA_ERR_WORKSPACE;
    const int64_t Mmax = hisa_Mmax(a);
    // Without device lengths every query may sit anywhere below max_len;
    // the append is folded into the index's launch only when that bound is
    // the appended length (the launch treats positions at or past a
    // sequence's appended length as invalid, which the two calls would not
    // when max_len is larger).
    const bool lengths_known = a->seq_len != nullptr || (n_new > 0 && a->max_len == seqs[0].len + n_new);
    const bool foldable = n_new > 0 && a->nq > 0 && hisa_split(a) && n_new <= a->B && a->nseq <= kDecodeJobs &&
                          chunk >= a->nq && lengths_known;
    const bool fuse = foldable && Mmax <= kStage1FusedMax;
    if (foldable && !fuse) {
        // more than 2048 blocks: the append joins the block-score launch,
        // then the selection with the token scores and the top-k as in
        // hisa_index
        const Layout L = layout_for(a, 0, chunk);
        hipStream_t stream = static_cast<hipStream_t>(stream_);
        const int lb = log2_of(a->B);
        PoolJob jobs[kDecodeJobs];
        for (int s = 0; s < a->nseq; ++s) {
            const hisa_seq& q = seqs[s];
            const int64_t first = q.len / a->B;
            const int64_t last = (q.len + n_new - 1) / a->B;
            jobs[s] = PoolJob{q.key_off, q.rep_off, (int32_t)q.len, (int32_t)(q.len + n_new), (int32_t)(s * n_new),
                              (int32_t)first, (int32_t)(last - first + 1), 0};
        }
        const StepAppend app{const_cast<uint16_t*>(a->keys), new_keys, a->B, jobs, a->nseq};
        const QueryMeta qm = meta_of(a);
        float* sigma = at<float>(a->workspace, L.sigma);
        int32_t* sel = at<int32_t>(a->workspace, L.sel);
        RowInfo* rinfo = at<RowInfo>(a->workspace, L.rinfo);
        uint32_t* ukeys = at<uint32_t>(a->workspace, L.ukeys);
        hipError_t err = launch_block_scores(qm, a->reps, 0, a->nq, lb, Mmax, sigma, stream, stage_timing(a, true, 0),
                                             &app);
        if (err == hipSuccess)
            err = launch_select_scores(qm, a->keys, 0, a->nq, lb, a->m, Mmax, sigma, sel, rinfo, a->out_blocks, ukeys,
                                       stream, stage_timing(a, true, 1));
        if (err == hipSuccess)
            err = launch_topk_small(ukeys, a->nq, a->m << lb, a->k, sel, a->m, lb, a->out_idx, a->out_scores, stream,
                                    stage_timing(a, true, 2));
        return err == hipSuccess ? HISA_OK : HISA_ERR_HIP;
    }
    if (!fuse) {
        // the same results as the two calls in order
        const int arc = hisa_append_keys(const_cast<uint16_t*>(a->keys), const_cast<uint16_t*>(a->reps), seqs,
                                         a->nseq, new_keys, n_new, a->d, a->B, stream_);
        if (arc != HISA_OK) return arc;
        return hisa_index(a, stream_);
    }
    const Layout L = layout_for(a, 0, chunk);
    hipStream_t stream = static_cast<hipStream_t>(stream_);
    const int lb = log2_of(a->B);
    PoolJob jobs[kDecodeJobs];
    for (int s = 0; s < a->nseq; ++s) {
        const hisa_seq& q = seqs[s];
        const int64_t first = q.len / a->B;
        const int64_t last = (q.len + n_new - 1) / a->B;
        jobs[s] = PoolJob{q.key_off, q.rep_off, (int32_t)q.len, (int32_t)(q.len + n_new), (int32_t)(s * n_new),
                          (int32_t)first, (int32_t)(last - first + 1), 0};
    }
    int32_t* sel = at<int32_t>(a->workspace, L.sel);
    RowInfo* rinfo = at<RowInfo>(a->workspace, L.rinfo);
    uint32_t* ukeys = at<uint32_t>(a->workspace, L.ukeys);
    // stage events as in hisa_index's fused case: stage 1 is the launch
    // (append included), stage 2 the top-k
    hipError_t err = launch_decode_step(meta_of(a), const_cast<uint16_t*>(a->reps), const_cast<uint16_t*>(a->keys),
                                        new_keys, a->B, jobs, a->nseq, a->nq, lb, a->m, Mmax, sel, rinfo,
                                        a->out_blocks, ukeys, stream, stage_timing(a, true, 1));
    if (err == hipSuccess)
        err = launch_topk_small(ukeys, a->nq, a->m << lb, a->k, sel, a->m, lb, a->out_idx, a->out_scores, stream,
                                stage_timing(a, true, 2));
    return err == hipSuccess ? HISA_OK : HISA_ERR_HIP;
}

int hisa_block_index(const hisa_index_args* a, void* stream_)
{
    const int rc = validate_index(a, 0);
    if (rc != HISA_OK) return rc;
    if ((int64_t)a->k != (int64_t)a->m * a->B || a->out_scores) return HISA_ERR_INVALID_ARG;
    if (a->nq == 0) return HISA_OK;
    if (!a->workspace) return HISA_ERR_WORKSPACE;
    if (!ws_aligned(a->workspace)) return HISA_ERR_INVALID_ARG;
    const int64_t chunk = chunk_for(a, 0, a->workspace_bytes);
    if (chunk < 1) return HISA_ERR_WORKSPACE;
    const Layout L = layout_for(a, 0, chunk);
    hipStream_t stream = static_cast<hipStream_t>(stream_);
    const QueryMeta qm = meta_of(a);
    const int64_t Mmax = hisa_Mmax(a);
    const int lb = log2_of(a->B);
    float* sigma = Mmax > kStage1FusedMax ? at<float>(a->workspace, L.sigma) : nullptr;
    int32_t* sel = at<int32_t>(a->workspace, L.sel);
    RowInfo* rinfo = at<RowInfo>(a->workspace, L.rinfo);
    for (int64_t q0 = 0; q0 < a->nq; q0 += chunk) {
        const int64_t nc = std::min(chunk, a->nq - q0);
        const bool last = q0 + nc >= a->nq;
        hipError_t err = launch_stage1(qm, a->reps, q0, nc, lb, a->m, Mmax, sigma, sel, rinfo, a->out_blocks, stream,
                                       stage_timing(a, last, 0));
        if (err == hipSuccess)
            err = launch_expand_blocks(sel, rinfo, nc, a->m, lb, a->out_idx + q0 * a->k, stream,
                                       stage_timing(a, last, 1));
        if (err != hipSuccess) return HISA_ERR_HIP;
    }
    return HISA_OK;
}

int hisa_flat_index(const hisa_index_args* a, void* stream_)
{
    const int rc = validate_index(a, 1);
    if (rc != HISA_OK) return rc;
    if (a->nq == 0) return HISA_OK;
    if (!a->workspace) return HISA_ERR_WORKSPACE;
    if (!ws_aligned(a->workspace)) return HISA_ERR_INVALID_ARG;
    const int64_t chunk = chunk_for(a, 1, a->workspace_bytes);
    if (chunk < 1) return HISA_ERR_WORKSPACE;
    const Layout L = layout_for(a, 1, chunk);
    hipStream_t stream = static_cast<hipStream_t>(stream_);
    const QueryMeta qm = meta_of(a);
    uint32_t* ukeys = at<uint32_t>(a->workspace, L.ukeys);
    for (int64_t q0 = 0; q0 < a->nq; q0 += chunk) {
        const int64_t nc = std::min(chunk, a->nq - q0);
        const bool last = q0 + nc >= a->nq;
        int32_t* oi = a->out_idx + q0 * a->k;
        float* os = a->out_scores ? a->out_scores + q0 * a->k : nullptr;
        // the radix top-k reads whole rows, so it needs the masked keys zeroed
        hipError_t err = launch_flat_scores(qm, a->keys, q0, nc, a->max_len, ukeys, flat_mfma(a),
                                            flat_plan_of(a).radix, stream, stage_timing(a, last, 0));
        if (err == hipSuccess) {
            if (!flat_plan_of(a).radix) {
                uint32_t* ck[2] = {at<uint32_t>(a->workspace, L.cand_key[0]), at<uint32_t>(a->workspace, L.cand_key[1])};
                int32_t* ct[2] = {at<int32_t>(a->workspace, L.cand_tok[0]), at<int32_t>(a->workspace, L.cand_tok[1])};
                err = launch_flat_topk(flat_plan_of(a), qm, q0, nc, ukeys, a->max_len, a->k, ck, ct, a->out_idx,
                                       a->out_scores, stream, stage_timing(a, last, 1));
            } else {
                RadixWorkspace ws{at<int>(a->workspace, L.hist), at<uint32_t>(a->workspace, L.state),
                                  at<int>(a->workspace, L.counts)};
                err = launch_topk_radix(ukeys, nc, a->max_len, a->k, ws, oi, os, stream, stage_timing(a, last, 1));
            }
        }
        if (err != hipSuccess) return HISA_ERR_HIP;
    }
    return HISA_OK;
}

}  // extern "C"
