// libhisa kernels of the flat DSA indexer: every visible key scored (one
// thread per pair, or 16-query tiles on the bf16 MFMA), then the top-k in
// levels of slice selections, or a radix select for few long rows.
//
// What is computed follows the "DSA" section of "Why long-context LLMs
// slow down and how sparse attention fixes it" (idea.jsleekr.com): every
// key is scored by a light dot product with the query and the best k are
// kept.
#include "kernels.h"

#include <math.h>

#include <algorithm>

#include "common.h"
#include "launch.h"
#include "select.h"

namespace hisa {

static __global__ __launch_bounds__(kThreads) void fill_u32_kernel(uint32_t* p, int64_t n, uint32_t v)
{
    const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (i < n) p[i] = v;
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
HISA_INLINE void flat_select_body(const QueryMeta& qm, int64_t q0, const uint32_t* ukeys, int64_t Lmax, int SL,
                                  int k, int K1, uint32_t* cand_key, int32_t* cand_tok, int32_t* out_idx,
                                  float* out_scores)
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
    // every item loads through a buffer resource of the slice's n keys (the
    // lane is the vector offset, the item a scalar one; past n reads 0)
    const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(src, (uint32_t)n * 4u);
    const int w0 = __builtin_amdgcn_readfirstlane(wave_id()) * ITEMS;
    uint32_t key[ITEMS];
#pragma unroll
    for (int it = 0; it < ITEMS; ++it) key[it] = __builtin_amdgcn_raw_buffer_load_b32(rs, lane_id() * 4, (w0 + it) * 256, 0);
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
HISA_INLINE void cand_select_body(int64_t q0, const uint32_t* in_key, const int32_t* in_tok, int S_in, int G, int k,
                                  int K1, uint32_t* out_key, int32_t* out_tok, int32_t* out_idx, float* out_scores)
{
    __shared__ BucketSmem<NT> sm;
    const int64_t row = blockIdx.x;
    const int g = blockIdx.y;
    const int s0 = g * G;
    const int n = max(0, min(G, S_in - s0)) * K1;
    const uint32_t* kin = in_key + ((int64_t)row * S_in + s0) * K1;
    const int32_t* tin = in_tok + ((int64_t)row * S_in + s0) * K1;
    const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(kin, (uint32_t)n * 4u);     // past n reads 0
    const int w0 = __builtin_amdgcn_readfirstlane(wave_id()) * ITEMS;
    uint32_t key[ITEMS];
#pragma unroll
    for (int it = 0; it < ITEMS; ++it) key[it] = __builtin_amdgcn_raw_buffer_load_b32(rs, lane_id() * 4, (w0 + it) * 256, 0);
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

template <int NT, int ITEMS, bool TO_CAND>
__global__ __launch_bounds__(NT) void flat_select_kernel(QueryMeta qm, int64_t q0, const uint32_t* ukeys,
                                                         int64_t Lmax, int SL, int k, int K1, uint32_t* cand_key,
                                                         int32_t* cand_tok, int32_t* out_idx, float* out_scores)
{
    flat_select_body<NT, ITEMS, TO_CAND>(qm, q0, ukeys, Lmax, SL, k, K1, cand_key, cand_tok, out_idx, out_scores);
}

template <int NT, int ITEMS, bool TO_CAND>
__global__ __launch_bounds__(NT) void cand_select_kernel(int64_t q0, const uint32_t* in_key, const int32_t* in_tok,
                                                         int S_in, int G, int k, int K1, uint32_t* out_key,
                                                         int32_t* out_tok, int32_t* out_idx, float* out_scores)
{
    cand_select_body<NT, ITEMS, TO_CAND>(q0, in_key, in_tok, S_in, G, k, K1, out_key, out_tok, out_idx, out_scores);
}

// The 512-thread forms (many rows, 32 keys per thread) held to six waves per
// SIMD, as the HISA top-k's many-row form: three slices share a CU instead
// of one (150 VGPRs) and hide each other's barrier and LDS latency
// (measured, 32K prefill: level selects 3.47 -> 2.95 ms; four waves per
// SIMD 3.51 ms).
template <int NT, int ITEMS, bool TO_CAND>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(6, 8))) void flat_select_many_kernel(
    QueryMeta qm, int64_t q0, const uint32_t* ukeys, int64_t Lmax, int SL, int k, int K1, uint32_t* cand_key,
    int32_t* cand_tok, int32_t* out_idx, float* out_scores)
{
    flat_select_body<NT, ITEMS, TO_CAND>(qm, q0, ukeys, Lmax, SL, k, K1, cand_key, cand_tok, out_idx, out_scores);
}

template <int NT, int ITEMS, bool TO_CAND>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(6, 8))) void cand_select_many_kernel(
    int64_t q0, const uint32_t* in_key, const int32_t* in_tok, int S_in, int G, int k, int K1, uint32_t* out_key,
    int32_t* out_tok, int32_t* out_idx, float* out_scores)
{
    cand_select_body<NT, ITEMS, TO_CAND>(q0, in_key, in_tok, S_in, G, k, K1, out_key, out_tok, out_idx, out_scores);
}

template <int NT, int ITEMS>
static hipError_t launch_flat_level(const QueryMeta& qm, int64_t q0, int64_t nq, const uint32_t* ukeys, int64_t Lmax,
                                    int SL, int S, int k, int K1, uint32_t* ck, int32_t* ct, int32_t* out_idx,
                                    float* out_scores, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1)
{
    if constexpr (NT == 512) {
        if (S > 1)
            return launch_k(flat_select_many_kernel<NT, ITEMS, true>, dim3((unsigned)nq, (unsigned)S), dim3(NT),
                            stream, ev0, ev1, qm, q0, ukeys, Lmax, SL, k, K1, ck, ct, out_idx, out_scores);
        return launch_k(flat_select_many_kernel<NT, ITEMS, false>, dim3((unsigned)nq, 1u), dim3(NT), stream, ev0,
                        ev1, qm, q0, ukeys, Lmax, SL, k, K1, ck, ct, out_idx, out_scores);
    } else {
        if (S > 1)
            return launch_k(flat_select_kernel<NT, ITEMS, true>, dim3((unsigned)nq, (unsigned)S), dim3(NT), stream,
                            ev0, ev1, qm, q0, ukeys, Lmax, SL, k, K1, ck, ct, out_idx, out_scores);
        return launch_k(flat_select_kernel<NT, ITEMS, false>, dim3((unsigned)nq, 1u), dim3(NT), stream, ev0, ev1, qm,
                        q0, ukeys, Lmax, SL, k, K1, ck, ct, out_idx, out_scores);
    }
}

template <int NT, int ITEMS>
static hipError_t launch_cand_level(int64_t q0, int64_t nq, const uint32_t* ik, const int32_t* itok, int S_in, int G,
                                    int S_out, int k, int K1, uint32_t* ok, int32_t* otok, int32_t* out_idx,
                                    float* out_scores, hipStream_t stream, hipEvent_t ev1)
{
    if constexpr (NT == 512) {
        if (S_out > 1)
            return launch_k(cand_select_many_kernel<NT, ITEMS, true>, dim3((unsigned)nq, (unsigned)S_out), dim3(NT),
                            stream, nullptr, ev1, q0, ik, itok, S_in, G, k, K1, ok, otok, out_idx, out_scores);
        return launch_k(cand_select_many_kernel<NT, ITEMS, false>, dim3((unsigned)nq, 1u), dim3(NT), stream, nullptr,
                        ev1, q0, ik, itok, S_in, G, k, K1, ok, otok, out_idx, out_scores);
    } else {
        if (S_out > 1)
            return launch_k(cand_select_kernel<NT, ITEMS, true>, dim3((unsigned)nq, (unsigned)S_out), dim3(NT),
                            stream, nullptr, ev1, q0, ik, itok, S_in, G, k, K1, ok, otok, out_idx, out_scores);
        return launch_k(cand_select_kernel<NT, ITEMS, false>, dim3((unsigned)nq, 1u), dim3(NT), stream, nullptr, ev1,
                        q0, ik, itok, S_in, G, k, K1, ok, otok, out_idx, out_scores);
    }
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
