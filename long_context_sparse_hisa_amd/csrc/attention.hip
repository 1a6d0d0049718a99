// Sparse attention over an index call's output: gather the keys and values
// at each query's token indices and apply softmax attention over that set
// (HISA summary, stage-2 paragraph: the indices feed the sparse attention
// operator; video summary, "HISA" section: only the selected key and value
// rows are gathered and attended).  One head of dimension 128, bf16 inputs,
// fp32 arithmetic.
//
// Each query's indices are cut into chunks of kAttnChunk; a workgroup takes
// one chunk and leaves its partial softmax state (chunk maximum m, sum of
// exp(s - m), and the exp-weighted value sum), so even a few queries spread
// over the chip; a second kernel merges the states of each query.
// Sixteen lanes share a key or value row (16 bytes each), so every wave
// load is four whole 256-byte rows.
#include "../../include/hisa.h"

#include <hip/hip_runtime.h>
#include <math.h>

#include <algorithm>
#include <cmath>

#include "common.h"

namespace hisa {
namespace {

constexpr int kAttnDim = 128;
constexpr int kAttnChunk = 128;                       // indices per workgroup
constexpr int kAttnThreads = 256;
constexpr int kAttnLanesPerRow = 16;                  // 16 x 16 bytes = one row
constexpr int kAttnRowsPerPass = kAttnThreads / kAttnLanesPerRow;
constexpr int kAttnPasses = kAttnChunk / kAttnRowsPerPass;
constexpr int kAttnState = kAttnDim + 2;              // m, l, weighted value sum
constexpr int kAttnMaxChunks = (HISA_MAX_K + kAttnChunk - 1) / kAttnChunk;

static_assert(HISA_ATTN_DIM == kAttnDim, "head dimension");

// Sum over the 16 lanes of a DPP row as a butterfly: xor 1 and 2 inside
// quads, then the half-row mirror (quad 0 with quad 1) and the row mirror
// (half 0 with half 1).  At every step a lane and its partner add the same
// two values, so all 16 lanes end with the bit-identical total; a rotation
// would group the additions differently per lane, and lanes that each use
// their own copy of a score would then weight their columns differently.
__device__ __forceinline__ float row16_sum(float x)
{
    x += __uint_as_float(dpp_u32<0xb1>(__float_as_uint(x)));
    x += __uint_as_float(dpp_u32<0x4e>(__float_as_uint(x)));
    x += __uint_as_float(dpp_u32<0x141>(__float_as_uint(x)));
    x += __uint_as_float(dpp_u32<0x140>(__float_as_uint(x)));
    return x;
}

__device__ __forceinline__ float dot8(const uint4& a, const uint4& b)
{
    float acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(a.x), as_bf16x2(b.x), 0.f, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(a.y), as_bf16x2(b.y), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(a.z), as_bf16x2(b.z), acc, false);
    return __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(a.w), as_bf16x2(b.w), acc, false);
}

// Sum over the wave: the four DPP-row sums added by readlane.
__device__ __forceinline__ float wave_sum_f32(float x)
{
    x = row16_sum(x);
    return (__uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(x), 0)) +
            __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(x), 16))) +
           (__uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(x), 32)) +
            __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(x), 48)));
}

__device__ __forceinline__ float wave_max_f32(float x)
{
    // scores are ordered by their ranking keys, so the unsigned maximum of
    // the keys is the float maximum
    return key_score(wave_max_u32(score_key(x)));
}

// Merge the chunk states of one query: with M the largest chunk maximum,
// out = sum_g exp(m_g - M) acc_g / sum_g exp(m_g - M) l_g (zero when no
// chunk saw a valid index).  One round trip for everything: thread g loads
// (m_g, l_g), and every thread loads its column of the first chunks of its
// half of the workgroup (even or odd g) before the maximum is known.
__device__ __forceinline__ void attn_merge(const float* st, int G, float* out_row, float* s_f, float* s_half)
{
    constexpr int kPre = 8;
    const int t = threadIdx.x;
    const int c = t & (kAttnDim - 1);
    const int h = t / kAttnDim;
    const float m = t < G ? st[(int64_t)t * kAttnState] : -INFINITY;
    const float lg = t < G ? st[(int64_t)t * kAttnState + 1] : 0.f;
    float av[kPre];
#pragma unroll
    for (int i = 0; i < kPre; ++i) {
        const int g = h + 2 * i;
        av[i] = g < G ? st[(int64_t)g * kAttnState + 2 + c] : 0.f;
    }
    float M = wave_max_f32(m);
    __shared__ float s_m[kAttnThreads / 64];
    if (lane_id() == 0) s_m[wave_id()] = M;
    __syncthreads();
#pragma unroll
    for (int w = 0; w < kAttnThreads / 64; ++w) M = fmaxf(M, s_m[w]);
    if (t < G) {
        const float f = m > -INFINITY ? expf(m - M) : 0.f;
        s_f[t] = f;
        s_f[kAttnMaxChunks + t] = f * lg;
    }
    __syncthreads();
    float a = 0.f;
#pragma unroll
    for (int i = 0; i < kPre; ++i) {
        const int g = h + 2 * i;
        if (g < G) a += s_f[g] * av[i];
    }
    for (int g = h + 2 * kPre; g < G; g += 2) a += s_f[g] * st[(int64_t)g * kAttnState + 2 + c];
    if (h == 1) s_half[c] = a;
    __syncthreads();
    if (h == 0) {
        float l = 0.f;
        for (int g = 0; g < G; ++g) l += s_f[kAttnMaxChunks + g];
        a += s_half[c];
        out_row[c] = l > 0.f ? a / l : 0.f;
    }
}

// One chunk of kAttnChunk indices of one query (grid: queries x chunks).
// With a single chunk the workgroup writes the output itself; otherwise it
// stores its partial state for attn_combine_kernel.
__global__ __launch_bounds__(kAttnThreads) void attn_partial_kernel(const uint16_t* q, const uint16_t* k,
                                                                    const uint16_t* v, const int32_t* idx,
                                                                    const int32_t* q_seq, const int64_t* seq_key_off,
                                                                    const int64_t* seq_len, int nseq, int kk,
                                                                    float scale, float* state, float* out)
{
    __shared__ float s_red[2][kAttnThreads / 64];
    __shared__ float s_acc[kAttnRowsPerPass][kAttnDim];
    const int64_t row = blockIdx.x;
    const int g = blockIdx.y;
    const int G = gridDim.y;
    const int sub = threadIdx.x & (kAttnLanesPerRow - 1);     // which 16 bytes (8 dims) of a row
    const int grp = threadIdx.x / kAttnLanesPerRow;           // which row of a pass
    const int s = q_seq ? q_seq[row] : 0;
    const bool qvalid = s >= 0 && s < nseq;
    const int64_t koff = qvalid && seq_key_off ? seq_key_off[s] : 0;
    const int64_t len = qvalid ? seq_len[s] : 0;
    const uint4 qv = reinterpret_cast<const uint4*>(q + row * kAttnDim)[sub];
    const int32_t* irow = idx + row * (int64_t)kk;
    // two round trips: every pass's index, then every pass's key and value
    // parts (lanes of an absent index load nothing and hold zeros)
    int32_t jj[kAttnPasses];
#pragma unroll
    for (int p = 0; p < kAttnPasses; ++p) jj[p] = irow[min(g * kAttnChunk + p * kAttnRowsPerPass + grp, kk - 1)];
    bool ok[kAttnPasses];
    uint4 kv[kAttnPasses], vv[kAttnPasses];
#pragma unroll
    for (int p = 0; p < kAttnPasses; ++p) {
        const int r = g * kAttnChunk + p * kAttnRowsPerPass + grp;
        ok[p] = r < kk && jj[p] >= 0 && jj[p] < len;
        kv[p] = make_uint4(0u, 0u, 0u, 0u);
        vv[p] = kv[p];
        if (ok[p]) {
            const int64_t rowk = koff + jj[p];
            kv[p] = reinterpret_cast<const uint4*>(k + rowk * kAttnDim)[sub];
            vv[p] = reinterpret_cast<const uint4*>(v + rowk * kAttnDim)[sub];
        }
    }
    // scores and the chunk maximum
    float sc[kAttnPasses];
    float mx = -INFINITY;
#pragma unroll
    for (int p = 0; p < kAttnPasses; ++p) {
        sc[p] = scale * row16_sum(dot8(qv, kv[p]));
        if (ok[p]) mx = fmaxf(mx, sc[p]);
    }
    mx = wave_max_f32(mx);
    if (lane_id() == 0) s_red[0][wave_id()] = mx;
    __syncthreads();
#pragma unroll
    for (int w = 0; w < kAttnThreads / 64; ++w) mx = fmaxf(mx, s_red[0][w]);
    // weights, their sum (one lane per row counts it) and the weighted values
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    float lsum = 0.f;
#pragma unroll
    for (int p = 0; p < kAttnPasses; ++p) {
        const float w = ok[p] ? expf(sc[p] - mx) : 0.f;
        lsum += sub == 0 ? w : 0.f;
        acc[0] += w * bf16_lo(vv[p].x);
        acc[1] += w * bf16_hi(vv[p].x);
        acc[2] += w * bf16_lo(vv[p].y);
        acc[3] += w * bf16_hi(vv[p].y);
        acc[4] += w * bf16_lo(vv[p].z);
        acc[5] += w * bf16_hi(vv[p].z);
        acc[6] += w * bf16_lo(vv[p].w);
        acc[7] += w * bf16_hi(vv[p].w);
    }
    lsum = wave_sum_f32(lsum);
    if (lane_id() == 0) s_red[1][wave_id()] = lsum;
#pragma unroll
    for (int e = 0; e < 8; ++e) s_acc[grp][sub * 8 + e] = acc[e];
    __syncthreads();
    float l = 0.f;
#pragma unroll
    for (int w = 0; w < kAttnThreads / 64; ++w) l += s_red[1][w];
    float a = 0.f;
    if (threadIdx.x < kAttnDim) {
#pragma unroll
        for (int r = 0; r < kAttnRowsPerPass; ++r) a += s_acc[r][threadIdx.x];
    }
    if (G == 1) {
        if (threadIdx.x < kAttnDim) out[row * kAttnDim + threadIdx.x] = l > 0.f ? a / l : 0.f;
        return;
    }
    float* st = state + (row * G + g) * kAttnState;
    if (threadIdx.x < kAttnDim) st[2 + threadIdx.x] = a;
    if (threadIdx.x == 0) {
        st[0] = mx;
        st[1] = l;
    }
}

// The chunk states of one query merged (grid: queries).  A separate launch:
// the kernel boundary makes every chunk's stores visible, which a counter
// in the partial kernel could only do with a device-scope fence per chunk
// (a write-back of its die's L2), measured slower than the second launch.
__global__ __launch_bounds__(kAttnThreads) void attn_combine_kernel(const float* state, int G, float* out)
{
    __shared__ float s_f[2 * kAttnMaxChunks];
    __shared__ float s_half[kAttnDim];
    static_assert(kAttnMaxChunks <= kAttnThreads, "one merging thread per chunk");
    attn_merge(state + (int64_t)blockIdx.x * G * kAttnState, G, out + (int64_t)blockIdx.x * kAttnDim, s_f, s_half);
}

// Workspace: the chunk states, G = ceil(kk / kAttnChunk) per query.
size_t state_bytes(int64_t nq, int kk)
{
    const int64_t G = (kk + kAttnChunk - 1) / kAttnChunk;
    return (size_t)std::max<int64_t>(nq, 1) * G * kAttnState * sizeof(float);
}

int validate_attn(const hisa_attn_args* a)
{
    if (!a) return HISA_ERR_INVALID_ARG;
    if (a->nq < 0 || a->nseq < 1 || a->kk < 1) return HISA_ERR_INVALID_ARG;
    if (a->nseq > 1 && !a->seq_key_off) return HISA_ERR_INVALID_ARG;
    if (a->dh != HISA_ATTN_DIM || a->kk > HISA_MAX_K) return HISA_ERR_UNSUPPORTED;
    if (!std::isfinite(a->scale)) return HISA_ERR_INVALID_ARG;
    if (a->nq > 0 && (!a->q || !a->k || !a->v || !a->idx || !a->seq_len || !a->out)) return HISA_ERR_INVALID_ARG;
    return HISA_OK;
}

}  // namespace
}  // namespace hisa

extern "C" {

int hisa_attention_workspace_bytes(const hisa_attn_args* a, size_t* bytes)
{
    if (!bytes) return HISA_ERR_INVALID_ARG;
    const int rc = hisa::validate_attn(a);
    if (rc != HISA_OK) return rc;
    *bytes = hisa::state_bytes(a->nq, a->kk);
    return HISA_OK;
}

int hisa_sparse_attention(const hisa_attn_args* a, void* stream_)
{
    using namespace hisa;
    const int rc = validate_attn(a);
    if (rc != HISA_OK) return rc;
    if (a->nq == 0) return HISA_OK;
    if (!a->workspace || a->workspace_bytes < state_bytes(a->nq, a->kk)) return HISA_ERR_WORKSPACE;
    if (a->nq > INT32_MAX) return HISA_ERR_UNSUPPORTED;
    hipStream_t stream = static_cast<hipStream_t>(stream_);
    const int G = (a->kk + kAttnChunk - 1) / kAttnChunk;
    float* state = static_cast<float*>(a->workspace);
    hipLaunchKernelGGL(attn_partial_kernel, dim3((unsigned)a->nq, (unsigned)G), dim3(kAttnThreads), 0, stream, a->q,
                       a->k, a->v, a->idx, a->q_seq, a->seq_key_off, a->seq_len, (int)a->nseq, (int)a->kk, a->scale,
                       state, a->out);
    if (hipGetLastError() != hipSuccess) return HISA_ERR_HIP;
    if (G > 1) {
        hipLaunchKernelGGL(attn_combine_kernel, dim3((unsigned)a->nq), dim3(kAttnThreads), 0, stream,
                           static_cast<const float*>(state), G, a->out);
        if (hipGetLastError() != hipSuccess) return HISA_ERR_HIP;
    }
    return HISA_OK;
}

}  // extern "C"
