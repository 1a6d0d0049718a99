// Device-side helpers shared by the libhisa kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hisa {

constexpr int kDim = 64;        // index-key dimension
constexpr int kThreads = 256;   // threads per workgroup of every kernel here
constexpr int kWaves = kThreads / 64;

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;   // one MFMA operand slice per lane
typedef __attribute__((ext_vector_type(4))) float f32x4_t;     // one 16x16 MFMA result slice per lane

// ---- bf16 ------------------------------------------------------------------

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ bf16x2_t as_bf16x2(uint32_t w) { return __builtin_bit_cast(bf16x2_t, w); }

// fp32 dot of two 64-element bf16 rows: the query as 32 packed words, the
// key row as eight 16-byte parts.  Each v_dot2 step adds two exact bf16
// products; four independent partial sums keep the rounding error of the
// 64-term sum small.
__device__ __forceinline__ float dot64_regs(const uint32_t (&q)[32], const uint4 (&v)[8])
{
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        acc[c & 3] = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(q[4 * c + 0]), as_bf16x2(v[c].x), acc[c & 3], false);
        acc[c & 3] = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(q[4 * c + 1]), as_bf16x2(v[c].y), acc[c & 3], false);
        acc[c & 3] = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(q[4 * c + 2]), as_bf16x2(v[c].z), acc[c & 3], false);
        acc[c & 3] = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(q[4 * c + 3]), as_bf16x2(v[c].w), acc[c & 3], false);
    }
    return (acc[0] + acc[1]) + (acc[2] + acc[3]);
}

// The same dot, loading the key row from memory.
__device__ __forceinline__ float dot64_packed(const uint32_t (&q)[32], const uint4* row)
{
    uint4 v[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) v[c] = row[c];
    return dot64_regs(q, v);
}

__device__ __forceinline__ void load_query(const uint16_t* q, uint32_t (&out)[32])
{
    const uint4* p = reinterpret_cast<const uint4*>(q);
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        uint4 v = p[c];
        out[4 * c + 0] = v.x;
        out[4 * c + 1] = v.y;
        out[4 * c + 2] = v.z;
        out[4 * c + 3] = v.w;
    }
}

// Round a double to bf16, nearest-even, from its bit fields.  Normal bf16
// results keep the top 8 significant bits of the 53; below 2^-126 the bf16
// spacing is 2^-133 and the scaled value is rounded to an integer.
__device__ __forceinline__ uint16_t f64_to_bf16_rne(double v)
{
    uint64_t u = (uint64_t)__double_as_longlong(v);
    uint16_t sign = (uint16_t)((u >> 48) & 0x8000u);
    uint64_t a = u & 0x7fffffffffffffffull;
    if (a > 0x7ff0000000000000ull) return 0x7fc0;            // NaN
    if (a == 0x7ff0000000000000ull) return sign | 0x7f80;    // inf
    int e = (int)(a >> 52) - 1023;
    if (e < -134) return sign;                               // below half the smallest step
    if (e < -126) {
        double n = __longlong_as_double((long long)a) * 0x1p133;   // exact scaling
        return sign | (uint16_t)__builtin_rint(n);
    }
    uint64_t mant = (a & 0x000fffffffffffffull) | 0x0010000000000000ull;
    uint32_t keep = (uint32_t)(mant >> 45);                   // 128 .. 255
    uint64_t rem = mant & ((1ull << 45) - 1);
    const uint64_t half = 1ull << 44;
    if (rem > half || (rem == half && (keep & 1u))) ++keep;
    if (keep == 256u) { keep = 128u; ++e; }
    if (e > 127) return sign | 0x7f80;
    return sign | (uint16_t)((e + 127) << 7) | (uint16_t)(keep & 0x7fu);
}

// ---- ranking keys ------------------------------------------------------------
// An order-preserving map of fp32 scores to u32; larger score, larger key.
// Key 0 marks "no candidate" and is never produced for a score.

__device__ __forceinline__ uint32_t score_key(float f)
{
    // negative: invert every bit; otherwise set the top bit.  Key 0 stays
    // free for "no candidate" (only the all-ones NaN would map to it).  -0
    // takes +0's key: the two compare equal, so they tie (lower index first)
    const uint32_t u0 = __float_as_uint(f);
    const uint32_t u = u0 == 0x80000000u ? 0u : u0;
    const uint32_t key = u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
    return max(key, 1u);
}

__device__ __forceinline__ float key_score(uint32_t key)
{
    // top bit set: a non-negative score, clear that bit; otherwise a
    // negative score, invert every bit
    const uint32_t t = (uint32_t)((int32_t)key >> 31);
    return __uint_as_float(key ^ 0x80000000u ^ (~t & 0x7fffffffu));
}

// ---- workgroup scans (256 threads) ------------------------------------------

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
__device__ __forceinline__ int wave_id() { return threadIdx.x >> 6; }

// Cross-lane steps through DPP (data-parallel primitives on the VALU):
// row_shr:n moves values n lanes up inside each row of 16 lanes; row_bcast
// 15 / 31 carry the last lane of a row into the following row(s).  Lanes
// with no source read 0.  Every lane of the wave must be active.
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROW_MASK, 0xf, true);
}

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ int wave_incl_scan(int v)
{
    uint32_t x = (uint32_t)v;
    x += dpp_u32<0x111>(x);          // row_shr:1
    x += dpp_u32<0x112>(x);          // row_shr:2
    x += dpp_u32<0x114>(x);          // row_shr:4
    x += dpp_u32<0x118>(x);          // row_shr:8
    x += dpp_u32<0x142, 0xa>(x);     // row_bcast:15 into rows 1 and 3
    x += dpp_u32<0x143, 0xc>(x);     // row_bcast:31 into rows 2 and 3
    return (int)x;
}

__device__ __forceinline__ int wave_sum(int v)
{
    return __builtin_amdgcn_readlane(wave_incl_scan(v), 63);
}

// Largest value over the wave (unsigned), the same ladder with max.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x)
{
    x = max(x, dpp_u32<0x111>(x));
    x = max(x, dpp_u32<0x112>(x));
    x = max(x, dpp_u32<0x114>(x));
    x = max(x, dpp_u32<0x118>(x));
    x = max(x, dpp_u32<0x142, 0xa>(x));
    x = max(x, dpp_u32<0x143, 0xc>(x));
    return (uint32_t)__builtin_amdgcn_readlane((int)x, 63);
}

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t x) { return ~wave_max_u32(~x); }

// Inclusive scan over the workgroup in thread order; scratch holds kWaves
// ints.  Contains barriers: every thread must call it.
__device__ __forceinline__ int block_incl_scan(int v, int* scratch)
{
    int s = wave_incl_scan(v);
    if (lane_id() == 63) scratch[wave_id()] = s;
    __syncthreads();
    int add = 0;
    for (int w = 0; w < wave_id(); ++w) add += scratch[w];
    __syncthreads();
    return s + add;
}

__device__ __forceinline__ int block_sum(int v, int* scratch)
{
    int s = wave_sum(v);
    if (lane_id() == 0) scratch[wave_id()] = s;
    __syncthreads();
    int tot = 0;
    for (int w = 0; w < kWaves; ++w) tot += scratch[w];
    __syncthreads();
    return tot;
}

// A raw buffer resource over `bytes` bytes from p (word 3 as CDNA
// expects for untyped dword access).  Loads through it take a vector
// offset and a scalar offset, so a wave's per-item addresses cost no
// vector instructions.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* p, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}

// How many lanes below this one have their bit set in b (v_mbcnt).
__device__ __forceinline__ int count_below(uint64_t b)
{
    return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(b >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)b, 0u));
}

// ---- query metadata ----------------------------------------------------------

struct QueryInfo {
    bool valid;
    int32_t seq;
    int64_t t;        // position in its sequence
    int64_t key_off;  // first key row of its sequence
    int64_t rep_off;  // first representative row of its sequence
};

__device__ __forceinline__ QueryInfo query_info(int64_t i, const int64_t* q_pos, const int32_t* q_seq,
                                                const int64_t* seq_key_off, const int64_t* seq_rep_off,
                                                const int64_t* seq_len, int32_t nseq, int64_t max_len)
{
    QueryInfo qi;
    qi.seq = q_seq ? q_seq[i] : 0;
    qi.t = q_pos[i];
    qi.valid = false;
    qi.key_off = 0;
    qi.rep_off = 0;
    if (qi.seq < 0 || qi.seq >= nseq) return qi;
    int64_t len = seq_len ? seq_len[qi.seq] : max_len;
    if (len > max_len || qi.t < 0 || qi.t >= len) return qi;
    qi.key_off = seq_key_off ? seq_key_off[qi.seq] : 0;
    qi.rep_off = seq_rep_off ? seq_rep_off[qi.seq] : 0;
    qi.valid = true;
    return qi;
}

}  // namespace hisa
