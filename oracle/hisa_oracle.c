/*
 * hisa_oracle.c -- CPU oracle for the HISA hierarchical indexer and for the
 * flat DSA indexer it replaces.
 *
 * TEST INFRASTRUCTURE ONLY.  This file defines what correct output is; it is
 * plain, slow and written to be checked by eye against the pages.  Only the
 * test suite, the smoke check and the bench's CPU-baseline leg may load it.
 * It shares no code, header, table or helper with the HIP library and it
 * includes nothing from it.
 *
 * Sources (cited by page title and passage):
 *   [HISA] "HISA: Efficient Hierarchical Indexing for Fine-Grained Sparse
 *          Attention" (aitrends.kr summary of the HISA paper):
 *          - structure paragraph: split the L keys into M contiguous blocks
 *            of size B; each block's representative is the sum of its
 *            indexing keys divided by their count (mean pooling);
 *          - stage-1 paragraph: inner product of the query with each block
 *            representative, causal mask, keep the top-m blocks, the first
 *            block and the last two blocks always kept;
 *          - stage-2 paragraph: the original DSA scoring applied only to the
 *            tokens of the m selected blocks, top-k token indices out;
 *          - maintenance paragraph: representatives are kept up to date
 *            incrementally when the KV cache grows;
 *          - kernel paragraph: no loss once m*B >= k.
 *   [VID]  "Why long-context LLMs slow down and how sparse attention fixes
 *          it" (idea.jsleekr.com, video summary), sections "DSA" and "HISA":
 *          DSA scores every key with a light dot product and keeps the top
 *          few; HISA uses 128-token blocks, about 1,000 block scores plus
 *          about 8,000 token scores at 128K.
 *
 * Readings taken where the pages are silent:
 *   - block representative: the sum is taken in fp64 (exact for the input
 *     class described below), divided by the count in fp64, and rounded to
 *     bf16 with round-to-nearest-even; a partial last block is averaged
 *     over the keys it holds;
 *   - block b is causal for a query at position t iff b*B <= t; key j is
 *     visible iff j <= t (a query sees its own key);
 *   - "last two blocks" are the last two causal blocks c = t/B and c-1;
 *     forced blocks count inside the m kept blocks; if c+1 <= m every
 *     causal block is kept;
 *   - the DSA token score is the plain dot product q . k_j (no scale);
 *   - scores are evaluated in fp64 and ranked on their fp32 rounding (the
 *     precision the GPU kernels decide in), ties going to the lower block
 *     or token index;
 *   - output: the selected token indices in ascending order followed by -1
 *     padding up to k; the selected blocks likewise, padded to m.
 *
 * Sparse attention over the selected tokens (the consumer of the indices):
 *   [HISA] stage-2 paragraph: the top-k token indices go to the sparse
 *   attention operator; [VID] "HISA" section: only the selected keys and
 *   values are gathered into smaller tensors and attention is computed on
 *   that set.  Readings: softmax attention of one head, weights
 *   softmax_j(scale * qa . ka_j) over the valid indices j of the row, output
 *   sum_j w_j v_j; an empty row (every index -1) gives a zero output; an
 *   index at or past its sequence's length counts as absent.
 *
 * Exactness precondition for pooling: every addition of the fp64 block sum
 * must be exact.  That holds when no nonzero |key| is below 2^-34 and the
 * block sums stay below 2^10 in magnitude; the synthetic generators flush
 * |x| < 2^-24 to zero.  oracle_pool reports any inexact addition (TwoSum
 * error term nonzero) through its flag so a test can refuse such inputs.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---- bf16 <-> double ---------------------------------------------------- */

/* A bf16 value is the upper half of an IEEE binary32 value; widening is
 * exact. */
static double bf16_value(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Round a double to the nearest bf16 value, ties to an even last mantissa
 * bit, written from the definition: find the two bf16 numbers that bracket
 * |v| on the bf16 grid (8 significant bits; quantum 2^-133 below 2^-126)
 * and pick the nearer one. */
static uint16_t bf16_round_nearest_even(double v)
{
    if (isnan(v)) return 0x7FC0;
    double a = fabs(v);
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    if (a == 0.0) return sign;
    if (isinf(a)) return sign | 0x7F80;

    int e;
    (void)frexp(a, &e);            /* a in [2^(e-1), 2^e) */
    int qexp = (e < -125 ? -125 : e) - 8;
    double q = ldexp(1.0, qexp);   /* spacing of bf16 numbers near a */
    double n_lo = floor(a / q);    /* a / q is exact (power-of-two scaling) */
    double lo = n_lo * q;
    double hi = lo + q;
    double r;
    double below = a - lo, above = hi - a;   /* both exact (Sterbenz) */
    if (below < above) r = lo;
    else if (above < below) r = hi;
    else r = (fmod(n_lo, 2.0) == 0.0) ? lo : hi;

    /* bf16 largest finite value is (2 - 2^-7) * 2^127; beyond it, inf */
    if (r > ldexp(255.0, 120)) return sign | 0x7F80;
    float f = (float)r;            /* exact: r is a bf16 number */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return sign | (uint16_t)(u >> 16);
}

/* fp32 rounding of a double (round to nearest even under the default
 * floating-point environment). */
static float to_f32(double x) { return (float)x; }

/* ---- pooling ([HISA] structure paragraph; maintenance paragraph) -------- */

/* Knuth's TwoSum: s = fl(a + b) and the exact rounding error of that sum. */
static double two_sum_err(double a, double b, double s)
{
    double bb = s - a;
    return (a - (s - bb)) + (b - bb);
}

/* Mean-pool blocks [b0, b1) of one sequence of L keys.  Returns 0, or -1
 * on bad arguments.  *inexact is set to 1 if any fp64 addition rounded. */
int oracle_pool_range(const uint16_t* keys, int64_t L, int d, int B,
                      int64_t b0, int64_t b1, uint16_t* reps, int* inexact)
{
    if (!keys || !reps || L < 0 || d <= 0 || B <= 0) return -1;
    int flag = 0;
    for (int64_t b = b0; b < b1; ++b) {
        int64_t start = b * (int64_t)B;
        int64_t count = L - start < B ? L - start : B;
        if (count <= 0) return -1;
        for (int c = 0; c < d; ++c) {
            double sum = 0.0;
            for (int64_t j = start; j < start + count; ++j) {
                double x = bf16_value(keys[j * d + c]);
                double s = sum + x;
                if (two_sum_err(sum, x, s) != 0.0) flag = 1;
                sum = s;
            }
            double mean = sum / (double)count;
            reps[b * d + c] = bf16_round_nearest_even(mean);
        }
    }
    if (inexact) *inexact = flag;
    return 0;
}

/* All M = ceil(L/B) blocks of one sequence. */
int oracle_pool(const uint16_t* keys, int64_t L, int d, int B,
                uint16_t* reps, int* inexact)
{
    if (B <= 0) return -1;
    int64_t M = (L + B - 1) / B;
    return oracle_pool_range(keys, L, d, B, 0, M, reps, inexact);
}

/* ---- scores ------------------------------------------------------------- */

/* The dot product of two d-vectors of bf16 values, accumulated in fp64 in
 * index order ([HISA] stage-1 inner product; [VID] DSA light dot product). */
static double dot_bf16(const uint16_t* a, const uint16_t* b, int d)
{
    double s = 0.0;
    for (int c = 0; c < d; ++c) s += bf16_value(a[c]) * bf16_value(b[c]);
    return s;
}

/* Block scores of one query against blocks [0, nblocks). */
int oracle_block_scores(const uint16_t* q, const uint16_t* reps,
                        int64_t nblocks, int d, double* out)
{
    if (!q || !reps || !out || d <= 0) return -1;
    for (int64_t b = 0; b < nblocks; ++b) out[b] = dot_bf16(q, reps + b * d, d);
    return 0;
}

/* ---- ranking -------------------------------------------------------------- */

typedef struct {
    float key;      /* fp32 rounding of the score: what ranking looks at */
    double score;   /* the fp64 score */
    int64_t id;     /* block or token index */
} cand_t;

/* Larger key first; equal keys: lower id first. */
static int cand_cmp(const void* pa, const void* pb)
{
    const cand_t* a = (const cand_t*)pa;
    const cand_t* b = (const cand_t*)pb;
    if (a->key > b->key) return -1;
    if (a->key < b->key) return 1;
    return (a->id < b->id) ? -1 : (a->id > b->id);
}

static int cand_cmp_id(const void* pa, const void* pb)
{
    const cand_t* a = (const cand_t*)pa;
    const cand_t* b = (const cand_t*)pb;
    return (a->id < b->id) ? -1 : (a->id > b->id);
}

static int i64_cmp(const void* pa, const void* pb)
{
    int64_t a = *(const int64_t*)pa, b = *(const int64_t*)pb;
    return (a < b) ? -1 : (a > b);
}

/* ---- stage 1: block selection ([HISA] stage-1 paragraph) ---------------- */

/* Select the blocks a query at position t keeps.  Writes up to m ascending
 * block ids to sel and returns how many.  Returns -1 on bad arguments. */
int oracle_select_blocks(const uint16_t* q, const uint16_t* reps, int64_t t,
                         int d, int B, int m, int64_t* sel,
                         int64_t* n_block_scores)
{
    if (t < 0 || m < 3 || B <= 0) return -1;
    int64_t c = t / B;                       /* the query's own block */
    if (n_block_scores) *n_block_scores = c + 1;
    if (c + 1 <= m) {                        /* every causal block fits */
        for (int64_t b = 0; b <= c; ++b) sel[b] = b;
        return (int)(c + 1);
    }
    /* c >= m >= 3: the forced blocks 0, c-1, c are distinct. */
    int64_t ncand = c - 2;                   /* blocks 1 .. c-2 */
    cand_t* cand = (cand_t*)malloc((size_t)ncand * sizeof(cand_t));
    if (!cand) return -1;
    for (int64_t b = 1; b <= c - 2; ++b) {
        double s = dot_bf16(q, reps + b * d, d);
        cand[b - 1].score = s;
        cand[b - 1].key = to_f32(s);
        cand[b - 1].id = b;
    }
    qsort(cand, (size_t)ncand, sizeof(cand_t), cand_cmp);
    int n = 0;
    sel[n++] = 0;
    for (int i = 0; i < m - 3; ++i) sel[n++] = cand[i].id;
    sel[n++] = c - 1;
    sel[n++] = c;
    free(cand);
    qsort(sel, (size_t)n, sizeof(int64_t), i64_cmp);
    return n;
}

/* ---- stage 2: token scoring and top-k ([HISA] stage-2 paragraph) -------- */

/* Top-k over the visible tokens (j <= t, j < L) of the given blocks. */
int oracle_tokens_on_blocks(const uint16_t* q, const uint16_t* keys, int64_t L,
                            int64_t t, int d, int B, const int64_t* blocks,
                            int nblocks, int k, int32_t* out_idx,
                            double* out_scores, int64_t* n_token_scores)
{
    if (k <= 0 || t < 0 || t >= L) return -1;
    int64_t cap = (int64_t)nblocks * B;
    cand_t* cand = (cand_t*)malloc((size_t)(cap > 0 ? cap : 1) * sizeof(cand_t));
    if (!cand) return -1;
    int64_t n = 0;
    for (int i = 0; i < nblocks; ++i) {
        int64_t b = blocks[i];
        for (int64_t j = b * B; j < (b + 1) * B; ++j) {
            if (j > t || j >= L) break;
            double s = dot_bf16(q, keys + j * d, d);
            cand[n].score = s;
            cand[n].key = to_f32(s);
            cand[n].id = j;
            ++n;
        }
    }
    if (n_token_scores) *n_token_scores = n;
    qsort(cand, (size_t)n, sizeof(cand_t), cand_cmp);
    int64_t take = n < k ? n : k;
    qsort(cand, (size_t)take, sizeof(cand_t), cand_cmp_id);
    for (int64_t i = 0; i < k; ++i) {
        out_idx[i] = i < take ? (int32_t)cand[i].id : -1;
        if (out_scores) out_scores[i] = i < take ? cand[i].score : NAN;
    }
    free(cand);
    return 0;
}

/* One HISA query: stage 1 then stage 2.  out_blocks (nullable) gets m
 * entries: the kept blocks ascending, then -1.  counts (nullable) gets the
 * number of block scores and token scores the query needed. */
int oracle_hisa_query(const uint16_t* q, const uint16_t* keys,
                      const uint16_t* reps, int64_t L, int64_t t, int d,
                      int B, int m, int k, int32_t* out_idx,
                      double* out_scores, int32_t* out_blocks, int64_t* counts)
{
    if (t < 0 || t >= L || m < 3 || k <= 0) return -1;
    int64_t* sel = (int64_t*)malloc((size_t)m * sizeof(int64_t));
    if (!sel) return -1;
    int64_t nb = 0, nt = 0;
    int ns = oracle_select_blocks(q, reps, t, d, B, m, sel, &nb);
    int rc = ns < 0 ? -1
                    : oracle_tokens_on_blocks(q, keys, L, t, d, B, sel, ns, k,
                                              out_idx, out_scores, &nt);
    if (rc == 0 && out_blocks)
        for (int i = 0; i < m; ++i) out_blocks[i] = i < ns ? (int32_t)sel[i] : -1;
    if (counts) { counts[0] = nb; counts[1] = nt; }
    free(sel);
    return rc;
}

/* One flat DSA query ([VID] DSA section): every visible key, then top-k. */
int oracle_flat_query(const uint16_t* q, const uint16_t* keys, int64_t L,
                      int64_t t, int d, int k, int32_t* out_idx,
                      double* out_scores, int64_t* counts)
{
    if (t < 0 || t >= L || k <= 0) return -1;
    /* the flat scan is stage 2 over one block that spans the whole prefix */
    int64_t whole = 0;
    int64_t nt = 0;
    int rc = oracle_tokens_on_blocks(q, keys, L, t, d, (int)(t + 1), &whole, 1,
                                     k, out_idx, out_scores, &nt);
    if (counts) { counts[0] = 0; counts[1] = nt; }
    return rc;
}

/* ---- block-only selection ---------------------------------------------- */

/* The variant HISA is contrasted with ([HISA] results paragraph: choosing
 * whole blocks without the token-level refinement loses accuracy at long
 * context).  Reading: stage 1 unchanged, then every visible token (j <= t)
 * of the kept blocks, ascending, followed by -1 up to m*B entries; no token
 * is scored. */
int oracle_block_only_query(const uint16_t* q, const uint16_t* reps, int64_t L, int64_t t, int d, int B, int m,
                            int32_t* out_idx, int32_t* out_blocks)
{
    if (t < 0 || t >= L || m < 3 || B <= 0) return -1;
    int64_t* sel = (int64_t*)malloc((size_t)m * sizeof(int64_t));
    if (!sel) return -1;
    const int ns = oracle_select_blocks(q, reps, t, d, B, m, sel, NULL);
    if (ns < 0) {
        free(sel);
        return -1;
    }
    int64_t n = 0;
    for (int i = 0; i < ns; ++i)
        for (int64_t j = sel[i] * B; j < (sel[i] + 1) * B; ++j)
            if (j <= t) out_idx[n++] = (int32_t)j;
    for (; n < (int64_t)m * B; ++n) out_idx[n] = -1;
    if (out_blocks)
        for (int i = 0; i < m; ++i) out_blocks[i] = i < ns ? (int32_t)sel[i] : -1;
    free(sel);
    return 0;
}

/* ---- batches over packed sequences -------------------------------------- */

static void fill_invalid(int32_t* idx, double* sc, int32_t* blk, int k, int m)
{
    for (int i = 0; i < k; ++i) {
        idx[i] = -1;
        if (sc) sc[i] = NAN;
    }
    if (blk) for (int i = 0; i < m; ++i) blk[i] = -1;
}

/* Queries of several sequences packed together.  Sequence s owns key rows
 * [seq_key_off[s], seq_key_off[s] + seq_len[s]) and block-representative
 * rows starting at seq_rep_off[s]; q_seq == NULL puts every query in
 * sequence 0.  A query whose sequence id or position is out of range gets a
 * row of -1.  mode 0 runs HISA, 1 the flat indexer (reps, B, m unused), 2
 * the block-only selection (k must be m*B; out_scores unused). */
int oracle_index_batch(int mode, const uint16_t* queries, const int64_t* q_pos,
                       const int32_t* q_seq, int64_t nq, const uint16_t* keys,
                       const uint16_t* reps, const int64_t* seq_key_off,
                       const int64_t* seq_rep_off, const int64_t* seq_len,
                       int nseq, int d, int B, int m, int k, int32_t* out_idx,
                       double* out_scores, int32_t* out_blocks)
{
    if (!queries || !q_pos || !keys || !seq_key_off || !seq_len || !out_idx)
        return -1;
    const int flat = mode == 1;
    if (mode < 0 || mode > 2) return -1;
    if (!flat && (!reps || !seq_rep_off)) return -1;
    if (mode == 2 && (int64_t)k != (int64_t)m * B) return -1;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 8) reduction(| : bad)
    for (int64_t i = 0; i < nq; ++i) {
        int32_t s = q_seq ? q_seq[i] : 0;
        int32_t* idx = out_idx + i * k;
        double* sc = (out_scores && mode != 2) ? out_scores + i * k : NULL;
        int32_t* blk = (out_blocks && !flat) ? out_blocks + i * m : NULL;
        if (s < 0 || s >= nseq || q_pos[i] < 0 || q_pos[i] >= seq_len[s]) {
            fill_invalid(idx, sc, blk, k, m);
            continue;
        }
        const uint16_t* q = queries + i * d;
        const uint16_t* K = keys + seq_key_off[s] * d;
        int rc;
        if (flat)
            rc = oracle_flat_query(q, K, seq_len[s], q_pos[i], d, k, idx, sc, NULL);
        else if (mode == 2)
            rc = oracle_block_only_query(q, reps + seq_rep_off[s] * d, seq_len[s], q_pos[i], d, B, m, idx, blk);
        else
            rc = oracle_hisa_query(q, K, reps + seq_rep_off[s] * d, seq_len[s],
                                   q_pos[i], d, B, m, k, idx, sc, blk, NULL);
        if (rc != 0) bad = 1;
    }
    return bad ? -1 : 0;
}

/* Sparse attention of one query row: qa [dh], ka / v [len, dh] (the
 * row's sequence), idx [kk].  fp64 throughout: s_j = scale * sum qa ka_j,
 * w_j = exp(s_j - max s), out = sum w_j v_j / sum w_j.  Returns the number
 * of indices used. */
int oracle_attention_row(const uint16_t* qa, const uint16_t* ka, const uint16_t* v, int64_t len, int dh,
                         const int32_t* idx, int kk, double scale, double* out)
{
    double smax = -INFINITY;
    int used = 0;
    double* s = (double*)malloc(sizeof(double) * (size_t)(kk > 0 ? kk : 1));
    for (int r = 0; r < kk; ++r) {
        const int64_t j = idx[r];
        s[r] = NAN;
        if (j < 0 || j >= len) continue;
        double dot = 0.0;
        for (int c = 0; c < dh; ++c) dot += bf16_value(qa[c]) * bf16_value(ka[j * dh + c]);
        s[r] = scale * dot;
        if (s[r] > smax) smax = s[r];
        ++used;
    }
    for (int c = 0; c < dh; ++c) out[c] = 0.0;
    if (used == 0) {
        free(s);
        return 0;
    }
    double wsum = 0.0;
    for (int r = 0; r < kk; ++r) {
        const int64_t j = idx[r];
        if (j < 0 || j >= len) continue;
        const double w = exp(s[r] - smax);
        wsum += w;
        for (int c = 0; c < dh; ++c) out[c] += w * bf16_value(v[j * dh + c]);
    }
    for (int c = 0; c < dh; ++c) out[c] /= wsum;
    free(s);
    return used;
}

/* A batch of rows: query i reads its sequence at key_off[i] with length
 * len[i] (len < 0: an invalid query, zero output). */
void oracle_attention_batch(const uint16_t* qa, const uint16_t* ka, const uint16_t* v, int64_t nq, int dh,
                            const int64_t* key_off, const int64_t* len, const int32_t* idx, int kk,
                            double scale, double* out)
{
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t i = 0; i < nq; ++i) {
        if (len[i] < 0) {
            for (int c = 0; c < dh; ++c) out[i * dh + c] = 0.0;
            continue;
        }
        oracle_attention_row(qa + i * dh, ka + key_off[i] * dh, v + key_off[i] * dh, len[i], dh, idx + i * kk,
                             kk, scale, out + i * dh);
    }
}

/* Threads an OpenMP parallel region will use. */
int oracle_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Threads later parallel regions of the calling thread use (n >= 1); the
 * timing harness sets 1 for its single-core figure.  Not arithmetic. */
void oracle_set_threads(int n)
{
#ifdef _OPENMP
    if (n >= 1) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* Exposed for the tests: the rounding rule used for representatives. */
uint16_t oracle_bf16_round(double v) { return bf16_round_nearest_even(v); }
