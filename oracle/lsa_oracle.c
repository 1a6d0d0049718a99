/*
 * lsa_oracle.c -- CPU oracle for LSA-Flat, the semantic-bucket indexer of
 * latent sparse attention, run on the same kind of index keys as HISA.
 *
 * TEST INFRASTRUCTURE ONLY, like hisa_oracle.c (same library): plain, slow,
 * fp64, written to be checked by eye against the page; shares nothing with
 * the HIP library.
 *
 * Source: [LSA] the latent sparse attention digest (seosoyoung), section
 * on how LSA works and Fig. 2 (Flat):
 *   step 1  every index key is L2-normalised (d = 64);
 *   step 2  four consecutive normalised keys are summed into one pool key;
 *   step 3  every 512 consecutive keys form a cluster block whose 128 pool
 *           keys start as buckets; mutually cheapest pairs of buckets (the
 *           pair whose merge grows the within-bucket sum of squared
 *           distances least, Ward's criterion) are merged in parallel,
 *           repeatedly, until the block has 64 buckets (8 keys on average);
 *           a merge that would give a bucket more than 16 keys is skipped;
 *   step 4  each bucket's centroid is its summed keys normalised; the
 *           centroid and the positions of the bucket's keys are cached;
 *   flat search: the query is scored against every centroid by inner
 *           product and the top p buckets are taken; footnote 3: bucket
 *           sizes vary, so keys are filled from the best bucket down and
 *           cut at exactly k.
 *
 * Readings where the page is silent:
 *   - fp64 throughout the build; a zero key stays zero when normalised;
 *   - Ward cost of buckets A, B with point sums S and point counts n (a
 *     point is a pool key): nA nB / (nA + nB) * |S_A/nA - S_B/nB|^2;
 *   - a bucket's cheapest partner is taken among the buckets it may merge
 *     with (at most 4 pool keys = 16 keys together); ties go to the lower
 *     bucket index.  A and B are a mutual pair when each is the other's
 *     cheapest partner.  When a round has more mutual pairs than merges
 *     left before 64 buckets, the cheapest pairs merge first (ties: lower
 *     first index), so a block always ends with exactly 64 buckets;
 *   - buckets are numbered within their block by their smallest pool key;
 *     a bucket's keys are listed in ascending position;
 *   - centroids are stored as bf16 (round to nearest even of the fp64
 *     normalised sum), as the page stores 64-dimensional bf16 vectors;
 *   - only complete cluster blocks are indexed; a query at t sees the
 *     blocks that end at or before t (floor((t + 1) / 512) of them);
 *   - scoring skips the query's normalisation: a positive scale does not
 *     change the ranking.  Scores are fp64 dot products of the bf16 values
 *     ranked on their fp32 rounding (the GPU's precision), ties to the
 *     lower global bucket id (block * 64 + local id);
 *   - fill: buckets in rank order, at most p of them, each bucket's keys in
 *     ascending position, until k keys; the row is those positions
 *     ascending, then -1.  Sinks and the sliding window that the page adds
 *     afterwards are a separate selection rule and are not part of it.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define LSA_BLOCK 512
#define LSA_POOL 4
#define LSA_POINTS (LSA_BLOCK / LSA_POOL) /* 128 pool keys per block */
#define LSA_BUCKETS 64
#define LSA_CAP 4                         /* pool keys per bucket: 16 keys */

uint16_t oracle_bf16_round(double v);     /* hisa_oracle.c */

static double bf16_val(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static double ward_cost(const double* SA, int nA, const double* SB, int nB, int d)
{
    double ss = 0.0;
    for (int c = 0; c < d; ++c) {
        const double diff = SA[c] / nA - SB[c] / nB;
        ss += diff * diff;
    }
    return (double)nA * nB / (nA + nB) * ss;
}

/* Agglomerate n points (rows of P, d dims) by rounds of mutual cheapest
 * pairs until `target` buckets remain, never joining more than `cap`
 * points.  label[i] gets the index of the bucket root point i belongs to
 * (its smallest point).  *margin (nullable) gets the smallest relative gap
 * between a decisive comparison's two sides.  If merges is not NULL, every
 * merge is appended as (root kept, root absorbed) pairs and *nmerges is set.
 * Returns the number of buckets left (target unless no admissible pair
 * remains). */
int oracle_lsa_ward(const double* P, int n, int d, int target, int cap, int32_t* label, double* margin,
                    int32_t* merges, int32_t* nmerges)
{
    double* S = (double*)malloc(sizeof(double) * (size_t)n * d);
    int* cnt = (int*)malloc(sizeof(int) * n);
    int* alive = (int*)malloc(sizeof(int) * n);
    int* best = (int*)malloc(sizeof(int) * n);
    double* bcost = (double*)malloc(sizeof(double) * n);
    int* pa = (int*)malloc(sizeof(int) * n);
    int* pb = (int*)malloc(sizeof(int) * n);
    double* pc = (double*)malloc(sizeof(double) * n);
    int32_t* parent = (int32_t*)malloc(sizeof(int32_t) * n);
    memcpy(S, P, sizeof(double) * (size_t)n * d);
    for (int i = 0; i < n; ++i) {
        cnt[i] = 1;
        alive[i] = 1;
        parent[i] = i;
    }
    double mg = INFINITY;
    int count = n, nm = 0;
    while (count > target) {
        /* every bucket's cheapest admissible partner */
        for (int a = 0; a < n; ++a) {
            best[a] = -1;
            if (!alive[a]) continue;
            double c1 = INFINITY, c2 = INFINITY;
            for (int b = 0; b < n; ++b) {
                if (b == a || !alive[b] || cnt[a] + cnt[b] > cap) continue;
                const double c = ward_cost(S + (size_t)a * d, cnt[a], S + (size_t)b * d, cnt[b], d);
                if (c < c1) {
                    c2 = c1;
                    c1 = c;
                    best[a] = b;
                } else if (c < c2) {
                    c2 = c;
                }
            }
            bcost[a] = c1;
            if (best[a] >= 0 && isfinite(c2)) {
                const double g = (c2 - c1) / (c1 > 0 ? c1 : 1.0);
                if (g < mg) mg = g;
            }
        }
        /* mutual pairs, cheapest first (insertion sort: few pairs) */
        int np = 0;
        for (int a = 0; a < n; ++a) {
            const int b = best[a];
            if (b > a && best[b] == a) {
                int j = np++;
                while (j > 0 && (pc[j - 1] > bcost[a] || (pc[j - 1] == bcost[a] && pa[j - 1] > a))) {
                    pa[j] = pa[j - 1];
                    pb[j] = pb[j - 1];
                    pc[j] = pc[j - 1];
                    --j;
                }
                pa[j] = a;
                pb[j] = b;
                pc[j] = bcost[a];
            }
        }
        if (np == 0) break;
        int take = np < count - target ? np : count - target;
        if (take < np) {
            const double g = (pc[take] - pc[take - 1]) / (pc[take - 1] > 0 ? pc[take - 1] : 1.0);
            if (g < mg) mg = g;
        }
        for (int i = 0; i < take; ++i) {
            const int a = pa[i], b = pb[i];
            for (int c = 0; c < d; ++c) S[(size_t)a * d + c] += S[(size_t)b * d + c];
            cnt[a] += cnt[b];
            alive[b] = 0;
            parent[b] = a;
            if (merges) {
                merges[2 * nm] = a;
                merges[2 * nm + 1] = b;
            }
            ++nm;
            --count;
        }
    }
    for (int i = 0; i < n; ++i) {
        int r = i;
        while (parent[r] != r) r = parent[r];
        label[i] = r;
    }
    if (margin) *margin = mg;
    if (nmerges) *nmerges = nm;
    free(S);
    free(cnt);
    free(alive);
    free(best);
    free(bcost);
    free(pa);
    free(pb);
    free(pc);
    free(parent);
    return count;
}

/* Build the buckets of one complete block of 512 keys (d dims, bf16):
 * centroids [64, d] bf16, members [128] pool-key indices grouped by bucket
 * (bucket order: smallest pool key; ascending inside a bucket), offs [65]
 * the start of each bucket in members.  *margin as in oracle_lsa_ward.
 * Returns 0, or -1 on bad arguments. */
int oracle_lsa_block(const uint16_t* keys, int d, uint16_t* centroids, uint8_t* members, uint8_t* offs,
                     double* margin)
{
    if (!keys || d <= 0 || !centroids || !members || !offs) return -1;
    double* P = (double*)calloc((size_t)LSA_POINTS * d, sizeof(double));
    for (int j = 0; j < LSA_BLOCK; ++j) {
        double nn = 0.0;
        for (int c = 0; c < d; ++c) nn += bf16_val(keys[(size_t)j * d + c]) * bf16_val(keys[(size_t)j * d + c]);
        const double norm = sqrt(nn);
        for (int c = 0; c < d; ++c)
            P[(size_t)(j / LSA_POOL) * d + c] += norm > 0 ? bf16_val(keys[(size_t)j * d + c]) / norm : 0.0;
    }
    int32_t label[LSA_POINTS];
    oracle_lsa_ward(P, LSA_POINTS, d, LSA_BUCKETS, LSA_CAP, label, margin, NULL, NULL);
    /* buckets in order of their smallest point (the root is that point) */
    int nb = 0, pos = 0;
    for (int r = 0; r < LSA_POINTS; ++r) {
        if (label[r] != r) continue;
        offs[nb] = (uint8_t)pos;
        double* s = (double*)calloc((size_t)d, sizeof(double));
        for (int i = 0; i < LSA_POINTS; ++i) {
            if (label[i] != r) continue;
            members[pos++] = (uint8_t)i;
            for (int c = 0; c < d; ++c) s[c] += P[(size_t)i * d + c];
        }
        double nn = 0.0;
        for (int c = 0; c < d; ++c) nn += s[c] * s[c];
        const double norm = sqrt(nn);
        for (int c = 0; c < d; ++c) centroids[(size_t)nb * d + c] = oracle_bf16_round(norm > 0 ? s[c] / norm : 0.0);
        free(s);
        ++nb;
    }
    offs[nb] = (uint8_t)pos;
    free(P);
    return nb == LSA_BUCKETS ? 0 : -1;
}

/* Every complete block of a sequence of L keys: centroids [nblk*64, d],
 * members [nblk*128], offs [nblk*65], margins [nblk] (nullable).  Returns
 * the number of blocks, or -1. */
int oracle_lsa_build(const uint16_t* keys, int64_t L, int d, uint16_t* centroids, uint8_t* members, uint8_t* offs,
                     double* margins)
{
    if (L < 0) return -1;
    const int64_t nblk = L / LSA_BLOCK;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int64_t b = 0; b < nblk; ++b) {
        double mg = 0.0;
        if (oracle_lsa_block(keys + (size_t)b * LSA_BLOCK * d, d, centroids + (size_t)b * LSA_BUCKETS * d,
                             members + (size_t)b * LSA_POINTS, offs + (size_t)b * (LSA_BUCKETS + 1), &mg) != 0)
            bad = 1;
        if (margins) margins[b] = mg;
    }
    return bad ? -1 : (int)nblk;
}

typedef struct {
    float key;
    int64_t id;
} lsa_cand;

static int lsa_cmp(const void* pa, const void* pb)
{
    const lsa_cand* a = (const lsa_cand*)pa;
    const lsa_cand* b = (const lsa_cand*)pb;
    if (a->key != b->key) return a->key > b->key ? -1 : 1;
    return a->id < b->id ? -1 : (a->id > b->id ? 1 : 0);
}

static int i32_cmp(const void* pa, const void* pb)
{
    const int32_t a = *(const int32_t*)pa, b = *(const int32_t*)pb;
    return a < b ? -1 : (a > b ? 1 : 0);
}

/* One flat-search query at position t over a sequence whose first nblk
 * complete blocks are built.  out_idx [k]: the filled positions ascending,
 * then -1; out_buckets [p] (nullable): the global ids of the buckets keys
 * were taken from, in rank order, then -1; out_scores [p] (nullable): their
 * fp64 scores.  Returns the number of keys, or -1. */
int oracle_lsa_query(const uint16_t* q, const uint16_t* centroids, const uint8_t* members, const uint8_t* offs,
                     int64_t nblk, int64_t t, int d, int p, int k, int32_t* out_idx, int32_t* out_buckets,
                     double* out_scores)
{
    if (t < 0 || p < 1 || k < 1 || nblk < 0) return -1;
    int64_t vis = (t + 1) / LSA_BLOCK;
    if (vis > nblk) vis = nblk;
    const int64_t nbk = vis * LSA_BUCKETS;
    lsa_cand* cand = (lsa_cand*)malloc(sizeof(lsa_cand) * (size_t)(nbk > 0 ? nbk : 1));
    double* sc = (double*)malloc(sizeof(double) * (size_t)(nbk > 0 ? nbk : 1));
    for (int64_t b = 0; b < nbk; ++b) {
        double s = 0.0;
        for (int c = 0; c < d; ++c) s += bf16_val(centroids[(size_t)b * d + c]) * bf16_val(q[c]);
        sc[b] = s;
        cand[b].key = (float)s;
        cand[b].id = b;
    }
    qsort(cand, (size_t)nbk, sizeof(lsa_cand), lsa_cmp);
    int n = 0, used = 0;
    for (int64_t r = 0; r < nbk && used < p && n < k; ++r) {
        const int64_t b = cand[r].id;
        const int64_t blk = b / LSA_BUCKETS, lb = b % LSA_BUCKETS;
        const uint8_t* off = offs + blk * (LSA_BUCKETS + 1);
        const uint8_t* mem = members + blk * LSA_POINTS;
        for (int i = off[lb]; i < off[lb + 1] && n < k; ++i)
            for (int r4 = 0; r4 < LSA_POOL && n < k; ++r4)
                out_idx[n++] = (int32_t)(blk * LSA_BLOCK + (int64_t)mem[i] * LSA_POOL + r4);
        if (out_buckets) out_buckets[used] = (int32_t)b;
        if (out_scores) out_scores[used] = sc[b];
        ++used;
    }
    qsort(out_idx, (size_t)n, sizeof(int32_t), i32_cmp);
    for (int i = n; i < k; ++i) out_idx[i] = -1;
    if (out_buckets)
        for (int i = used; i < p; ++i) out_buckets[i] = -1;
    if (out_scores)
        for (int i = used; i < p; ++i) out_scores[i] = NAN;
    free(cand);
    free(sc);
    return n;
}

/* A batch of queries over packed sequences: sequence s has its keys' built
 * blocks starting at block row seq_blk_off[s] (centroid rows * 64, member
 * rows * 128, offset rows * 65) and seq_nblk[s] built blocks and seq_len[s]
 * keys; a query whose sequence or position is out of range gets -1 rows.
 * Bucket ids in out_buckets are relative to the query's sequence. */
int oracle_lsa_batch(const uint16_t* queries, const int64_t* q_pos, const int32_t* q_seq, int64_t nq,
                     const uint16_t* centroids, const uint8_t* members, const uint8_t* offs,
                     const int64_t* seq_blk_off, const int64_t* seq_nblk, const int64_t* seq_len, int nseq, int d,
                     int p, int k, int32_t* out_idx, int32_t* out_buckets)
{
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 4) reduction(| : bad)
    for (int64_t i = 0; i < nq; ++i) {
        const int32_t s = q_seq ? q_seq[i] : 0;
        int32_t* oi = out_idx + i * k;
        int32_t* ob = out_buckets ? out_buckets + i * p : NULL;
        if (s < 0 || s >= nseq || q_pos[i] < 0 || q_pos[i] >= seq_len[s]) {
            for (int j = 0; j < k; ++j) oi[j] = -1;
            if (ob)
                for (int j = 0; j < p; ++j) ob[j] = -1;
            continue;
        }
        const int64_t bo = seq_blk_off[s];
        /* bucket ids come out relative to the sequence's first block */
        if (oracle_lsa_query(queries + i * d, centroids + (size_t)bo * LSA_BUCKETS * d,
                             members + (size_t)bo * LSA_POINTS, offs + (size_t)bo * (LSA_BUCKETS + 1), seq_nblk[s],
                             q_pos[i], d, p, k, oi, ob, NULL) < 0)
            bad = 1;
    }
    return bad ? -1 : 0;
}
