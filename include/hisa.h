/*
 * hisa.h -- C ABI of libhisa, the MI355X (gfx950) HISA hierarchical indexer
 * and flat DSA indexer.
 *
 * What is computed (pages cited by title and passage):
 *   "HISA: Efficient Hierarchical Indexing for Fine-Grained Sparse
 *   Attention" (aitrends.kr summary of the HISA paper):
 *     structure paragraph   -- the L index keys of a sequence are split into
 *                              contiguous blocks of B; a block's
 *                              representative is the mean of its keys;
 *     stage-1 paragraph     -- each query scores the representatives by
 *                              inner product under a causal mask and keeps
 *                              the top m blocks, always including the first
 *                              block and the last two;
 *     stage-2 paragraph     -- the token-level score is applied only to the
 *                              m*B tokens of the kept blocks and the top k
 *                              token indices are returned for the sparse
 *                              attention operator;
 *     maintenance paragraph -- representatives are updated incrementally
 *                              when keys are appended to the cache; the
 *                              output layout is the flat indexer's;
 *     kernel paragraph      -- no loss once m*B >= k.
 *   "Why long-context LLMs slow down and how sparse attention fixes it"
 *   (idea.jsleekr.com), section "DSA": the flat indexer scores every key
 *   with a light dot product and keeps the best few.
 *
 * Conventions shared by every call
 *   - bf16 values are passed as their 16-bit patterns (uint16_t).
 *   - d (index-key dimension) must be 64.
 *   - Every array pointer is a DEVICE pointer owned by the caller, unless a
 *     parameter says "host".  The library allocates nothing and keeps no
 *     mutable global state; calls on different streams are independent.
 *   - `stream` is a hipStream_t (NULL = the null stream).  Every call only
 *     enqueues work and returns; the library never synchronises.  A device
 *     fault shows up at the caller's next synchronisation.
 *   - Return value: HISA_OK or a negative HISA_ERR_* code.  Arguments are
 *     validated on the host before anything is enqueued; on error nothing
 *     is written.  HISA_ERR_HIP means a launch was rejected by the runtime
 *     (earlier launches of the same call may have run).
 *
 * Representatives (the readings taken where the pages are silent):
 *   R_b = RNE_bf16( fp64( S_b / n_b ) ), S_b the fp64 sum of the n_b keys
 *   of block b (n_b = B except for a partial last block), added exactly
 *   whenever every nonzero |key| >= 2^-34 and |S_b| < 2^10, so that the
 *   result is independent of summation order.
 *
 * Selection (readings): key j is visible to a query at position t iff
 *   j <= t; block b is causal iff b*B <= t; with c = t / B the forced blocks
 *   are 0, c-1 and c, counted among the m kept blocks; if c+1 <= m every
 *   causal block is kept.  Scores are fp32 sums of exact bf16 products.
 *   Ties at the m-th block / k-th token go to the lower block / token index
 *   (scores compare as fp32 values, so -0.0 ties with +0.0).
 *
 * Output layout (identical for HISA and flat):
 *   out_idx[i*k + r]: the selected token indices of query i, relative to the
 *   start of its sequence, in ascending order, then -1 up to k.  A row holds
 *   min(k, number of candidate tokens) valid entries.
 *   out_scores[i*k + r] (optional): the fp32 score of out_idx[i*k + r]
 *   (NaN where out_idx is -1).
 *   out_blocks[i*m + r] (optional, HISA only): the kept block ids of query
 *   i in ascending order, then -1 up to m.
 *   A query whose sequence id is outside [0, nseq) or whose position is
 *   outside [0, seq_len) gets an all -1 row (NaN scores); that is not an
 *   error the host can see, since positions live on the device.
 */
#ifndef HISA_H
#define HISA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define HISA_ABI_VERSION 1

enum {
    HISA_OK = 0,
    HISA_ERR_INVALID_ARG = -1,  /* null required pointer, bad size, m < 3, m*B < k, ... */
    HISA_ERR_UNSUPPORTED = -2,  /* d != 64, B not a power of two in [16, 256], limits */
    HISA_ERR_WORKSPACE = -3,    /* workspace smaller than one query needs */
    HISA_ERR_HIP = -4           /* the HIP runtime rejected a launch */
};

/* Largest k and largest m*B the index calls accept. */
#define HISA_MAX_K 16384
#define HISA_MAX_CANDIDATES 16384
/* Largest sequence length (token indices are int32). */
#define HISA_MAX_LEN ((int64_t)1 << 30)

/* Host-side description of one sequence in a packed key cache, for the
 * append call.  key rows [key_off, key_off + capacity) belong to the
 * sequence, of which the first `len` are filled; its representatives occupy
 * rows [rep_off, rep_off + ceil(capacity / B)). */
typedef struct hisa_seq {
    int64_t key_off;
    int64_t rep_off;
    int64_t len;
    int64_t capacity;
} hisa_seq;

/*
 * hisa_pool_blocks -- mean-pool one sequence's keys into representatives
 * (structure paragraph of the HISA summary).
 *   keys  [L, d] bf16, read.
 *   reps  [ceil(L / B), d] bf16, written.
 *   L >= 0 (0 is a no-op), d == 64, B a power of two in [16, 256].
 * Errors: INVALID_ARG (null pointer with L > 0, L < 0 or L > HISA_MAX_LEN),
 *         UNSUPPORTED (d, B).
 */
int hisa_pool_blocks(const uint16_t* keys, int64_t L, int d, int B, uint16_t* reps,
                     void* stream);

/*
 * hisa_append_keys -- append n_new keys to each of nseq sequences and bring
 * the representatives of every block the new keys touch up to date
 * (maintenance paragraph of the HISA summary).  The result equals pooling
 * the grown sequences from scratch, bit for bit.
 *   keys      packed key cache, rows written at [key_off + len, + n_new).
 *   reps      packed representatives, rows of the touched blocks written.
 *   seqs      HOST array of nseq descriptors (len = length before the call;
 *             the library does not update it).
 *   new_keys  [nseq, n_new, d] bf16, read.
 *   n_new >= 0 (0 is a no-op), nseq >= 0.
 * Errors: INVALID_ARG (null pointer, negative sizes, len + n_new > capacity,
 *         capacity > HISA_MAX_LEN), UNSUPPORTED (d, B).
 */
int hisa_append_keys(uint16_t* keys, uint16_t* reps, const hisa_seq* seqs, int nseq,
                     const uint16_t* new_keys, int64_t n_new, int d, int B, void* stream);

/* Arguments of the two index calls. */
typedef struct hisa_index_args {
    const uint16_t* queries;     /* [nq, d] bf16 index queries */
    const int64_t* q_pos;        /* [nq] position of each query in its sequence */
    const int32_t* q_seq;        /* [nq] sequence id of each query; NULL: all in sequence 0 */
    int64_t nq;                  /* number of queries, >= 0 (0 is a no-op) */
    const uint16_t* keys;        /* packed keys, [*, d] bf16 */
    const uint16_t* reps;        /* packed representatives, [*, d] bf16 (HISA only) */
    const int64_t* seq_key_off;  /* [nseq] first key row of each sequence; NULL if nseq == 1: 0 */
    const int64_t* seq_rep_off;  /* [nseq] first rep row of each sequence; NULL if nseq == 1: 0 */
    const int64_t* seq_len;      /* [nseq] keys in each sequence; NULL if nseq == 1: max_len */
    int32_t nseq;                /* >= 1 */
    int64_t max_len;             /* HOST bound: every seq_len <= max_len <= HISA_MAX_LEN;
                                    HISA also ceil(max_len / B) <= HISA_MAX_CANDIDATES
                                    blocks (2M keys at B = 128, 256K at B = 16) */
    int32_t d;                   /* 64 */
    int32_t B;                   /* block size (HISA), power of two in [16, 256] */
    int32_t m;                   /* kept blocks (HISA), 3 <= m, m*B <= HISA_MAX_CANDIDATES */
    int32_t k;                   /* tokens returned, 1 <= k <= HISA_MAX_K; HISA: k <= m*B */
    int32_t* out_idx;            /* [nq, k] */
    float* out_scores;           /* [nq, k] or NULL */
    int32_t* out_blocks;         /* [nq, m] or NULL (HISA only) */
    void* workspace;             /* device scratch owned by the caller, 16-byte aligned
                                    (HISA_ERR_INVALID_ARG otherwise: the kernels move it
                                    as 16-byte vectors) */
    size_t workspace_bytes;      /* its size; see hisa_workspace_bytes */
    void* const* stage_events;   /* NULL, or 2 * HISA_STAGES hipEvent_t handles (profiling aid,
                                    created with timing enabled).  Events 2s and 2s+1 record
                                    when the first kernel of stage s starts and its last kernel
                                    ends, for the call's last query chunk, from the dispatch
                                    itself.  HISA stages: 0 block scores and top-m; 1 token
                                    scores; 2 token top-k.  With fewer than 512 queries and
                                    at most 2048 blocks, stages 0 and 1 are one kernel,
                                    recorded as stage 1 (0 not recorded).  Flat stages:
                                    0 scores, 1 top-k (2 not recorded). */
} hisa_index_args;

#define HISA_STAGES 3


/*
 * hisa_workspace_bytes -- workspace an index call wants for these
 * arguments (flat != 0: the flat indexer).  Only the sizes in `a` are
 * read.  Any workspace of at least the one-query size is accepted: the call
 * then works through the queries in as many chunks as it needs.
 *   *bytes          the recommended size: the largest chunk that fits in
 *                   1 GiB (all queries if they fit);
 *   *min_bytes      (nullable) the one-query size;
 *   *all_bytes      (nullable) the size that takes every query in one chunk.
 */
int hisa_workspace_bytes(const hisa_index_args* a, int flat, size_t* bytes, size_t* min_bytes,
                         size_t* all_bytes);

/*
 * hisa_index -- HISA: block scores, causal + forced top-m, token scores in
 * the kept blocks, top-k (stage-1 and stage-2 paragraphs of the HISA
 * summary).
 * Errors: INVALID_ARG (null required pointer, nq < 0, nseq < 1, m < 3,
 *         k < 1, m*B < k, max_len < 1), UNSUPPORTED (d, B, k, m*B,
 *         max_len or its block count beyond the limits above), WORKSPACE.
 */
int hisa_index(const hisa_index_args* a, void* stream);

/*
 * hisa_index_static -- hisa_index for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation): the same results, with the library's own device
 * scratch in place of a caller workspace.  a->workspace and
 * a->workspace_bytes are ignored; nothing is allocated.
 *   The scratch is a static device array of HISA_STATIC_SCRATCH_BYTES per
 *   GPU, held from the first call on that GPU until the process ends.  Its
 *   contents need not start at any value.  Every call on one GPU uses the
 *   same array, so calls that may overlap on one GPU (different streams,
 *   threads or processes' shared contexts) race: serialise them.  Queries
 *   that do not fit at once run in chunks, in order, on `stream`.
 *   The stream must belong to the current device.
 * Errors: those of hisa_index, HISA_ERR_WORKSPACE when one query's scratch
 *         would exceed HISA_STATIC_SCRATCH_BYTES (not reachable within the
 *         limits above), HISA_ERR_HIP when the scratch cannot be located.
 */
#define HISA_STATIC_SCRATCH_BYTES ((size_t)64 << 20)
int hisa_index_static(const hisa_index_args* a, void* stream);

/*
 * hisa_flat_index -- the flat DSA indexer: every visible key scored, top-k
 * ("DSA" section of the video summary).  B, m, reps and out_blocks are
 * ignored.  Same errors as hisa_index, less those about B and m.
 */
int hisa_flat_index(const hisa_index_args* a, void* stream);

/*
 * hisa_decode_step -- hisa_append_keys(keys, reps, seqs, nseq, new_keys,
 * n_new, d, B) followed by hisa_index(a): the same outputs, keys and
 * representatives, in fewer launches.  The append writes a->keys and
 * a->reps (the const of hisa_index_args does not hold for this call).
 * seqs[s] describes sequence s of `a` (the same key and representative
 * offsets) with its length BEFORE the append; a->seq_len holds the lengths
 * AFTER it.  With fewer than 512 queries, n_new <= B, at most 64
 * sequences and a workspace that holds every query, the append runs inside
 * the index's first launch: with at most 2048 blocks the launch that
 * selects the blocks and scores the tokens (which reads the new keys from
 * new_keys; stage event 1 covers it, 2 the top-k), with more the
 * block-score launch (stage events 0, 1, 2 as in hisa_index).  Either way
 * the blocks the append re-pools are the queries' forced last two, whose
 * representatives stage 1 never scores.  Otherwise the two calls run one
 * after the other.  The append is folded in only when the lengths the
 * queries see are known to be the appended ones: a->seq_len is given, or
 * (one sequence, seq_len NULL) max_len == seqs[0].len + n_new.  A device
 * length larger than len + n_new breaks that precondition: in the folded
 * launch a query at or past len + n_new of its sequence then gets a -1 row
 * (where the two calls would index it).
 * Errors: those of hisa_index and hisa_append_keys; INVALID_ARG also when
 *         an appended length exceeds max_len.
 */
int hisa_decode_step(const hisa_index_args* a, const hisa_seq* seqs, const uint16_t* new_keys, int64_t n_new,
                     void* stream);

/*
 * hisa_block_index -- block-only selection, the variant the HISA summary's
 * results paragraph contrasts with HISA (whole blocks chosen without the
 * token-level refinement): stage 1 exactly as in hisa_index, then each
 * out_idx row holds every visible token (j <= t) of the kept blocks in
 * ascending order, followed by -1.  No token is scored.  The row width
 * must be the whole candidate set: k == m*B.  out_blocks as in hisa_index;
 * out_scores must be NULL.  Workspace: what hisa_workspace_bytes reports
 * for hisa_index (flat = 0).  Stage events 0 (stage 1) and 1 (the
 * expansion).
 * Errors: those of hisa_index, and INVALID_ARG for k != m*B or a non-NULL
 *         out_scores.
 */
int hisa_block_index(const hisa_index_args* a, void* stream);

/*
 * Sparse attention over an index call's output -- the operator the indices
 * are for: [HISA] stage-2 paragraph (the top-k indices go to the sparse
 * attention operator) and the video summary's "HISA" section (gather only
 * the selected keys and values, attend over that small set).
 * Per query i with valid indices J (entries of idx row i that are >= 0 and
 * below its sequence's length):
 *     w_j = softmax over J of  scale * (q_i . ka_j),   out_i = sum_j w_j v_j,
 * one head, fp32 arithmetic on bf16 inputs; a row with no valid index (or a
 * query whose sequence id is outside [0, nseq)) gets a zero output.
 */
#define HISA_ATTN_DIM 128

typedef struct hisa_attn_args {
    const uint16_t* q;           /* [nq, 128] bf16 attention queries */
    const uint16_t* k;           /* [rows, 128] bf16 attention keys, packed per sequence like the index keys */
    const uint16_t* v;           /* [rows, 128] bf16 values, the same rows */
    const int32_t* idx;          /* [nq, kk] token indices relative to the sequence start, -1 = none
                                    (out_idx of hisa_index / hisa_flat_index) */
    const int32_t* q_seq;        /* [nq] sequence of each query, or NULL: sequence 0 */
    const int64_t* seq_key_off;  /* [nseq] first row of each sequence, or NULL if nseq == 1: 0 */
    const int64_t* seq_len;      /* [nseq] rows of each sequence (required) */
    int32_t nseq;
    int64_t nq;
    int32_t kk;                  /* indices per query, 1 <= kk <= HISA_MAX_K */
    int32_t dh;                  /* head dimension, must be HISA_ATTN_DIM */
    float scale;                 /* softmax scale, e.g. 1/sqrt(128) */
    float* out;                  /* [nq, 128] fp32 */
    void* workspace;             /* device scratch owned by the caller */
    size_t workspace_bytes;      /* at least hisa_attention_workspace_bytes */
} hisa_attn_args;

/* Workspace hisa_sparse_attention needs for these sizes (nq, kk): the
 * per-chunk partial softmax states (nq * ceil(kk / 128) * 130 floats).  No
 * initial contents are required; calls that share a workspace must not
 * overlap. */
int hisa_attention_workspace_bytes(const hisa_attn_args* a, size_t* bytes);

/*
 * hisa_sparse_attention -- gather the keys and values at each query's
 * indices, softmax attention over them.  Every query's indices are split
 * into chunks of 128 handled by separate workgroups (partial max, sum and
 * weighted value sum), then a second kernel merges each query's chunks
 * (one launch when kk <= 128).  Both on `stream`.
 * Errors: INVALID_ARG (null q, k, v, idx, seq_len or out with nq > 0;
 *         nq < 0; nseq < 1; nseq > 1 without seq_key_off; kk < 1;
 *         non-finite scale), UNSUPPORTED
 *         (dh != 128, kk > HISA_MAX_K), WORKSPACE.
 */
int hisa_sparse_attention(const hisa_attn_args* a, void* stream);

/*
 * LSA-Flat: semantic buckets instead of positional blocks, the indexer of
 * the latent sparse attention digest (section on how LSA works, steps 1-4
 * and Fig. 2, Flat search; footnote 3 for the fill to exactly k), on the
 * same d = 64 bf16 index keys.
 *
 * Cache of one sequence, per complete block of HISA_LSA_BLOCK keys
 * (block b covers keys 512 b .. 512 b + 511):
 *   centroids [nblk * 64, 64] bf16   unit centroid of each bucket
 *   members   [nblk, 128] uint8      the block's pool keys (pool key i =
 *                                    keys 4i .. 4i+3) grouped by bucket,
 *                                    ascending inside a bucket
 *   offs      [nblk, 65] uint8       bucket j holds members[offs[j] ..
 *                                    offs[j+1]); 1 to 4 pool keys each
 * Buckets are numbered by their smallest pool key.  Several sequences pack
 * their block rows back to back (seq_blk_off below).
 */
#define HISA_LSA_BLOCK 512
#define HISA_LSA_BUCKETS 64
#define HISA_LSA_POOL_KEYS 128
#define HISA_LSA_MAX_P 2048
#define HISA_LSA_MAX_LEN (1LL << 20)

/*
 * hisa_lsa_build -- buckets of blocks first_block .. len/512 - 1 of one
 * sequence: keys [len, 64] bf16 (16-byte aligned) are L2-normalised, summed
 * four at a time into 128 pool keys per block, and merged by rounds of
 * mutually cheapest pairs under Ward's criterion (fp64), at most 16 keys
 * per bucket, down to 64 buckets; the cheapest pairs merge first when a
 * round offers more than are needed.  centroids, members and offs point at
 * the sequence's block row 0.  A block whose keys hold non-finite values
 * gets 64 empty buckets.  One workgroup per block.
 * Errors: INVALID_ARG (null pointer with blocks to build, len < 0,
 *         first_block < 0), UNSUPPORTED (d != 64, len > HISA_LSA_MAX_LEN,
 *         misaligned keys).
 */
int hisa_lsa_build(const uint16_t* keys, int64_t len, int64_t first_block, int d, uint16_t* centroids,
                   uint8_t* members, uint8_t* offs, void* stream);

typedef struct hisa_lsa_args {
    const uint16_t* queries;     /* [nq, 64] bf16 index queries */
    const int64_t* q_pos;        /* [nq] position of each query in its sequence */
    const int32_t* q_seq;        /* [nq] sequence of each query, or NULL: sequence 0 */
    int64_t nq;
    const uint16_t* centroids;   /* the cache above, all sequences' block rows */
    const uint8_t* members;
    const uint8_t* offs;
    const int64_t* seq_blk_off;  /* [nseq] first block row of each sequence */
    const int64_t* seq_nblk;     /* [nseq] built blocks of each sequence */
    const int64_t* seq_len;      /* [nseq] keys of each sequence */
    int32_t nseq;
    int64_t max_len;             /* HOST bound: every seq_len <= max_len <= HISA_LSA_MAX_LEN */
    int32_t d;                   /* must be 64 */
    int32_t p;                   /* buckets searched, 1 .. HISA_LSA_MAX_P */
    int32_t k;                   /* keys out, 1 .. HISA_MAX_K */
    int32_t* out_idx;            /* [nq, k] positions ascending, then -1 */
    int32_t* out_buckets;        /* [nq, p] or NULL: the buckets keys came from, in rank order
                                    (ids relative to the sequence: block * 64 + bucket), then -1 */
    void* workspace;
    size_t workspace_bytes;      /* at least hisa_lsa_workspace_bytes */
} hisa_lsa_args;

/* Workspace for hisa_lsa_index with these sizes. */
int hisa_lsa_workspace_bytes(const hisa_lsa_args* a, size_t* bytes);

/*
 * hisa_lsa_index -- LSA flat search.  A query at t sees the built blocks
 * that end at or before t (min(floor((t+1)/512), seq_nblk) of them); every
 * visible centroid is scored by its dot product with the query (fp32; the
 * query's normalisation would not change the order), the p best buckets
 * are ranked (score descending, lower id first), and their keys are taken
 * bucket by bucket, each in ascending position, until k: the row is those
 * positions ascending, then -1.  A query with no visible block, or whose
 * position or sequence is out of range, gets a row of -1.  Three kernels
 * and the flat indexer's selection on `stream`.
 * Errors: INVALID_ARG (null required pointer with nq > 0, nq < 0, nseq < 1,
 *         p < 1, k < 1, max_len < 1), UNSUPPORTED (d, p, k, max_len beyond
 *         the limits), WORKSPACE.
 */
int hisa_lsa_index(const hisa_lsa_args* a, void* stream);

/* Human-readable name of a status code (static string). */
const char* hisa_status_str(int status);

/* HISA_ABI_VERSION of the built library. */
int hisa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* HISA_H */
