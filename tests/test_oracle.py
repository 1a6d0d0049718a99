"""Pins of the CPU oracle against what the pages and the mathematics fix.

Every check here compares the oracle with something other than itself:
exact rational arithmetic, dense numpy brute force, closed forms, the work
counts printed on the pages, and invariants the method guarantees.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from bruteforce import (bf16_bits_to_fraction, bf16_round_exact, bf16_values, hisa_dense,
                        pool_exact)
from long_context_sparse_hisa_amd import synth

D = 64


def _int_bf16(g, shape, lo=-6, hi=6):
    """Small integers as bf16 bits: every sum and product of a few of them
    is exact in fp64, so ties are real and frequent."""
    return synth.to_bf16(g.integers(lo, hi + 1, size=shape).astype(np.float32))


# --- the representative's rounding rule ------------------------------------

def test_bf16_round_matches_exact_definition():
    g = np.random.default_rng(0)
    vals = list(g.standard_normal(300) * 10.0 ** g.integers(-40, 39, 300))
    # exact midpoints between neighbouring bf16 values, both parities
    for h in [0x3F80, 0x3F81, 0x4000, 0x0001, 0x0080, 0x7F7E, 0x7F7F, 0x1234]:
        a = bf16_bits_to_fraction(h)
        b = bf16_bits_to_fraction(h + 1) if h < 0x7F7F else a + (a - bf16_bits_to_fraction(h - 1))
        vals.append(float((a + b) / 2))
        vals.append(-float((a + b) / 2))
    vals += [0.0, -0.0, 1e-45, 3.4e38, 3.39e38, 1e300, 2.0 ** -133, 2.0 ** -134, 1.5 * 2.0 ** -134]
    for v in vals:
        if v == 0.0:                                      # rationals carry no sign of zero
            assert oracle.bf16_round(v) == (0x8000 if math.copysign(1, v) < 0 else 0)
            continue
        assert oracle.bf16_round(v) == bf16_round_exact(Fraction(v)), v


def test_bf16_round_ties_to_even():
    one, up = 1.0, 1.0 + 2.0 ** -7                       # 0x3F80, 0x3F81
    assert oracle.bf16_round((one + up) / 2) == 0x3F80   # tie -> even pattern
    up2 = 1.0 + 2.0 ** -6                                 # 0x3F82
    assert oracle.bf16_round((up + up2) / 2) == 0x3F82


# --- pooling: closed forms (HISA summary, structure paragraph) ---------------

def test_pool_constant_blocks():
    g = np.random.default_rng(1)
    B, M = 16, 7
    vals = synth.to_bf16(g.standard_normal((M, D)).astype(np.float32))
    keys = np.repeat(vals, B, axis=0)
    assert np.array_equal(oracle.pool(keys, B), vals)


def test_pool_arithmetic_progression():
    # keys j: every coordinate equals j (integers are exact in bf16 up to 256)
    B = 8
    L = 64
    keys = synth.to_bf16(np.repeat(np.arange(L, dtype=np.float32)[:, None], D, axis=1))
    reps = oracle.pool(keys, B)
    for b in range(L // B):
        mean = b * B + (B - 1) / 2.0                     # mean of an arithmetic run
        assert np.all(reps[b] == synth.to_bf16(np.float32(mean)))


def test_pool_matches_exact_rational_mean():
    g = np.random.default_rng(2)
    for B, L in [(4, 37), (8, 64), (16, 33), (128, 300)]:
        keys = synth.to_bf16(g.standard_normal((L, 8)).astype(np.float32))
        reps, inexact = oracle.pool(keys, B, return_flag=True)
        assert not inexact
        assert np.array_equal(reps, pool_exact(keys, B))


def test_pool_partial_block_divides_by_its_count():
    B = 128
    keys = np.zeros((130, D), np.uint16)
    keys[128] = synth.to_bf16(np.full(D, 1.0, np.float32))
    keys[129] = synth.to_bf16(np.full(D, 2.0, np.float32))
    reps = oracle.pool(keys, B)
    assert reps.shape == (2, D)
    assert np.all(reps[1] == synth.to_bf16(np.float32(1.5)))   # (1 + 2) / 2, not / 128
    assert np.all(reps[0] == 0)


def test_pool_reports_inexact_sums():
    keys = np.zeros((4, D), np.uint16)
    keys[0] = synth.to_bf16(np.full(D, 1.0, np.float32))
    keys[1] = 0x0001                                      # 2^-133: far below the exact range
    _, inexact = oracle.pool(keys, 4, return_flag=True)
    assert inexact


def test_incremental_equals_one_shot():
    """Representatives kept up to date at append (HISA summary, maintenance
    paragraph) equal pooling everything at once, for any split."""
    g = np.random.default_rng(3)
    B = 16
    keys = synth.to_bf16(g.standard_normal((203, D)).astype(np.float32))
    want = oracle.pool(keys, B)
    for trial in range(5):
        cuts = np.sort(g.choice(np.arange(1, 203), size=6, replace=False))
        bounds = [0] + list(cuts) + [203]
        reps = np.zeros(((203 + B - 1) // B, D), np.uint16)
        for lo, hi in zip(bounds[:-1], bounds[1:]):
            cur = keys[:hi]
            oracle.pool_range(cur, B, lo // B, (hi + B - 1) // B, reps)
        assert np.array_equal(reps, want)


# --- scores -----------------------------------------------------------------

def test_block_scores_exact_on_integers():
    g = np.random.default_rng(4)
    reps = _int_bf16(g, (50, D))
    q = _int_bf16(g, (D,))
    want = bf16_values(reps) @ bf16_values(q)
    assert np.array_equal(oracle.block_scores(q, reps), want)


def test_block_scores_against_numpy_random():
    g = np.random.default_rng(5)
    reps = synth.to_bf16(g.standard_normal((40, D)).astype(np.float32))
    q = synth.to_bf16(g.standard_normal(D).astype(np.float32))
    want = bf16_values(reps) @ bf16_values(q)
    assert np.allclose(oracle.block_scores(q, reps), want, rtol=0, atol=1e-12)


# --- whole indexer vs dense brute force --------------------------------------

@pytest.mark.parametrize("B,d,m,k", [(2, 4, 3, 1), (4, 8, 4, 5), (8, 64, 5, 16), (4, 4, 6, 9),
                                     (8, 8, 3, 24)])
def test_hisa_equals_dense_bruteforce_integer(B, d, m, k):
    """Integer data: scores are exact on both sides, ties are frequent, so
    the tie rule (lower index first) is pinned too."""
    g = np.random.default_rng(100 + B * 10 + m)
    for trial in range(12):
        L = int(g.integers(1, 65))
        keys = _int_bf16(g, (L, d), -3, 3)
        queries = _int_bf16(g, (L, d), -3, 3)
        pos = np.arange(L, dtype=np.int64)
        reps = oracle.pool(keys, B)
        for flat in (False, True):
            idx, _, blk = oracle.index_batch(flat, queries, pos, keys, k, reps=reps, B=B, m=m)
            want_idx, want_blk = hisa_dense(queries, keys, reps, pos, B, m, k, flat=flat)
            assert np.array_equal(idx, want_idx)
            if not flat:
                assert np.array_equal(blk, want_blk)


def test_hisa_matches_dense_bruteforce_random():
    g = np.random.default_rng(7)
    B, m, k = 8, 4, 12
    keys = synth.to_bf16(g.standard_normal((96, D)).astype(np.float32))
    queries = synth.to_bf16(g.standard_normal((96, D)).astype(np.float32))
    pos = np.arange(96, dtype=np.int64)
    reps = oracle.pool(keys, B)
    idx, _, blk = oracle.index_batch(False, queries, pos, keys, k, reps=reps, B=B, m=m)
    want_idx, want_blk = hisa_dense(queries, keys, reps, pos, B, m, k)
    assert np.array_equal(idx, want_idx) and np.array_equal(blk, want_blk)


def _certify(q, keys, reps, t, B, m, k, idx, sc, blk):
    """Selection certificates that do not trust any sort."""
    qv = bf16_values(q)
    c = t // B
    kept = [b for b in blk if b >= 0]
    assert kept == sorted(kept) and len(set(kept)) == len(kept)
    assert len(kept) == min(m, c + 1)
    assert all(0 <= b <= c for b in kept)
    if c + 1 > m:
        assert {0, c - 1, c} <= set(kept)                 # forced blocks present
        sig = (bf16_values(reps[: c + 1]) @ qv).astype(np.float32)
        free_kept = [b for b in kept if b not in (0, c - 1, c)]
        free_drop = [b for b in range(1, c - 1) if b not in kept]
        if free_kept and free_drop:
            assert min(sig[free_kept]) >= max(sig[free_drop])
    cand = [j for b in kept for j in range(b * B, min((b + 1) * B, t + 1))]
    got = [j for j in idx if j >= 0]
    assert got == sorted(got) and len(set(got)) == len(got)
    assert len(got) == min(k, len(cand))
    assert set(got) <= set(cand) and max(got) <= t
    u = (bf16_values(keys[cand]) @ qv).astype(np.float32)
    emitted = np.isin(cand, got)
    if emitted.any() and (~emitted).any():
        assert u[emitted].min() >= u[~emitted].max()
    # emitted scores are the fp64 dot products
    for j, s in zip(idx, sc):
        if j >= 0:
            assert abs(s - float(bf16_values(keys[j]) @ qv)) < 1e-9


def test_selection_certificates_tiny_random():
    g = np.random.default_rng(8)
    for trial in range(1500):
        B = int(g.choice([2, 4, 8]))
        d = int(g.choice([4, 8, 64]))
        m = int(g.integers(3, 7))
        k = int(g.integers(1, 17))
        L = int(g.integers(1, 65))
        keys = synth.to_bf16(g.standard_normal((L, d)).astype(np.float32))
        q = synth.to_bf16(g.standard_normal(d).astype(np.float32))
        t = int(g.integers(0, L))
        reps = oracle.pool(keys, B)
        idx, sc, blk, _ = oracle.hisa_query(q, keys, reps, t, B, m, k)
        _certify(q, keys, reps, t, B, m, k, idx, sc, blk)


# --- causality, forced blocks, padding, reduction to flat --------------------

def test_causality_and_flat_prefix():
    g = np.random.default_rng(9)
    keys = synth.to_bf16(g.standard_normal((300, D)).astype(np.float32))
    q = synth.to_bf16(g.standard_normal(D).astype(np.float32))
    reps = oracle.pool(keys, 16)
    for t in [0, 1, 15, 16, 17, 100, 299]:
        idx, _, _, _ = oracle.hisa_query(q, keys, reps, t, 16, 4, 40)
        assert idx.max() <= t
        fidx, _, _ = oracle.flat_query(q, keys, t, t + 1)
        assert np.array_equal(fidx, np.arange(t + 1))          # k >= t+1: the whole prefix
        fidx, _, _ = oracle.flat_query(q, keys, t, t + 5)
        assert np.array_equal(fidx[: t + 1], np.arange(t + 1)) and np.all(fidx[t + 1:] == -1)


def test_forced_blocks_survive_adversarial_keys():
    """First block and the last two causal blocks are kept even when they
    score worst (HISA summary, stage-1 paragraph)."""
    g = np.random.default_rng(10)
    B, m, L = 16, 5, 320
    q = synth.to_bf16(np.abs(g.standard_normal(D)).astype(np.float32) + 0.5)
    qv = synth.from_bf16(q)
    keys = synth.to_bf16(g.standard_normal((L, D)).astype(np.float32) * 0.1 + qv * 0.2)
    t = 250
    c = t // B
    for b in (0, c - 1, c):
        keys[b * B:(b + 1) * B] = synth.to_bf16(-qv)[None, :]
    # make blocks 5 and 9 clearly the best free blocks
    keys[5 * B:6 * B] = synth.to_bf16(qv * 2)[None, :]
    keys[9 * B:10 * B] = synth.to_bf16(qv * 1.5)[None, :]
    reps = oracle.pool(keys, B)
    _, _, blk, _ = oracle.hisa_query(q, keys, reps, t, B, m, 64)
    assert list(blk) == sorted([0, c - 1, c, 5, 9])


def test_all_causal_blocks_when_they_fit():
    g = np.random.default_rng(11)
    keys = synth.to_bf16(g.standard_normal((100, D)).astype(np.float32))
    q = synth.to_bf16(g.standard_normal(D).astype(np.float32))
    reps = oracle.pool(keys, 16)
    _, _, blk, _ = oracle.hisa_query(q, keys, reps, 40, 16, 6, 8)
    assert list(blk) == [0, 1, 2, -1, -1, -1]


def test_hisa_with_m_covering_all_blocks_is_flat():
    """With m >= c+1 HISA keeps every causal block and equals the flat
    indexer; flat equals an argsort of the dense score row."""
    g = np.random.default_rng(12)
    w = synth.chunked_prefill(L=1024, seed=12, q_positions=np.arange(0, 1024, 37))
    ph = w.phases[0]
    reps = oracle.pool(w.keys, 128)
    k = 100
    hidx, hsc, _ = oracle.index_batch(False, ph.queries, ph.q_pos, w.keys, k, reps=reps, B=128,
                                      m=8)
    fidx, fsc, _ = oracle.index_batch(True, ph.queries, ph.q_pos, w.keys, k)
    assert np.array_equal(hidx, fidx)
    np.testing.assert_array_equal(hsc, fsc)
    row = (bf16_values(ph.queries) @ bf16_values(w.keys).T).astype(np.float32)
    for i, t in enumerate(ph.q_pos):
        ids = np.arange(t + 1)
        order = np.lexsort((ids, -row[i, : t + 1]))
        want = np.sort(ids[order[:k]])
        assert np.array_equal(fidx[i, : len(want)], want)


def test_work_counts_match_pages():
    """About 1,000 block scores and 8,000 token scores at 128K."""
    path = os.path.join(os.path.dirname(__file__), "golden", "work_counts_128k.txt")
    rows = [l.split() for l in open(path) if l.strip() and not l.startswith("#")]
    L, t, B, m, nb, nt, nflat = map(int, rows[0])
    g = np.random.default_rng(13)
    # one query at L-1 needs only the blocks and keys it touches; random
    # data of the full length keeps the count honest
    keys = synth.to_bf16(g.standard_normal((L, D)).astype(np.float32))
    q = synth.to_bf16(g.standard_normal(D).astype(np.float32))
    reps = oracle.pool(keys, B)
    _, _, _, counts = oracle.hisa_query(q, keys, reps, t, B, m, 2048)
    assert counts == (nb, nt)
    _, _, fcounts = oracle.flat_query(q, keys, t, 2048)
    assert fcounts[1] == nflat


def test_planted_needles_found_by_flat():
    w = synth.long_context(L=8192, chunk=64, ndecode=2, nneedles=16, seed=14, k=256)
    ph = w.phases[1]
    idx, _, _ = oracle.index_batch(True, ph.queries[:1], ph.q_pos[:1], w.keys, 256)
    assert set(w.needles.tolist()) <= set(idx[0].tolist())


def test_batch_packing_and_invalid_queries():
    g = np.random.default_rng(15)
    w = synth.decode_batch(nseq=3, L=700, seed=15, m=4, k=50, spare=30)
    ph = w.phases[0]
    B, m, k = 64, 4, 50
    rep_off = w.seq_rep_off(B)
    reps = np.zeros((w.total_rep_rows(B), D), np.uint16)
    for s in range(w.nseq):
        o = int(w.seq_key_off[s])
        r = oracle.pool(w.keys[o: o + w.seq_len[s]], B)
        reps[rep_off[s]: rep_off[s] + len(r)] = r
    q_pos = ph.q_pos.copy()
    q_pos[1] = 700                               # past the end: invalid
    idx, sc, blk = oracle.index_batch(False, ph.queries, q_pos, w.keys, k, reps=reps,
                                      q_seq=ph.q_seq, seq_key_off=w.seq_key_off,
                                      seq_rep_off=rep_off, seq_len=w.seq_len, B=B, m=m)
    assert np.all(idx[1] == -1) and np.all(blk[1] == -1)
    for s in (0, 2):
        o = int(w.seq_key_off[s])
        K = w.keys[o: o + w.seq_len[s]]
        r = reps[rep_off[s]: rep_off[s] + (700 + B - 1) // B]
        want, wsc, wblk, _ = oracle.hisa_query(ph.queries[s], K, r, int(q_pos[s]), B, m, k)
        assert np.array_equal(idx[s], want) and np.array_equal(blk[s], wblk)


def test_mog_generator_is_deterministic():
    a = synth.decode_batch(nseq=2, L=512, seed=2)
    b = synth.decode_batch(nseq=2, L=512, seed=2)
    assert synth.sha256(a.keys, a.phases[0].queries) == synth.sha256(b.keys, b.phases[0].queries)
    assert np.all(np.abs(synth.from_bf16(a.keys)) < 16)


def test_signed_zero_scores_tie_to_lower_index():
    """-0.0 and +0.0 are equal fp32 values: a key whose every product is -0
    (score -0.0) ties with one of score +0.0, and the lower index is taken.
    Expected rows written by hand."""
    L = 600
    keys = np.full((L, synth.D), synth.to_bf16(np.float32(-1.0)), np.uint16)
    keys[10:15] = synth.to_bf16(np.float32(1.0))
    keys[20] = 0x8000                                      # bf16 -0.0
    keys[30] = 0x0000                                      # bf16 +0.0
    q = np.full(synth.D, synth.to_bf16(np.float32(1.0)), np.uint16)
    want = [10, 11, 12, 13, 14, 20]
    idx, sc, _ = oracle.flat_query(q, keys, L - 1, 6)
    assert sorted(idx.tolist()) == want
    assert sc[list(idx).index(20)] == 0.0
    idx, _, _ = oracle.hisa_query(q, keys, oracle.pool(keys, 64), L - 1, 64, 10, 6)[:3]
    assert sorted(idx.tolist()) == want
    # with the zeros swapped the +0 row is the lower one
    keys[20], keys[30] = 0x0000, 0x8000
    idx, _, _ = oracle.flat_query(q, keys, L - 1, 6)
    assert sorted(idx.tolist()) == want
