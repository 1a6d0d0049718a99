"""Pins of the LSA-Flat oracle (CPU), each against something other than the
oracle itself: scipy's Ward linkage, hand-derived merges, planted
clusters, closed forms and a numpy brute force of the flat search."""
import numpy as np
import pytest

import oracle
from long_context_sparse_hisa_amd import synth

D = 64


def _clusters_formed(n, merges):
    members = {i: frozenset([i]) for i in range(n)}
    out = []
    for a, b in merges:
        members[a] = members[a] | members[b]
        out.append(members[a])
    return out


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_full_hierarchy_equals_scipy_ward(seed):
    """Without a size cap and down to one bucket, rounds of mutual cheapest
    pairs form exactly the clusters of Ward's greedy linkage (Ward's
    criterion is reducible, so the two orders give one hierarchy)."""
    from scipy.cluster.hierarchy import linkage
    g = np.random.default_rng(seed)
    n = 60
    P = g.standard_normal((n, 12))
    _, merges, _, left = oracle.lsa_ward(P, 1, 10 ** 6)
    assert left == 1
    Z = linkage(P, method="ward")
    cl = {i: frozenset([i]) for i in range(n)}
    theirs = []
    for i, (x, y, _, _) in enumerate(Z):
        cl[n + i] = cl[int(x)] | cl[int(y)]
        theirs.append(cl[n + i])
    assert set(_clusters_formed(n, merges)) == set(theirs)


def test_size_cap_changes_the_merge_by_hand():
    """1-D points 0, 1, 2.5, 50, 51.2, 53, 100, 101.7 with at most 2 points
    per bucket, down to 4 buckets.  Round 1: {0,1}, {50,51.2}, {100,101.7}
    are mutual cheapest pairs (2.5's cheapest is 1, 53's is 51.2, neither
    mutual).  Round 2: only 2.5 and 53 may still merge.  Without the cap 2.5
    would join {0, 1}."""
    x = np.array([0, 1, 2.5, 50, 51.2, 53, 100, 101.7])
    P = np.zeros((8, 4))
    P[:, 0] = x
    lab, merges, _, left = oracle.lsa_ward(P, 4, 2)
    assert left == 4
    assert [tuple(m) for m in merges] == [(0, 1), (3, 4), (6, 7), (2, 5)]
    assert list(lab) == [0, 0, 2, 3, 3, 2, 6, 6]
    lab, _, _, _ = oracle.lsa_ward(P, 4, 10)
    assert lab[2] == 0


def test_last_round_merges_the_cheapest_pairs_only():
    """Four well separated pairs with spreads 1, 2, 3, 4, down to 6 buckets:
    all four pairs are mutual in round 1, only the two cheapest merge."""
    P = np.zeros((8, 2))
    P[:, 0] = [0, 4, 100, 101, 200, 203, 300, 302]
    lab, merges, _, left = oracle.lsa_ward(P, 6, 4)
    assert left == 6
    assert sorted(map(tuple, merges)) == [(2, 3), (6, 7)]


def _block_keys(g, n=512):
    return synth.to_bf16(g.standard_normal((n, D)).astype(np.float32))


def test_block_invariants_and_centroids():
    g = np.random.default_rng(4)
    keys = _block_keys(g, 1024 + 300)            # two complete blocks and a ragged tail
    cen, mem, off, _ = oracle.lsa_build(keys)
    assert cen.shape == (128, D) and mem.shape == (2, 128) and off.shape == (2, 65)
    for b in range(2):
        o = off[b].astype(int)
        assert o[0] == 0 and o[-1] == 128 and np.all(np.diff(o) >= 1) and np.all(np.diff(o) <= 4)
        assert sorted(mem[b]) == list(range(128))
        firsts = [mem[b][o[i]] for i in range(64)]
        assert firsts == sorted(firsts)
        kv = synth.from_bf16(keys[b * 512:(b + 1) * 512]).astype(np.float64)
        unit = kv / np.linalg.norm(kv, axis=1, keepdims=True)
        for i in range(64):
            pts = mem[b][o[i]:o[i + 1]].astype(int)
            assert np.all(np.diff(pts) > 0)
            rows = np.concatenate([np.arange(4 * p, 4 * p + 4) for p in pts])
            s = unit[rows].sum(0)
            want = np.array([oracle.bf16_round(v) for v in s / np.linalg.norm(s)], np.uint16)
            got = cen[b * 64 + i]
            # the fp64 sums differ from numpy's in the last bits at most, so a
            # component may round to the neighbouring bf16 value only at a
            # rounding midpoint
            assert np.sum(got != want) <= 1


def test_scaling_keys_changes_nothing():
    g = np.random.default_rng(5)
    keys = _block_keys(g)
    a = oracle.lsa_build(keys)
    b = oracle.lsa_build(synth.to_bf16(synth.from_bf16(keys) * np.float32(4.0)))
    for x, y in zip(a[:3], b[:3]):
        assert np.array_equal(x, y)


def test_planted_groups_of_eight_keys_become_the_buckets():
    """64 directions far apart, each shared (with small noise) by 8
    consecutive keys = 2 pool keys: Ward pairs exactly those pool keys."""
    g = np.random.default_rng(6)
    dirs = g.standard_normal((64, D))
    keys = np.repeat(dirs, 8, axis=0) + 0.01 * g.standard_normal((512, D))
    cen, mem, off, _ = oracle.lsa_build(synth.to_bf16(keys.astype(np.float32)))
    assert np.array_equal(off[0], np.arange(0, 129, 2))
    assert np.array_equal(mem[0], np.arange(128))
    d = dirs / np.linalg.norm(dirs, axis=1, keepdims=True)
    c = synth.from_bf16(cen).astype(np.float64)
    assert np.all(np.sum(c * d, axis=1) > 0.999)


def _brute_query(q, cen, mem, off, t, p, k):
    """Rank every visible centroid by the fp32 rounding of its fp64 score
    (ties: lower id) with numpy, then fill."""
    vis = min((t + 1) // 512, mem.shape[0])
    nb = vis * 64
    s = (synth.from_bf16(cen[:nb]).astype(np.float64) @ synth.from_bf16(q).astype(np.float64)).astype(np.float32)
    order = np.lexsort((np.arange(nb), -s))
    toks = []
    used = []
    for b in order[:p]:
        if len(toks) >= k:
            break
        blk, lb = divmod(int(b), 64)
        pts = mem[blk][off[blk][lb]:off[blk][lb + 1]].astype(int)
        for pt in pts:
            toks.extend(range(blk * 512 + 4 * pt, blk * 512 + 4 * pt + 4))
        used.append(int(b))
    toks = sorted(toks[:k])
    return np.array(toks + [-1] * (k - len(toks)), np.int32), used


@pytest.mark.parametrize("t,p,k", [(4095, 32, 256), (4095, 8, 4096), (3000, 64, 300), (600, 5, 40), (511, 3, 17)])
def test_query_matches_numpy_bruteforce(t, p, k):
    g = np.random.default_rng(7)
    keys = _block_keys(g, 4096)
    cen, mem, off, _ = oracle.lsa_build(keys)
    for trial in range(4):
        q = synth.to_bf16(g.standard_normal(D).astype(np.float32))
        idx, bk, _ = oracle.lsa_query(q, cen, mem, off, t, p, k)
        want, used = _brute_query(q, cen, mem, off, t, p, k)
        assert np.array_equal(idx, want)
        assert list(bk[bk >= 0]) == used


def test_query_closed_forms_and_causality():
    g = np.random.default_rng(8)
    keys = _block_keys(g, 2048)
    cen, mem, off, _ = oracle.lsa_build(keys)
    q = synth.to_bf16(g.standard_normal(D).astype(np.float32))
    # nothing complete before position 511
    idx, bk, _ = oracle.lsa_query(q, cen, mem, off, 510, 10, 50)
    assert np.all(idx == -1) and np.all(bk == -1)
    # every bucket and room for every key: all keys of the visible blocks
    for t, vis in ((511, 1), (1500, 2), (2047, 4)):
        idx, _, _ = oracle.lsa_query(q, cen, mem, off, t, 10 ** 6, 4096)
        assert np.array_equal(idx[: vis * 512], np.arange(vis * 512)) and np.all(idx[vis * 512:] == -1)
    # exactly k keys when the p buckets hold more
    idx, bk, _ = oracle.lsa_query(q, cen, mem, off, 2047, 64, 100)
    assert (idx >= 0).sum() == 100


def test_query_along_a_centroid_takes_its_bucket_first():
    g = np.random.default_rng(9)
    keys = _block_keys(g, 1024)
    cen, mem, off, _ = oracle.lsa_build(keys)
    q = synth.to_bf16(synth.from_bf16(cen[77]) * np.float32(8.0))
    _, bk, _ = oracle.lsa_query(q, cen, mem, off, 1023, 4, 16)
    assert bk[0] == 77


def test_batch_rows_read_their_own_sequence():
    g = np.random.default_rng(10)
    k1, k2 = _block_keys(g, 1536), _block_keys(g, 1100)
    c1, m1, o1, _ = oracle.lsa_build(k1)
    c2, m2, o2, _ = oracle.lsa_build(k2)
    cen = np.concatenate([c1, c2])
    mem = np.concatenate([m1, m2])
    off = np.concatenate([o1, o2])
    queries = synth.to_bf16(g.standard_normal((4, D)).astype(np.float32))
    q_pos = np.array([1535, 1099, 1100, 700], np.int64)
    q_seq = np.array([0, 1, 1, 5], np.int32)
    idx, bk = oracle.lsa_batch(queries, q_pos, q_seq, cen, mem, off, np.array([0, 3]), np.array([3, 2]),
                               np.array([1536, 1100]), 20, 120)
    w0, b0, _ = oracle.lsa_query(queries[0], c1, m1, o1, 1535, 20, 120)
    w1, b1, _ = oracle.lsa_query(queries[1], c2, m2, o2, 1099, 20, 120)
    assert np.array_equal(idx[0], w0) and np.array_equal(bk[0], b0)
    assert np.array_equal(idx[1], w1) and np.array_equal(bk[1], b1)
    assert np.all(idx[2:] == -1) and np.all(bk[2:] == -1)
