"""Pins of the oracle's block-only selection (stage 1 expanded to every
visible token of the kept blocks, no token refinement), each against
something other than itself."""
import numpy as np
import pytest

import oracle
from bruteforce import hisa_dense
from long_context_sparse_hisa_amd import synth

D = 64


def _int_bf16(g, shape, lo=-3, hi=3):
    return synth.to_bf16(g.integers(lo, hi + 1, size=shape).astype(np.float32))


def test_all_causal_blocks_when_they_fit_is_the_prefix():
    """c + 1 <= m: every causal block is kept, so the row is 0..t."""
    g = np.random.default_rng(1)
    B, m, L = 16, 6, 200
    keys = synth.to_bf16(g.standard_normal((L, D)).astype(np.float32))
    reps = oracle.pool(keys, B)
    for t in (0, 1, 15, 16, 50, 95):
        idx, blk = oracle.block_only_query(keys[t], reps, L, t, B, m)
        assert np.array_equal(idx[: t + 1], np.arange(t + 1))
        assert np.all(idx[t + 1:] == -1)
        c = t // B
        assert np.array_equal(blk[: c + 1], np.arange(c + 1)) and np.all(blk[c + 1:] == -1)


@pytest.mark.parametrize("B,d,m", [(2, 4, 3), (4, 8, 4), (8, 64, 5), (4, 4, 6)])
def test_equals_dense_bruteforce_with_every_candidate_kept(B, d, m):
    """The dense whole-matrix construction with k = m*B keeps every
    candidate token, which is exactly the block-only row.  Integer data:
    block-score ties are frequent, so the lower-index rule is pinned."""
    g = np.random.default_rng(200 + B * 10 + m)
    for _ in range(10):
        L = int(g.integers(1, 80))
        keys = _int_bf16(g, (L, d))
        queries = _int_bf16(g, (L, d))
        pos = np.arange(L, dtype=np.int64)
        reps = oracle.pool(keys, B)
        idx, sc, blk = oracle.index_batch(False, queries, pos, keys, m * B, reps=reps, B=B, m=m,
                                          block_only=True)
        assert sc is None
        want_idx, want_blk = hisa_dense(queries, keys, reps, pos, B, m, m * B)
        assert np.array_equal(idx, want_idx)
        assert np.array_equal(blk, want_blk)


def test_hisa_rows_lie_inside_the_block_only_rows():
    """HISA refines the same candidate set: its top-k tokens are a subset,
    and with k = m*B it returns the whole set."""
    g = np.random.default_rng(3)
    B, m, k, L = 32, 5, 40, 1000
    keys = synth.to_bf16(g.standard_normal((L, D)).astype(np.float32))
    queries = synth.to_bf16(g.standard_normal((60, D)).astype(np.float32))
    pos = np.sort(g.integers(0, L, 60)).astype(np.int64)
    reps = oracle.pool(keys, B)
    bo, _, bblk = oracle.index_batch(False, queries, pos, keys, m * B, reps=reps, B=B, m=m, block_only=True)
    hi, _, hblk = oracle.index_batch(False, queries, pos, keys, k, reps=reps, B=B, m=m)
    full, _, _ = oracle.index_batch(False, queries, pos, keys, m * B, reps=reps, B=B, m=m)
    assert np.array_equal(bblk, hblk)
    assert np.array_equal(full, bo)
    for i in range(len(pos)):
        assert set(hi[i][hi[i] >= 0]) <= set(bo[i][bo[i] >= 0])


def test_batch_packing_invalid_queries_and_width():
    g = np.random.default_rng(4)
    B, m = 16, 4
    lens = np.array([300, 200], np.int64)
    offs = np.array([0, 300], np.int64)
    keys = synth.to_bf16(g.standard_normal((500, D)).astype(np.float32))
    reps = np.concatenate([oracle.pool(keys[:300], B), oracle.pool(keys[300:], B)])
    rep_off = np.array([0, (300 + B - 1) // B], np.int64)
    queries = synth.to_bf16(g.standard_normal((4, D)).astype(np.float32))
    q_pos = np.array([299, 199, 200, 10], np.int64)
    q_seq = np.array([0, 1, 1, 2], np.int32)      # position 200 and sequence 2 are out of range
    idx, _, blk = oracle.index_batch(False, queries, q_pos, keys, m * B, reps=reps, q_seq=q_seq,
                                     seq_key_off=offs, seq_rep_off=rep_off, seq_len=lens, B=B, m=m,
                                     block_only=True)
    want0, wb0 = oracle.block_only_query(queries[0], reps[:rep_off[1]], 300, 299, B, m)
    want1, wb1 = oracle.block_only_query(queries[1], reps[rep_off[1]:], 200, 199, B, m)
    assert np.array_equal(idx[0], want0) and np.array_equal(blk[0], wb0)
    assert np.array_equal(idx[1], want1) and np.array_equal(blk[1], wb1)
    assert np.all(idx[2:] == -1) and np.all(blk[2:] == -1)
    with pytest.raises(ValueError):
        oracle.index_batch(False, queries, q_pos, keys, m * B - 1, reps=reps, q_seq=q_seq, seq_key_off=offs,
                           seq_rep_off=rep_off, seq_len=lens, B=B, m=m, block_only=True)
