"""GPU-vs-oracle comparison rule for index results (tests only).

Rule (tolerance TOL = 1e-3 absolute on scores):
  * every exported GPU score is within TOL of the fp64 dot product of its
    index;
  * kept block sets equal the oracle's, except blocks whose fp64 score lies
    within TOL of the oracle's m-th (boundary) block score; when they differ
    the oracle's stage 2 is re-run on the GPU's block set and tokens are
    compared against that;
  * token sets equal the oracle's, except tokens whose fp64 score lies within
    TOL of the oracle's k-th score; the number of valid entries is exact;
  * rows are ascending, duplicate-free, causal, and -1 padded.
"""
from __future__ import annotations

import numpy as np

import oracle
from bruteforce import bf16_values

TOL = 1e-3


class Mismatch(AssertionError):
    pass


def _u(q, K, ids):
    return bf16_values(K[ids]) @ bf16_values(q)


def check_row_shape(idx_row, t, what):
    valid = idx_row[idx_row >= 0]
    n = len(valid)
    if not np.all(idx_row[n:] == -1):
        raise Mismatch("%s: -1 padding not at the end" % what)
    if n and (np.any(np.diff(valid) <= 0) or valid[-1] > t or valid[0] < 0):
        raise Mismatch("%s: row not ascending/unique/causal" % what)
    return valid


def check_query(q, K, R, t, B, m, k, g_idx, g_sc, g_blk, flat, what=""):
    """Compare one query's GPU row with the oracle.  Returns 'exact' or
    'excused' (differences inside the tolerance band)."""
    verdict = "exact"
    valid = check_row_shape(g_idx, t, what)
    if g_sc is not None and len(valid):
        err = np.abs(g_sc[: len(valid)].astype(np.float64) - _u(q, K, valid))
        if err.max() > TOL:
            raise Mismatch("%s: score error %.3g > %g" % (what, err.max(), TOL))
    if flat:
        o_idx, _, _ = oracle.flat_query(q, K, t, k)
        blocks = None
    else:
        o_idx, _, o_blk, _ = oracle.hisa_query(q, K, R, t, B, m, k)
        if g_blk is not None and not np.array_equal(g_blk, o_blk):
            gb = g_blk[g_blk >= 0]
            ob = o_blk[o_blk >= 0]
            if len(gb) != len(ob) or np.any(np.diff(gb) <= 0):
                raise Mismatch("%s: block row malformed %s vs %s" % (what, gb, ob))
            c = t // B
            forced = {0, c - 1, c}
            if not forced <= set(gb.tolist()):
                raise Mismatch("%s: forced block missing" % what)
            sig = bf16_values(R[: c + 1]) @ bf16_values(q)
            free_o = [b for b in ob if b not in forced]
            boundary = min(sig[free_o])
            for b in set(gb.tolist()) ^ set(ob.tolist()):
                if abs(sig[b] - boundary) > TOL:
                    raise Mismatch("%s: block %d differs, score %.6f vs boundary %.6f"
                                   % (what, b, sig[b], boundary))
            o_idx, _ = oracle.tokens_on_blocks(q, K, t, B, gb, k)
            verdict = "excused"
        blocks = g_blk
    o_valid = o_idx[o_idx >= 0]
    if len(o_valid) != len(valid):
        raise Mismatch("%s: %d valid tokens vs oracle %d" % (what, len(valid), len(o_valid)))
    if not np.array_equal(valid, o_valid):
        if len(o_valid) < k:
            raise Mismatch("%s: all candidates fit in k but sets differ" % what)
        boundary = _u(q, K, o_valid).min()
        diff = np.setxor1d(valid, o_valid)
        # a token the GPU took must be a candidate of the kept blocks
        if blocks is not None:
            kept = set(blocks[blocks >= 0].tolist())
            if any((j // B) not in kept for j in valid):
                raise Mismatch("%s: token outside the kept blocks" % what)
        ud = _u(q, K, diff)
        if np.abs(ud - boundary).max() > TOL:
            raise Mismatch("%s: tokens %s differ beyond tolerance (scores %s, boundary %.6f)"
                           % (what, diff[:8], ud[:8], boundary))
        verdict = "excused"
    return verdict


def check_rows(rows, queries, q_pos, K_of, R_of, B, m, k, g_idx, g_sc, g_blk, flat, label=""):
    """Check the given query rows; K_of(i) / R_of(i) give the sequence's
    key / representative arrays of query i.  Returns counts per verdict."""
    counts = {"exact": 0, "excused": 0}
    for i in rows:
        v = check_query(queries[i], K_of(i), None if flat else R_of(i), int(q_pos[i]), B, m, k,
                        g_idx[i], None if g_sc is None else g_sc[i],
                        None if g_blk is None else g_blk[i], flat, "%s row %d" % (label, i))
        counts[v] += 1
    return counts


def check_all_rows_properties(g_idx, g_blk, q_pos, B, m, k, flat, seq_len=None):
    """Properties every row must have at any size (vectorised)."""
    nq = g_idx.shape[0]
    valid = g_idx >= 0
    nvalid = valid.sum(1)
    # padding only at the end
    assert np.all(valid[:, :-1] >= valid[:, 1:]), "padding not at the end"
    # ascending and causal
    big = np.where(valid, g_idx, np.iinfo(np.int32).max)
    assert np.all(np.diff(big, axis=1)[valid[:, 1:]] > 0), "rows not ascending"
    bad = np.nonzero(g_idx.max(1) > q_pos)[0]
    assert len(bad) == 0, "non-causal index: row %d t=%d idx>t: %s" % (
        bad[0], q_pos[bad[0]], g_idx[bad[0]][g_idx[bad[0]] > q_pos[bad[0]]][:10])
    if flat:
        assert np.all(nvalid == np.minimum(k, q_pos + 1)), "flat row count"
    else:
        c = q_pos // B
        nb = (g_blk >= 0).sum(1)
        assert np.all(nb == np.minimum(m, c + 1)), "kept block count"
        assert np.all(g_blk[:, 0] == 0), "first block not kept"
        last = g_blk[np.arange(nq), nb - 1]
        assert np.all(last == c), "own block not kept"
        # the block before the query's own is forced too: second to last of
        # the ascending list whenever it exists
        has_prev = c >= 1
        prev = g_blk[np.arange(nq), np.maximum(nb - 2, 0)]
        assert np.all(prev[has_prev] == c[has_prev] - 1), "block c-1 not kept"
        # tokens sit inside kept blocks
        M = int(q_pos.max()) // B + 2
        kept = np.zeros((nq, M), bool)
        r = np.repeat(np.arange(nq), g_blk.shape[1])
        b = g_blk.ravel()
        kept[r[b >= 0], b[b >= 0]] = True
        tb = np.where(valid, g_idx // B, M - 1)
        inside = kept[np.arange(nq)[:, None], tb] | ~valid
        assert inside.all(), "token outside kept blocks"
        cand = np.where(g_blk >= 0, np.minimum(B, q_pos[:, None] - g_blk * B + 1), 0).sum(1)
        assert np.all(nvalid == np.minimum(k, cand)), "hisa row count"


def check_batch(ph, keys, lens, seq_key_off, reps, rep_off, B, m, k, g_idx, g_sc, g_blk, flat, K_of, R_of,
                label=""):
    """Every row of a phase against one batched oracle call: rows whose
    indices (and kept blocks) equal the oracle's exactly pass, with every
    exported score within TOL of the oracle's fp64 value; the other rows go
    through the per-row tolerance rule of check_query.  Returns counts per
    verdict."""
    o_idx, o_sc, o_blk = oracle.index_batch(flat, ph.queries, ph.q_pos, keys, k, reps=reps, q_seq=ph.q_seq,
                                            seq_key_off=seq_key_off, seq_rep_off=rep_off, seq_len=lens, B=B, m=m)
    same = np.all(g_idx == o_idx, axis=1)
    if not flat and g_blk is not None:
        same &= np.all(g_blk == o_blk, axis=1)
    if g_sc is not None:
        v = same[:, None] & (o_idx >= 0)
        err = np.abs(np.where(v, g_sc.astype(np.float64) - o_sc, 0.0))
        if err.max() > TOL:
            r = int(np.argmax(err.max(1)))
            raise Mismatch("%s row %d: score error %.3g > %g" % (label, r, err[r].max(), TOL))
    counts = {"exact": int(same.sum()), "excused": 0}
    rest = np.nonzero(~same)[0]
    if len(rest):
        c = check_rows(rest, ph.queries, ph.q_pos, K_of, R_of, B, m, k, g_idx, g_sc, g_blk, flat, label)
        counts["exact"] += c["exact"]
        counts["excused"] += c["excused"]
    return counts
