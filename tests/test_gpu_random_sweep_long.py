"""A seeded sweep of random long-row shapes on the GPU against the oracle:
many queries (256 to 900) over rows of more than 1,024 blocks, where stage 1
is the two-walk selection (m - 3 <= 64) or the score row (larger m), and
one-sequence calls whose sparse kept lists take the block-major token
scores.  Block sizes 16..256, m from 4 to 90, k from 1 to min(m*B, 2048),
one or two sequences of ragged lengths, queries anywhere in them (some
invalid).  Each case checks every row's properties and a sample of rows
against the oracle, HISA only (the flat indexer's long rows have tests of
their own)."""
import numpy as np
import pytest

import oracle
from long_context_sparse_hisa_amd import synth
from parity import check_all_rows_properties, check_rows

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

N_CASES = 48


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from long_context_sparse_hisa_amd import hisa
    hisa.lib()                                  # raises if the library is missing


def _case(seed):
    g = np.random.default_rng(5000 + seed)
    B = int(g.choice([16, 32, 64, 128, 256]))
    nseq = 1 if seed % 3 else 2
    # more than 1,024 blocks in the longest sequence, at most 16,384
    lo, hi = 1100 * B, min(16000 * B, 400000)
    lens = g.integers(lo // 2, hi, nseq).astype(np.int64)
    lens[0] = max(int(lens[0]), lo)
    m = int(g.choice([int(g.integers(4, 68)), int(g.integers(1, 17)) * 4, int(g.integers(1, 17)) * 4,
                      int(g.integers(68, 91))]))
    if m * B > 16384:
        m = 16384 // B
    k = int(min(g.integers(1, m * B + 1), 2048))
    nq = int(g.integers(256, 901))
    return g, B, nseq, lens, m, k, nq


@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_long_shape(seed):
    g, B, nseq, lens, m, k, nq = _case(seed)
    print("long sweep %d: B=%d nseq=%d lens=%s m=%d k=%d nq=%d" % (seed, B, nseq, lens.tolist(), m, k, nq),
          flush=True)
    from long_context_sparse_hisa_amd import device as dv
    w = synth.decode_batch(nseq=nseq, L=int(lens.max()), seed=6000 + seed, B=B, m=m, k=k)
    cache = dv.DeviceCache(w, B=B)
    cache.set_lengths(lens)
    cache.pool()
    q_seq = g.integers(0, nseq, nq).astype(np.int32)
    q_pos = np.array([g.integers(0, lens[s]) for s in q_seq], np.int64)
    q_pos[:2] = [0, min(int(lens[q_seq[1]]) - 1, B * m - 1)]     # rows that keep every causal block
    bad = g.random(nq) < 0.03                      # a few invalid queries
    bad[:2] = False
    q_pos[bad] = lens[q_seq[bad]] + 1
    queries = synth.to_bf16(g.standard_normal((nq, synth.D)).astype(np.float32))
    reps = [oracle.pool(w.keys[int(w.seq_key_off[s]):int(w.seq_key_off[s]) + int(lens[s])], B) for s in range(nseq)]
    call = dv.IndexCall(cache, queries, q_pos, q_seq, k=k, m=m, flat=False)
    call.run()
    idx, sc, blk = call.results()
    for i in np.nonzero(bad)[0]:
        assert np.all(idx[i] == -1) and np.all(blk[i] == -1), "invalid query %d" % i
    ok = ~bad
    check_all_rows_properties(idx[ok], blk[ok], q_pos[ok], B, m, k, False)
    rows = sorted(set(g.choice(nq, min(nq, 120), replace=False).tolist()) | {0, 1, nq - 1})
    good = [i for i in rows if ok[i]]
    check_rows(good, queries, q_pos,
               lambda i: w.keys[int(w.seq_key_off[q_seq[i]]):int(w.seq_key_off[q_seq[i]]) + int(lens[q_seq[i]])],
               lambda i: reps[int(q_seq[i])], B, m, k, idx, sc, blk, False, "longsweep%d" % seed)
