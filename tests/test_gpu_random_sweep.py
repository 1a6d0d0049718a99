"""A seeded sweep of random index shapes on the GPU against the oracle:
block sizes 16..256, kept-block counts from 3 to past the causal range, k
from 1 to m*B, query counts on both sides of the few-/many-query split
(512) and the many-row top-k threshold (256), packed sequences of ragged
lengths with queries anywhere in them (and some invalid ones).  Each case
checks every row's properties and a sample of rows against the oracle."""
import numpy as np
import pytest

import oracle
from long_context_sparse_hisa_amd import synth
from parity import check_all_rows_properties, check_rows

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

N_CASES = 64


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from long_context_sparse_hisa_amd import hisa
    hisa.lib()                                  # raises if the library is missing


def _case(seed):
    g = np.random.default_rng(1000 + seed)
    B = int(g.choice([16, 32, 64, 128, 256]))
    nseq = int(g.integers(1, 5))
    lens = g.integers(1, 6000, nseq).astype(np.int64)
    m = int(g.integers(3, 80))
    if m * B > 16384:
        m = 16384 // B
    k = int(g.integers(1, m * B + 1))
    k = min(k, 2048)
    nq = int(g.choice([int(g.integers(1, 40)), int(g.integers(200, 300)), int(g.integers(500, 700))]))
    return g, B, nseq, lens, m, k, nq


@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_shape(seed):
    g, B, nseq, lens, m, k, nq = _case(seed)
    print("sweep %d: B=%d nseq=%d lens=%s m=%d k=%d nq=%d" % (seed, B, nseq, lens.tolist(), m, k, nq), flush=True)
    from long_context_sparse_hisa_amd import device as dv
    w = synth.decode_batch(nseq=nseq, L=int(lens.max()), seed=2000 + seed, B=B, m=m, k=k)
    cache = dv.DeviceCache(w, B=B)
    cache.set_lengths(lens)
    cache.pool()
    q_seq = g.integers(0, nseq, nq).astype(np.int32)
    q_pos = np.array([g.integers(0, lens[s]) for s in q_seq], np.int64)
    bad = g.random(nq) < 0.03                      # a few invalid queries
    q_seq[bad] = nseq
    queries = synth.to_bf16(g.standard_normal((nq, synth.D)).astype(np.float32))
    reps = [oracle.pool(w.keys[int(w.seq_key_off[s]):int(w.seq_key_off[s]) + int(lens[s])], B) for s in range(nseq)]
    rows = sorted(set(g.choice(nq, min(nq, 40), replace=False).tolist()) | {0, nq - 1})
    for flat in (False, True):
        call = dv.IndexCall(cache, queries, q_pos, q_seq, k=k, m=m, flat=flat)
        call.run()
        idx, sc, blk = call.results()
        for i in np.nonzero(bad)[0]:
            assert np.all(idx[i] == -1), "invalid query %d" % i
        ok = ~bad
        check_all_rows_properties(idx[ok], None if flat else blk[ok], q_pos[ok], B, m, k, flat)
        good = [i for i in rows if ok[i]]
        check_rows(good, queries, q_pos,
                   lambda i: w.keys[int(w.seq_key_off[q_seq[i]]):int(w.seq_key_off[q_seq[i]]) + int(lens[q_seq[i]])],
                   lambda i: reps[int(q_seq[i])], B, m, k, idx, sc, blk, flat, "sweep%d" % seed)
