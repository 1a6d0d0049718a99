"""Token scores of sparse kept lists, block-major (many queries of one
sequence, 8m <= blocks <= 128m, m <= 64 and a multiple of 4): each kept
(row, block) pair scored once by the workgroup that holds the block's
keepers.  Every row against the oracle, through the C ABI."""
import numpy as np
import pytest

import oracle
from long_context_sparse_hisa_amd import synth
from parity import check_all_rows_properties, check_batch

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from long_context_sparse_hisa_amd import hisa
    hisa.lib()                                  # raises if the library is missing


def _dev():
    from long_context_sparse_hisa_amd import device
    return device


def _check_all(w, cache, ph, k, m, label, bad=None):
    call = _dev().IndexCall(cache, ph.queries, ph.q_pos, ph.q_seq, k=k, m=m, flat=False)
    call.run()
    idx, sc, blk = call.results()
    if bad is not None:
        assert np.all(idx[bad] == -1) and np.all(blk[bad] == -1) and np.all(np.isnan(sc[bad]))
        keep = np.nonzero(~bad)[0]
        ph = synth.Phase("p", ph.queries[keep], ph.q_pos[keep], ph.q_seq[keep])
        idx, sc, blk = idx[keep], sc[keep], blk[keep]
    B = cache.B
    lens = np.asarray(cache.seq_len, np.int64)
    check_all_rows_properties(idx, blk, ph.q_pos, B, m, k, False)
    reps = oracle.pool(w.keys[:int(lens[0])], B)

    def K_of(i):
        return w.keys[:int(lens[0])]

    def R_of(i):
        return reps

    counts = check_batch(ph, w.keys, lens, w.seq_key_off, reps, np.zeros(1, np.int64), B, m, k, idx, sc, blk, False,
                         K_of, R_of, label)
    print(label, counts, flush=True)
    assert counts["exact"] + counts["excused"] == len(ph.q_pos)


@pytest.mark.parametrize("L,B,m,k", [(20000, 32, 40, 1000), (60000, 64, 32, 1500), (32768, 16, 64, 1024),
                                     (131072, 16, 64, 1024)])
def test_gather_every_row_with_invalid_queries(L, B, m, k):
    """700 queries (a ragged last tile of 188 rows) at random positions of
    one MoG sequence, one in 13 past the sequence's end (a -1 row), the
    first few keeping every causal block; the last shape sits at the
    largest block count the block-major form takes (128m: about two
    keepers per block and tile)."""
    print("gather L=%d B=%d m=%d k=%d" % (L, B, m, k), flush=True)
    dv = _dev()
    Mb = (L + B - 1) // B
    assert 8 * m <= Mb <= 128 * m and m % 4 == 0
    g = np.random.default_rng(L + m)
    nq = 700
    pos = np.sort(g.choice(np.arange(L), nq, replace=False)).astype(np.int64)
    pos[:3] = [0, B * (m - 1), B * m - 1]                # every causal block kept
    bad = np.zeros(nq, bool)
    bad[7::13] = True
    w = synth.chunked_prefill(L=L, seed=71, B=B, m=m, k=k, q_positions=pos)
    q_pos = pos.copy()
    q_pos[bad] = L + 5
    ph = synth.Phase("p", w.phases[0].queries, q_pos, np.zeros(nq, np.int32))
    cache = dv.DeviceCache(w, B=B)
    cache.pool()
    _check_all(w, cache, ph, k, m, "gather", bad=bad)
