"""The many-row, many-block stage 1 (rows of more than 1,024 blocks, m - 3
at most 64): two MFMA walks over the representatives with no score row in
memory, a per-row threshold from the first walk, the exact top m-3 of the
blocks the second walk lists, and the from-scratch reselection of rows
whose list cannot certify the result.  HIP path against the oracle,
through the C ABI."""
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


def _run(cache, ph, k, m, **kw):
    call = _dev().IndexCall(cache, ph.queries, ph.q_pos, ph.q_seq, k=k, m=m, flat=False, **kw)
    call.run()
    return call.results()


def _check_all(w, cache, ph, k, m, label, **kw):
    """Every row against one batched oracle call, plus the row properties."""
    idx, sc, blk = _run(cache, ph, k, m, **kw)
    B = cache.B
    lens = np.asarray(cache.seq_len, np.int64)
    check_all_rows_properties(idx, blk, ph.q_pos, B, m, k, False)
    reps_list = [oracle.pool(w.keys[int(w.seq_key_off[s]):int(w.seq_key_off[s]) + int(lens[s])], B)
                 for s in range(len(lens))]
    reps = np.concatenate(reps_list)
    rep_off = np.concatenate([[0], np.cumsum([len(r) for r in reps_list])[:-1]]).astype(np.int64)

    def K_of(i):
        s = int(ph.q_seq[i])
        o = int(w.seq_key_off[s])
        return w.keys[o:o + int(lens[s])]

    def R_of(i):
        return reps_list[int(ph.q_seq[i])]

    counts = check_batch(ph, w.keys, lens, w.seq_key_off, reps, rep_off, B, m, k, idx, sc, blk, False, K_of, R_of,
                         label)
    print(label, counts, flush=True)
    assert counts["exact"] + counts["excused"] == len(ph.q_pos)
    return idx, sc, blk


@pytest.mark.parametrize("L,B,m,k,iid", [
    (200000, 128, 64, 2048, False),     # 1,563 blocks: formerly the 256-thread fused select
    (70000, 16, 67, 1000, False),       # 4,375 blocks, m - 3 = 64: the largest the walks take
    (70000, 16, 4, 64, False),          # m - 3 = 1
    (90000, 32, 20, 512, True),         # i.i.d. keys and queries, 2,813 blocks
])
def test_walks_every_row(L, B, m, k, iid):
    """600 queries at random positions past 1,024 blocks (the first of them
    keeps every causal block when c + 1 <= m is reached), every row against
    the oracle."""
    print("walks L=%d B=%d m=%d k=%d iid=%s" % (L, B, m, k, iid), flush=True)
    dv = _dev()
    g = np.random.default_rng(L + B + m)
    nq = 600
    pos = np.sort(g.choice(np.arange(1024 * B, L), nq - 1, replace=False)).astype(np.int64)
    pos = np.concatenate([[min(L - 1, B * (m - 1))], pos]).astype(np.int64)    # one row keeps every block
    w = synth.chunked_prefill(L=L, seed=61, B=B, m=m, k=k, q_positions=pos)
    if iid:
        keys = synth.to_bf16(g.standard_normal((L, synth.D)).astype(np.float32))
        queries = synth.to_bf16(g.standard_normal((nq, synth.D)).astype(np.float32))
        w = synth.Workload("iid", keys, w.seq_key_off, w.seq_len, w.seq_cap, B, m, k)
        w.phases.append(synth.Phase("p", queries, pos, np.zeros(nq, np.int32)))
    cache = dv.DeviceCache(w, B=B)
    cache.pool()
    _check_all(w, cache, w.phases[0], k, m, "walks")


@pytest.mark.parametrize("kind", ["constant", "quantized", "half_zero_queries"])
def test_walks_ties(kind):
    """Scores with heavy ties at the threshold: one score for every block
    (every free block passes the threshold, more than a list holds: every
    row is reselected from scratch and keeps the lowest free blocks), five
    score values, and MoG rows where every other query is zero (those rows
    tie everywhere, the others take the walks' lists)."""
    print("walk ties %s" % kind, flush=True)
    dv = _dev()
    L, B, m, k = 150000, 128, 64, 2048
    g = np.random.default_rng(62)
    nq = 320 if kind != "half_zero_queries" else 600
    pos = np.sort(g.choice(np.arange(140000, L), nq, replace=False)).astype(np.int64)
    w = synth.chunked_prefill(L=L, seed=63, B=B, m=m, k=k, q_positions=pos)
    keys, queries = w.keys, w.phases[0].queries
    if kind == "constant":
        kf = np.zeros((L, synth.D), np.float32)
        kf[:, :4] = 1.0
        keys = synth.to_bf16(kf)
        qf = np.zeros((nq, synth.D), np.float32)
        qf[:, :4] = 1.0
        queries = synth.to_bf16(qf)
    elif kind == "quantized":
        kf = np.zeros((L, synth.D), np.float32)
        kf[:, :4] = g.choice([-1.0, 1.0], size=(L, 4))
        keys = synth.to_bf16(kf)
        qf = np.zeros((nq, synth.D), np.float32)
        qf[:, :4] = 1.0
        queries = synth.to_bf16(qf)
    else:
        queries = queries.copy()
        queries[::2] = 0
    w2 = synth.Workload(kind, keys, w.seq_key_off, w.seq_len, w.seq_cap, B, m, k)
    ph = synth.Phase("p", queries, pos, np.zeros(nq, np.int32))
    w2.phases.append(ph)
    cache = dv.DeviceCache(w2, B=B)
    cache.pool()
    nrows_many = nq >= 256                      # the many-row stage 1
    assert nrows_many
    idx, _, blk = _check_all(w2, cache, ph, k, m, "ties-" + kind)
    tie_rows = np.arange(nq) if kind == "constant" else (np.arange(0, nq, 2) if kind == "half_zero_queries" else [])
    for i in tie_rows:
        c = int(pos[i]) // B
        want = list(range(0, m - 2)) + [c - 1, c]
        assert list(blk[i]) == want, (i, list(blk[i])[:8])


def test_walks_packed_with_invalid_queries():
    """Queries in random order over packed sequences whose declared max_len
    gives 16,384 blocks of 16 (so every call takes the walks), with invalid
    queries (past their sequence) and rows that keep every causal block
    mixed in: 64-row tiles span several sequences and are walked one
    sequence at a time."""
    print("walks packed", flush=True)
    dv = _dev()
    nseq, B, m, k = 5, 16, 40, 512
    g = np.random.default_rng(64)
    lens = g.integers(3000, 60000, nseq).astype(np.int64)
    w = synth.decode_batch(nseq=nseq, L=int(lens.max()), seed=65, B=B, m=m, k=k)
    cache = dv.DeviceCache(w, B=B)
    cache.set_lengths(lens)
    cache.pool()
    nq = 900
    q_seq = g.integers(0, nseq, nq).astype(np.int32)
    q_pos = (g.random(nq) * lens[q_seq]).astype(np.int64)
    q_pos[5::53] = g.integers(0, B * m, len(q_pos[5::53]))   # every causal block kept
    q_pos[::41] = lens[q_seq[::41]] + 3                 # past the sequence: a -1 row
    queries = synth.to_bf16(g.standard_normal((nq, synth.D)).astype(np.float32))
    ph = synth.Phase("p", queries, q_pos, q_seq)
    bad = np.zeros(nq, bool)
    bad[::41] = True
    idx, sc, blk = _run(cache, ph, k, m, max_len=262144)
    assert np.all(idx[bad] == -1) and np.all(blk[bad] == -1)
    good = np.nonzero(~bad)[0]
    ph_good = synth.Phase("p", queries[good], q_pos[good], q_seq[good])
    _check_all(w, cache, ph_good, k, m, "walks-packed", max_len=262144)
