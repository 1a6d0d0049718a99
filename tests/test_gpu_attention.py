"""Sparse attention over the selected tokens: the HIP path vs the fp64 CPU
oracle, through the C ABI, on the GPU.

Tolerance.  The kernel computes in fp32 on bf16 inputs.  A score is a sum of
128 exact bf16 products over a chain of at most 12 fp32 additions, so its
error is below 12 u sum|q_i k_i| (u = 2^-24); for N(0, 1) rows and scale
1/sqrt(128) that is about 5e-6, which moves a weight by the same relative
amount and the output by at most twice that times max|v| (about 5).  The
weighted value sums and the weight sum pass through at most 40 fp32
additions (8 per lane, 16 row groups, 16 chunks), another 40 u max|v| in
numerator and denominator.  Together below 1e-4; ATOL doubles it.  With a
zero query every weight is exactly 1 and only the sums remain: ATOL_MEAN.
"""
import numpy as np
import pytest

import oracle
from long_context_sparse_hisa_amd import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

ATOL = 2e-4
ATOL_MEAN = 3e-5
SCALE = 1.0 / np.sqrt(synth.DA)


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from long_context_sparse_hisa_amd import hisa
    hisa.lib()                                  # raises if the library is missing


def _gpu(qa, ka, va, idx, scale=SCALE, **kw):
    from long_context_sparse_hisa_amd import device
    call = device.AttentionCall(qa, ka, va, idx, scale, **kw)
    call.run()
    return call.result()


def _random_rows(g, nq, kk, L, fill):
    """Index rows with `fill` of kk entries drawn from [0, L) (distinct),
    the rest -1 or out of range, mixed in at random positions."""
    idx = np.full((nq, kk), -1, np.int32)
    for i in range(nq):
        n = int(min(fill[i], L, kk))
        row = np.full(kk, -1, np.int32)
        row[:n] = g.choice(L, n, replace=False)
        extra = kk - n
        if extra:
            row[n:] = np.where(g.random(extra) < 0.5, -1, L + g.integers(0, 1000, extra))
        idx[i] = g.permutation(row)
    return idx


def _check(got, want, atol=ATOL, label=""):
    err = np.abs(got - want)
    i, c = np.unravel_index(np.argmax(err), err.shape)
    assert err[i, c] <= atol, "%s row %d col %d: got %r want %r" % (label, i, c, got[i, c], want[i, c])


@pytest.mark.parametrize("L,kk,nq", [(1, 1, 4), (100, 50, 16), (1000, 128, 16), (1000, 129, 16),
                                     (5000, 300, 24), (5000, 2048, 8), (20000, 16384, 2)])
def test_small_grid(L, kk, nq):
    print("attention L=%d kk=%d nq=%d" % (L, kk, nq), flush=True)
    g = np.random.default_rng(L + kk)
    qa, ka, va = synth.attention_inputs(L, nq, seed=40 + kk)
    fill = g.integers(0, kk + 1, nq)
    fill[0] = kk                                  # one full row
    if nq > 1:
        fill[1] = 0                               # one empty row
    idx = _random_rows(g, nq, kk, L, fill)
    got = _gpu(qa, ka, va, idx)
    want = oracle.attention_batch(qa, ka, va, np.zeros(nq, np.int64), np.full(nq, L, np.int64), idx, SCALE)
    _check(got, want, label="L=%d kk=%d" % (L, kk))
    empty = ~((idx >= 0) & (idx < L)).any(1)
    assert np.all(got[empty] == 0.0)


def test_packed_sequences_and_invalid_queries():
    print("attention packed", flush=True)
    g = np.random.default_rng(50)
    lens = np.array([3000, 1, 700], np.int64)
    offs = np.array([0, 3000, 3001], np.int64)
    rows = int(offs[-1] + lens[-1])
    nq, kk = 12, 256
    qa, ka, va = synth.attention_inputs(rows, nq, seed=51)
    q_seq = np.array([0, 1, 2, 0, -1, 2, 3, 1, 0, 2, 2, 0], np.int32)
    L_of = np.array([lens[s] if 0 <= s < 3 else 1 for s in q_seq])
    idx = np.stack([_random_rows(g, 1, kk, int(L_of[i]), [int(g.integers(1, kk + 1))])[0] for i in range(nq)])
    got = _gpu(qa, ka, va, idx, q_seq=q_seq, seq_key_off=offs, seq_len=lens)
    key_off = np.array([offs[s] if 0 <= s < 3 else 0 for s in q_seq], np.int64)
    q_len = np.array([lens[s] if 0 <= s < 3 else -1 for s in q_seq], np.int64)
    want = oracle.attention_batch(qa, ka, va, key_off, q_len, idx, SCALE)
    _check(got, want, label="packed")
    assert np.all(got[(q_seq < 0) | (q_seq >= 3)] == 0.0)


def test_zero_query_gives_the_mean():
    print("attention zero query", flush=True)
    g = np.random.default_rng(52)
    L, kk = 40000, 2048
    _, ka, va = synth.attention_inputs(L, 1, seed=53)
    qa = np.zeros((3, synth.DA), np.uint16)
    idx = np.stack([np.sort(g.choice(L, kk, replace=False)) for _ in range(3)]).astype(np.int32)
    got = _gpu(qa, ka, va, idx)
    want = np.stack([synth.from_bf16(va[idx[i]]).astype(np.float64).mean(0) for i in range(3)])
    _check(got, want, atol=ATOL_MEAN, label="mean")


def test_large_scores_pick_the_matching_key():
    """Scores in the thousands: only the running-maximum subtraction keeps
    the exponentials finite."""
    print("attention large scores", flush=True)
    L, kk = 3000, 512
    qa, ka, va = synth.attention_inputs(L, 4, seed=54)
    g = np.random.default_rng(55)
    idx = np.stack([g.choice(L, kk, replace=False) for _ in range(4)]).astype(np.int32)
    hit = idx[np.arange(4), [0, 130, 300, 511]]
    qa = synth.to_bf16(synth.from_bf16(ka[hit]) * np.float32(30.0))
    got = _gpu(qa, ka, va, idx, scale=1.0)
    assert np.all(np.isfinite(got))
    want = oracle.attention_batch(qa, ka, va, np.zeros(4, np.int64), np.full(4, L, np.int64), idx, 1.0)
    _check(got, want, label="large")


@pytest.mark.parametrize("flat", [False, True])
def test_decode_32k_x16_over_oracle_indices(flat):
    """The decode workload end to end at full size: the oracle's index rows
    for the 16 queries (HISA and flat) feed both attentions."""
    print("attention decode 32K x16 flat=%d" % flat, flush=True)
    w = synth.decode_batch()
    ph = w.phases[0]
    reps = None
    if not flat:
        reps = np.concatenate([oracle.pool(w.keys[int(o):int(o) + int(n)], w.B)
                               for o, n in zip(w.seq_key_off, w.seq_len)])
    idx, _, _ = oracle.index_batch(flat, ph.queries, ph.q_pos, w.keys, w.k, reps=reps, q_seq=ph.q_seq,
                                   seq_key_off=w.seq_key_off, seq_rep_off=w.seq_rep_off(),
                                   seq_len=w.seq_len, B=w.B, m=w.m)
    qa, ka, va = synth.attention_inputs(w.keys.shape[0], len(ph.queries), seed=56)
    got = _gpu(qa, ka, va, idx, q_seq=ph.q_seq, seq_key_off=w.seq_key_off, seq_len=w.seq_len)
    want = oracle.attention_batch(qa, ka, va, w.seq_key_off[ph.q_seq], w.seq_len[ph.q_seq], idx, SCALE)
    _check(got, want, label="decode flat=%d" % flat)


def test_repeated_calls_and_graph_replays_agree():
    """Eager calls and replays of a captured call on one workspace give
    bit-identical outputs, also when the indices change between replays."""
    print("attention repeats + graph", flush=True)
    from long_context_sparse_hisa_amd import device
    g = np.random.default_rng(57)
    L, kk, nq = 9000, 1000, 20
    qa, ka, va = synth.attention_inputs(L, nq, seed=58)
    idx1 = _random_rows(g, nq, kk, L, g.integers(1, kk + 1, nq))
    idx2 = _random_rows(g, nq, kk, L, g.integers(1, kk + 1, nq))
    call = device.AttentionCall(qa, ka, va, idx1, SCALE)
    first = None
    for _ in range(3):
        call.run()
        r = call.result()
        first = r if first is None else first
        assert np.array_equal(r, first)
    want1 = oracle.attention_batch(qa, ka, va, np.zeros(nq, np.int64), np.full(nq, L, np.int64), idx1, SCALE)
    want2 = oracle.attention_batch(qa, ka, va, np.zeros(nq, np.int64), np.full(nq, L, np.int64), idx2, SCALE)
    _check(first, want1, label="repeat")
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call.run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        call.run()
    d1 = device.to_dev(idx1, "cuda:0")
    d2 = device.to_dev(idx2, "cuda:0")
    for rep in range(4):
        call.idx.copy_(d2 if rep % 2 else d1)
        graph.replay()
        torch.cuda.synchronize()
        got = call.out.cpu().numpy()
        if rep % 2:
            _check(got, want2, label="replay %d" % rep)
        else:
            assert np.array_equal(got, first)
