"""HIP path vs the CPU oracle, through the C ABI, on the GPU."""
import numpy as np
import pytest

import oracle
from long_context_sparse_hisa_amd import synth
from parity import check_all_rows_properties, check_batch, check_rows

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


def _oracle_reps(w, B, lengths=None):
    lengths = w.seq_len if lengths is None else lengths
    out = []
    for s in range(w.nseq):
        o = int(w.seq_key_off[s])
        out.append(oracle.pool(w.keys[o:o + int(lengths[s])], B))
    return out


def _gpu_reps(cache, s, n):
    r = int(cache.seq_rep_off[s])
    nb = (n + cache.B - 1) // cache.B
    return cache.reps[r:r + nb].cpu().numpy().view(np.uint16)


# ---- pooling and append -------------------------------------------------------

@pytest.mark.parametrize("L,B", [(1, 16), (100, 16), (128, 128), (1000, 64), (4097, 128), (5000, 256),
                                 (70000, 128)])
def test_pool_bitwise(L, B):
    print("pool L=%d B=%d" % (L, B), flush=True)
    dv = _dev()
    w = synth.chunked_prefill(L=L, seed=21, B=B, q_positions=[0])
    cache = dv.DeviceCache(w, B=B)
    cache.pool()
    torch.cuda.synchronize()
    assert np.array_equal(_gpu_reps(cache, 0, L), oracle.pool(w.keys, B))


def test_pool_rounding_ties():
    print("pool ties", flush=True)
    dv = _dev()
    B = 16
    vals = []
    for x in (1.0625, 1.1875, -1.0625, -1.1875, 3.0, 0.0):   # the first four give exact midpoints
        blk = np.full((B, synth.D), 1.0 if x >= 0 else -1.0, np.float32)
        blk[0] = x
        vals.append(blk)
    keys = synth.to_bf16(np.concatenate(vals + [np.full((5, synth.D), 2.5, np.float32)]))
    w = synth.Workload("ties", keys, np.zeros(1, np.int64), np.array([len(keys)], np.int64),
                       np.array([len(keys)], np.int64), B, 3, 1)
    cache = dv.DeviceCache(w, B=B)
    cache.pool()
    torch.cuda.synchronize()
    got = _gpu_reps(cache, 0, len(keys))
    want = oracle.pool(keys, B)
    assert np.array_equal(got, want)
    assert got[0, 0] == 0x3F80 and got[1, 0] == 0x3F82            # ties to even


def test_append_matches_one_shot_pooling():
    print("append", flush=True)
    dv = _dev()
    B = 64
    g = np.random.default_rng(22)
    caps = np.array([900, 700, 1000], np.int64)
    init = np.array([0, 77, 128], np.int64)
    offs = np.concatenate([[0], np.cumsum(caps)[:-1]]).astype(np.int64)
    full = synth.to_bf16(g.standard_normal((int(caps.sum()), synth.D)).astype(np.float32))
    keys = np.zeros_like(full)
    for s in range(3):
        keys[offs[s]:offs[s] + init[s]] = full[offs[s]:offs[s] + init[s]]
    w = synth.Workload("append", keys, offs, init.copy(), caps, B, 3, 1)
    cache = dv.DeviceCache(w, B=B)
    cache.pool()
    lens = init.copy()
    for n_new in (1, 37, 64, 128, 200, 5):
        new = np.stack([full[offs[s] + lens[s]: offs[s] + lens[s] + n_new] for s in range(3)])
        cache.append(new)
        lens += n_new
        torch.cuda.synchronize()
        kk = cache.keys.cpu().numpy().view(np.uint16)
        for s in range(3):
            o = int(offs[s])
            assert np.array_equal(kk[o:o + lens[s]], full[o:o + lens[s]])
            assert np.array_equal(_gpu_reps(cache, s, int(lens[s])), oracle.pool(full[o:o + lens[s]], B))


# ---- index: small grids checked row by row ----------------------------------------

def _run(cache, ph, k, m, flat, **kw):
    call = _dev().IndexCall(cache, ph.queries, ph.q_pos, ph.q_seq, k=k, m=m, flat=flat, **kw)
    call.run()
    return call.results()


def _check_phase(w, cache, ph, k, m, flat, rows=None, label="", props=True, **kw):
    idx, sc, blk = _run(cache, ph, k, m, flat, **kw)
    B = cache.B
    lens = cache.seq_len
    reps = None if flat else _oracle_reps(w, B, lens)
    if props:
        check_all_rows_properties(idx, blk, ph.q_pos, B, m, k, flat)

    def K_of(i):                       # host keys: nothing the oracle reads comes from the GPU
        s = int(ph.q_seq[i])
        o = int(w.seq_key_off[s])
        return w.keys[o:o + int(lens[s])]

    def R_of(i):
        return reps[int(ph.q_seq[i])]

    rows = range(len(ph.q_pos)) if rows is None else rows
    counts = check_rows(rows, ph.queries, ph.q_pos, K_of, R_of, B, m, k, idx, sc, blk, flat, label)
    print(label, "flat" if flat else "hisa", counts, flush=True)
    return idx, sc, blk


@pytest.mark.parametrize("L,B,m,k,iid", [
    (300, 16, 3, 1, True), (300, 16, 5, 17, False), (1000, 64, 4, 100, False),
    (1000, 128, 8, 256, True), (2500, 32, 6, 150, False), (4097, 128, 8, 300, False),
    (3000, 256, 3, 700, False), (1500, 16, 64, 1024, False)])
def test_index_small_grid(L, B, m, k, iid):
    print("grid L=%d B=%d m=%d k=%d iid=%s" % (L, B, m, k, iid), flush=True)
    dv = _dev()
    if iid:
        w = synth.tiny_prefill(L=L, seed=23, B=B, m=m, k=k)
    else:
        w = synth.chunked_prefill(L=L, seed=23, B=B, m=m, k=k)
    cache = dv.DeviceCache(w, B=B)
    cache.pool()
    ph = w.phases[0]
    for flat in (False, True):
        _check_phase(w, cache, ph, k, m, flat, label="grid%d" % L)


@pytest.mark.parametrize("B,m,k", [(16, 1024, 2048), (16, 500, 1000), (32, 300, 4000), (128, 128, 4096),
                                   (64, 256, 3000)])
def test_many_queries_long_kept_lists(B, m, k):
    """Enough queries for the matrix-core token scores, with kept-block
    lists long enough that a wave serves one (m = 1024), two (m = 500, 256)
    or four (m = 300, 128) 16-query sub-tiles; the last two also take the
    16,384-candidate rows of the 512-thread top-k with per-wave token
    bases (B >= 64)."""
    print("long kept lists B=%d m=%d k=%d" % (B, m, k), flush=True)
    dv = _dev()
    L = 20000
    pos = np.arange(3, L, 33, dtype=np.int64)       # 606 queries, every block size of row
    w = synth.chunked_prefill(L=L, seed=29, B=B, m=m, k=k, q_positions=pos)
    cache = dv.DeviceCache(w, B=B)
    cache.pool()
    g = np.random.default_rng(B + m)
    rows = sorted(set([0, 1, 15, 16, 63, 64, len(pos) - 1] + list(g.choice(len(pos), 80, replace=False))))
    _check_phase(w, cache, w.phases[0], k, m, False, rows=rows, label="longlists")


@pytest.mark.parametrize("B,m,k", [(32, 40, 1000), (64, 16, 900), (128, 16, 2000), (256, 8, 1500), (16, 60, 700)])
def test_many_queries_sparse_kept_lists(B, m, k):
    """Matrix-core token scores where the kept lists cover a small part of
    the block range (at least 8 blocks per kept block), which the tile walk
    takes in pieces of one 16-key tile with the next piece loading while
    one is scored (B = 16 has a single tile per block)."""
    print("sparse kept lists B=%d m=%d k=%d" % (B, m, k), flush=True)
    dv = _dev()
    L = 20000
    assert (L + B - 1) // B >= 8 * m
    pos = np.arange(5, L, 31, dtype=np.int64)       # 645 queries
    w = synth.chunked_prefill(L=L, seed=33, B=B, m=m, k=k, q_positions=pos)
    cache = dv.DeviceCache(w, B=B)
    cache.pool()
    g = np.random.default_rng(B * 7 + m)
    rows = sorted(set([0, 1, 15, 16, 63, 64, len(pos) - 1] + list(g.choice(len(pos), 80, replace=False))))
    _check_phase(w, cache, w.phases[0], k, m, False, rows=rows, label="sparselists")


@pytest.mark.parametrize("kind,B,m,k", [("prefill", 128, 8, 256), ("prefill", 32, 12, 300), ("prefill", 64, 128, 4096),
                                         ("decode", 128, 16, 512), ("decode", 32, 40, 900)])
def test_indices_without_scores_equal_with_scores(kind, B, m, k):
    """The index rows do not depend on whether the optional scores are
    written (the calls the benchmark times request none); the rows with
    scores are checked against the oracle elsewhere."""
    print("no-scores %s B=%d m=%d k=%d" % (kind, B, m, k), flush=True)
    dv = _dev()
    if kind == "prefill":
        w = synth.chunked_prefill(L=9000, seed=31, B=B, m=m, k=k, q_positions=np.arange(0, 9000, 7))
    else:
        w = synth.decode_batch(nseq=6, L=20000, seed=31, B=B, m=m, k=k)
    cache = dv.DeviceCache(w, B=B)
    cache.pool()
    ph = w.phases[0]
    for flat in (False, True):
        a = dv.IndexCall(cache, ph.queries, ph.q_pos, ph.q_seq, k=k, m=m, flat=flat)
        b = dv.IndexCall(cache, ph.queries, ph.q_pos, ph.q_seq, k=k, m=m, flat=flat, scores=False)
        a.run()
        b.run()
        ia = a.results()[0]
        ib = b.results()[0]
        assert np.array_equal(ia, ib), "%s flat=%s: rows differ without scores" % (kind, flat)


def test_small_workspace_forces_chunks():
    print("chunked workspace", flush=True)
    dv = _dev()
    w = synth.chunked_prefill(L=2000, seed=24, B=64, m=6, k=200)
    cache = dv.DeviceCache(w, B=64)
    cache.pool()
    ph = w.phases[0]
    full_h, _, full_b = _run(cache, ph, 200, 6, False)
    from long_context_sparse_hisa_amd import hisa
    probe = dv.IndexCall(cache, ph.queries, ph.q_pos, ph.q_seq, k=200, m=6)
    _, least = hisa.hisa_workspace_bytes(probe.args)
    small_h, _, small_b = _run(cache, ph, 200, 6, False, workspace_bytes=least * 7 + 100)
    assert np.array_equal(full_h, small_h) and np.array_equal(full_b, small_b)
    full_f, _, _ = _run(cache, ph, 200, 6, True)
    probe = dv.IndexCall(cache, ph.queries, ph.q_pos, ph.q_seq, k=200, m=6, flat=True)
    _, least = hisa.hisa_workspace_bytes(probe.args, True)
    small_f, _, _ = _run(cache, ph, 200, 6, True, workspace_bytes=least * 3)
    assert np.array_equal(full_f, small_f)


def test_packed_sequences_and_invalid_queries():
    print("packed", flush=True)
    dv = _dev()
    w = synth.decode_batch(nseq=5, L=3000, seed=25, B=64, m=5, k=300, spare=100)
    cache = dv.DeviceCache(w, B=64)
    cache.set_lengths([3000, 1, 640, 2999, 1500])
    cache.pool()
    ph = w.phases[0]
    q_pos = np.array([2999, 0, 639, 2000, 1500], np.int64)      # the last is past its end
    q_seq = np.array([0, 1, 2, 3, 4], np.int32)
    ph2 = synth.Phase("p", ph.queries, q_pos, q_seq)
    for flat in (False, True):
        idx, sc, blk = _run(cache, ph2, 300, 5, flat)
        assert np.all(idx[4] == -1) and np.all(np.isnan(sc[4]))
        if not flat:
            assert np.all(blk[4] == -1)
        _check_phase(w, cache, ph2, 300, 5, flat, rows=[0, 1, 2, 3], label="packed", props=False)
    bad = synth.Phase("bad", ph.queries[:2], np.array([5, 5], np.int64), np.array([-1, 7], np.int32))
    for flat in (False, True):
        idx, _, _ = _run(cache, bad, 300, 5, flat)
        assert np.all(idx == -1)


def test_degenerate_ties_pick_lowest_indices():
    print("ties", flush=True)
    dv = _dev()
    L, B = 3000, 64
    keys = np.tile(synth.to_bf16(np.linspace(-1, 1, synth.D).astype(np.float32)), (L, 1))
    q = synth.to_bf16(np.ones((3, synth.D), np.float32))
    q[2] = 0                                               # zero query: every score is 0
    w = synth.Workload("ties", keys, np.zeros(1, np.int64), np.array([L], np.int64),
                       np.array([L], np.int64), B, 6, 100)
    ph = synth.Phase("p", q, np.array([2999, 1234, 2500], np.int64), np.zeros(3, np.int32))
    cache = dv.DeviceCache(w, B=B)
    cache.pool()
    for flat in (False, True):
        idx, _, blk = _check_phase(w, cache, ph, 100, 6, flat, label="ties")
        if flat:
            assert np.array_equal(idx[0], np.arange(100))


def test_signed_zero_scores_tie():
    """Scores -0.0 and +0.0 compare equal, so the two tie and the lower
    index goes first (the oracle sorts the fp32 values).  Query all ones;
    keys all -1 except five rows of +1 (scores 64), row 20 of -0.0 (score
    -0.0: every product is -0) and row 30 of +0.0 (score +0.0); k = 6 takes
    the five positives and one zero, which must be row 20."""
    print("signed zeros", flush=True)
    dv = _dev()
    L, B = 600, 64
    keys = np.full((L, synth.D), synth.to_bf16(np.float32(-1.0)), np.uint16)
    keys[10:15] = synth.to_bf16(np.float32(1.0))
    keys[20] = 0x8000                                      # bf16 -0.0
    keys[30] = 0x0000                                      # bf16 +0.0
    q = np.full((1, synth.D), synth.to_bf16(np.float32(1.0)), np.uint16)
    w = synth.Workload("zeros", keys, np.zeros(1, np.int64), np.array([L], np.int64),
                       np.array([L], np.int64), B, 10, 6)
    ph = synth.Phase("p", q, np.array([L - 1], np.int64), np.zeros(1, np.int32))
    cache = dv.DeviceCache(w, B=B)
    cache.pool()
    want = np.array([10, 11, 12, 13, 14, 20], np.int32)
    o_idx = oracle.flat_query(q[0], keys, L - 1, 6)[0]
    assert np.array_equal(np.sort(o_idx), want), o_idx
    for flat in (False, True):
        idx, sc, _ = _run(cache, ph, 6, 10, flat)
        assert np.array_equal(np.sort(idx[0]), want), (flat, idx[0])


def test_hisa_with_m_covering_every_block_equals_flat():
    """With m covering every causal block HISA is the flat indexer: its rows
    must pass the parity rule against the oracle's flat result, and where
    the GPU's HISA and flat rows share an index their scores agree (they
    are summed by different units, v_dot2 and MFMA, so not bit for bit)."""
    print("m covers all", flush=True)
    dv = _dev()
    w = synth.chunked_prefill(L=2048, seed=26, B=128, m=16, k=512)
    cache = dv.DeviceCache(w, B=128)
    cache.pool()
    ph = w.phases[0]
    h_idx, h_sc, _ = _run(cache, ph, 512, 16, False)
    f_idx, f_sc, _ = _run(cache, ph, 512, 16, True)
    counts = check_rows(range(len(ph.q_pos)), ph.queries, ph.q_pos, lambda i: w.keys, None, 128, 16, 512,
                        h_idx, h_sc, None, True, "hisa-as-flat")
    print("hisa as flat", counts, flush=True)
    for i in range(len(ph.q_pos)):
        common, hi, fi = np.intersect1d(h_idx[i], f_idx[i], return_indices=True)
        keep = common >= 0
        assert np.all(np.abs(h_sc[i][hi[keep]] - f_sc[i][fi[keep]]) <= 1e-3)


@pytest.mark.parametrize("L,k,nq", [(20000, 2048, 8), (70000, 2048, 8), (70000, 2048, 40), (20000, 5000, 8),
                                    (300000, 1000, 3)])
def test_flat_long_rows(L, k, nq):
    """Rows longer than one workgroup's selection: slices merged in levels
    (few queries: 8192-key slices; many: 16384 and matrix-core scores), or
    the several-workgroup radix select when k is too large to merge."""
    print("flat long L=%d k=%d nq=%d" % (L, k, nq), flush=True)
    dv = _dev()
    g = np.random.default_rng(L + nq)
    pos = np.concatenate([[0, 5, 2047, 2048, 9999 % L, L // 2, L - 2, L - 1],
                          g.integers(0, L, max(0, nq - 8))])[:nq].astype(np.int64)
    w = synth.chunked_prefill(L=L, seed=27, B=128, m=16, k=k, q_positions=pos)
    cache = dv.DeviceCache(w, B=128)
    cache.pool()
    _check_phase(w, cache, w.phases[0], k, 16, True, label="flatlong")
    # ties across slices: a run of equal keys longer than k
    keys = w.keys.copy()
    keys[1000:9000] = keys[1000]
    w2 = synth.Workload("ties", keys, w.seq_key_off, w.seq_len, w.seq_cap, 128, 16, 2048)
    cache2 = dv.DeviceCache(w2, B=128)
    q = np.repeat(keys[1000:1001], 2, axis=0)
    ph = synth.Phase("p", q, np.array([L - 1, 8999], np.int64), np.zeros(2, np.int32))
    _check_phase(w2, cache2, ph, 2048, 16, True, label="flatties")


# ---- the five workloads at full size ----------------------------------------------

def test_tiny_prefill_4k_full():
    print("tiny prefill 4K", flush=True)
    dv = _dev()
    w = synth.tiny_prefill()
    cache = dv.DeviceCache(w)
    cache.pool()
    torch.cuda.synchronize()
    assert np.array_equal(_gpu_reps(cache, 0, 4096), oracle.pool(w.keys, 128))
    for flat in (False, True):
        _check_phase(w, cache, w.phases[0], w.k, w.m, flat, label="cfg1")


def test_decode_32k_x16_full():
    print("decode 32K x16", flush=True)
    dv = _dev()
    w = synth.decode_batch()
    cache = dv.DeviceCache(w)
    cache.pool()
    for flat in (False, True):
        _check_phase(w, cache, w.phases[0], w.k, w.m, flat, label="cfg2")


def test_decode_32k_x256_batch():
    """The decode step at 256 sequences (the batch sweep's largest point):
    the stage-1 MFMA tiles, the split token stage and the many-row top-k
    shapes, every query checked."""
    print("decode 32K x256", flush=True)
    dv = _dev()
    w = synth.decode_batch(nseq=256)
    cache = dv.DeviceCache(w)
    cache.pool()
    for flat in (False, True):
        _check_phase(w, cache, w.phases[0], w.k, w.m, flat, label="dec256")


def test_decode_varlen_x64_full():
    """64 sequences of mixed length (4K to 128K keys, log-uniform) in one
    decode launch, every query checked: per-sequence causal bounds and
    forced blocks inside one call."""
    print("decode varlen x64", flush=True)
    dv = _dev()
    w = synth.decode_varlen()
    cache = dv.DeviceCache(w)
    cache.pool()
    for flat in (False, True):
        _check_phase(w, cache, w.phases[0], w.k, w.m, flat, label="varlen")


def _check_phase_all(w, cache, ph, k, m, flat, label="", **kw):
    """Every row of a phase against one batched oracle call (exact rows
    pass at once, the rest through the per-row tolerance rule), plus the
    vectorised row properties."""
    idx, sc, blk = _run(cache, ph, k, m, flat, **kw)
    B = cache.B
    lens = np.asarray(cache.seq_len, np.int64)
    check_all_rows_properties(idx, blk, ph.q_pos, B, m, k, flat)
    reps_list = None if flat else _oracle_reps(w, B, lens)
    reps = None if flat else np.concatenate(reps_list)
    rep_off = None if flat else np.concatenate([[0], np.cumsum([len(r) for r in reps_list])[:-1]]).astype(np.int64)

    def K_of(i):
        s = int(ph.q_seq[i])
        o = int(w.seq_key_off[s])
        return w.keys[o:o + int(lens[s])]

    def R_of(i):
        return reps_list[int(ph.q_seq[i])]

    counts = check_batch(ph, w.keys, lens, w.seq_key_off, reps, rep_off, B, m, k, idx, sc, blk, flat, K_of, R_of,
                         label)
    print(label, "flat" if flat else "hisa", "all rows", counts, flush=True)
    assert counts["exact"] + counts["excused"] == len(ph.q_pos)
    return idx, sc, blk


def test_chunked_prefill_32k_all_rows():
    """All 32768 causal queries of the 32K prefill, every row against the
    oracle (HISA and flat)."""
    print("chunked prefill 32K, all rows", flush=True)
    dv = _dev()
    w = synth.chunked_prefill()
    cache = dv.DeviceCache(w)
    cache.pool()
    for flat in (False, True):
        _check_phase_all(w, cache, w.phases[0], w.k, w.m, flat, label="cfg3")


def test_long_context_128k_all_rows():
    """The 128K context: every row of the 4096-query chunk and of the
    32-query decode batch against the oracle; the flat rows of the decode
    batch hold every planted needle."""
    print("long context 128K, all rows", flush=True)
    dv = _dev()
    w = synth.long_context()
    cache = dv.DeviceCache(w)
    cache.pool()
    chunk, dec = w.phases
    for flat in (False, True):
        _check_phase_all(w, cache, chunk, w.k, w.m, flat, label="cfg4chunk")
        idx, _, _ = _check_phase_all(w, cache, dec, w.k, w.m, flat, label="cfg4decode")
        if flat:
            assert set(w.needles.tolist()) <= set(idx[0].tolist())


def test_long_decode_1m_with_appends():
    print("1M decode + append", flush=True)
    dv = _dev()
    w = synth.long_decode_append()
    cache = dv.DeviceCache(w)
    cache.pool()
    full = w.keys.copy()
    L = int(w.seq_len[0])
    want_reps = oracle.pool(full[:L], 128)
    torch.cuda.synchronize()
    assert np.array_equal(_gpu_reps(cache, 0, L), want_reps)
    for ph in w.phases:
        cache.append(ph.append)
        n_new = ph.append.shape[1]
        full[L:L + n_new] = ph.append[0]
        L += n_new
        torch.cuda.synchronize()
        got = _gpu_reps(cache, 0, L)
        b0 = (L - n_new) // 128
        want = oracle.pool(full[b0 * 128:L], 128)
        assert np.array_equal(got[b0:], want)
        w.keys = full                                    # the oracle reads the grown cache
        for flat in (False, True):
            _check_phase(w, cache, ph, w.k, w.m, flat, label="cfg5 " + ph.name, props=True)


def test_graph_replays_match_eager():
    """A decode step (append + HISA + flat) captured in a HIP graph gives the
    eager result on every replay, with other eager work in between."""
    print("graph replay", flush=True)
    dv = _dev()
    w = synth.decode_batch(nseq=4, L=20000, seed=30, B=128, m=16, k=512, spare=8)
    cache = dv.DeviceCache(w)
    cache.set_lengths(w.seq_len - 1)
    cache.pool()
    last = np.stack([w.keys[int(o) + int(L) - 1] for o, L in zip(w.seq_key_off, w.seq_len)])[:, None]
    new = dv.to_dev(last, cache.device)
    seqs = [(cache.seq_key_off[s], cache.seq_rep_off[s], cache.seq_len[s], cache.seq_cap[s])
            for s in range(cache.nseq)]
    cache.append(new)                        # lengths the queries see
    ph = w.phases[0]
    hcall = dv.IndexCall(cache, ph.queries, ph.q_pos, ph.q_seq, k=512, m=16)
    fcall = dv.IndexCall(cache, ph.queries, ph.q_pos, ph.q_seq, k=512, m=16, flat=True)
    from long_context_sparse_hisa_amd import hisa

    def step():
        hisa.hisa_append_keys(cache.keys, cache.reps, seqs, new, cache.B)
        hcall.run()
        fcall.run()

    step()
    want = [x.copy() for x in hcall.results() + fcall.results() if x is not None]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(4):
        for t in [hcall.out_idx, fcall.out_idx, hcall.out_scores, fcall.out_scores, hcall.out_blocks]:
            t.fill_(7)                        # eager work that the replay must overwrite
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [x for x in hcall.results() + fcall.results() if x is not None]
        for a, b in zip(got, want):
            assert np.array_equal(np.nan_to_num(a, nan=-9), np.nan_to_num(b, nan=-9)), "replay %d" % rep


def test_tie_bin_taken_whole():
    """A run of 600 equal scores (more than the threshold bin's exact-rank
    list holds) that is exactly what the top-k still needs after the larger
    scores: the tie fallback must take that run and nothing below it."""
    print("tie bin taken whole", flush=True)
    dv = _dev()
    L, k = 2000, 1000
    g = np.random.default_rng(31)
    v = np.empty(L, np.float32)
    order = g.permutation(L)
    v[order[:400]] = 8.0 + np.arange(400, dtype=np.float32) / 64.0      # 400 larger, distinct
    v[order[400:1000]] = 4.0                                            # 600 tied
    v[order[1000:]] = -4.0 + np.arange(1000, dtype=np.float32) / 256.0  # 1000 smaller
    keys = np.zeros((L, synth.D), np.float32)
    keys[:, 0] = v
    keys = synth.to_bf16(keys)
    q = np.zeros((1, synth.D), np.float32)
    q[0, 0] = 1.0                                                       # score = first coordinate
    q = synth.to_bf16(q)
    w = synth.Workload("tiebin", keys, np.zeros(1, np.int64), np.array([L], np.int64),
                       np.array([L], np.int64), 64, 32, k)
    ph = synth.Phase("p", q, np.array([L - 1], np.int64), np.zeros(1, np.int32))
    cache = dv.DeviceCache(w, B=64)
    cache.pool()
    for flat in (False, True):                  # m = 32 keeps all 32 blocks: HISA sees every key
        idx, _, _ = _check_phase(w, cache, ph, k, 32, flat, label="tiebin")
        assert np.array_equal(np.sort(idx[0]), np.sort(order[:1000]))


@pytest.mark.parametrize("force_fallback", [False, True])
def test_many_queries_packed_sequences(force_fallback):
    """Hundreds of queries in random order over packed sequences of
    different lengths: 16-query tiles span several sequences, so the MFMA
    tile kernels walk one sequence at a time.  With a declared max_len of
    more blocks than the stage-1 tile kernel holds, stage 1 scores into a
    row per query and selects with one workgroup per query instead."""
    print("many packed queries fallback=%s" % force_fallback, flush=True)
    dv = _dev()
    nseq = 70 if force_fallback else 6
    B = 16 if force_fallback else 64
    m, k = 8, 64
    g = np.random.default_rng(32)
    lens = g.integers(40, 400, nseq).astype(np.int64)
    w = synth.decode_batch(nseq=nseq, L=int(lens.max()), seed=32, B=B, m=m, k=k)
    cache = dv.DeviceCache(w, B=B)
    cache.set_lengths(lens)
    cache.pool()
    nq = 700
    q_seq = g.integers(0, nseq, nq).astype(np.int32)
    q_pos = (g.random(nq) * lens[q_seq]).astype(np.int64)
    queries = synth.to_bf16(g.standard_normal((nq, synth.D)).astype(np.float32))
    ph = synth.Phase("p", queries, q_pos, q_seq)
    max_len = 262144 if force_fallback else None
    for flat in (False, True):
        _check_phase(w, cache, ph, k, m, flat, label="manypacked", props=False, max_len=max_len)


@pytest.mark.parametrize("kind", ["mog", "quantized", "constant"])
def test_many_rows_topk_ties(kind):
    """Hundreds of prefill rows of up to 8,192 candidates (B = 128, m = 64,
    k = 2048) through the many-row top-k (one 256-thread workgroup per row):
    plain keys; scores from five values only (block and token ties across
    the threshold, resolved by the lower index); one score for every key
    (the lowest blocks and tokens win).  The early positions keep every
    causal block."""
    print("many-row top-k %s" % kind, flush=True)
    dv = _dev()
    L, B, m, k = 20000, 128, 64, 2048
    pos = np.concatenate([np.arange(2100, 5400, 97), np.arange(9001, L, 37)]).astype(np.int64)
    w = synth.chunked_prefill(L=L, seed=41, B=B, m=m, k=k, q_positions=pos)
    keys, queries = w.keys, w.phases[0].queries
    if kind != "mog":
        g = np.random.default_rng(42)
        kf = np.zeros((L, synth.D), np.float32)
        if kind == "quantized":
            kf[:, :4] = g.choice([-1.0, 1.0], size=(L, 4))
        else:
            kf[:, :4] = 1.0
        keys = synth.to_bf16(kf)
        qf = np.zeros((len(pos), synth.D), np.float32)
        qf[:, :4] = 1.0
        queries = synth.to_bf16(qf)
    w2 = synth.Workload(kind, keys, w.seq_key_off, w.seq_len, w.seq_cap, B, m, k)
    ph = synth.Phase("p", queries, pos, np.zeros(len(pos), np.int32))
    cache = dv.DeviceCache(w2, B=B)
    cache.pool()
    idx, _, _ = _check_phase(w2, cache, ph, k, m, False, label="pf-" + kind)
    if kind == "constant":
        # every score ties: the lowest blocks and, inside them, the lowest tokens
        t = int(pos[-1])
        c = t // B
        blocks = list(range(0, m - 2)) + [c - 1, c]
        want = np.concatenate([np.arange(b * B, b * B + B) for b in blocks])[:k]
        assert np.array_equal(idx[-1], want)


@pytest.mark.parametrize("nq", [320, 600])
def test_many_queries_long_rows(nq):
    """Hundreds of queries with more representatives than the stage-1 tile
    kernel holds (2,345 blocks of 128 over 300,100 keys; a count not
    divisible by four): with 600 queries the two MFMA walks that select
    without a score row; with 320 (fewer than 512, every query split over
    several workgroups) the representative scores into a row per query
    (the last scores of a row stored one by one), then the selection fused
    with the token scores."""
    print("long rows nq=%d" % nq, flush=True)
    dv = _dev()
    L, B, m, k = 300100, 128, 64, 2048
    g = np.random.default_rng(43 + nq)
    pos = np.sort(g.choice(np.arange(200000, L), nq, replace=False)).astype(np.int64)
    pos[-1] = L - 1
    w = synth.chunked_prefill(L=L, seed=44, B=B, m=m, k=k, q_positions=pos)
    cache = dv.DeviceCache(w, B=B)
    cache.pool()
    _check_phase(w, cache, w.phases[0], k, m, False, label="longrows%d" % nq)


@pytest.mark.parametrize("nq", [12, 600])
def test_largest_block_count(nq):
    """A sequence of exactly the most blocks the index calls accept (16,384
    blocks of 16 over 262,144 keys): the last query sees every block.  With
    12 queries each gets its own score row; with 600 the two MFMA walks
    select from 16,384 blocks per row.  Sampled rows, HISA and flat,
    against the oracle."""
    print("largest block count nq=%d" % nq, flush=True)
    dv = _dev()
    L, B, m, k = 262144, 16, 64, 512
    g = np.random.default_rng(46 + nq)
    pos = np.sort(g.choice(np.arange(1000, L), nq, replace=False)).astype(np.int64)
    pos[-1] = L - 1
    w = synth.chunked_prefill(L=L, seed=47, B=B, m=m, k=k, q_positions=pos)
    cache = dv.DeviceCache(w, B=B)
    cache.pool()
    rows = sorted(set([0, nq - 1] + list(g.choice(nq, min(nq, 30), replace=False))))
    for flat in (False, True):
        _check_phase(w, cache, w.phases[0], k, m, flat, rows=rows, label="maxblocks%d" % nq)


@pytest.mark.parametrize("nq", [8, 600])
def test_largest_k(nq):
    """The largest k the index calls accept, 16,384, equal to m*B (128
    blocks of 128): HISA returns every visible token of its kept blocks, and
    the flat indexer the 16,384 best of up to 40,000 keys.  Few queries (one
    workgroup per row of 16,384 candidates) and many (the many-row forms).
    Sampled rows, HISA and flat, against the oracle."""
    print("largest k nq=%d" % nq, flush=True)
    dv = _dev()
    L, B, m, k = 40000, 128, 128, 16384
    g = np.random.default_rng(48 + nq)
    pos = np.sort(g.choice(np.arange(100, L), nq, replace=False)).astype(np.int64)
    pos[-1] = L - 1
    w = synth.chunked_prefill(L=L, seed=49, B=B, m=m, k=k, q_positions=pos)
    cache = dv.DeviceCache(w, B=B)
    cache.pool()
    rows = sorted(set([0, nq - 1] + list(g.choice(nq, min(nq, 24), replace=False))))
    for flat in (False, True):
        _check_phase(w, cache, w.phases[0], k, m, flat, rows=rows, label="maxk%d" % nq)


def test_supplementary_block_scoring_shape_sampled():
    """The supplementary block-scoring shape at full size: the last 32,768
    positions of a 1,048,576-key MoG sequence in one call (8,064-8,192
    causal blocks per query, selected by the two MFMA walks).  Every row's properties; 48 rows (the first, the last and 46
    random ones) against the oracle."""
    print("supplementary 32768 x 8192", flush=True)
    dv = _dev()
    L, nq = 1 << 20, 32768
    pos = np.arange(L - nq, L, dtype=np.int64)
    w = synth.chunked_prefill(L=L, seed=13, q_positions=pos)
    cache = dv.DeviceCache(w)
    cache.pool()
    g = np.random.default_rng(45)
    rows = sorted(set([0, nq - 1] + list(g.choice(nq, 46, replace=False))))
    _check_phase(w, cache, w.phases[0], w.k, w.m, False, rows=rows, label="supp", one_chunk_limit=16 << 30)


@pytest.mark.parametrize("B,m,k", [(64, 12, 500), (128, 64, 2048), (16, 40, 640)])
def test_few_hundred_packed_queries(B, m, k):
    """A few hundred queries (300, fewer than 512: every query split over
    several workgroups) over packed sequences of ragged lengths with invalid
    queries mixed in, with at most 2048 blocks: the fused selection and
    token scores, then the many-row top-k."""
    print("few hundred packed B=%d m=%d k=%d" % (B, m, k), flush=True)
    dv = _dev()
    nseq = 9
    g = np.random.default_rng(B * 3 + m)
    lens = g.integers(300, 6000, nseq).astype(np.int64)
    w = synth.decode_batch(nseq=nseq, L=int(lens.max()), seed=46, B=B, m=m, k=k)
    cache = dv.DeviceCache(w, B=B)
    cache.set_lengths(lens)
    cache.pool()
    nq = 300
    q_seq = g.integers(0, nseq, nq).astype(np.int32)
    q_pos = (g.random(nq) * lens[q_seq]).astype(np.int64)
    q_pos[::37] = lens[q_seq[::37]] + 5                 # past the sequence: invalid, a -1 row
    queries = synth.to_bf16(g.standard_normal((nq, synth.D)).astype(np.float32))
    ph = synth.Phase("p", queries, q_pos, q_seq)
    bad = np.zeros(nq, bool)
    bad[::37] = True
    for flat in (False, True):
        idx, sc, blk = _run(cache, ph, k, m, flat)
        assert np.all(idx[bad] == -1) and np.all(np.isnan(sc[bad]))
        if not flat:
            assert np.all(blk[bad] == -1)
        _check_phase(w, cache, ph, k, m, flat, rows=np.nonzero(~bad)[0], label="fewhundred", props=False)


@pytest.mark.parametrize("n_out", [16, 300])
def test_outlier_scores_stretch_the_bins(n_out):
    """A few keys along each decode query (score about 6 |q|^2, far above
    the rest) stretch the selects' bins, so the threshold bin holds well
    over 64 members (ranked through the member list); 300 outliers per
    sequence also put them among the kept tokens."""
    print("outliers %d" % n_out, flush=True)
    dv = _dev()
    w = synth.decode_batch(nseq=4, L=20000, seed=35, B=128, m=64, k=2048)
    keys = w.keys.copy()
    g = np.random.default_rng(36 + n_out)
    for s in range(4):
        o = int(w.seq_key_off[s])
        q = synth.from_bf16(w.phases[0].queries[s])
        pos = g.choice(int(w.seq_len[s]) - 1, n_out, replace=False)
        keys[o + pos] = synth.to_bf16((6.0 * q).astype(np.float32))
    w2 = synth.Workload("outliers", keys, w.seq_key_off, w.seq_len, w.seq_cap, 128, 64, 2048)
    cache = dv.DeviceCache(w2, B=128)
    cache.pool()
    for flat in (False, True):
        _check_phase(w2, cache, w.phases[0], 2048, 64, flat, label="outliers%d" % n_out)
