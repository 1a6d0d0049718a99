"""LSA-Flat on the GPU (hisa_lsa_build, hisa_lsa_index) against the CPU
oracle, through the C ABI.

Build rule: members, offsets and bf16 centroids equal the oracle's bit for
bit, block by block.  The Ward costs that decide the merges are fp64 on
both sides but summed in different orders (about 1e-15 relative apart);
the oracle reports the smallest relative gap between the two sides of any
comparison it made in a block, and only a block whose gap is below MARGIN
may differ (then its buckets must still be a valid partition).

Query rule: the ranked bucket list equals the oracle's, except at ranks
where both buckets' fp64 scores lie within TOL of each other (fp32 scores
of near-equal buckets may order either way); the row must then be the fill
of the GPU's own ranked list.
"""
import numpy as np
import pytest

import oracle
from long_context_sparse_hisa_amd import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

MARGIN = 1e-9
TOL = 1e-3


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from long_context_sparse_hisa_amd import hisa
    hisa.lib()                                  # raises if the library is missing


def _setup(w, build=True):
    from long_context_sparse_hisa_amd import device
    cache = device.DeviceCache(w)
    lsa = device.LsaCache(cache)
    if build:
        lsa.build()
    return cache, lsa


def _seq_keys(w, cache, s):
    o = int(w.seq_key_off[s])
    return w.keys[o:o + int(cache.seq_len[s])]


def _valid_partition(mem, off):
    o = off.astype(int)
    return (o[0] == 0 and o[-1] == 128 and np.all(np.diff(o) >= 1) and np.all(np.diff(o) <= 4)
            and sorted(mem) == list(range(128)))


def _check_build(w, cache, lsa, label=""):
    """Returns the oracle caches per sequence and the number of excused blocks."""
    out, excused = [], 0
    for s in range(cache.nseq):
        cen, mem, off, margins = oracle.lsa_build(_seq_keys(w, cache, s))
        gc, gm, go = lsa.host(s)
        assert gm.shape == mem.shape, "%s seq %d: %s blocks vs %s" % (label, s, gm.shape, mem.shape)
        for b in range(mem.shape[0]):
            same = (np.array_equal(gm[b], mem[b]) and np.array_equal(go[b], off[b])
                    and np.array_equal(gc[b * 64:(b + 1) * 64], cen[b * 64:(b + 1) * 64]))
            if not same:
                assert margins[b] < MARGIN, "%s seq %d block %d differs (oracle margin %.3g)" % (
                    label, s, b, margins[b])
                assert _valid_partition(gm[b], go[b])
                excused += 1
        out.append((cen, mem, off))
    return out, excused


def _fill(bk, mem, off, k):
    toks = []
    for b in bk[bk >= 0]:
        blk, lb = divmod(int(b), 64)
        for pt in mem[blk][off[blk][lb]:off[blk][lb + 1]].astype(int):
            toks.extend(range(blk * 512 + 4 * pt, blk * 512 + 4 * pt + 4))
    toks = sorted(toks[:k])
    return np.array(toks + [-1] * (k - len(toks)), np.int32)


def _check_query(q, t, cen, mem, off, p, k, g_idx, g_bk, what):
    o_idx, o_bk, _ = oracle.lsa_query(q, cen, mem, off, t, p, k)
    if np.array_equal(g_idx, o_idx) and np.array_equal(g_bk, o_bk):
        return "exact"
    sc = synth.from_bf16(cen).astype(np.float64) @ synth.from_bf16(q).astype(np.float64)
    ng, no = int((g_bk >= 0).sum()), int((o_bk >= 0).sum())
    differ = False
    for r in range(min(ng, no)):
        gb, ob = int(g_bk[r]), int(o_bk[r])
        if gb != ob:
            differ = True
            assert abs(sc[gb] - sc[ob]) <= TOL, "%s rank %d: bucket %d (%.6f) vs oracle %d (%.6f)" % (
                what, r, gb, sc[gb], ob, sc[ob])
    # the same buckets in the same order fill to the same cut
    assert differ or ng == no, "%s: %d buckets used vs oracle %d" % (what, ng, no)
    assert np.array_equal(g_idx, _fill(g_bk, mem, off, k)), "%s: row is not the fill of its buckets" % what
    return "excused"


def _run_query(lsa, ph, p, k, max_len=None):
    from long_context_sparse_hisa_amd import device
    call = device.LsaCall(lsa, ph.queries, ph.q_pos, ph.q_seq, p, k, max_len=max_len)
    call.run()
    return call.results()


def _check_all(w, cache, caches, ph, g_idx, g_bk, p, k, rows=None, label=""):
    counts = {"exact": 0, "excused": 0}
    rows = range(len(ph.q_pos)) if rows is None else rows
    for i in rows:
        s = int(ph.q_seq[i])
        t = int(ph.q_pos[i])
        if s < 0 or s >= cache.nseq or t < 0 or t >= cache.seq_len[s]:
            assert np.all(g_idx[i] == -1) and np.all(g_bk[i] == -1), "%s row %d invalid" % (label, i)
            continue
        cen, mem, off = caches[s]
        counts[_check_query(ph.queries[i], t, cen, mem, off, p, k, g_idx[i], g_bk[i],
                            "%s row %d" % (label, i))] += 1
    print(label, counts, flush=True)
    return counts


@pytest.mark.parametrize("L,iid", [(512, True), (512 * 8 + 77, False), (4096, True), (9000, False)])
def test_build_matches_oracle(L, iid):
    print("lsa build L=%d iid=%s" % (L, iid), flush=True)
    w = synth.tiny_prefill(L=L, seed=61, nq=1) if iid else synth.chunked_prefill(L=L, seed=61, q_positions=[0])
    cache, lsa = _setup(w)
    _, excused = _check_build(w, cache, lsa, "build")
    assert excused == 0


def test_incremental_build_equals_one_shot():
    print("lsa incremental build", flush=True)
    w = synth.decode_batch(nseq=2, L=6000, seed=62, spare=0)
    cache, lsa = _setup(w, build=False)
    cache.set_lengths([1600, 2100])          # 3 and 4 complete blocks
    lsa.build()
    cache.set_lengths([6000, 6000])          # 11 each
    lsa.build()
    once_cache, once = _setup(w)
    for s in range(2):
        for a, b in zip(lsa.host(s), once.host(s)):
            assert np.array_equal(a, b)
    _check_build(w, cache, lsa, "incremental")


def test_planted_groups_become_buckets():
    print("lsa planted", flush=True)
    g = np.random.default_rng(63)
    dirs = g.standard_normal((128, 64))
    keys = np.repeat(dirs, 8, axis=0) + 0.01 * g.standard_normal((1024, 64))
    kb = synth.to_bf16(keys.astype(np.float32))
    w = synth.Workload("planted", kb, np.zeros(1, np.int64), np.array([1024], np.int64),
                       np.array([1024], np.int64), 128, 64, 2048)
    cache, lsa = _setup(w)
    _, mem, off = lsa.host(0)
    for b in range(2):
        assert np.array_equal(off[b], np.arange(0, 129, 2)) and np.array_equal(mem[b], np.arange(128))
    _check_build(w, cache, lsa, "planted")


@pytest.mark.parametrize("p,k", [(1, 1), (7, 33), (64, 256), (256, 2045), (300, 2048), (513, 3000), (700, 2047),
                                 (2048, 5000)])
def test_query_grid(p, k):
    print("lsa query p=%d k=%d" % (p, k), flush=True)
    L = 8192
    pos = np.arange(0, L, 37, dtype=np.int64)
    w = synth.chunked_prefill(L=L, seed=64, q_positions=pos)
    cache, lsa = _setup(w)
    caches, _ = _check_build(w, cache, lsa, "grid")
    ph = w.phases[0]
    g_idx, g_bk = _run_query(lsa, ph, p, k)
    _check_all(w, cache, caches, ph, g_idx, g_bk, p, k, label="grid")
    # before the first complete block: nothing visible
    assert np.all(g_idx[pos < 511] == -1)


def test_packed_sequences_and_invalid_queries():
    print("lsa packed", flush=True)
    w = synth.decode_batch(nseq=4, L=5000, seed=65, spare=0)
    cache, lsa = _setup(w, build=False)
    cache.set_lengths([5000, 300, 2600, 4000])
    lsa.build()
    caches, _ = _check_build(w, cache, lsa, "packed")
    g = np.random.default_rng(66)
    q_seq = np.array([0, 1, 2, 3, 0, 2, -1, 4, 3, 1], np.int32)
    q_pos = np.array([4999, 299, 2599, 1000, 511, 2048, 10, 10, 4000, 0], np.int64)   # row 8 is past its end
    queries = synth.to_bf16(g.standard_normal((10, 64)).astype(np.float32))
    ph = synth.Phase("p", queries, q_pos, q_seq)
    g_idx, g_bk = _run_query(lsa, ph, 40, 300)
    _check_all(w, cache, caches, ph, g_idx, g_bk, 40, 300, label="packed")
    for i in (1, 6, 7, 8, 9):
        assert np.all(g_idx[i] == -1)


def test_decode_32k_x16_full():
    """The decode batch's keys and queries: p = 256 buckets, k = 2048."""
    print("lsa decode 32K x16", flush=True)
    w = synth.decode_batch()
    cache, lsa = _setup(w)
    caches, excused = _check_build(w, cache, lsa, "decode")
    print("build blocks excused:", excused, flush=True)
    ph = w.phases[0]
    g_idx, g_bk = _run_query(lsa, ph, 256, 2048)
    _check_all(w, cache, caches, ph, g_idx, g_bk, 256, 2048, label="decode")


def test_long_context_128k_decode_queries():
    """131,072 keys (256 blocks, 16,384 buckets), the 32 decode queries at
    the end: p = 512, k = 4096 (the page's example sizes)."""
    print("lsa 128K", flush=True)
    w = synth.long_context()
    cache, lsa = _setup(w)
    caches, excused = _check_build(w, cache, lsa, "128K")
    print("build blocks excused:", excused, flush=True)
    ph = w.phases[1]
    g_idx, g_bk = _run_query(lsa, ph, 512, 4096)
    _check_all(w, cache, caches, ph, g_idx, g_bk, 512, 4096, label="128K")
