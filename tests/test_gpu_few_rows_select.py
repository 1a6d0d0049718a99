"""Stage 1 of few queries (fewer than 256) over rows of more than 2,048
blocks: the representative scores come from their own launch, and each of a
query's workgroups selects the kept blocks from its score row (the bucket
select over up to 16,384 keys) before scoring its share of the kept tokens.
Shapes from m - 3 = 1 to 65, i.i.d. and MoG keys, and exact integer block
scores with ties where the kept blocks end.  HIP path against the oracle,
every row, through the C ABI."""
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


def _check_all(w, ph, k, m, label):
    from long_context_sparse_hisa_amd import device as dv
    cache = dv.DeviceCache(w, B=w.B)
    cache.pool()
    call = dv.IndexCall(cache, ph.queries, ph.q_pos, ph.q_seq, k=k, m=m, flat=False)
    call.run()
    idx, sc, blk = call.results()
    B = w.B
    lens = np.asarray(cache.seq_len, np.int64)
    check_all_rows_properties(idx, blk, ph.q_pos, B, m, k, False)
    reps = oracle.pool(w.keys[:int(lens[0])], B)

    def K_of(i):
        return w.keys[:int(lens[0])]

    def R_of(i):
        return reps

    counts = check_batch(ph, w.keys, lens, w.seq_key_off, reps, np.zeros(1, np.int64), B, m, k, idx, sc, blk,
                         False, K_of, R_of, label)
    print(label, counts, flush=True)
    assert counts["exact"] + counts["excused"] == len(ph.q_pos)
    return idx, blk


@pytest.mark.parametrize("L,B,m,k,iid", [
    (70000, 16, 67, 1000, False),       # 4,375 blocks, m - 3 = 64
    (70000, 16, 4, 64, False),          # m - 3 = 1
    (300000, 128, 64, 2048, False),     # 2,344 blocks
    (70000, 16, 68, 1000, False),       # m - 3 = 65
    (262144, 16, 40, 512, True),        # 16,384 blocks, i.i.d. keys and queries
])
def test_few_rows_every_row(L, B, m, k, iid):
    """12 queries past 2,048 blocks at random positions (one of them at the
    last key), every row against the oracle."""
    print("few rows L=%d B=%d m=%d k=%d iid=%s" % (L, B, m, k, iid), flush=True)
    g = np.random.default_rng(L + B + m)
    nq = 12
    pos = np.sort(g.choice(np.arange(2049 * B, L - 1), nq - 1, replace=False)).astype(np.int64)
    pos = np.concatenate([pos, [L - 1]]).astype(np.int64)
    w = synth.chunked_prefill(L=L, seed=81, B=B, m=m, k=k, q_positions=pos)
    ph = w.phases[0]
    if iid:
        keys = synth.to_bf16(g.standard_normal((L, synth.D)).astype(np.float32))
        queries = synth.to_bf16(g.standard_normal((nq, synth.D)).astype(np.float32))
        w = synth.Workload("iid", keys, w.seq_key_off, w.seq_len, w.seq_cap, B, m, k)
        ph = synth.Phase("p", queries, pos, np.zeros(nq, np.int32))
        w.phases.append(ph)
    _check_all(w, ph, k, m, "fewrows")


def _tiered(L, B, nq, tiers, seed):
    """Keys whose every block scores one small integer against the query
    e0 (a block's keys are all equal, so its representative is that key):
    `tiers` lists (value, count) pairs for the top blocks, placed at random
    free blocks; every other block scores 0..3."""
    g = np.random.default_rng(seed)
    nb = L // B
    val = g.integers(0, 4, nb).astype(np.float32)
    free = g.permutation(np.arange(1, nb - 40))         # blocks every query sees as free
    at = 0
    for v, n in tiers:
        val[free[at:at + n]] = v
        at += n
    kf = np.zeros((L, synth.D), np.float32)
    kf[:, 0] = np.repeat(val, B)
    qf = np.zeros((nq, synth.D), np.float32)
    qf[:, 0] = 1.0
    return synth.to_bf16(kf), synth.to_bf16(qf), val


@pytest.mark.parametrize("kind", ["small_tie", "large_tie", "all_equal"])
def test_few_rows_ties(kind):
    """Exact integer block scores with ties where the m - 3 free blocks end:
    a small tie (10 blocks at 8, then 15 at 7 of which 7 are kept: the
    lowest 7), a tie of 300 equal blocks of which 44 are kept, and one
    score for every block (the lowest free blocks are kept).  The kept
    blocks are also checked against the rule itself: the highest scores,
    equal scores to the lower block."""
    print("few rows ties %s" % kind, flush=True)
    L, B, nq = 70000, 16, 10
    m = 20 if kind == "small_tie" else 67
    k = 256 if kind == "small_tie" else 512       # k <= m*B
    g = np.random.default_rng(82)
    pos = np.sort(g.choice(np.arange(L - 600, L), nq, replace=False)).astype(np.int64)
    tiers = {"small_tie": [(8.0, 10), (7.0, 15)], "large_tie": [(9.0, 20), (8.0, 300)],
             "all_equal": []}[kind]
    keys, queries, val = _tiered(L, B, nq, tiers, 83)
    if kind == "all_equal":
        keys = synth.to_bf16(np.where(np.arange(synth.D) == 0, 1.0, 0.0).astype(np.float32)[None].repeat(L, 0))
        val = np.ones(L // B, np.float32)
    base = synth.chunked_prefill(L=L, seed=84, B=B, m=m, k=k, q_positions=pos)
    w = synth.Workload(kind, keys, base.seq_key_off, base.seq_len, base.seq_cap, B, m, k)
    ph = synth.Phase("p", queries, pos, np.zeros(nq, np.int32))
    w.phases.append(ph)
    _, blk = _check_all(w, ph, k, m, "fewties-" + kind)
    for i in range(nq):
        c = int(pos[i]) // B
        free = np.arange(1, c - 1)
        order = sorted(free.tolist(), key=lambda b: (-val[b], b))
        want = [0] + sorted(order[:m - 3]) + [c - 1, c]
        assert list(blk[i]) == want, (i, list(blk[i])[:8], want[:8])
