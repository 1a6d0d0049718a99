"""Forced blocks under adversarial keys, and recovery of corrupted
representatives, on the GPU through the C ABI.

Forced blocks: the HISA summary's stage-1 paragraph keeps the first block
and the last two blocks whatever their scores.  Here the keys of those
blocks point exactly away from the query (bf16(-q)), so their block scores
are the lowest of all; every path must still keep them, and every row must
equal the oracle's.

Recovery: the maintenance paragraph makes the representatives state derived
from the keys; overwriting them and pooling again restores them bit for bit
(and the index results with them).
"""
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


def _adversarial(L, own_blocks, nq, seed, B=128):
    """L i.i.d. keys; nq copies of one query placed in the given own blocks;
    the keys of block 0 and of blocks c-1 and c for every own block c are
    bf16(-q)."""
    g = np.random.default_rng(seed)
    keys = g.standard_normal((L, synth.D)).astype(np.float32)
    q = g.standard_normal(synth.D).astype(np.float32)
    bad = {0}
    for c in own_blocks:
        bad |= {c - 1, c}
    for b in bad:
        keys[b * B:(b + 1) * B] = -q
    keys = synth.to_bf16(keys)
    cs = np.asarray(own_blocks)[np.arange(nq) % len(own_blocks)]
    q_pos = np.minimum(cs * B + g.integers(0, B, nq), L - 1).astype(np.int64)
    queries = np.repeat(synth.to_bf16(q)[None], nq, axis=0)
    w = synth.Workload("adversarial", keys, np.zeros(1, np.int64), np.array([L], np.int64),
                       np.array([L], np.int64), B, 64, 2048)
    ph = synth.Phase("p", queries, q_pos, np.zeros(nq, np.int32))
    return w, ph, sorted(bad)


@pytest.mark.parametrize("L,nq", [(40000, 16), (40000, 600), (300000, 4)],
                         ids=["decode-fused", "prefill-tiles", "long-rows"])
def test_forced_blocks_kept_against_adversarial_keys(L, nq):
    """16 queries take the fused decode launch, 600 the MFMA tile kernels,
    4 queries over 300,000 keys (more than 2048 blocks) the block-score
    launch and the select-and-score launch."""
    print("adversarial forced blocks L=%d nq=%d" % (L, nq), flush=True)
    from long_context_sparse_hisa_amd import device
    B, m, k = 128, 64, 2048
    own = [100, 150, 200, 250, 300] if L < 100000 else [1000, 2343]
    w, ph, bad = _adversarial(L, own, nq, seed=L + nq)
    cache = device.DeviceCache(w, B=B)
    cache.pool()
    call = device.IndexCall(cache, ph.queries, ph.q_pos, ph.q_seq, k=k, m=m)
    call.run()
    idx, sc, blk = call.results()
    reps = oracle.pool(w.keys, B)
    # the adversarial blocks score below every other causal block
    qv = synth.from_bf16(ph.queries[0]).astype(np.float64)
    sig = synth.from_bf16(reps).astype(np.float64) @ qv
    c0 = int(ph.q_pos[0]) // B
    others = [b for b in range(c0 + 1) if b not in bad]
    assert max(sig[b] for b in bad if b <= c0) < min(sig[others])
    check_all_rows_properties(idx, blk, ph.q_pos, B, m, k, False)
    for i in range(nq):
        c = int(ph.q_pos[i]) // B
        assert {0, c - 1, c} <= set(blk[i].tolist()), "row %d lost a forced block" % i
    counts = check_batch(ph, w.keys, w.seq_len, w.seq_key_off, reps, np.zeros(1, np.int64), B, m, k, idx, sc, blk,
                         False, lambda i: w.keys, lambda i: reps, "adversarial")
    print("adversarial", counts, flush=True)


def test_corrupted_representatives_recovered_by_pooling():
    """Pool, index; overwrite every representative with random bits (NaNs
    and infinities among them) and also zero a few; pool again: the
    representatives equal the oracle's bit for bit and the index results
    equal the first ones bit for bit."""
    print("representative recovery", flush=True)
    from long_context_sparse_hisa_amd import device, hisa
    w = synth.chunked_prefill(L=20000, seed=81, B=128, m=16, k=512, q_positions=np.arange(5, 20000, 37))
    cache = device.DeviceCache(w, B=128)
    cache.pool()
    ph = w.phases[0]
    call = device.IndexCall(cache, ph.queries, ph.q_pos, ph.q_seq, k=512, m=16)
    call.run()
    first = [x.copy() for x in call.results()]
    want = oracle.pool(w.keys, 128)
    nrep = len(want)
    g = np.random.default_rng(82)
    junk = g.integers(0, 1 << 16, (nrep, synth.D), dtype=np.uint16)
    junk[::7] = 0
    cache.reps[:nrep].copy_(torch.from_numpy(junk.view(np.int16)).to(cache.reps.device))
    torch.cuda.synchronize()
    assert not np.array_equal(cache.reps[:nrep].cpu().numpy().view(np.uint16), want)
    hisa.hisa_pool_blocks(cache.keys[:20000], 128, cache.reps[:nrep], cache.stream)
    torch.cuda.synchronize()
    assert np.array_equal(cache.reps[:nrep].cpu().numpy().view(np.uint16), want)
    call.run()
    again = call.results()
    for a, b, what in zip(first, again, ("indices", "scores", "blocks")):
        assert np.array_equal(a, b, equal_nan=True), "%s differ after recovery" % what
