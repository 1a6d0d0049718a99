"""hisa_index_static (the index call on the library's own static device
scratch, for callers that cannot allocate) against hisa_index with a caller
workspace, through the C ABI: equal bit for bit on two calls in a row, the
second smaller than the first, so the second runs over what the first left
in the scratch."""
import numpy as np
import pytest

from long_context_sparse_hisa_amd import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from long_context_sparse_hisa_amd import hisa
    hisa.lib()                                  # raises if the library is missing


def _both(w, ph, B, m, k):
    """(hisa_index with a workspace, hisa_index_static) results."""
    from long_context_sparse_hisa_amd import device, hisa
    cache = device.DeviceCache(w, B=B)
    cache.pool()
    call = device.IndexCall(cache, ph.queries, ph.q_pos, ph.q_seq, k=k, m=m, one_chunk_limit=16 << 30)
    call.run()
    want = [x.copy() for x in call.results()]
    for t in (call.out_idx, call.out_scores, call.out_blocks):
        t.fill_(7)                                 # the static call must write every entry
    a = call.args
    saved = (a.workspace, a.workspace_bytes)
    a.workspace, a.workspace_bytes = None, 0       # the static call ignores them
    try:
        hisa.hisa_index_static(a, cache.stream)
    finally:
        a.workspace, a.workspace_bytes = saved
    got = call.results()
    return want, got


def _same(want, got, label):
    for x, y, what in zip(want, got, ("indices", "scores", "blocks")):
        assert np.array_equal(x, y, equal_nan=True), "%s: %s differ" % (label, what)


def test_static_scratch_equals_workspace_call_twice():
    from long_context_sparse_hisa_amd import hisa
    # call 1: 2,500 prefill queries over 20,000 keys: their candidate rows
    # (2,500 x 8,192 x 4 bytes) exceed the 64 MiB scratch, so the call runs
    # in chunks; the workspace call takes them in one
    print("static scratch: 2500 prefill queries, L=20000", flush=True)
    pos = np.linspace(0, 19999, 2500).astype(np.int64)
    w1 = synth.chunked_prefill(L=20000, seed=61, B=128, m=64, k=2048, q_positions=pos)
    want, got = _both(w1, w1.phases[0], 128, 64, 2048)
    _same(want, got, "call 1")
    # call 2: smaller, a decode batch of 16 sequences x 12,000 keys
    print("static scratch: 16 decode queries, L=12000", flush=True)
    w2 = synth.decode_batch(nseq=16, L=12000, seed=62, B=64, m=32, k=1000)
    want, got = _both(w2, w2.phases[0], 64, 32, 1000)
    _same(want, got, "call 2")
    # the validation is hisa_index's
    a = hisa.hisa_index_args()
    a.nq, a.nseq, a.max_len, a.d, a.B, a.m, a.k = 1, 1, 100, 32, 128, 4, 10
    assert hisa.lib().hisa_index_static(a, None) == hisa.HISA_ERR_UNSUPPORTED
