"""Block-only selection (hisa_block_index) vs the CPU oracle, through the C
ABI, on the GPU.  Rows hold every visible token of the kept blocks, so
k = m*B; the comparison rule is the index rule of parity.py (kept blocks
equal the oracle's, or differ only inside the near-tie band, in which case
the row must be the expansion of the GPU's own blocks)."""
import numpy as np
import pytest

import oracle
from long_context_sparse_hisa_amd import synth
from parity import check_all_rows_properties, check_rows

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from long_context_sparse_hisa_amd import hisa
    hisa.lib()                                  # raises if the library is missing


def _expand(blk, t, B):
    """The row a kept-block list stands for (host arithmetic on GPU blocks)."""
    toks = [j for b in blk if b >= 0 for j in range(b * B, (b + 1) * B) if j <= t]
    return np.array(toks + [-1] * (len(blk) * B - len(toks)), np.int32)


def _block_run(w, ph, B, m, rows=None, label="", out_offset=0, **kw):
    from long_context_sparse_hisa_amd import device
    cache = device.DeviceCache(w, B=B)
    cache.pool()
    k = m * B
    call = device.IndexCall(cache, ph.queries, ph.q_pos, ph.q_seq, k=k, m=m, block_only=True, **kw)
    if out_offset:
        # a row buffer that starts off the 16-byte grid: the one-entry store path
        nq = len(ph.q_pos)
        buf = torch.full((nq * k + out_offset,), -7, dtype=torch.int32, device=cache.device)
        call.out_idx = buf[out_offset:].view(nq, k)
        call.args = call._args(call.workspace)
        call.args.workspace_bytes = call.workspace.numel()
    call.run()
    idx, sc, blk = call.results()
    assert sc is None
    lens = cache.seq_len
    reps = []
    for s in range(w.nseq):
        o = int(w.seq_key_off[s])
        reps.append(oracle.pool(w.keys[o:o + int(lens[s])], B))

    def K_of(i):
        s = int(ph.q_seq[i])
        o = int(w.seq_key_off[s])
        return w.keys[o:o + int(lens[s])]

    rows = range(len(ph.q_pos)) if rows is None else rows
    counts = check_rows(rows, ph.queries, ph.q_pos, K_of, lambda i: reps[int(ph.q_seq[i])], B, m, k, idx, None,
                        blk, False, label)
    print(label, counts, flush=True)
    return idx, blk


@pytest.mark.parametrize("L,B,m", [(1, 16, 3), (300, 16, 3), (1000, 64, 4), (1000, 128, 8), (4097, 128, 8),
                                   (3000, 256, 3), (1500, 16, 64)])
def test_small_grid(L, B, m):
    print("block-only L=%d B=%d m=%d" % (L, B, m), flush=True)
    w = synth.chunked_prefill(L=L, seed=31, B=B, m=m, k=m * B)
    ph = w.phases[0]
    idx, blk = _block_run(w, ph, B, m, label="bo%d" % L)
    check_all_rows_properties(idx, blk, ph.q_pos, B, m, m * B, False)
    for i in range(0, len(ph.q_pos), max(1, len(ph.q_pos) // 50)):
        assert np.array_equal(idx[i], _expand(blk[i], int(ph.q_pos[i]), B))


def test_unaligned_output_rows():
    print("block-only unaligned", flush=True)
    w = synth.chunked_prefill(L=2000, seed=32, B=32, m=5, k=160, q_positions=np.arange(0, 2000, 7))
    ph = w.phases[0]
    a, _ = _block_run(w, ph, 32, 5, label="aligned")
    b, _ = _block_run(w, ph, 32, 5, label="unaligned", out_offset=1)
    assert np.array_equal(a, b)


def test_packed_sequences_and_invalid_queries():
    print("block-only packed", flush=True)
    w = synth.decode_batch(nseq=5, L=3000, seed=33, B=64, m=5, k=320, spare=100)
    ph = w.phases[0]
    w.seq_len[:] = [3000, 1, 640, 2999, 1500]
    q_pos = np.array([2999, 0, 639, 2000, 1500], np.int64)      # the last is past its end
    ph2 = synth.Phase("p", ph.queries, q_pos, np.arange(5, dtype=np.int32))
    idx, blk = _block_run(w, ph2, 64, 5, rows=[0, 1, 2, 3], label="packed")
    assert np.all(idx[4] == -1) and np.all(blk[4] == -1)


def test_many_queries_tile_path_sampled():
    """4096 queries: stage 1 in MFMA tiles, then the expansion."""
    print("block-only 32K prefill sample", flush=True)
    pos = np.arange(7, 32768, 8, dtype=np.int64)
    w = synth.chunked_prefill(L=32768, seed=34, m=64, k=8192, q_positions=pos)
    ph = w.phases[0]
    rows = np.linspace(0, len(pos) - 1, 48).astype(int)
    idx, blk = _block_run(w, ph, 128, 64, rows=rows, label="prefill")
    check_all_rows_properties(idx, blk, ph.q_pos, 128, 64, 8192, False)


@pytest.mark.parametrize("m", [16, 64])
def test_decode_32k_x16_full(m):
    """The decode batch at full size; m = 16 spends the same 2048-token
    budget as HISA's k, m = 64 keeps HISA's candidate set."""
    print("block-only decode 32K x16 m=%d" % m, flush=True)
    w = synth.decode_batch()
    idx, blk = _block_run(w, w.phases[0], 128, m, label="decode")
    check_all_rows_properties(idx, blk, w.phases[0].q_pos, 128, m, m * 128, False)


def test_long_rows_use_the_separate_block_score_pass():
    """More than 2048 blocks (300,000 keys, B = 128): block scores in their
    own kernel before the selection."""
    print("block-only 300K", flush=True)
    L = 300_000
    w = synth.chunked_prefill(L=L, seed=35, m=16, k=2048, q_positions=np.array([L - 1, L // 2, 5000, 127]))
    _block_run(w, w.phases[0], 128, 16, label="300K")
