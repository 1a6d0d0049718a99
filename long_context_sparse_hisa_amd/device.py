"""Device-side state of a workload: packed keys, representatives, lengths,
and the buffers the index calls write.  Marshalling only: every computation
is a libhisa call.
"""
from __future__ import annotations

import numpy as np
import torch

from . import hisa
from .synth import D, Workload


def to_dev(a: np.ndarray, device) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(device)


class DeviceCache:
    """Packed key cache and block representatives of a workload's sequences."""

    def __init__(self, w: Workload, B: int | None = None, device: str = "cuda:0", stream=None):
        self.w = w
        self.B = B or w.B
        self.device = torch.device(device)
        self.stream = stream
        self.keys = to_dev(w.keys, self.device)
        self.seq_key_off = np.asarray(w.seq_key_off, np.int64)
        self.seq_rep_off = w.seq_rep_off(self.B)
        self.seq_cap = np.asarray(w.seq_cap, np.int64)
        self.seq_len = np.asarray(w.seq_len, np.int64).copy()
        self.reps = torch.zeros((w.total_rep_rows(self.B), D), dtype=torch.int16, device=self.device)
        self.d_key_off = to_dev(self.seq_key_off, self.device)
        self.d_rep_off = to_dev(self.seq_rep_off, self.device)
        self.d_len = to_dev(self.seq_len, self.device)
        self._ws = {}

    @property
    def nseq(self) -> int:
        return len(self.seq_len)

    def pool(self):
        for s in range(self.nseq):
            o, n, r = int(self.seq_key_off[s]), int(self.seq_len[s]), int(self.seq_rep_off[s])
            nb = (n + self.B - 1) // self.B
            hisa.hisa_pool_blocks(self.keys[o:o + n], self.B, self.reps[r:r + max(nb, 1)], self.stream)

    def append(self, new_keys: np.ndarray | torch.Tensor, update_lengths: bool = True):
        """Append new_keys [nseq, n_new, D] (bf16 bits) to every sequence."""
        nk = new_keys if isinstance(new_keys, torch.Tensor) else to_dev(new_keys, self.device)
        seqs = [(self.seq_key_off[s], self.seq_rep_off[s], self.seq_len[s], self.seq_cap[s])
                for s in range(self.nseq)]
        hisa.hisa_append_keys(self.keys, self.reps, seqs, nk, self.B, self.stream)
        if update_lengths:
            self.seq_len += nk.shape[1]
            self.d_len.copy_(torch.from_numpy(self.seq_len))

    def decode_step(self, call: "IndexCall", new_keys: np.ndarray | torch.Tensor, stream=None):
        """Append new_keys [nseq, n_new, D] to every sequence and run the
        index call in one hisa_decode_step (the call's queries should sit at
        positions valid after the append)."""
        nk = new_keys if isinstance(new_keys, torch.Tensor) else to_dev(new_keys, self.device)
        seqs = [(self.seq_key_off[s], self.seq_rep_off[s], self.seq_len[s], self.seq_cap[s])
                for s in range(self.nseq)]
        self.seq_len += nk.shape[1]
        self.d_len.copy_(torch.from_numpy(self.seq_len))
        hisa.hisa_decode_step(call.args, seqs, nk, stream or self.stream)

    def set_lengths(self, lengths):
        self.seq_len = np.asarray(lengths, np.int64).copy()
        self.d_len.copy_(torch.from_numpy(self.seq_len))

    def workspace(self, nbytes: int, tag: str = "") -> torch.Tensor:
        ws = self._ws.get(tag)
        if ws is None or ws.numel() < nbytes:
            ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=self.device)
            self._ws[tag] = ws
        return ws


class IndexCall:
    """Buffers and arguments of one index call, reusable across launches."""

    def __init__(self, cache: DeviceCache, queries, q_pos, q_seq, k: int, m: int | None = None,
                 flat: bool = False, scores: bool = True, blocks: bool = True,
                 max_len: int | None = None, workspace_bytes: int | None = None,
                 one_chunk_limit: int = 0, block_only: bool = False):
        """block_only: the block-only selection (k must be m*B; no scores)."""
        dev = cache.device
        self.cache = cache
        self.flat = flat
        self.block_only = block_only
        if block_only:
            scores = False
        self.queries = queries if isinstance(queries, torch.Tensor) else to_dev(queries, dev)
        self.q_pos = q_pos if isinstance(q_pos, torch.Tensor) else to_dev(np.asarray(q_pos, np.int64), dev)
        self.q_seq = q_seq if isinstance(q_seq, torch.Tensor) else to_dev(np.asarray(q_seq, np.int32), dev)
        nq = self.queries.shape[0]
        self.k = k
        self.m = m if m is not None else cache.w.m
        self.out_idx = torch.empty((nq, k), dtype=torch.int32, device=dev)
        self.out_scores = torch.empty((nq, k), dtype=torch.float32, device=dev) if scores else None
        self.out_blocks = (torch.empty((nq, self.m), dtype=torch.int32, device=dev)
                           if (blocks and not flat) else None)
        self.max_len = int(max_len if max_len is not None else cache.seq_cap.max())
        args = self._args(None)
        want, _, whole = hisa.hisa_workspace_bytes(args, flat, all_queries=True)
        if whole <= one_chunk_limit:           # every query in one chunk
            want = whole
        nbytes = want if workspace_bytes is None else workspace_bytes
        self.workspace = cache.workspace(nbytes, "flat" if flat else "hisa")
        self.args = self._args(self.workspace)
        self.args.workspace_bytes = nbytes

    def _args(self, ws):
        c = self.cache
        return hisa.make_args(self.queries, self.q_pos, c.keys, self.k, reps=c.reps, q_seq=self.q_seq,
                              seq_key_off=c.d_key_off, seq_rep_off=c.d_rep_off, seq_len=c.d_len,
                              max_len=self.max_len, B=c.B, m=self.m, out_idx=self.out_idx,
                              out_scores=self.out_scores, out_blocks=self.out_blocks, workspace=ws)

    def run(self, stream=None):
        if self.flat:
            hisa.hisa_flat_index(self.args, stream or self.cache.stream)
        elif self.block_only:
            hisa.hisa_block_index(self.args, stream or self.cache.stream)
        else:
            hisa.hisa_index(self.args, stream or self.cache.stream)

    def results(self):
        """(idx, scores or None, blocks or None) as numpy arrays."""
        torch.cuda.synchronize()
        idx = self.out_idx.cpu().numpy()
        sc = None if self.out_scores is None else self.out_scores.cpu().numpy()
        blk = None if self.out_blocks is None else self.out_blocks.cpu().numpy()
        return idx, sc, blk


class AttentionCall:
    """Buffers and arguments of one sparse-attention call over index rows
    idx [nq, kk] (a torch tensor, e.g. an IndexCall's out_idx, or numpy)."""

    def __init__(self, qa, ka, va, idx, scale: float, *, q_seq=None, seq_key_off=None, seq_len=None,
                 device: str = "cuda:0", stream=None):
        dev = torch.device(device)
        self.stream = stream
        def t(a, dtype=None):
            if a is None or isinstance(a, torch.Tensor):
                return a
            return to_dev(np.asarray(a, dtype) if dtype else a, dev)
        self.qa, self.ka, self.va = t(qa), t(ka), t(va)
        self.idx = t(idx, np.int32)
        if seq_len is None:
            seq_len = np.array([self.ka.shape[0]], np.int64)
        self.q_seq = t(q_seq, np.int32)
        self.seq_key_off = t(seq_key_off, np.int64)
        self.seq_len = t(seq_len, np.int64)
        nq = self.qa.shape[0]
        self.out = torch.empty((nq, self.qa.shape[1]), dtype=torch.float32, device=dev)
        args = self._args(None, scale)
        nbytes = hisa.hisa_attention_workspace_bytes(args)
        self.workspace = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=dev)
        self.args = self._args(self.workspace, scale)

    def _args(self, ws, scale):
        return hisa.make_attn_args(self.qa, self.ka, self.va, self.idx, scale, q_seq=self.q_seq,
                                   seq_key_off=self.seq_key_off, seq_len=self.seq_len, out=self.out,
                                   workspace=ws)

    def run(self, stream=None):
        hisa.hisa_sparse_attention(self.args, stream or self.stream)

    def result(self) -> np.ndarray:
        torch.cuda.synchronize()
        return self.out.cpu().numpy()


class LsaCache:
    """Bucket cache (centroids, members, offsets) of a DeviceCache's
    sequences, built by hisa_lsa_build over each sequence's complete
    512-key blocks."""

    def __init__(self, cache: DeviceCache):
        self.cache = cache
        dev = cache.device
        cap_blocks = cache.seq_cap // hisa.HISA_LSA_BLOCK
        self.seq_blk_off = np.concatenate([[0], np.cumsum(cap_blocks)[:-1]]).astype(np.int64)
        nb = max(int(cap_blocks.sum()), 1)
        self.centroids = torch.zeros((nb * hisa.HISA_LSA_BUCKETS, D), dtype=torch.int16, device=dev)
        self.members = torch.zeros((nb, hisa.HISA_LSA_POOL_KEYS), dtype=torch.uint8, device=dev)
        self.offs = torch.zeros((nb, hisa.HISA_LSA_BUCKETS + 1), dtype=torch.uint8, device=dev)
        self.nblk = np.zeros(cache.nseq, np.int64)
        self.d_blk_off = to_dev(self.seq_blk_off, dev)
        self.d_nblk = to_dev(self.nblk, dev)

    def build(self, stream=None):
        """Build every complete block not built yet."""
        c = self.cache
        for s in range(c.nseq):
            o, n, b = int(c.seq_key_off[s]), int(c.seq_len[s]), int(self.seq_blk_off[s])
            full = n // hisa.HISA_LSA_BLOCK
            if full > self.nblk[s]:
                hisa.hisa_lsa_build(c.keys[o:o + n], int(self.nblk[s]), self.centroids[b * hisa.HISA_LSA_BUCKETS:],
                                    self.members[b:], self.offs[b:], stream)
                self.nblk[s] = full
        self.d_nblk.copy_(torch.from_numpy(self.nblk))

    def host(self, s: int):
        """(centroids, members, offs) of sequence s as numpy arrays."""
        b, n = int(self.seq_blk_off[s]), int(self.nblk[s])
        torch.cuda.synchronize()
        return (self.centroids[b * hisa.HISA_LSA_BUCKETS:(b + n) * hisa.HISA_LSA_BUCKETS].cpu().numpy().view(np.uint16),
                self.members[b:b + n].cpu().numpy(), self.offs[b:b + n].cpu().numpy())


class LsaCall:
    """Buffers and arguments of one LSA flat-search call."""

    def __init__(self, lsa: LsaCache, queries, q_pos, q_seq, p: int, k: int, max_len: int | None = None,
                 buckets: bool = True):
        c = lsa.cache
        dev = c.device
        self.lsa = lsa
        self.queries = queries if isinstance(queries, torch.Tensor) else to_dev(queries, dev)
        self.q_pos = q_pos if isinstance(q_pos, torch.Tensor) else to_dev(np.asarray(q_pos, np.int64), dev)
        self.q_seq = q_seq if isinstance(q_seq, torch.Tensor) else to_dev(np.asarray(q_seq, np.int32), dev)
        nq = self.queries.shape[0]
        self.p, self.k = p, k
        self.out_idx = torch.empty((nq, k), dtype=torch.int32, device=dev)
        self.out_buckets = torch.empty((nq, p), dtype=torch.int32, device=dev) if buckets else None
        self.max_len = int(max_len if max_len is not None else c.seq_cap.max())
        nbytes = hisa.hisa_lsa_workspace_bytes(self._args(None))
        self.workspace = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=dev)
        self.args = self._args(self.workspace)

    def _args(self, ws):
        lsa, c = self.lsa, self.lsa.cache
        return hisa.make_lsa_args(self.queries, self.q_pos, lsa.centroids, lsa.members, lsa.offs, lsa.d_blk_off,
                                  lsa.d_nblk, c.d_len, self.max_len, self.p, self.k, q_seq=self.q_seq,
                                  out_idx=self.out_idx, out_buckets=self.out_buckets, workspace=ws)

    def run(self, stream=None):
        hisa.hisa_lsa_index(self.args, stream or self.lsa.cache.stream)

    def results(self):
        torch.cuda.synchronize()
        return (self.out_idx.cpu().numpy(),
                None if self.out_buckets is None else self.out_buckets.cpu().numpy())
