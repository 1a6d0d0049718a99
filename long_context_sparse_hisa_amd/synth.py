"""Seeded synthetic inputs for the indexer workloads.

This module only draws random numbers and lays them out; it holds none of
the indexer's arithmetic.  The CPU oracle (in the tests) and the HIP library
consume the same bytes it produces.

Values are drawn in fp32 and rounded to bf16 with round-to-nearest-even;
magnitudes below 2^-24 are flushed to zero first, so that a block sum of
keys is exact in fp64 (the representative's exactness precondition).

Key distributions:
  * i.i.d.: every key and query coordinate ~ N(0, 1);
  * mixture of Gaussians (MoG): each run of 128 consecutive keys shares a
    centroid c ~ N(0, I_64); a key is its centroid plus 0.5 * N(0, I_64); a
    query at position t is the centroid of a block drawn uniformly from the
    blocks 0 .. t // 128, plus 0.5 * N(0, I_64).

Random streams per workload seed: 0 centroids and keys, 1 queries, 2 needle
positions, 3 appended keys; 4, 5, 6 the attention queries, keys and values;
7 the sequence lengths of a mixed-length batch.

Attention inputs (the consumer of the indices) are i.i.d. N(0, 1) rows of
DA = 128 coordinates, one key and one value row beside each index key.
"""
from __future__ import annotations

import hashlib
from dataclasses import dataclass, field

import numpy as np

D = 64                 # index-key dimension of every workload
DA = 128               # attention head dimension
CENTROID_RUN = 128     # keys sharing one mixture centroid


def rng(seed: int, stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, stream])))


def to_bf16(x) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest even, after
    flushing |x| < 2^-24 to zero."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    x = np.where(np.abs(x) < np.float32(2.0 ** -24), np.float32(0.0), x)
    u = x.view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return (u >> 16).astype(np.uint16)


def from_bf16(h) -> np.ndarray:
    """bf16 bit patterns -> fp32 values (exact)."""
    return (np.asarray(h, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def sha256(*arrays) -> str:
    h = hashlib.sha256()
    for a in arrays:
        h.update(np.ascontiguousarray(a).view(np.uint8).tobytes())
    return h.hexdigest()[:16]


@dataclass
class Phase:
    """One index call: the queries, plus keys appended just before it."""
    name: str
    queries: np.ndarray            # [nq, D] bf16 bits
    q_pos: np.ndarray              # [nq] int64
    q_seq: np.ndarray              # [nq] int32
    append: np.ndarray | None = None   # [nseq, n_new, D] bf16 bits, or None


@dataclass
class Workload:
    name: str
    keys: np.ndarray               # packed keys [capacity_total, D] bf16 bits
    seq_key_off: np.ndarray        # [nseq] int64
    seq_len: np.ndarray            # [nseq] int64, lengths before any append
    seq_cap: np.ndarray            # [nseq] int64, key rows reserved per sequence
    B: int
    m: int
    k: int
    phases: list = field(default_factory=list)
    needles: np.ndarray | None = None

    @property
    def nseq(self) -> int:
        return len(self.seq_len)

    def seq_rep_off(self, B: int | None = None) -> np.ndarray:
        """Representative rows start at each sequence's key 0; reserve
        ceil(capacity / B) rows per sequence."""
        B = B or self.B
        nblk = (self.seq_cap + B - 1) // B
        return np.concatenate([[0], np.cumsum(nblk)[:-1]]).astype(np.int64)

    def total_rep_rows(self, B: int | None = None) -> int:
        B = B or self.B
        return int(((self.seq_cap + B - 1) // B).sum())


def _mog_keys(g: np.random.Generator, centroids: np.ndarray, start: int, n: int) -> np.ndarray:
    blk = (np.arange(start, start + n) // CENTROID_RUN)
    noise = g.standard_normal((n, D), dtype=np.float32)
    return centroids[blk] + np.float32(0.5) * noise


def _mog_queries(g: np.random.Generator, centroids: np.ndarray, pos: np.ndarray) -> np.ndarray:
    hi = pos // CENTROID_RUN + 1
    pick = (g.random(len(pos)) * hi).astype(np.int64)
    pick = np.minimum(pick, hi - 1)
    noise = g.standard_normal((len(pos), D), dtype=np.float32)
    return centroids[pick] + np.float32(0.5) * noise


def tiny_prefill(L: int = 4096, nq: int | None = None, seed: int = 1, B: int = 128,
                 m: int = 8, k: int = 256) -> Workload:
    """Causal prefill on i.i.d. N(0,1) keys and queries; query i sits at
    position i."""
    nq = L if nq is None else nq
    keys = to_bf16(rng(seed, 0).standard_normal((L, D), dtype=np.float32))
    queries = to_bf16(rng(seed, 1).standard_normal((nq, D), dtype=np.float32))
    q_pos = np.arange(nq, dtype=np.int64) * max(1, L // nq) if nq != L else np.arange(L, dtype=np.int64)
    w = Workload("tiny_prefill", keys, np.zeros(1, np.int64), np.array([L], np.int64),
                 np.array([L], np.int64), B, m, k)
    w.phases.append(Phase("prefill", queries, q_pos, np.zeros(nq, np.int32)))
    return w


def decode_batch(nseq: int = 16, L: int = 32768, seed: int = 2, B: int = 128, m: int = 64,
                 k: int = 2048, spare: int = 0) -> Workload:
    """nseq independent MoG sequences of L keys, one query per sequence at
    position L-1.  `spare` extra key rows are reserved per sequence."""
    gk, gq = rng(seed, 0), rng(seed, 1)
    cap = L + spare
    keys = np.zeros((nseq * cap, D), np.uint16)
    queries = np.zeros((nseq, D), np.uint16)
    nblk = (cap + CENTROID_RUN - 1) // CENTROID_RUN
    pos = np.full(nseq, L - 1, np.int64)
    for s in range(nseq):
        cent = gk.standard_normal((nblk, D), dtype=np.float32)
        keys[s * cap: s * cap + L] = to_bf16(_mog_keys(gk, cent, 0, L))
        queries[s] = to_bf16(_mog_queries(gq, cent, pos[s:s + 1]))[0]
    w = Workload("decode_batch", keys, np.arange(nseq, dtype=np.int64) * cap,
                 np.full(nseq, L, np.int64), np.full(nseq, cap, np.int64), B, m, k)
    w.phases.append(Phase("decode", queries, pos, np.arange(nseq, dtype=np.int32)))
    return w


def decode_varlen(nseq: int = 64, lo: int = 4096, hi: int = 131072, seed: int = 7, B: int = 128, m: int = 64,
                  k: int = 2048) -> Workload:
    """nseq MoG sequences whose lengths are drawn log-uniformly from
    [lo, hi] (stream 7), packed back to back, one query per sequence at its
    last position: a decode batch of mixed lengths in one launch."""
    gl, gk, gq = rng(seed, 7), rng(seed, 0), rng(seed, 1)
    lens = np.exp(gl.uniform(np.log(lo), np.log(hi), nseq)).astype(np.int64)
    lens = np.clip(lens, lo, hi)
    offs = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int64)
    keys = np.zeros((int(lens.sum()), D), np.uint16)
    queries = np.zeros((nseq, D), np.uint16)
    pos = lens - 1
    for s in range(nseq):
        L = int(lens[s])
        cent = gk.standard_normal(((L + CENTROID_RUN - 1) // CENTROID_RUN, D), dtype=np.float32)
        keys[offs[s]: offs[s] + L] = to_bf16(_mog_keys(gk, cent, 0, L))
        queries[s] = to_bf16(_mog_queries(gq, cent, pos[s:s + 1]))[0]
    w = Workload("decode_varlen", keys, offs, lens.copy(), lens.copy(), B, m, k)
    w.phases.append(Phase("decode", queries, pos.astype(np.int64), np.arange(nseq, dtype=np.int32)))
    return w


def chunked_prefill(L: int = 32768, seed: int = 3, B: int = 128, m: int = 64, k: int = 2048,
                    q_positions: np.ndarray | None = None) -> Workload:
    """One MoG sequence of L keys with a query at every position (or at the
    given positions)."""
    gk, gq = rng(seed, 0), rng(seed, 1)
    nblk = (L + CENTROID_RUN - 1) // CENTROID_RUN
    cent = gk.standard_normal((nblk, D), dtype=np.float32)
    keys = to_bf16(_mog_keys(gk, cent, 0, L))
    pos = np.arange(L, dtype=np.int64) if q_positions is None else np.asarray(q_positions, np.int64)
    queries = to_bf16(_mog_queries(gq, cent, pos))
    w = Workload("chunked_prefill", keys, np.zeros(1, np.int64), np.array([L], np.int64),
                 np.array([L], np.int64), B, m, k)
    w.phases.append(Phase("prefill", queries, pos, np.zeros(len(pos), np.int32)))
    return w


def long_context(L: int = 131072, chunk: int = 4096, ndecode: int = 32, nneedles: int = 64,
                 seed: int = 4, B: int = 128, m: int = 64, k: int = 2048) -> Workload:
    """One MoG sequence of L keys; a prefill chunk of the last `chunk`
    positions and a decode batch of `ndecode` queries at L-1.  `nneedles`
    keys at distinct uniform positions are replaced by 3x the first decode
    query."""
    gk, gq, gn = rng(seed, 0), rng(seed, 1), rng(seed, 2)
    nblk = (L + CENTROID_RUN - 1) // CENTROID_RUN
    cent = gk.standard_normal((nblk, D), dtype=np.float32)
    keys = to_bf16(_mog_keys(gk, cent, 0, L))
    dpos = np.full(ndecode, L - 1, np.int64)
    dq = to_bf16(_mog_queries(gq, cent, dpos))
    cpos = np.arange(L - chunk, L, dtype=np.int64)
    cq = to_bf16(_mog_queries(gq, cent, cpos))
    needles = np.sort(gn.choice(L, size=nneedles, replace=False)).astype(np.int64)
    keys[needles] = to_bf16(np.float32(3.0) * from_bf16(dq[0]))[None, :]
    w = Workload("long_context", keys, np.zeros(1, np.int64), np.array([L], np.int64),
                 np.array([L], np.int64), B, m, k, needles=needles)
    w.phases.append(Phase("prefill_chunk", cq, cpos, np.zeros(chunk, np.int32)))
    w.phases.append(Phase("decode", dq, dpos, np.zeros(ndecode, np.int32)))
    return w


def long_decode_append(L0: int = 1_047_552, steps: int = 8, n_new: int = 128, seed: int = 5,
                       B: int = 128, m: int = 64, k: int = 2048) -> Workload:
    """One MoG sequence of L0 keys; `steps` times: append n_new MoG keys,
    then one query at the new last position."""
    gk, gq, ga = rng(seed, 0), rng(seed, 1), rng(seed, 3)
    cap = L0 + steps * n_new
    nblk = (cap + CENTROID_RUN - 1) // CENTROID_RUN
    cent = gk.standard_normal((nblk, D), dtype=np.float32)
    keys = np.zeros((cap, D), np.uint16)
    keys[:L0] = to_bf16(_mog_keys(gk, cent, 0, L0))
    w = Workload("long_decode_append", keys, np.zeros(1, np.int64), np.array([L0], np.int64),
                 np.array([cap], np.int64), B, m, k)
    L = L0
    for s in range(steps):
        new = to_bf16(_mog_keys(ga, cent, L, n_new))[None]
        L += n_new
        pos = np.array([L - 1], np.int64)
        q = to_bf16(_mog_queries(gq, cent, pos))
        w.phases.append(Phase("step%d" % s, q, pos, np.zeros(1, np.int32), append=new))
    return w


def attention_inputs(rows: int, nq: int, seed: int):
    """(queries [nq, DA], keys [rows, DA], values [rows, DA]) as bf16 bits,
    i.i.d. N(0, 1), from streams 4, 5 and 6 of the seed."""
    qa = to_bf16(rng(seed, 4).standard_normal((nq, DA), dtype=np.float32))
    ka = to_bf16(rng(seed, 5).standard_normal((rows, DA), dtype=np.float32))
    va = to_bf16(rng(seed, 6).standard_normal((rows, DA), dtype=np.float32))
    return qa, ka, va


# The five workloads at full size, by short name.
FULL = {
    "tiny_prefill_4k": lambda: tiny_prefill(),
    "decode_32k_x16": lambda: decode_batch(),
    "chunked_prefill_32k": lambda: chunked_prefill(),
    "long_context_128k": lambda: long_context(),
    "long_decode_1m_append": lambda: long_decode_append(),
}
