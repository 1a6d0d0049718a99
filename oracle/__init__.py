"""CPU oracle for the HISA indexer and the flat DSA indexer (numpy front end).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the bench's
CPU-baseline leg are the only callers.  The product path never imports this
package, and this package imports nothing from the product package.

The arithmetic lives in ``hisa_oracle.c`` and ``lsa_oracle.c`` (LSA-Flat)
(plain C, fp64, OpenMP over queries); this module compiles them with gcc on
first use and marshals numpy arrays.  See the headers of the C files for the
passages of the pages each step follows and for the readings taken where
the pages are silent.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRCS = [os.path.join(_HERE, "hisa_oracle.c"), os.path.join(_HERE, "lsa_oracle.c")]
_LIB = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int


def build(force: bool = True) -> str:
    """Compile the oracle into ``oracle/liboracle.so`` (IEEE semantics kept:
    no fast-math, no FMA contraction)."""
    if not force and os.path.exists(_LIB) and all(os.path.getmtime(_LIB) >= os.path.getmtime(s) for s in _SRCS):
        return _LIB
    tmp = _LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
           "-fno-fast-math", "-ffp-contract=off", "-o", tmp] + _SRCS + ["-lm"]
    subprocess.check_call(cmd)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build(force=False)
            lib = ctypes.CDLL(_LIB)
            lib.oracle_pool.argtypes = [_P, _I64, _I32, _I32, _P, _P]
            lib.oracle_pool_range.argtypes = [_P, _I64, _I32, _I32, _I64, _I64, _P, _P]
            lib.oracle_block_scores.argtypes = [_P, _P, _I64, _I32, _P]
            lib.oracle_select_blocks.argtypes = [_P, _P, _I64, _I32, _I32, _I32, _P, _P]
            lib.oracle_tokens_on_blocks.argtypes = [_P, _P, _I64, _I64, _I32, _I32, _P, _I32,
                                                    _I32, _P, _P, _P]
            lib.oracle_hisa_query.argtypes = [_P, _P, _P, _I64, _I64, _I32, _I32, _I32, _I32,
                                              _P, _P, _P, _P]
            lib.oracle_flat_query.argtypes = [_P, _P, _I64, _I64, _I32, _I32, _P, _P, _P]
            lib.oracle_block_only_query.argtypes = [_P, _P, _I64, _I64, _I32, _I32, _I32, _P, _P]
            lib.oracle_attention_row.argtypes = [_P, _P, _P, _I64, _I32, _P, _I32, ctypes.c_double, _P]
            lib.oracle_attention_row.restype = _I32
            lib.oracle_attention_batch.argtypes = [_P, _P, _P, _I64, _I32, _P, _P, _P, _I32,
                                                   ctypes.c_double, _P]
            lib.oracle_index_batch.argtypes = [_I32, _P, _P, _P, _I64, _P, _P, _P, _P, _P,
                                               _I32, _I32, _I32, _I32, _I32, _P, _P, _P]
            lib.oracle_lsa_ward.argtypes = [_P, _I32, _I32, _I32, _I32, _P, _P, _P, _P]
            lib.oracle_lsa_ward.restype = _I32
            lib.oracle_lsa_block.argtypes = [_P, _I32, _P, _P, _P, _P]
            lib.oracle_lsa_build.argtypes = [_P, _I64, _I32, _P, _P, _P, _P]
            lib.oracle_lsa_query.argtypes = [_P, _P, _P, _P, _I64, _I64, _I32, _I32, _I32, _P, _P, _P]
            lib.oracle_lsa_batch.argtypes = [_P, _P, _P, _I64, _P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _I32,
                                             _P, _P]
            lib.oracle_bf16_round.argtypes = [ctypes.c_double]
            lib.oracle_bf16_round.restype = ctypes.c_uint16
            lib.oracle_threads.restype = ctypes.c_int
            lib.oracle_set_threads.argtypes = [_I32]
            _lib = lib
    return _lib


def _ptr(a: np.ndarray | None):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _u16(a) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint16:
        raise TypeError("bf16 arrays are passed as their uint16 bit patterns")
    return a


def threads() -> int:
    return int(_load().oracle_threads())


def set_threads(n: int) -> None:
    """OpenMP threads of later oracle calls from this thread (timing only)."""
    _load().oracle_set_threads(int(n))


def bf16_round(v: float) -> int:
    """Round-to-nearest-even of a double to bf16 bits (the representative
    rounding rule)."""
    return int(_load().oracle_bf16_round(float(v)))


def pool(keys, B: int, return_flag: bool = False):
    """Block representatives of one sequence: keys [L, d] bf16 bits ->
    reps [ceil(L/B), d] bf16 bits."""
    keys = _u16(keys)
    L, d = keys.shape
    M = (L + B - 1) // B
    reps = np.zeros((M, d), np.uint16)
    flag = ctypes.c_int(0)
    rc = _load().oracle_pool(_ptr(keys), L, d, B, _ptr(reps), ctypes.byref(flag))
    if rc != 0:
        raise ValueError("oracle_pool: bad arguments")
    return (reps, bool(flag.value)) if return_flag else reps


def pool_range(keys, B: int, b0: int, b1: int, reps: np.ndarray) -> bool:
    """Re-pool blocks [b0, b1) in place (the incremental update at append)."""
    keys = _u16(keys)
    L, d = keys.shape
    assert reps.dtype == np.uint16 and reps.flags.c_contiguous
    flag = ctypes.c_int(0)
    rc = _load().oracle_pool_range(_ptr(keys), L, d, B, b0, b1, _ptr(reps), ctypes.byref(flag))
    if rc != 0:
        raise ValueError("oracle_pool_range: bad arguments")
    return bool(flag.value)


def block_scores(q, reps) -> np.ndarray:
    q = _u16(q)
    reps = _u16(reps)
    out = np.zeros(reps.shape[0], np.float64)
    _load().oracle_block_scores(_ptr(q), _ptr(reps), reps.shape[0], reps.shape[1], _ptr(out))
    return out


def select_blocks(q, reps, t: int, B: int, m: int):
    """Ascending block ids a query at position t keeps, and how many block
    scores that took."""
    q = _u16(q)
    reps = _u16(reps)
    sel = np.zeros(m, np.int64)
    nb = ctypes.c_int64(0)
    n = _load().oracle_select_blocks(_ptr(q), _ptr(reps), t, reps.shape[1], B, m,
                                     _ptr(sel), ctypes.byref(nb))
    if n < 0:
        raise ValueError("oracle_select_blocks: bad arguments")
    return sel[:n].copy(), int(nb.value)


def tokens_on_blocks(q, keys, t: int, B: int, blocks, k: int):
    """Stage 2 on a given block set: (idx[k], scores[k])."""
    q = _u16(q)
    keys = _u16(keys)
    blocks = np.ascontiguousarray(blocks, np.int64)
    idx = np.zeros(k, np.int32)
    sc = np.zeros(k, np.float64)
    rc = _load().oracle_tokens_on_blocks(_ptr(q), _ptr(keys), keys.shape[0], t, keys.shape[1],
                                         B, _ptr(blocks), len(blocks), k, _ptr(idx), _ptr(sc),
                                         None)
    if rc != 0:
        raise ValueError("oracle_tokens_on_blocks: bad arguments")
    return idx, sc


def hisa_query(q, keys, reps, t: int, B: int, m: int, k: int):
    """One HISA query: (idx[k], scores[k], blocks[m], (n_block_scores,
    n_token_scores))."""
    q = _u16(q)
    keys = _u16(keys)
    reps = _u16(reps)
    idx = np.zeros(k, np.int32)
    sc = np.zeros(k, np.float64)
    blk = np.zeros(m, np.int32)
    counts = np.zeros(2, np.int64)
    rc = _load().oracle_hisa_query(_ptr(q), _ptr(keys), _ptr(reps), keys.shape[0], t,
                                   keys.shape[1], B, m, k, _ptr(idx), _ptr(sc), _ptr(blk),
                                   _ptr(counts))
    if rc != 0:
        raise ValueError("oracle_hisa_query: bad arguments")
    return idx, sc, blk, (int(counts[0]), int(counts[1]))


def flat_query(q, keys, t: int, k: int):
    q = _u16(q)
    keys = _u16(keys)
    idx = np.zeros(k, np.int32)
    sc = np.zeros(k, np.float64)
    counts = np.zeros(2, np.int64)
    rc = _load().oracle_flat_query(_ptr(q), _ptr(keys), keys.shape[0], t, keys.shape[1], k,
                                   _ptr(idx), _ptr(sc), _ptr(counts))
    if rc != 0:
        raise ValueError("oracle_flat_query: bad arguments")
    return idx, sc, (int(counts[0]), int(counts[1]))


def block_only_query(q, reps, L: int, t: int, B: int, m: int):
    """Block-only selection of one query: (idx[m*B], blocks[m])."""
    q = _u16(q)
    reps = _u16(reps)
    idx = np.zeros(m * B, np.int32)
    blk = np.zeros(m, np.int32)
    rc = _load().oracle_block_only_query(_ptr(q), _ptr(reps), L, t, q.shape[-1], B, m, _ptr(idx), _ptr(blk))
    if rc != 0:
        raise ValueError("oracle_block_only_query: bad arguments")
    return idx, blk


def index_batch(flat: bool, queries, q_pos, keys, k: int, *, reps=None, q_seq=None,
                seq_key_off=None, seq_rep_off=None, seq_len=None, B: int = 128, m: int = 3,
                block_only: bool = False):
    """Batched HISA (flat=False) or flat (flat=True) over packed sequences,
    or with block_only the block-only selection (k = m*B, no scores).
    Returns (idx[nq,k] int32, scores[nq,k] fp64 or None, blocks[nq,m]
    int32 or None)."""
    queries = _u16(queries)
    keys = _u16(keys)
    nq, d = queries.shape
    q_pos = np.ascontiguousarray(q_pos, np.int64)
    if seq_key_off is None:
        seq_key_off = np.zeros(1, np.int64)
        seq_rep_off = np.zeros(1, np.int64)
        seq_len = np.array([keys.shape[0]], np.int64)
    seq_key_off = np.ascontiguousarray(seq_key_off, np.int64)
    seq_len = np.ascontiguousarray(seq_len, np.int64)
    seq_rep_off = None if seq_rep_off is None else np.ascontiguousarray(seq_rep_off, np.int64)
    q_seq = None if q_seq is None else np.ascontiguousarray(q_seq, np.int32)
    if reps is not None:
        reps = _u16(reps)
    idx = np.zeros((nq, k), np.int32)
    sc = None if block_only else np.zeros((nq, k), np.float64)
    blk = None if flat else np.zeros((nq, m), np.int32)
    mode = 2 if block_only else int(bool(flat))
    rc = _load().oracle_index_batch(mode, _ptr(queries), _ptr(q_pos), _ptr(q_seq), nq,
                                    _ptr(keys), _ptr(reps), _ptr(seq_key_off), _ptr(seq_rep_off),
                                    _ptr(seq_len), len(seq_len), d, B, m, k, _ptr(idx), _ptr(sc),
                                    _ptr(blk))
    if rc != 0:
        raise ValueError("oracle_index_batch: bad arguments")
    return idx, sc, blk


def attention_row(qa, ka, v, idx, scale: float) -> np.ndarray:
    """Sparse attention of one row (fp64): softmax over the valid indices of
    idx of scale * qa . ka_j, applied to the v rows.  ka, v: [len, dh]."""
    qa, ka, v = _u16(qa), _u16(ka), _u16(v)
    idx = np.ascontiguousarray(idx, np.int32)
    dh = qa.shape[-1]
    out = np.zeros(dh, np.float64)
    _load().oracle_attention_row(_ptr(qa), _ptr(ka), _ptr(v), ka.shape[0], dh, _ptr(idx), len(idx), scale,
                                 _ptr(out))
    return out


def attention_batch(qa, ka, v, key_off, lens, idx, scale: float) -> np.ndarray:
    """Rows i of qa [nq, dh] over the sequence at key_off[i] of length
    lens[i] (negative: zero output) in ka / v [rows, dh]; idx [nq, kk]."""
    qa, ka, v = _u16(qa), _u16(ka), _u16(v)
    idx = np.ascontiguousarray(idx, np.int32)
    key_off = np.ascontiguousarray(key_off, np.int64)
    lens = np.ascontiguousarray(lens, np.int64)
    nq, dh = qa.shape
    out = np.zeros((nq, dh), np.float64)
    _load().oracle_attention_batch(_ptr(qa), _ptr(ka), _ptr(v), nq, dh, _ptr(key_off), _ptr(lens), _ptr(idx),
                                   idx.shape[1], scale, _ptr(out))
    return out


# ---- LSA-Flat (lsa_oracle.c) ----------------------------------------------------

LSA_BLOCK = 512
LSA_POINTS = 128
LSA_BUCKETS = 64


def lsa_ward(points, target: int, cap: int):
    """Agglomerate the rows of points (fp64) by rounds of mutual cheapest
    pairs down to `target` buckets of at most `cap` points.  Returns
    (labels [n] -- each point's bucket root, the bucket's smallest point --,
    merges [(kept, absorbed), ...] in merge order, margin, buckets left)."""
    P = np.ascontiguousarray(points, np.float64)
    n, d = P.shape
    label = np.zeros(n, np.int32)
    margin = np.zeros(1, np.float64)
    merges = np.zeros(2 * n, np.int32)
    nm = np.zeros(1, np.int32)
    left = _load().oracle_lsa_ward(_ptr(P), n, d, target, cap, _ptr(label), _ptr(margin), _ptr(merges), _ptr(nm))
    return label, merges[: 2 * int(nm[0])].reshape(-1, 2), float(margin[0]), int(left)


def lsa_build(keys):
    """Buckets of every complete 512-key block of one sequence: (centroids
    [nblk*64, d] bf16 bits, members [nblk, 128] uint8, offs [nblk, 65]
    uint8, margins [nblk])."""
    keys = _u16(keys)
    L, d = keys.shape
    nblk = L // LSA_BLOCK
    cen = np.zeros((max(nblk, 1) * LSA_BUCKETS, d), np.uint16)
    mem = np.zeros((max(nblk, 1), LSA_POINTS), np.uint8)
    off = np.zeros((max(nblk, 1), LSA_BUCKETS + 1), np.uint8)
    mg = np.zeros(max(nblk, 1), np.float64)
    rc = _load().oracle_lsa_build(_ptr(keys), L, d, _ptr(cen), _ptr(mem), _ptr(off), _ptr(mg))
    if rc < 0:
        raise ValueError("oracle_lsa_build failed")
    return cen[: nblk * LSA_BUCKETS], mem[:nblk], off[:nblk], mg[:nblk]


def lsa_query(q, cen, mem, off, t: int, p: int, k: int):
    """One flat-search query: (idx [k], buckets [p], scores [p])."""
    q = _u16(q)
    cen = _u16(cen)
    mem = np.ascontiguousarray(mem, np.uint8)
    off = np.ascontiguousarray(off, np.uint8)
    idx = np.zeros(k, np.int32)
    bk = np.zeros(p, np.int32)
    sc = np.zeros(p, np.float64)
    rc = _load().oracle_lsa_query(_ptr(q), _ptr(cen), _ptr(mem), _ptr(off), mem.shape[0], t, q.shape[-1], p, k,
                                  _ptr(idx), _ptr(bk), _ptr(sc))
    if rc < 0:
        raise ValueError("oracle_lsa_query: bad arguments")
    return idx, bk, sc


def lsa_batch(queries, q_pos, q_seq, cen, mem, off, seq_blk_off, seq_nblk, seq_len, p: int, k: int):
    """Batched flat search over packed sequences: (idx [nq, k], buckets
    [nq, p], ids relative to each query's sequence)."""
    queries = _u16(queries)
    nq, d = queries.shape
    idx = np.zeros((nq, k), np.int32)
    bk = np.zeros((nq, p), np.int32)
    seq_len = np.ascontiguousarray(seq_len, np.int64)
    rc = _load().oracle_lsa_batch(_ptr(queries), _ptr(np.ascontiguousarray(q_pos, np.int64)),
                                  _ptr(None if q_seq is None else np.ascontiguousarray(q_seq, np.int32)), nq,
                                  _ptr(_u16(cen)), _ptr(np.ascontiguousarray(mem, np.uint8)),
                                  _ptr(np.ascontiguousarray(off, np.uint8)),
                                  _ptr(np.ascontiguousarray(seq_blk_off, np.int64)),
                                  _ptr(np.ascontiguousarray(seq_nblk, np.int64)), _ptr(seq_len), len(seq_len), d, p,
                                  k, _ptr(idx), _ptr(bk))
    if rc != 0:
        raise ValueError("oracle_lsa_batch: bad arguments")
    return idx, bk
