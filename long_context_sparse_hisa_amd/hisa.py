"""Thin ctypes binding of libhisa (include/hisa.h).

Argument marshalling only: torch tensors supply device pointers and the
current HIP stream; every step of the indexer runs in the HIP library.
The library must have been built (``python -m long_context_sparse_hisa_amd.build``);
if it is missing, or a tensor is not on the GPU, the calls raise.
"""
from __future__ import annotations

import ctypes
import os
import re

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libhisa.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "hisa.h")

HISA_OK = 0
HISA_ERR_INVALID_ARG = -1
HISA_ERR_UNSUPPORTED = -2
HISA_ERR_WORKSPACE = -3
HISA_ERR_HIP = -4

_P = ctypes.c_void_p
_lib = None


class HisaError(RuntimeError):
    def __init__(self, status: int, call: str):
        self.status = status
        super().__init__("%s: %s (%d)" % (call, status_str(status), status))


class hisa_seq(ctypes.Structure):
    _fields_ = [("key_off", ctypes.c_int64), ("rep_off", ctypes.c_int64), ("len", ctypes.c_int64),
                ("capacity", ctypes.c_int64)]


class hisa_index_args(ctypes.Structure):
    _fields_ = [
        ("queries", _P), ("q_pos", _P), ("q_seq", _P), ("nq", ctypes.c_int64),
        ("keys", _P), ("reps", _P), ("seq_key_off", _P), ("seq_rep_off", _P), ("seq_len", _P),
        ("nseq", ctypes.c_int32), ("max_len", ctypes.c_int64),
        ("d", ctypes.c_int32), ("B", ctypes.c_int32), ("m", ctypes.c_int32), ("k", ctypes.c_int32),
        ("out_idx", _P), ("out_scores", _P), ("out_blocks", _P),
        ("workspace", _P), ("workspace_bytes", ctypes.c_size_t),
        ("stage_events", ctypes.POINTER(_P)),
    ]


HISA_STAGES = 3
HISA_ATTN_DIM = 128
HISA_LSA_BLOCK = 512
HISA_LSA_BUCKETS = 64
HISA_LSA_POOL_KEYS = 128


class hisa_lsa_args(ctypes.Structure):
    _fields_ = [
        ("queries", _P), ("q_pos", _P), ("q_seq", _P), ("nq", ctypes.c_int64),
        ("centroids", _P), ("members", _P), ("offs", _P),
        ("seq_blk_off", _P), ("seq_nblk", _P), ("seq_len", _P), ("nseq", ctypes.c_int32),
        ("max_len", ctypes.c_int64), ("d", ctypes.c_int32), ("p", ctypes.c_int32), ("k", ctypes.c_int32),
        ("out_idx", _P), ("out_buckets", _P), ("workspace", _P), ("workspace_bytes", ctypes.c_size_t),
    ]


class hisa_attn_args(ctypes.Structure):
    _fields_ = [
        ("q", _P), ("k", _P), ("v", _P), ("idx", _P), ("q_seq", _P), ("seq_key_off", _P), ("seq_len", _P),
        ("nseq", ctypes.c_int32), ("nq", ctypes.c_int64), ("kk", ctypes.c_int32), ("dh", ctypes.c_int32),
        ("scale", ctypes.c_float), ("out", _P), ("workspace", _P), ("workspace_bytes", ctypes.c_size_t),
    ]


def lib():
    """The loaded libhisa (raises if it was not built)."""
    global _lib
    if _lib is None:
        import torch  # noqa: F401  (one HIP runtime: libhisa binds to the one torch loaded)
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libhisa.so is not built: run python -m long_context_sparse_hisa_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        L.hisa_pool_blocks.argtypes = [_P, ctypes.c_int64, ctypes.c_int, ctypes.c_int, _P, _P]
        L.hisa_append_keys.argtypes = [_P, _P, ctypes.POINTER(hisa_seq), ctypes.c_int, _P,
                                       ctypes.c_int64, ctypes.c_int, ctypes.c_int, _P]
        L.hisa_workspace_bytes.argtypes = [ctypes.POINTER(hisa_index_args), ctypes.c_int,
                                           ctypes.POINTER(ctypes.c_size_t),
                                           ctypes.POINTER(ctypes.c_size_t),
                                           ctypes.POINTER(ctypes.c_size_t)]
        L.hisa_index.argtypes = [ctypes.POINTER(hisa_index_args), _P]
        L.hisa_index_static.argtypes = [ctypes.POINTER(hisa_index_args), _P]
        L.hisa_flat_index.argtypes = [ctypes.POINTER(hisa_index_args), _P]
        L.hisa_block_index.argtypes = [ctypes.POINTER(hisa_index_args), _P]
        L.hisa_decode_step.argtypes = [ctypes.POINTER(hisa_index_args), ctypes.POINTER(hisa_seq), _P,
                                       ctypes.c_int64, _P]
        L.hisa_attention_workspace_bytes.argtypes = [ctypes.POINTER(hisa_attn_args),
                                                     ctypes.POINTER(ctypes.c_size_t)]
        L.hisa_sparse_attention.argtypes = [ctypes.POINTER(hisa_attn_args), _P]
        L.hisa_lsa_build.argtypes = [_P, ctypes.c_int64, ctypes.c_int64, ctypes.c_int, _P, _P, _P, _P]
        L.hisa_lsa_workspace_bytes.argtypes = [ctypes.POINTER(hisa_lsa_args), ctypes.POINTER(ctypes.c_size_t)]
        L.hisa_lsa_index.argtypes = [ctypes.POINTER(hisa_lsa_args), _P]
        L.hisa_status_str.restype = ctypes.c_char_p
        L.hisa_status_str.argtypes = [ctypes.c_int]
        L.hisa_abi_version.restype = ctypes.c_int
        _lib = L
    return _lib


def header_functions() -> list:
    """Names of the functions include/hisa.h declares."""
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(hisa_\w+)\s*\(", text, re.M)))


def status_str(status: int) -> str:
    return lib().hisa_status_str(int(status)).decode()


def abi_version() -> int:
    return int(lib().hisa_abi_version())


def _check(rc: int, call: str):
    if rc != HISA_OK:
        raise HisaError(rc, call)


def _dev(t, what: str, nbytes_per_elem=None):
    """Device pointer of a contiguous GPU tensor (or None)."""
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("%s must be a GPU tensor" % what)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % what)
    if nbytes_per_elem is not None and t.element_size() != nbytes_per_elem:
        raise ValueError("%s must have %d-byte elements" % (what, nbytes_per_elem))
    return t.data_ptr()


def _stream(stream):
    """A torch stream, a raw hipStream_t handle (int), or None for torch's
    current stream."""
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def seq_array(seqs):
    """The host hisa_seq array of the append calls from (key_off, rep_off,
    len, capacity) tuples; an existing hisa_seq array is returned as it is
    (build it once to keep per-call marshalling out of a decode loop)."""
    if isinstance(seqs, ctypes.Array) and seqs._type_ is hisa_seq:
        return seqs
    return (hisa_seq * max(1, len(seqs)))(*[hisa_seq(*map(int, s)) for s in seqs])


def hisa_pool_blocks(keys, B: int, reps, stream=None):
    """reps[:ceil(L/B)] = block means of keys [L, 64] (bf16 bits)."""
    rc = lib().hisa_pool_blocks(_dev(keys, "keys", 2), keys.shape[0], keys.shape[1], B,
                                _dev(reps, "reps", 2), _stream(stream))
    _check(rc, "hisa_pool_blocks")


def hisa_append_keys(keys, reps, seqs, new_keys, B: int, stream=None):
    """Append new_keys [nseq, n_new, 64] to each sequence; seqs is a list of
    (key_off, rep_off, len, capacity) with the lengths before the append."""
    arr = seq_array(seqs)
    n_new = new_keys.shape[1] if new_keys.dim() == 3 else new_keys.shape[0]
    rc = lib().hisa_append_keys(_dev(keys, "keys", 2), _dev(reps, "reps", 2), arr, len(seqs),
                                _dev(new_keys, "new_keys", 2), n_new, keys.shape[-1], B,
                                _stream(stream))
    _check(rc, "hisa_append_keys")


def make_args(queries, q_pos, keys, k: int, *, reps=None, q_seq=None, seq_key_off=None,
              seq_rep_off=None, seq_len=None, max_len=None, B: int = 128, m: int = 64,
              out_idx=None, out_scores=None, out_blocks=None, workspace=None) -> hisa_index_args:
    a = hisa_index_args()
    a.queries = _dev(queries, "queries", 2)
    a.q_pos = _dev(q_pos, "q_pos", 8)
    a.q_seq = _dev(q_seq, "q_seq", 4)
    a.nq = queries.shape[0]
    a.keys = _dev(keys, "keys", 2)
    a.reps = _dev(reps, "reps", 2)
    a.seq_key_off = _dev(seq_key_off, "seq_key_off", 8)
    a.seq_rep_off = _dev(seq_rep_off, "seq_rep_off", 8)
    a.seq_len = _dev(seq_len, "seq_len", 8)
    a.nseq = 1 if seq_len is None else seq_len.shape[0]
    a.max_len = keys.shape[0] if max_len is None else int(max_len)
    a.d = queries.shape[1]
    a.B, a.m, a.k = B, m, k
    a.out_idx = _dev(out_idx, "out_idx", 4)
    a.out_scores = _dev(out_scores, "out_scores", 4)
    a.out_blocks = _dev(out_blocks, "out_blocks", 4)
    if workspace is not None:
        a.workspace = _dev(workspace, "workspace")
        a.workspace_bytes = workspace.numel() * workspace.element_size()
    return a


def hisa_workspace_bytes(args: hisa_index_args, flat: bool = False, all_queries: bool = False):
    """(recommended bytes, minimum bytes) of workspace for these args, or
    with all_queries (recommended, minimum, one-chunk bytes)."""
    b = ctypes.c_size_t(0)
    mb = ctypes.c_size_t(0)
    ab = ctypes.c_size_t(0)
    rc = lib().hisa_workspace_bytes(ctypes.byref(args), int(flat), ctypes.byref(b), ctypes.byref(mb),
                                    ctypes.byref(ab))
    _check(rc, "hisa_workspace_bytes")
    if all_queries:
        return int(b.value), int(mb.value), int(ab.value)
    return int(b.value), int(mb.value)


def hisa_index(args: hisa_index_args, stream=None):
    _check(lib().hisa_index(ctypes.byref(args), _stream(stream)), "hisa_index")


def hisa_index_static(args: hisa_index_args, stream=None):
    """hisa_index on the library's own device scratch (args.workspace is
    ignored; nothing is allocated)."""
    _check(lib().hisa_index_static(ctypes.byref(args), _stream(stream)), "hisa_index_static")


def hisa_flat_index(args: hisa_index_args, stream=None):
    _check(lib().hisa_flat_index(ctypes.byref(args), _stream(stream)), "hisa_flat_index")


def hisa_decode_step(args: hisa_index_args, seqs, new_keys, stream=None):
    """Append new_keys [nseq, n_new, 64] to every sequence (seqs: host
    (key_off, rep_off, len before, capacity) per sequence) and index."""
    arr = seq_array(seqs)
    n_new = 0 if new_keys is None else (new_keys.shape[1] if new_keys.dim() == 3 else new_keys.shape[0])
    rc = lib().hisa_decode_step(ctypes.byref(args), arr, _dev(new_keys, "new_keys", 2), n_new, _stream(stream))
    _check(rc, "hisa_decode_step")


def hisa_block_index(args: hisa_index_args, stream=None):
    _check(lib().hisa_block_index(ctypes.byref(args), _stream(stream)), "hisa_block_index")


def make_attn_args(q, k, v, idx, scale: float, *, q_seq=None, seq_key_off=None, seq_len=None,
                   out=None, workspace=None) -> hisa_attn_args:
    """Arguments of hisa_sparse_attention: q [nq, 128], k and v [L, 128]
    (bf16 bits), idx [nq, kk] int32, seq_len [nseq] int64 (required),
    out [nq, 128] float32."""
    if seq_len is None:
        raise ValueError("seq_len is required")
    a = hisa_attn_args()
    a.q = _dev(q, "q", 2)
    a.k = _dev(k, "k", 2)
    a.v = _dev(v, "v", 2)
    a.idx = _dev(idx, "idx", 4)
    a.q_seq = _dev(q_seq, "q_seq", 4)
    a.seq_key_off = _dev(seq_key_off, "seq_key_off", 8)
    a.seq_len = _dev(seq_len, "seq_len", 8)
    a.nseq = seq_len.shape[0]
    a.nq = q.shape[0]
    a.kk = idx.shape[1]
    a.dh = q.shape[1]
    a.scale = float(scale)
    a.out = _dev(out, "out", 4)
    if workspace is not None:
        a.workspace = _dev(workspace, "workspace")
        a.workspace_bytes = workspace.numel() * workspace.element_size()
    return a


def hisa_attention_workspace_bytes(args: hisa_attn_args) -> int:
    b = ctypes.c_size_t(0)
    _check(lib().hisa_attention_workspace_bytes(ctypes.byref(args), ctypes.byref(b)),
           "hisa_attention_workspace_bytes")
    return int(b.value)


def hisa_sparse_attention(args: hisa_attn_args, stream=None):
    _check(lib().hisa_sparse_attention(ctypes.byref(args), _stream(stream)), "hisa_sparse_attention")


def hisa_lsa_build(keys, first_block: int, centroids, members, offs, stream=None):
    """Buckets of blocks first_block .. len(keys)//512 - 1 of one sequence
    (keys [L, 64] bf16 bits; cache arrays start at the sequence's block 0)."""
    rc = lib().hisa_lsa_build(_dev(keys, "keys", 2), keys.shape[0], int(first_block), keys.shape[1],
                              _dev(centroids, "centroids", 2), _dev(members, "members", 1),
                              _dev(offs, "offs", 1), _stream(stream))
    _check(rc, "hisa_lsa_build")


def make_lsa_args(queries, q_pos, centroids, members, offs, seq_blk_off, seq_nblk, seq_len, max_len: int, p: int,
                  k: int, *, q_seq=None, out_idx=None, out_buckets=None, workspace=None) -> hisa_lsa_args:
    a = hisa_lsa_args()
    a.queries = _dev(queries, "queries", 2)
    a.q_pos = _dev(q_pos, "q_pos", 8)
    a.q_seq = _dev(q_seq, "q_seq", 4)
    a.nq = queries.shape[0]
    a.centroids = _dev(centroids, "centroids", 2)
    a.members = _dev(members, "members", 1)
    a.offs = _dev(offs, "offs", 1)
    a.seq_blk_off = _dev(seq_blk_off, "seq_blk_off", 8)
    a.seq_nblk = _dev(seq_nblk, "seq_nblk", 8)
    a.seq_len = _dev(seq_len, "seq_len", 8)
    a.nseq = seq_len.shape[0]
    a.max_len = int(max_len)
    a.d = queries.shape[1]
    a.p, a.k = p, k
    a.out_idx = _dev(out_idx, "out_idx", 4)
    a.out_buckets = _dev(out_buckets, "out_buckets", 4)
    if workspace is not None:
        a.workspace = _dev(workspace, "workspace")
        a.workspace_bytes = workspace.numel() * workspace.element_size()
    return a


def hisa_lsa_workspace_bytes(args: hisa_lsa_args) -> int:
    b = ctypes.c_size_t(0)
    _check(lib().hisa_lsa_workspace_bytes(ctypes.byref(args), ctypes.byref(b)), "hisa_lsa_workspace_bytes")
    return int(b.value)


def hisa_lsa_index(args: hisa_lsa_args, stream=None):
    _check(lib().hisa_lsa_index(ctypes.byref(args), _stream(stream)), "hisa_lsa_index")


# ---- HIP events (stage timing) -------------------------------------------------

_hip = None


def _hiprt():
    global _hip
    if _hip is None:
        lib()                                  # the HIP runtime torch loaded
        h = ctypes.CDLL("libamdhip64.so.7")
        h.hipEventCreate.argtypes = [ctypes.POINTER(_P)]
        h.hipEventDestroy.argtypes = [_P]
        h.hipEventSynchronize.argtypes = [_P]
        h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), _P, _P]
        h.hipEventRecord.argtypes = [_P, _P]
        _hip = h
    return _hip


class StageEvents:
    """2 * HISA_STAGES hipEvent_t handles to hang on hisa_index_args: the
    start and stop of every stage, taken from the kernel dispatches."""

    def __init__(self):
        h = _hiprt()
        n = 2 * HISA_STAGES
        self.handles = (_P * n)()
        for i in range(n):
            e = _P()
            if h.hipEventCreate(ctypes.byref(e)) != 0:
                raise RuntimeError("hipEventCreate failed")
            self.handles[i] = e

    def attach(self, args: hisa_index_args):
        args.stage_events = ctypes.cast(self.handles, ctypes.POINTER(_P))

    def stage_ms(self, s: int) -> float:
        """Duration of stage s (start of its first kernel to end of its last)."""
        h = _hiprt()
        h.hipEventSynchronize(self.handles[2 * s + 1])
        f = ctypes.c_float(0.0)
        if h.hipEventElapsedTime(ctypes.byref(f), self.handles[2 * s], self.handles[2 * s + 1]) != 0:
            raise RuntimeError("hipEventElapsedTime failed (stage %d not recorded?)" % s)
        return float(f.value)

    def __del__(self):
        try:
            h = _hiprt()
            for i in range(2 * HISA_STAGES):
                h.hipEventDestroy(self.handles[i])
        except Exception:
            pass
