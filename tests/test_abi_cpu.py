"""The C-ABI library without a GPU: it loads, exports what include/hisa.h
declares, and rejects bad arguments on the host before touching a device."""
import ctypes
import os

import pytest

from long_context_sparse_hisa_amd import hisa

FAKE = 0x1000          # never dereferenced: validation fails first


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(hisa.LIB_PATH):
        from long_context_sparse_hisa_amd import build
        build.build()
    return hisa.lib()


def test_exports_every_declared_function(lib):
    names = hisa.header_functions()
    assert {"hisa_pool_blocks", "hisa_append_keys", "hisa_index", "hisa_flat_index",
            "hisa_workspace_bytes", "hisa_status_str", "hisa_abi_version", "hisa_sparse_attention",
            "hisa_attention_workspace_bytes", "hisa_block_index"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_status_strings(lib):
    assert hisa.abi_version() == 1
    for code in (0, -1, -2, -3, -4):
        assert hisa.status_str(code) != "unknown status"
    assert hisa.status_str(7) == "unknown status"


def _args(**kw):
    a = hisa.hisa_index_args()
    a.queries = FAKE
    a.q_pos = FAKE
    a.keys = FAKE
    a.reps = FAKE
    a.out_idx = FAKE
    a.nq = 16
    a.nseq = 1
    a.max_len = 32768
    a.d, a.B, a.m, a.k = 64, 128, 64, 2048
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def _rc(fn, a):
    return fn(ctypes.byref(a), None)


@pytest.mark.parametrize("field,value,code", [
    ("d", 32, hisa.HISA_ERR_UNSUPPORTED),
    ("B", 100, hisa.HISA_ERR_UNSUPPORTED),
    ("B", 512, hisa.HISA_ERR_UNSUPPORTED),
    ("m", 2, hisa.HISA_ERR_INVALID_ARG),
    ("k", 0, hisa.HISA_ERR_INVALID_ARG),
    ("k", 8193, hisa.HISA_ERR_INVALID_ARG),        # m*B < k: the no-loss condition
    ("m", 200, hisa.HISA_ERR_UNSUPPORTED),         # m*B beyond the candidate limit
    ("nq", -1, hisa.HISA_ERR_INVALID_ARG),
    ("nseq", 0, hisa.HISA_ERR_INVALID_ARG),
    ("nseq", 2, hisa.HISA_ERR_INVALID_ARG),        # several sequences need offsets
    ("max_len", 0, hisa.HISA_ERR_INVALID_ARG),
    ("max_len", (1 << 30) + 1, hisa.HISA_ERR_UNSUPPORTED),
    ("max_len", 16384 * 128 + 1, hisa.HISA_ERR_UNSUPPORTED),  # 16385 blocks of 128
    ("queries", None, hisa.HISA_ERR_INVALID_ARG),
    ("reps", None, hisa.HISA_ERR_INVALID_ARG),
    ("out_idx", None, hisa.HISA_ERR_INVALID_ARG),
])
def test_index_validation(lib, field, value, code):
    assert _rc(lib.hisa_index, _args(**{field: value})) == code


def test_flat_ignores_block_arguments(lib):
    a = _args(B=100, m=0, reps=None, workspace=FAKE, workspace_bytes=16)
    assert _rc(lib.hisa_flat_index, a) == hisa.HISA_ERR_WORKSPACE
    assert _rc(lib.hisa_flat_index, _args(d=16)) == hisa.HISA_ERR_UNSUPPORTED


def test_workspace_checks(lib):
    a = _args()
    assert _rc(lib.hisa_index, a) == hisa.HISA_ERR_WORKSPACE          # none given
    want, least, whole = hisa.hisa_workspace_bytes(a, all_queries=True)
    assert 0 < least <= want <= whole
    a = _args(workspace=FAKE, workspace_bytes=least - 1)
    assert _rc(lib.hisa_index, a) == hisa.HISA_ERR_WORKSPACE
    fw, fl = hisa.hisa_workspace_bytes(_args(), flat=True)
    assert 0 < fl <= fw
    # one query of a 32K flat row needs its 32768 ranking keys
    assert fl >= 32768 * 4


def test_zero_queries_is_a_no_op(lib):
    a = _args(nq=0, queries=None, q_pos=None, out_idx=None)
    assert _rc(lib.hisa_index, a) == hisa.HISA_OK
    assert _rc(lib.hisa_flat_index, a) == hisa.HISA_OK


def test_pool_and_append_validation(lib):
    P = ctypes.c_void_p
    assert lib.hisa_pool_blocks(P(FAKE), 0, 64, 128, P(FAKE), None) == hisa.HISA_OK
    assert lib.hisa_pool_blocks(P(FAKE), -1, 64, 128, P(FAKE), None) == hisa.HISA_ERR_INVALID_ARG
    assert lib.hisa_pool_blocks(P(FAKE), 10, 32, 128, P(FAKE), None) == hisa.HISA_ERR_UNSUPPORTED
    assert lib.hisa_pool_blocks(P(FAKE), 10, 64, 96, P(FAKE), None) == hisa.HISA_ERR_UNSUPPORTED
    assert lib.hisa_pool_blocks(None, 10, 64, 128, P(FAKE), None) == hisa.HISA_ERR_INVALID_ARG
    seqs = (hisa.hisa_seq * 2)(hisa.hisa_seq(0, 0, 100, 228), hisa.hisa_seq(228, 2, 200, 228))
    # the second sequence has room for 28 keys only
    assert lib.hisa_append_keys(P(FAKE), P(FAKE), seqs, 2, P(FAKE), 29, 64, 128, None) == \
        hisa.HISA_ERR_INVALID_ARG
    assert lib.hisa_append_keys(P(FAKE), P(FAKE), seqs, 2, P(FAKE), 0, 64, 128, None) == hisa.HISA_OK
    assert lib.hisa_append_keys(P(FAKE), P(FAKE), seqs, 2, P(FAKE), 8, 64, 48, None) == \
        hisa.HISA_ERR_UNSUPPORTED
    assert lib.hisa_append_keys(P(FAKE), P(FAKE), seqs, -1, P(FAKE), 8, 64, 128, None) == \
        hisa.HISA_ERR_INVALID_ARG


def _attn(**kw):
    a = hisa.hisa_attn_args()
    a.q = a.k = a.v = a.idx = a.seq_len = a.out = FAKE
    a.nq, a.nseq, a.kk, a.dh, a.scale = 16, 1, 2048, 128, 0.088
    for k, v in kw.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("field,value,code", [
    ("dh", 64, hisa.HISA_ERR_UNSUPPORTED),
    ("kk", 0, hisa.HISA_ERR_INVALID_ARG),
    ("kk", 16385, hisa.HISA_ERR_UNSUPPORTED),
    ("nq", -1, hisa.HISA_ERR_INVALID_ARG),
    ("nseq", 0, hisa.HISA_ERR_INVALID_ARG),
    ("nseq", 2, hisa.HISA_ERR_INVALID_ARG),        # several sequences need offsets
    ("scale", float("nan"), hisa.HISA_ERR_INVALID_ARG),
    ("scale", float("inf"), hisa.HISA_ERR_INVALID_ARG),
    ("v", None, hisa.HISA_ERR_INVALID_ARG),
    ("seq_len", None, hisa.HISA_ERR_INVALID_ARG),
    ("out", None, hisa.HISA_ERR_INVALID_ARG),
])
def test_attention_validation(lib, field, value, code):
    a = _attn(**{field: value})
    assert lib.hisa_sparse_attention(ctypes.byref(a), None) == code


def test_attention_workspace(lib):
    a = _attn()
    assert lib.hisa_sparse_attention(ctypes.byref(a), None) == hisa.HISA_ERR_WORKSPACE
    # 16 queries x 16 chunks of 128 indices x (max, sum, 128 weighted values)
    assert hisa.hisa_attention_workspace_bytes(a) == 16 * 16 * 130 * 4
    a = _attn(workspace=FAKE, workspace_bytes=16 * 16 * 130 * 4 - 1)
    assert lib.hisa_sparse_attention(ctypes.byref(a), None) == hisa.HISA_ERR_WORKSPACE
    a = _attn(nq=0, q=None, out=None)
    assert lib.hisa_sparse_attention(ctypes.byref(a), None) == hisa.HISA_OK


def test_block_index_validation(lib):
    a = _args(k=64 * 128)                       # the whole candidate set
    assert _rc(lib.hisa_block_index, a) == hisa.HISA_ERR_WORKSPACE
    assert _rc(lib.hisa_block_index, _args(k=2048)) == hisa.HISA_ERR_INVALID_ARG       # k != m*B
    assert _rc(lib.hisa_block_index, _args(k=64 * 128, out_scores=FAKE)) == hisa.HISA_ERR_INVALID_ARG
    assert _rc(lib.hisa_block_index, _args(k=64 * 128, B=100)) == hisa.HISA_ERR_UNSUPPORTED
    assert _rc(lib.hisa_block_index, _args(k=64 * 128, nq=0, queries=None)) == hisa.HISA_OK


def _lsa(**kw):
    a = hisa.hisa_lsa_args()
    a.queries = a.q_pos = a.centroids = a.members = a.offs = FAKE
    a.seq_blk_off = a.seq_nblk = a.seq_len = a.out_idx = FAKE
    a.nq, a.nseq, a.max_len, a.d, a.p, a.k = 16, 1, 32768, 64, 256, 2048
    for k, v in kw.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("field,value,code", [
    ("d", 32, hisa.HISA_ERR_UNSUPPORTED),
    ("p", 0, hisa.HISA_ERR_INVALID_ARG),
    ("p", 2049, hisa.HISA_ERR_UNSUPPORTED),
    ("k", 0, hisa.HISA_ERR_INVALID_ARG),
    ("k", 16385, hisa.HISA_ERR_UNSUPPORTED),
    ("max_len", (1 << 20) + 1, hisa.HISA_ERR_UNSUPPORTED),
    ("nseq", 0, hisa.HISA_ERR_INVALID_ARG),
    ("centroids", None, hisa.HISA_ERR_INVALID_ARG),
    ("seq_nblk", None, hisa.HISA_ERR_INVALID_ARG),
])
def test_lsa_index_validation(lib, field, value, code):
    a = _lsa(**{field: value})
    assert lib.hisa_lsa_index(ctypes.byref(a), None) == code


def test_lsa_workspace_and_build_validation(lib):
    a = _lsa()
    assert lib.hisa_lsa_index(ctypes.byref(a), None) == hisa.HISA_ERR_WORKSPACE
    n = hisa.hisa_lsa_workspace_bytes(a)
    # the ranked bucket lists (ids and scores) of every query come first
    assert n > 16 * 256 * 8
    a = _lsa(nq=0, queries=None)
    assert lib.hisa_lsa_index(ctypes.byref(a), None) == hisa.HISA_OK
    P = ctypes.c_void_p
    assert lib.hisa_lsa_build(P(FAKE), 4096, 0, 32, P(FAKE), P(FAKE), P(FAKE), None) == hisa.HISA_ERR_UNSUPPORTED
    assert lib.hisa_lsa_build(P(FAKE), -1, 0, 64, P(FAKE), P(FAKE), P(FAKE), None) == hisa.HISA_ERR_INVALID_ARG
    assert lib.hisa_lsa_build(P(FAKE + 2), 4096, 0, 64, P(FAKE), P(FAKE), P(FAKE), None) == hisa.HISA_ERR_UNSUPPORTED
    assert lib.hisa_lsa_build(P(FAKE), 511, 0, 64, P(FAKE), P(FAKE), P(FAKE), None) == hisa.HISA_OK
    assert lib.hisa_lsa_build(P(FAKE), 4096, 8, 64, P(FAKE), P(FAKE), P(FAKE), None) == hisa.HISA_OK
    assert lib.hisa_lsa_build(None, 4096, 0, 64, P(FAKE), P(FAKE), P(FAKE), None) == hisa.HISA_ERR_INVALID_ARG


def test_decode_step_validation(lib):
    seqs = (hisa.hisa_seq * 1)(hisa.hisa_seq(0, 0, 100, 200))
    P = ctypes.c_void_p
    a = _args(max_len=200)
    assert lib.hisa_decode_step(ctypes.byref(a), seqs, P(FAKE), -1, None) == hisa.HISA_ERR_INVALID_ARG
    assert lib.hisa_decode_step(ctypes.byref(a), seqs, P(FAKE), 101, None) == hisa.HISA_ERR_INVALID_ARG   # capacity
    a = _args(max_len=150)
    assert lib.hisa_decode_step(ctypes.byref(a), seqs, P(FAKE), 60, None) == hisa.HISA_ERR_INVALID_ARG    # max_len
    a = _args(max_len=200)
    assert lib.hisa_decode_step(ctypes.byref(a), seqs, None, 5, None) == hisa.HISA_ERR_INVALID_ARG
    assert lib.hisa_decode_step(ctypes.byref(a), seqs, P(FAKE), 5, None) == hisa.HISA_ERR_WORKSPACE
    assert lib.hisa_decode_step(ctypes.byref(_args(d=32)), seqs, P(FAKE), 5, None) == hisa.HISA_ERR_UNSUPPORTED


def test_seq_array_marshalling():
    # tuples become hisa_seq rows; an array already built passes through as it is
    arr = hisa.seq_array([(0, 0, 100, 128), (128, 1, 7, 64)])
    assert len(arr) == 2
    assert (arr[1].key_off, arr[1].rep_off, arr[1].len, arr[1].capacity) == (128, 1, 7, 64)
    assert hisa.seq_array(arr) is arr
    # a raw stream handle is passed on unchanged
    assert hisa._stream(0x1234).value == 0x1234


def test_workspace_must_be_16_byte_aligned(lib):
    # the kernels read and write the workspace as 16-byte vectors: a
    # misaligned one is refused before any launch
    a = _args(max_len=200)
    want, least, whole = hisa.hisa_workspace_bytes(a, all_queries=True)
    bad = _args(max_len=200, workspace=FAKE + 4, workspace_bytes=whole)
    assert _rc(lib.hisa_index, bad) == hisa.HISA_ERR_INVALID_ARG
    assert _rc(lib.hisa_block_index, bad) == hisa.HISA_ERR_INVALID_ARG
    fw, fl = hisa.hisa_workspace_bytes(a, flat=True)
    assert _rc(lib.hisa_flat_index, _args(max_len=200, workspace=FAKE + 8, workspace_bytes=fw)) == \
        hisa.HISA_ERR_INVALID_ARG
    seqs = (hisa.hisa_seq * 1)(hisa.hisa_seq(0, 0, 100, 200))
    assert lib.hisa_decode_step(ctypes.byref(bad), seqs, ctypes.c_void_p(FAKE), 5, None) == hisa.HISA_ERR_INVALID_ARG
