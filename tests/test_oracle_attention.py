"""Pins of the sparse-attention oracle (CPU): each compares it with something
other than itself -- exact values, a dense brute force built a different
way, and invariants the definition fixes."""
from fractions import Fraction

import numpy as np

import oracle
from long_context_sparse_hisa_amd import synth

DH = 128


def _rows(g, n, scale=1.0):
    return synth.to_bf16((g.standard_normal((n, DH)) * scale).astype(np.float32))


def _val(h):
    return synth.from_bf16(h).astype(np.float64)


def test_single_index_returns_its_value_row():
    g = np.random.default_rng(1)
    q, k, v = _rows(g, 1)[0], _rows(g, 50), _rows(g, 50)
    out = oracle.attention_row(q, k, v, np.array([-1, 17, -1], np.int32), 0.088)
    assert np.array_equal(out, _val(v[17]))


def test_zero_query_gives_the_exact_mean_of_the_selected_values():
    g = np.random.default_rng(2)
    k, v = _rows(g, 300), _rows(g, 300)
    idx = np.sort(g.choice(300, 97, replace=False)).astype(np.int32)
    out = oracle.attention_row(np.zeros(DH, np.uint16), k, v, idx, 0.088)
    vals = _val(v[idx])
    for c in range(DH):
        exact = sum(Fraction(float(x)) for x in vals[:, c]) / len(idx)
        assert out[c] == float(exact)


def test_matches_a_dense_masked_softmax():
    """Full score matrix, -inf outside each row's index set, softmax, then
    a matrix product: a different construction of the same quantity."""
    g = np.random.default_rng(3)
    L, nq, kk = 400, 12, 40
    k, v = _rows(g, L), _rows(g, L)
    q = _rows(g, nq)
    idx = np.full((nq, kk), -1, np.int32)
    for i in range(nq):
        n = int(g.integers(1, kk + 1))
        idx[i, :n] = g.choice(L, n, replace=False)
    scale = 1.0 / np.sqrt(DH)
    S = scale * (_val(q) @ _val(k).T)
    mask = np.zeros((nq, L), bool)
    for i in range(nq):
        mask[i, idx[i][idx[i] >= 0]] = True
    S = np.where(mask, S, -np.inf)
    P = np.exp(S - S.max(axis=1, keepdims=True))
    P /= P.sum(axis=1, keepdims=True)
    want = P @ _val(v)
    got = oracle.attention_batch(q, k, v, np.zeros(nq, np.int64), np.full(nq, L, np.int64), idx, scale)
    assert np.allclose(got, want, rtol=1e-12, atol=1e-12)


def test_order_of_the_indices_does_not_matter():
    g = np.random.default_rng(4)
    k, v, q = _rows(g, 500), _rows(g, 500), _rows(g, 1)[0]
    idx = g.choice(500, 200, replace=False).astype(np.int32)
    a = oracle.attention_row(q, k, v, idx, 0.088)
    b = oracle.attention_row(q, k, v, g.permutation(idx).astype(np.int32), 0.088)
    assert np.allclose(a, b, rtol=1e-12, atol=1e-14)


def test_large_scores_stay_finite_and_pick_the_best_key():
    """Scores near 4e3: without subtracting the maximum exp would overflow."""
    g = np.random.default_rng(5)
    k = _rows(g, 64)
    q = synth.to_bf16(synth.from_bf16(k[9]) * np.float32(30.0))
    v = _rows(g, 64)
    out = oracle.attention_row(q, k, v, np.arange(64, dtype=np.int32), 1.0)
    assert np.all(np.isfinite(out))
    assert np.allclose(out, _val(v[9]), atol=1e-9)


def test_absent_indices_are_ignored_and_an_empty_row_is_zero():
    g = np.random.default_rng(6)
    k, v, q = _rows(g, 30), _rows(g, 30), _rows(g, 1)[0]
    a = oracle.attention_row(q, k, v, np.array([3, 7, 11], np.int32), 0.1)
    b = oracle.attention_row(q, k, v, np.array([-1, 3, 30, 7, 99, 11, -1], np.int32), 0.1)
    assert np.array_equal(a, b)
    assert np.array_equal(oracle.attention_row(q, k, v, np.array([-1, 30], np.int32), 0.1), np.zeros(DH))


def test_batch_rows_read_their_own_sequence():
    g = np.random.default_rng(7)
    k, v = _rows(g, 700), _rows(g, 700)
    q = _rows(g, 3)
    key_off = np.array([0, 300, 450], np.int64)
    lens = np.array([300, 150, -1], np.int64)
    idx = np.array([[5, 299, -1], [0, 149, 7], [1, 2, 3]], np.int32)
    got = oracle.attention_batch(q, k, v, key_off, lens, idx, 0.09)
    assert np.array_equal(got[0], oracle.attention_row(q[0], k[:300], v[:300], idx[0], 0.09))
    assert np.array_equal(got[1], oracle.attention_row(q[1], k[300:450], v[300:450], idx[1], 0.09))
    assert np.array_equal(got[2], np.zeros(DH))
