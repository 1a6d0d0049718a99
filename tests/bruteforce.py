"""Independent brute-force checks used to pin the oracle (tests only).

Written from the pages' definitions with a different structure from the
oracle: exact rational arithmetic (fractions) for means and rounding, and
dense score matrices with masks (numpy) for selection.  Nothing here is
shared with the oracle or with the HIP library.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np


def bf16_bits_to_fraction(h: int) -> Fraction:
    """Exact value of a finite bf16 bit pattern."""
    sign = -1 if h & 0x8000 else 1
    e = (h >> 7) & 0xFF
    f = h & 0x7F
    assert e != 0xFF, "finite values only"
    if e == 0:
        return sign * Fraction(f, 1 << 7) * Fraction(1, 1 << 126)
    return sign * (1 + Fraction(f, 1 << 7)) * (Fraction(2) ** (e - 127))


def _all_bf16_positive_sorted():
    vals = [(bf16_bits_to_fraction(h), h) for h in range(0x0000, 0x7F80)]
    return vals


_POS = None


def bf16_round_exact(x: Fraction) -> int:
    """Round an exact rational to bf16 bits: nearest value, ties to the
    pattern with an even last bit; beyond the largest finite value by at
    least half a spacing, infinity."""
    global _POS
    if _POS is None:
        _POS = _all_bf16_positive_sorted()
    sign = 0x8000 if x < 0 else 0
    a = abs(x)
    if a == 0:
        return sign
    lo_i, hi_i = 0, len(_POS) - 1
    if a >= _POS[-1][0]:
        top = _POS[-1][0]
        half_ulp = (top - _POS[-2][0]) / 2
        return sign | (0x7F80 if a >= top + half_ulp else _POS[-1][1])
    while hi_i - lo_i > 1:                      # _POS[lo] <= a < _POS[hi]
        mid = (lo_i + hi_i) // 2
        if _POS[mid][0] <= a:
            lo_i = mid
        else:
            hi_i = mid
    lo, hi = _POS[lo_i], _POS[hi_i]
    if a - lo[0] < hi[0] - a:
        return sign | lo[1]
    if a - lo[0] > hi[0] - a:
        return sign | hi[1]
    return sign | (lo[1] if lo[1] % 2 == 0 else hi[1])


def bf16_values(h: np.ndarray) -> np.ndarray:
    return (np.asarray(h, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def pool_exact(keys: np.ndarray, B: int) -> np.ndarray:
    """Representatives by exact rational mean, then exact RNE to bf16."""
    L, d = keys.shape
    M = (L + B - 1) // B
    out = np.zeros((M, d), np.uint16)
    for b in range(M):
        rows = keys[b * B: min(L, (b + 1) * B)]
        for c in range(d):
            s = sum(bf16_bits_to_fraction(int(h)) for h in rows[:, c])
            out[b, c] = bf16_round_exact(s / len(rows))
    return out


def hisa_dense(Q: np.ndarray, K: np.ndarray, R: np.ndarray, pos: np.ndarray, B: int, m: int,
               k: int, flat: bool = False):
    """Whole-matrix HISA / flat: dense score matrices, masks, lexsort.
    Returns (idx[nq,k], blocks[nq,m]) with -1 padding, idx ascending."""
    q = bf16_values(Q)
    kk = bf16_values(K)
    L = K.shape[0]
    tok = (q @ kk.T).astype(np.float32)            # [nq, L] ranking keys
    nq = Q.shape[0]
    idx = np.full((nq, k), -1, np.int32)
    blocks = np.full((nq, m), -1, np.int32)
    if not flat:
        rr = bf16_values(R)
        blk = (q @ rr.T).astype(np.float32)        # [nq, M]
        M = R.shape[0]
    for i in range(nq):
        t = int(pos[i])
        visible = np.arange(L) <= t
        if flat:
            allowed = visible
        else:
            c = t // B
            causal = np.arange(M) <= c
            if c + 1 <= m:
                keep = causal.copy()
            else:
                forced = np.zeros(M, bool)
                forced[[0, c - 1, c]] = True
                free = causal & ~forced
                ids = np.nonzero(free)[0]
                order = np.lexsort((ids, -blk[i, ids]))   # score desc, id asc
                keep = forced.copy()
                keep[ids[order[: m - 3]]] = True
            kept = np.nonzero(keep)[0]
            blocks[i, : len(kept)] = kept
            allowed = visible & keep[np.arange(L) // B]
        ids = np.nonzero(allowed)[0]
        order = np.lexsort((ids, -tok[i, ids]))
        top = np.sort(ids[order[:k]])
        idx[i, : len(top)] = top
    return idx, blocks
