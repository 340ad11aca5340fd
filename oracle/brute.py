"""Brute-force characterisations used to pin the oracle (test infrastructure only).

These do not share the oracle's rank rule: each selection is found by
enumerating every admissible subset with exact rational arithmetic and taking
the one that keeps the most magnitude, the lexicographically smallest sorted
index tuple among equal totals.  For magnitude N:M pruning ("Success story:
ESPLAG", Highlights and Solution; "To 2:4 Sparsity and Beyond", abstract) that
subset is exactly the one the rank rule keeps: every maximiser holds all keys
above the N-th largest plus some of the keys tied with it, and trading a tied
index for a lower tied one makes the sorted tuple smaller.
"""

from __future__ import annotations

import itertools
from fractions import Fraction

import numpy as np


def _frac(x: float) -> Fraction:
    return Fraction(float(x))


def best_subset(keys, N: int):
    """Sorted tuple of N indices maximising the exact key sum (lexicographic tie-break)."""
    best, best_sum = None, None
    for sub in itertools.combinations(range(len(keys)), N):   # lexicographic order
        s = sum((_frac(keys[i]) for i in sub), Fraction(0))
        if best_sum is None or s > best_sum:
            best, best_sum = sub, s
    return best


def nm_mask(values64: np.ndarray, N: int, M: int) -> np.ndarray:
    """uint8 mask of a float64 matrix, chosen group by group by best_subset on |values|."""
    R, K = values64.shape
    out = np.zeros((R, K), np.uint8)
    for r in range(R):
        for g in range(K // M):
            sub = best_subset([abs(v) for v in values64[r, g * M:(g + 1) * M]], N)
            for p in sub:
                out[r, g * M + p] = 1
    return out


def venom_select(values64: np.ndarray, V: int, M: int):
    """(colsel [R/V, K/M, 4], mask [R, K]) for V:N:M with 4 columns kept, then 2:4.

    Stage 1 enumerates all C(M, 4) column subsets of a group and keeps the one
    with the largest exact sum of the block's column L1 norms; stage 2 runs
    best_subset with N = 2 on each row's 4 selected values.
    """
    R, K = values64.shape
    G = K // M
    colsel = np.zeros((R // V, G, 4), np.uint8)
    mask = np.zeros((R, K), np.uint8)
    for blk in range(R // V):
        rows = range(blk * V, (blk + 1) * V)
        for g in range(G):
            l1 = [sum((abs(_frac(values64[r, g * M + c])) for r in rows), Fraction(0))
                  for c in range(M)]
            cols = best_subset(l1, 4)
            colsel[blk, g] = cols
            for r in rows:
                js = best_subset([abs(values64[r, g * M + c]) for c in cols], 2)
                for j in js:
                    mask[r, g * M + cols[j]] = 1
    return colsel, mask


def dense_product(A64: np.ndarray, B64: np.ndarray) -> np.ndarray:
    """Exact A @ B with Fractions, rounded once to float64 (tiny inputs only)."""
    R, K = A64.shape
    Nc = B64.shape[1]
    out = np.zeros((R, Nc))
    for i in range(R):
        for j in range(Nc):
            acc = Fraction(0)
            for k in range(K):
                if A64[i, k] != 0 and B64[k, j] != 0:
                    acc += _frac(A64[i, k]) * _frac(B64[k, j])
            out[i, j] = float(acc)
    return out
