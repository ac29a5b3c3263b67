"""Cumulative indicator table (test infrastructure; see package docstring).

Source: "Precision As You Need" paper notes, Key design 1: the table
K[b, l] = 1[r_l <= b] is generated once and sliced by prefix for any stream
length.  Here rows are indexed by the level u = b + 1 in [0, P], so
K[u][l] = 1[r_l < u]; row u = 0 is the all-zero stream that the most negative
bipolar value needs.
"""

import numpy as np


def indicator_table(r: np.ndarray, P: int) -> np.ndarray:
    """K[u][l] = 1 if r_l < u else 0, for u in [0, P] and l < len(r).

    Returned as uint8 of shape (P + 1, len(r)).
    """
    r = np.asarray(r, dtype=np.int64)
    K = np.zeros((P + 1, r.shape[0]), dtype=np.uint8)
    for u in range(P + 1):
        for l in range(r.shape[0]):
            K[u, l] = 1 if r[l] < u else 0
    return K


def cumulative_table(K: np.ndarray) -> np.ndarray:
    """cum[u][n] = sum over l < n of K[u][l], for n in [0, len(r)].

    Returned as int64 of shape (P + 1, len(r) + 1).
    """
    rows, n = K.shape
    cum = np.zeros((rows, n + 1), dtype=np.int64)
    for u in range(rows):
        total = 0
        for l in range(n):
            total += int(K[u, l])
            cum[u, l + 1] = total
    return cum
