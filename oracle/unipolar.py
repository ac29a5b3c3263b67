"""Unipolar (AND-gate) SC mode, materialised bit by bit (test
infrastructure; see package docstring).

Sources:
* "Precision As You Need" paper notes, "Research background and motivation":
  SC represents a value by the frequency of ones in a bitstream, so a
  multiplier becomes one AND gate (unipolar) or one XNOR gate (bipolar);
  Key design 3 compares the unipolar AND gate with an unsigned INT8
  multiplier.
* scmp_vit README, the SC compensation driver flags: the compensation
  matmul's per-row SC quantisation mode is bipolar or unipolar.
* "Precision As You Need" Key design 1: the C-BSG streams and the Sobol
  cumulative table, used here unchanged.

Readings (the pages give neither the unipolar level map nor a sign rule):
* The same per-row (or per-chunk) quantiser as the bipolar mode: x_int in
  [-q, q] with s = a / q.
* Sign-magnitude: a stream carries |x_int| at level u = round(P |x| / q),
  computed exactly in integers (q is odd, so no value falls on a tie): 0 maps
  to 0 and q to P, so a stream's density is |x| / q.  The signs of the two
  operands multiply the count.  For non-negative operands (softmax
  probabilities) every sign is +1 and this is plain unipolar SC.
* The streams are those of the bipolar mode (A: the L-prefix of K[u_A]; B:
  two counters gated by A's bits); the gate is AND, so a position counts
  when both bits are 1.
* Decode per chunk c: s^A_ic s^B_jc q^2 (sum over d in c of
  sign_A sign_B count_d) / L_c, since count / L estimates
  (|x_A| / q)(|x_B| / q).
"""

import numpy as np

from .cbsg import _streams_for_row, conditional_stream_b, stream_a
from .quant import QMAX


def unipolar_level(x_int, p: int = 8):
    """Level u in [0, P] of the magnitude of an integer x in [-q, q]:
    u = floor((2 P |x| + q) / (2 q)) = round(P |x| / q)."""
    q = QMAX(p)
    P = 1 << p
    x = np.abs(np.asarray(x_int, dtype=np.int64))
    return (2 * P * x + q) // (2 * q)


def and_count(K_a: np.ndarray, K_b: np.ndarray, u_a, u_b, L: int) -> int:
    """Sum over d of the AND count of one (row, column) pair: positions
    l < L where A's bit and B's conditional bit are both 1."""
    u_a = np.atleast_1d(np.asarray(u_a, dtype=np.int64))
    u_b = np.atleast_1d(np.asarray(u_b, dtype=np.int64))
    total = 0
    for d in range(u_a.shape[0]):
        a = stream_a(K_a, int(u_a[d]), L)
        b = conditional_stream_b(K_b, a, int(u_b[d]))
        total += int(np.sum(a & b))
    return total


def and_count_row(K: np.ndarray, u_a_row, u_b, L_per_d, col_block: int = 32):
    """AND counts of one A row against every B row, materialising B's
    conditional stream for each (column j, index d, position l).  Shapes as
    the bipolar row count: ``u_a_row`` (D,), ``u_b`` (N, D), ``L_per_d``
    (D,); returns int64 (N, D)."""
    u_a_row = np.asarray(u_a_row, dtype=np.int64)
    u_b = np.asarray(u_b, dtype=np.int64)
    L_per_d = np.asarray(L_per_d, dtype=np.int64)
    N, D = u_b.shape
    a, idx, valid = _streams_for_row(K, u_a_row, L_per_d)
    Lm = a.shape[1]
    out = np.zeros((N, D), dtype=np.int64)
    if Lm == 0:
        return out
    width = K.shape[1]
    flatK = K.reshape(-1)
    for j0 in range(0, N, col_block):
        ub = u_b[j0:j0 + col_block]
        b = flatK[ub[:, :, None] * width + idx[None, :, :]]
        both = (b == 1) & (a[None, :, :] == 1) & valid[None, :, :]
        out[j0:j0 + col_block] = both.sum(axis=2)
    return out


def sign_of(x_int) -> np.ndarray:
    """+1 for x >= 0, -1 for x < 0 (a zero has level 0, so its sign never
    matters)."""
    return np.where(np.asarray(x_int) < 0, -1, 1).astype(np.int64)


def decode_unipolar(signed_counts, sA, sB, L, q: int):
    """Sum over chunks of s^A s^B q^2 count_c / L_c in float64.

    ``signed_counts``: (rows, N, n_chunks) sums of sign_A sign_B count;
    ``sA`` (rows, n_chunks); ``sB`` (N, n_chunks); ``L`` (rows, n_chunks).
    Returns (C, sum of the chunk terms' absolute values)."""
    terms = (np.asarray(sA, dtype=np.float64)[:, None, :]
             * np.asarray(sB, dtype=np.float64)[None, :, :]
             * float(q * q)
             * np.asarray(signed_counts, dtype=np.float64)
             / np.asarray(L, dtype=np.float64)[:, None, :])
    return terms.sum(axis=2), np.abs(terms).sum(axis=2)
