"""Conditional bitstream generator (C-BSG) and the bipolar XNOR count,
materialised bit by bit (test infrastructure; see package docstring).

Source: "Precision As You Need" paper notes, Key design 1: the second
operand's random-number generator is driven by the first operand's
bitstream, which makes the conditional probability equal the marginal one
and the bipolar XNOR product unbiased at any finite length L; the streams are
prefix slices of the cumulative indicator table.  The scmp_vit README
("Why it works") describes the count as an "enable-signal" count over a Sobol
prefix.

Reading taken (where the pages leave the mechanism open):
* A (the row side, X) emits a_l = K[u_A][l] for l < L: its stream at length
  L is the L-prefix of its full-length stream (early termination).
* B (the weight side, W) keeps two counters c1 and c0, both starting at 0.
  When a_l = 1 it emits K[u_B][c1] and advances c1; when a_l = 0 it emits
  K[u_B][c0] and advances c0.  B's randomness is thus indexed by A's bits.
* The count is the number of positions where the streams agree,
  XNOR(a, b) = 1 - (a XOR b), summed over l < L and over the contraction
  index d.
"""

import numpy as np


def stream_a(K: np.ndarray, u_a: int, L: int) -> np.ndarray:
    """A's stream at length L: the first L bits of table row u_a."""
    if L > K.shape[1]:
        raise ValueError("L exceeds the table length")
    return K[u_a, :L].astype(np.uint8)


def conditional_stream_b(K_b: np.ndarray, a: np.ndarray, u_b: int) -> np.ndarray:
    """B's stream given A's stream ``a``: two counters gated by A's bit."""
    b = np.zeros(a.shape[0], dtype=np.uint8)
    c1 = 0
    c0 = 0
    for l in range(a.shape[0]):
        if a[l]:
            b[l] = K_b[u_b, c1]
            c1 += 1
        else:
            b[l] = K_b[u_b, c0]
            c0 += 1
    return b


def xnor_count(K_a: np.ndarray, K_b: np.ndarray, u_a, u_b, L: int) -> int:
    """Sum over d of the XNOR count of one (row, column) pair.

    ``u_a`` and ``u_b`` are sequences of levels along the contraction axis
    (or scalars); ``K_a`` drives A's stream and ``K_b`` is the table B's
    counters index (the same table in the method; tests pass shifted copies
    to check unbiasedness).
    """
    u_a = np.atleast_1d(np.asarray(u_a, dtype=np.int64))
    u_b = np.atleast_1d(np.asarray(u_b, dtype=np.int64))
    total = 0
    for d in range(u_a.shape[0]):
        a = stream_a(K_a, int(u_a[d]), L)
        b = conditional_stream_b(K_b, a, int(u_b[d]))
        total += int(np.sum(1 - (a ^ b)))
    return total


def _streams_for_row(K: np.ndarray, u_a_row: np.ndarray, L_per_d: np.ndarray):
    """For one A row: the materialised A bits and B's counter index at every
    (d, l), padded to the longest L.  Positions l >= L_d are marked invalid.

    The counter index is the value of c1 (when a_l = 1) or c0 (when a_l = 0)
    at step l, i.e. the number of earlier positions whose A bit equals a_l.
    """
    D = u_a_row.shape[0]
    Lm = int(L_per_d.max()) if D else 0
    a = np.zeros((D, Lm), dtype=np.uint8)
    idx = np.zeros((D, Lm), dtype=np.int64)
    valid = np.zeros((D, Lm), dtype=bool)
    for d in range(D):
        L = int(L_per_d[d])
        ad = K[int(u_a_row[d]), :L]
        ones_before = np.concatenate(([0], np.cumsum(ad)[:-1])) if L else ad
        zeros_before = np.arange(L) - ones_before
        a[d, :L] = ad
        idx[d, :L] = np.where(ad == 1, ones_before, zeros_before)
        valid[d, :L] = True
    return a, idx, valid


def xnor_count_row(K: np.ndarray, u_a_row, u_b, L_per_d, col_block: int = 32):
    """XNOR counts of one A row against every B row, materialising B's
    conditional stream for each (column j, contraction index d, position l).

    ``u_a_row``: levels of the A row, shape (D,).
    ``u_b``: levels of the B rows, shape (N, D).
    ``L_per_d``: stream length used at each contraction index, shape (D,)
    (one value everywhere for per-row MP; per band for K-bands).

    Returns int64 counts of shape (N, D): the count at each contraction index,
    so callers can sum over any chunk or band.
    """
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
        ub = u_b[j0:j0 + col_block]                     # (nb, D)
        flat_index = ub[:, :, None] * width + idx[None, :, :]
        b = flatK[flat_index]                           # (nb, D, Lm)
        agree = (b == a[None, :, :]) & valid[None, :, :]
        out[j0:j0 + col_block] = agree.sum(axis=2)
    return out
