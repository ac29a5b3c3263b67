"""Bipolar decode of XNOR counts (test infrastructure; see package
docstring).

Source: "Precision As You Need" paper notes, Key design 1, the decode
equation: C_ij = s^A_i s^B_j q_max^2 [ (2 / L) sum_l sum_d XNOR - D ].
With per-(row, chunk) scales (K-band pull request, "How the banding works":
bands are made of whole quantisation chunks) the same equation applies to
each chunk c of width |c| with its own length L_c, and the chunk terms add:
C_ij = sum_c s^A_ic s^B_jc q^2 (2 count_ijc - L_c |c|) / L_c.
Evaluated in float64.
"""

import numpy as np


def decode_terms(count_c, sA_c, sB_c, L_c, width_c, q: int):
    """One chunk's term s^A s^B q^2 (2 count - L |c|) / L in float64.

    All arguments broadcast; ``count_c`` is an integer array.
    """
    num = 2.0 * np.asarray(count_c, dtype=np.float64) - (
        np.asarray(L_c, dtype=np.float64) * np.asarray(width_c, dtype=np.float64)
    )
    return (
        np.asarray(sA_c, dtype=np.float64)
        * np.asarray(sB_c, dtype=np.float64)
        * float(q * q)
        * num
        / np.asarray(L_c, dtype=np.float64)
    )


def decode(counts, sA, sB, L, widths, q: int):
    """Sum of chunk terms.

    ``counts``: (rows, N, n_chunks) integers; ``sA``: (rows, n_chunks);
    ``sB``: (N, n_chunks); ``L``: (rows, n_chunks) lengths; ``widths``:
    (n_chunks,).  Returns (rows, N) float64 and the per-chunk terms'
    absolute sum (used as the tolerance scale).
    """
    counts = np.asarray(counts)
    terms = decode_terms(
        counts,
        np.asarray(sA)[:, None, :],
        np.asarray(sB)[None, :, :],
        np.asarray(L)[:, None, :],
        np.asarray(widths)[None, None, :],
        q,
    )
    return terms.sum(axis=2), np.abs(terms).sum(axis=2)
