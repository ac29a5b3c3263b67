"""Range-based per-weight-group mixed precision (test infrastructure; see
package docstring).

Sources: the scmp_vit README's mixed-precision flag table (range MP on or
off, its stream-length levels with default 256,128, and a normalised range
threshold, default 0.3, where a higher threshold puts more groups at low
precision); the K-band pull request, "Guards" (range MP has no
contraction-axis dispatch, so it cannot be combined with K-bands).

Readings (the pages give neither the groups nor the range):
* A weight group is ``group_size`` consecutive rows of W (output features,
  the columns of C = A W^T); the last group may be short.  Range MP has no
  contraction-axis dispatch, so a group spans the whole contraction axis.
* A group's range is max - min over its float32 weights; the normalised
  range divides it by the largest group range (float32; all zero when that
  is 0), as the row metric is normalised ("Precision As You Need", Key
  design 2).
* Two levels: groups whose normalised range is below the threshold run at
  the second (lower) level, the others at the first.
* Every row of A runs at its column's group length (no per-row rungs).
"""

import numpy as np

from .matmul import OraclePlan, rows_product


def range_levels(W, group_size: int, threshold: float):
    """Per group of ``group_size`` rows of W (N x D): ``range`` (float32
    max - min), ``norm`` (float32 range / largest range) and ``level`` (0 =
    first level, 1 = second, when norm < threshold)."""
    W = np.asarray(W, dtype=np.float32)
    N = W.shape[0]
    starts = list(range(0, N, group_size))
    rng = np.array([np.max(W[s:s + group_size]) - np.min(W[s:s + group_size]) for s in starts],
                   dtype=np.float32)
    top = np.float32(rng.max()) if len(rng) else np.float32(0.0)
    if top == np.float32(0.0):
        norm = np.zeros_like(rng)
    else:
        norm = (rng / top).astype(np.float32)
    level = (norm < np.float32(threshold)).astype(np.int64)
    return {"range": rng, "norm": norm, "level": level}


def range_mp_rows(A, W, levels, threshold: float, group_size: int, p: int = 8, chunk_d: int = 0, rows=None):
    """C = A W^T with each column j at the length of its weight group's
    level (``levels`` = (L_high, L_low)); restricted to the rows ``rows``
    (all when None).  Returns ``C``, ``C_abs``, ``counts`` (R, N, n_chunks),
    the per-column length ``L_col`` and ``range_levels``' dict."""
    A = np.asarray(A, dtype=np.float32)
    W = np.asarray(W, dtype=np.float32)
    if len(levels) != 2:
        raise ValueError("range MP takes two levels")
    rl = range_levels(W, group_size, threshold)
    col_level = np.repeat(rl["level"], group_size)[: W.shape[0]]
    rows = np.arange(A.shape[0]) if rows is None else np.asarray(rows, dtype=np.int64)
    R, N = len(rows), W.shape[0]
    C = np.zeros((R, N), dtype=np.float64)
    C_abs = np.zeros_like(C)
    n_chunks = 1 if chunk_d <= 0 else -(-A.shape[1] // chunk_d)
    counts = np.zeros((R, N, n_chunks), dtype=np.int64)
    for k, L in enumerate(levels):
        cols = np.nonzero(col_level == k)[0]
        if len(cols) == 0:
            continue
        plan = OraclePlan(p=p, Lmax=1 << p, D=A.shape[1], chunk_d=chunk_d, levels=(L,))
        out = rows_product(A[rows], np.zeros(R, dtype=np.int64), W[cols], plan)
        C[:, cols] = out["C"]
        C_abs[:, cols] = out["C_abs"]
        counts[:, cols] = out["counts"]
    return {"C": C, "C_abs": C_abs, "counts": counts, "L_col": np.asarray(levels)[col_level], **rl}
