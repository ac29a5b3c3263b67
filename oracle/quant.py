"""Symmetric per-row (or per row-chunk) quantisation and the bipolar level
map (test infrastructure; see package docstring).

Sources:
* scmp_vit README, "Why it works": per-row bipolar quantisation sets the
  scale to the row's absolute maximum divided by 127.
* "Precision As You Need" paper notes, Key design 1 and its decode equation:
  the integers are symmetric p-bit values scaled by q_max = 2^(p-1) - 1, and
  the decode multiplies by q_max^2.
* K-band pull request, "How the banding works": with chunk_d set, each
  contraction chunk has its own quantisation, so scales are per (row, chunk).

Readings where the pages are silent: IEEE float32 divisions (a / q, then
x / s), round-half-to-even, clamp to +-q, and an all-zero row (or chunk) gets
scale 0 and integers 0.  The bipolar level map u = round(P (x + q) / (2 q)),
computed exactly in integers, sends -q to 0, 0 to P/2 and +q to P.
"""

import numpy as np


def QMAX(p: int) -> int:
    """q_max = 2^(p-1) - 1."""
    return (1 << (p - 1)) - 1


def quantize(X: np.ndarray, p: int = 8, chunk_d: int = 0):
    """Quantise each row of ``X`` (shape R x D) symmetrically.

    Returns ``(x_int, scales)``: x_int is int64 of shape (R, D) with values in
    [-q, q]; scales is float32 of shape (R, n_chunks) where n_chunks = 1 when
    ``chunk_d`` is 0 and ceil(D / chunk_d) otherwise (the last chunk may be
    short).

    For each row (or chunk): a = max |x| in float32, s = float32(a) / q by
    float32 division; if a == 0 then s = 0 and every integer is 0, otherwise
    x_int = clamp(rint(float32(x) / s), -q, q) with float32 division and
    round-half-to-even.
    """
    X = np.asarray(X, dtype=np.float32)
    if X.ndim != 2:
        raise ValueError("X must be 2-D")
    q = QMAX(p)
    R, D = X.shape
    if chunk_d <= 0:
        bounds = [(0, D)]
    else:
        bounds = [(c, min(c + chunk_d, D)) for c in range(0, D, chunk_d)]
    x_int = np.zeros((R, D), dtype=np.int64)
    scales = np.zeros((R, len(bounds)), dtype=np.float32)
    qf = np.float32(q)
    for ci, (c0, c1) in enumerate(bounds):
        block = X[:, c0:c1]
        a = np.max(np.abs(block), axis=1).astype(np.float32)     # (R,)
        s = (a / qf).astype(np.float32)                          # float32 division
        scales[:, ci] = s
        nz = a != np.float32(0.0)
        with np.errstate(divide="ignore", invalid="ignore"):
            v = np.rint(block / s[:, None])                      # float32 / float32
        v = np.clip(v, -q, q)
        x_int[:, c0:c1] = np.where(nz[:, None], v, 0).astype(np.int64)
        scales[~nz, ci] = np.float32(0.0)
    return x_int, scales


def bipolar_level(x_int, p: int = 8):
    """Level u in [0, P] of a bipolar integer x in [-q, q].

    u = floor((P (x + q) + q) / (2 q)), which is round(P (x + q) / (2 q));
    q is odd, so no value falls on a tie.
    """
    q = QMAX(p)
    P = 1 << p
    x = np.asarray(x_int, dtype=np.int64)
    return (P * (x + q) + q) // (2 * q)
