"""Dynamic mixed precision: row metrics, rung assignment and the K-band
length ladder (test infrastructure; see package docstring).

Sources:
* "Precision As You Need" paper notes, Key design 2: the row metric is the
  row's infinity norm for projection and MLP inputs and max_j A_ij for the
  attention-times-value product; it is normalised to [0, 1] and compared
  against descending thresholds tau_1 >= ... >= tau_(K-1) to pick a length
  from a ladder such as 64, 96, 128, 192, 256.
* scmp_vit README, MP flag table: levels are listed in descending order with
  one row fraction per level (an empty fraction list means an equal split).
* K-band pull request, "How the banding works", "Guards" and "Tooling": band
  b runs rung k at its own length L[b][k]; the per-rung iso-compute identity
  must hold and is never overspent; the tilt is a straight line, rounded
  down, with single units handed back to the bands that lost the largest
  fraction; tilt 0 reproduces the parent ladder; a rung already at the
  ceiling cannot be tilted; a band length above the ceiling is rejected.

Readings where the pages are silent:
* Normalisation divides by the largest metric of the group (the whole matrix
  for linear ops, one (batch, head) for attention), in float32; an all-zero
  group normalises to 0.
* Thresholds are the empirical quantiles of the input itself: rows are
  sorted by normalised metric, descending, ties by row index, and rung k
  takes sorted positions [c_(k-1), c_k) with c_k = floor(F_k M + 0.5),
  F_k = f_0 + ... + f_k in float64 (the last cut is M).
* The tilt is linear in the band index: raw = L_k (1 + t x_b) with
  x_b = (2b - (B - 1)) / (B - 1), for bands of equal width.
"""

import math

import numpy as np


def row_metric(X: np.ndarray) -> np.ndarray:
    """g_i = max_d |X_id| (float32) for projection and MLP inputs."""
    X = np.asarray(X, dtype=np.float32)
    return np.max(np.abs(X), axis=-1).astype(np.float32)


def attention_row_metric(A: np.ndarray) -> np.ndarray:
    """g_i = max_j A_ij (float32) for attention probabilities."""
    A = np.asarray(A, dtype=np.float32)
    return np.max(A, axis=-1).astype(np.float32)


def normalise_metric(g: np.ndarray) -> np.ndarray:
    """g_hat = g / max(g) in float32 (all zeros when max(g) is 0)."""
    g = np.asarray(g, dtype=np.float32)
    m = np.float32(np.max(g)) if g.size else np.float32(0.0)
    if m == np.float32(0.0):
        return np.zeros_like(g, dtype=np.float32)
    return (g / m).astype(np.float32)


def sorted_order(g_hat: np.ndarray) -> np.ndarray:
    """Row indices sorted by g_hat descending, ties by row index ascending.

    order[pos] is the row at sorted position pos.
    """
    g_hat = np.asarray(g_hat, dtype=np.float32)
    keyed = sorted(range(g_hat.shape[0]), key=lambda i: (-float(g_hat[i]), i))
    return np.asarray(keyed, dtype=np.int64)


def _fractions(n_rungs: int, fractions):
    if fractions is None or len(fractions) == 0:
        return [1.0 / n_rungs] * n_rungs
    if len(fractions) != n_rungs:
        raise ValueError("one fraction per rung")
    return [float(f) for f in fractions]


def rung_cuts(M: int, n_rungs: int, fractions=None) -> np.ndarray:
    """Sorted-position cuts c_(-1) = 0 <= c_0 <= ... <= c_(K-1) = M.

    c_k = floor(F_k * M + 0.5) with F_k the running float64 sum of the
    fractions, added left to right; the last cut is M.
    Returns int64 array of length n_rungs + 1 (leading 0).
    """
    fr = _fractions(n_rungs, fractions)
    cuts = [0]
    F = 0.0
    for k in range(n_rungs):
        F = F + fr[k]
        c = M if k == n_rungs - 1 else int(math.floor(F * M + 0.5))
        c = max(cuts[-1], min(M, c))
        cuts.append(c)
    return np.asarray(cuts, dtype=np.int64)


def assign_rungs(g_hat: np.ndarray, n_rungs: int, fractions=None):
    """Rung of each row (0 = longest stream) and the sorted order.

    Returns ``(rung, order)``: rung[i] = k when row i sits at a sorted
    position in [c_(k-1), c_k).
    """
    g_hat = np.asarray(g_hat, dtype=np.float32)
    M = g_hat.shape[0]
    order = sorted_order(g_hat)
    cuts = rung_cuts(M, n_rungs, fractions)
    rung = np.zeros(M, dtype=np.int64)
    for k in range(n_rungs):
        for pos in range(int(cuts[k]), int(cuts[k + 1])):
            rung[order[pos]] = k
    return rung, order


def thresholds(g_hat: np.ndarray, order: np.ndarray, cuts: np.ndarray):
    """tau_k (k = 1 .. K-1): the normalised metric of the last row admitted
    to rungs 0 .. k-1, i.e. g_hat at sorted position c_(k-1) - 1 (1.0 when
    that position does not exist).  Returned as float32, length K-1.
    """
    K = len(cuts) - 1
    out = np.ones(max(K - 1, 0), dtype=np.float32)
    for k in range(1, K):
        pos = int(cuts[k]) - 1
        if pos >= 0:
            out[k - 1] = g_hat[order[pos]]
    return out


def tilt_band_ladder(levels, n_bands: int, tilt: float, ceiling: int):
    """Band lengths L[b][k] for equal-width bands under a straight-line tilt.

    For a rung below the ceiling: raw_b = L_k (1 + tilt x_b),
    x_b = (2b - (B-1)) / (B-1); L[b][k] = floor(raw_b), then one unit is
    handed back to each of the (B L_k - sum floor(raw_b)) bands with the
    largest lost fraction raw_b - floor(raw_b), ties to the lower band.
    A rung at (or above) the ceiling keeps L_k in every band.
    Returns int64 array of shape (n_bands, n_rungs).
    """
    levels = [int(v) for v in levels]
    B = int(n_bands)
    out = np.zeros((B, len(levels)), dtype=np.int64)
    for k, Lk in enumerate(levels):
        if B == 1 or Lk >= ceiling:
            out[:, k] = Lk
            continue
        raw = []
        for b in range(B):
            x_b = (2.0 * b - (B - 1)) / (B - 1)
            raw.append(Lk * (1.0 + tilt * x_b))
        floors = [int(math.floor(v)) for v in raw]
        give = B * Lk - sum(floors)
        lost = sorted(range(B), key=lambda b: (-(raw[b] - floors[b]), b))
        for b in lost[:give]:
            floors[b] += 1
        out[:, k] = floors
    return out


def band_columns(D: int, chunk_d: int, band_chunks) -> np.ndarray:
    """Column boundaries of the bands: band b covers [start_b, start_(b+1)).

    Bands are made of whole chunks of ``chunk_d`` columns; the last chunk may
    be short.  Returns int64 of length n_bands + 1.
    """
    n_chunks = (D + chunk_d - 1) // chunk_d
    if sum(band_chunks) != n_chunks:
        raise ValueError("band widths must cover every chunk")
    starts = [0]
    c = 0
    for w in band_chunks:
        c += int(w)
        starts.append(min(c * chunk_d, D))
    return np.asarray(starts, dtype=np.int64)


def budget_use(band_L: np.ndarray, band_cols: np.ndarray, levels) -> np.ndarray:
    """Per-rung iso-compute budget use: sum_b D_b L[b][k] / (D L_k)."""
    widths = np.diff(np.asarray(band_cols, dtype=np.int64))
    D = int(widths.sum())
    out = np.zeros(len(levels), dtype=np.float64)
    for k, Lk in enumerate(levels):
        out[k] = float(np.sum(widths * band_L[:, k])) / float(D * int(Lk))
    return out


def check_band_ladder(band_L: np.ndarray, band_cols, levels, ceiling: int):
    """Reject a band ladder the way the K-band pull request's guards do:
    any length above the ceiling, any length below 1, or a rung whose
    column-weighted length sum exceeds D L_k (overspending the per-rung
    iso-compute identity).  Returns the per-rung budget use."""
    band_L = np.asarray(band_L, dtype=np.int64)
    if np.any(band_L > ceiling):
        raise ValueError("band length above the ceiling")
    if np.any(band_L < 1):
        raise ValueError("band length below 1")
    widths = np.diff(np.asarray(band_cols, dtype=np.int64))
    D = int(widths.sum())
    for k, Lk in enumerate(levels):
        if int(np.sum(widths * band_L[:, k])) > D * int(Lk):
            raise ValueError("iso-compute identity overspent")
    return budget_use(band_L, band_cols, levels)
