"""The whole SC matmul for a chosen set of output rows (test
infrastructure; see package docstring).

Steps, in the order the pages give them ("Precision As You Need" paper
notes, Key designs 1-3; K-band pull request, "How the banding works"):
Sobol table -> symmetric quantisation -> bipolar levels -> row metric and
rung -> per-(band, rung) stream length -> materialised C-BSG streams and
XNOR counts -> decode.

Output rows are independent of one another once their length and scales are
known, so a subset of rows is an exact sub-problem of the full product.
"""

from dataclasses import dataclass, field
from typing import Optional, Sequence

import numpy as np

from .cbsg import xnor_count_row
from .decode import decode
from .mp import (
    assign_rungs,
    attention_row_metric,
    band_columns,
    normalise_metric,
    row_metric,
    rung_cuts,
    tilt_band_ladder,
)
from .quant import QMAX, bipolar_level, quantize
from .sobol import sobol_points
from .table import indicator_table
from .unipolar import and_count_row, decode_unipolar, sign_of, unipolar_level


@dataclass
class OraclePlan:
    """What one SC matmul needs: precision, ladder, fractions and bands."""

    p: int = 8
    Lmax: int = 256
    D: int = 64
    chunk_d: int = 0
    levels: Sequence[int] = (256,)
    fractions: Optional[Sequence[float]] = None
    n_bands: int = 1
    band_chunks: Optional[Sequence[int]] = None
    tilt: float = 0.0
    band_L: Optional[np.ndarray] = None
    ceiling: int = 0
    metric: str = "linear"  # "linear": max |X_i|; "av": max_j A_ij
    mode: str = "bipolar"   # "bipolar" (XNOR) or "unipolar" (AND, sign-magnitude)
    _cache: dict = field(default_factory=dict, repr=False)

    @property
    def n_rungs(self) -> int:
        return len(self.levels)

    @property
    def n_chunks(self) -> int:
        return 1 if self.chunk_d <= 0 else (self.D + self.chunk_d - 1) // self.chunk_d

    def chunk_bounds(self):
        if self.chunk_d <= 0:
            return [(0, self.D)]
        return [(c, min(c + self.chunk_d, self.D)) for c in range(0, self.D, self.chunk_d)]

    def bands(self):
        """(band column starts, band of each chunk)."""
        if self.n_bands == 1:
            return np.asarray([0, self.D]), np.zeros(self.n_chunks, dtype=np.int64)
        widths = self.band_chunks
        if widths is None:
            if self.n_chunks % self.n_bands:
                raise ValueError("equal split needs n_chunks divisible by n_bands")
            widths = [self.n_chunks // self.n_bands] * self.n_bands
        cols = band_columns(self.D, self.chunk_d, widths)
        owner = np.repeat(np.arange(self.n_bands), widths)
        return cols, owner

    def ladder(self) -> np.ndarray:
        """L[b][k] (n_bands x n_rungs)."""
        if self.band_L is not None:
            return np.asarray(self.band_L, dtype=np.int64)
        ceiling = self.ceiling if self.ceiling > 0 else self.Lmax
        return tilt_band_ladder(self.levels, self.n_bands, self.tilt, ceiling)

    def table(self):
        key = (self.p, self.Lmax)
        if key not in self._cache:
            r = sobol_points(self.p, self.Lmax)
            self._cache[key] = indicator_table(r, 1 << self.p)
        return self._cache[key]


def rows_product(A_rows, rung_rows, B, plan: OraclePlan):
    """Counts and decoded products of some A rows whose rungs are known.

    ``A_rows``: (R, D) float32 rows of A; ``rung_rows``: (R,) their rungs;
    ``B``: (N, D).  Returns a dict with ``x_a``, ``s_a`` (of these rows),
    ``x_b``, ``s_b``, ``counts`` (R, N, n_chunks), ``band_counts``
    (R, N, n_bands), ``L`` (R, n_chunks), ``C`` and ``C_abs`` (R, N).
    In the unipolar mode the counts are the signed sums of
    sign_A sign_B AND-count over each chunk's indices.
    """
    A_rows = np.asarray(A_rows, dtype=np.float32)
    B = np.asarray(B, dtype=np.float32)
    R, D = A_rows.shape
    N, D2 = B.shape
    if D != plan.D or D2 != plan.D:
        raise ValueError("contraction length does not match the plan")
    q = QMAX(plan.p)
    K = plan.table()
    x_a, s_a = quantize(A_rows, plan.p, plan.chunk_d)
    x_b, s_b = quantize(B, plan.p, plan.chunk_d)
    unipolar = plan.mode == "unipolar"
    if unipolar:
        u_a = unipolar_level(x_a, plan.p)
        u_b = unipolar_level(x_b, plan.p)
        sg_b = sign_of(x_b)
    elif plan.mode == "bipolar":
        u_a = bipolar_level(x_a, plan.p)
        u_b = bipolar_level(x_b, plan.p)
    else:
        raise ValueError("mode must be bipolar or unipolar")

    ladder = plan.ladder()
    band_cols, chunk_band = plan.bands()
    bounds = plan.chunk_bounds()
    widths = np.asarray([c1 - c0 for c0, c1 in bounds], dtype=np.int64)
    band_of_d = np.zeros(D, dtype=np.int64)
    for b in range(plan.n_bands):
        band_of_d[band_cols[b]:band_cols[b + 1]] = b

    counts = np.zeros((R, N, len(bounds)), dtype=np.int64)
    Lrc = np.zeros((R, len(bounds)), dtype=np.int64)
    for t in range(R):
        k = int(rung_rows[t])
        L_per_d = ladder[band_of_d, k]
        if unipolar:
            per_d = and_count_row(K, u_a[t], u_b, L_per_d) * sign_of(x_a[t])[None, :] * sg_b
        else:
            per_d = xnor_count_row(K, u_a[t], u_b, L_per_d)
        for c, (c0, c1) in enumerate(bounds):
            counts[t, :, c] = per_d[:, c0:c1].sum(axis=1)
            Lrc[t, c] = ladder[chunk_band[c], k]

    band_counts = np.zeros((R, N, plan.n_bands), dtype=np.int64)
    for c in range(len(bounds)):
        band_counts[:, :, chunk_band[c]] += counts[:, :, c]

    if unipolar:
        C, C_abs = decode_unipolar(counts, s_a, s_b, Lrc, q)
    else:
        C, C_abs = decode(counts, s_a, s_b, Lrc, widths, q)
    return {"x_a": x_a, "s_a": s_a, "x_b": x_b, "s_b": s_b, "counts": counts,
            "band_counts": band_counts, "L": Lrc, "C": C, "C_abs": C_abs, "ladder": ladder}


def classify(A, plan: OraclePlan, metric=None):
    """Row metric, normalised metric, rung of every row, sorted order, cuts."""
    A = np.asarray(A, dtype=np.float32)
    M = A.shape[0]
    if metric is None:
        metric = attention_row_metric(A) if plan.metric == "av" else row_metric(A)
    g_hat = normalise_metric(metric)
    if plan.n_rungs > 1:
        rung, order = assign_rungs(g_hat, plan.n_rungs, plan.fractions)
    else:
        rung = np.zeros(M, dtype=np.int64)
        order = np.arange(M, dtype=np.int64)
    cuts = rung_cuts(M, plan.n_rungs, plan.fractions)
    return {"metric": np.asarray(metric, dtype=np.float32), "g_hat": g_hat, "rung": rung,
            "order": order, "cuts": cuts}


def sc_matmul_rows(A, B, plan: OraclePlan, rows=None, metric=None):
    """SC product of A (M x D, the row side) with B (N x D, the weight side)
    restricted to the output rows ``rows`` (all rows when None).

    Returns the union of ``classify`` (metric, g_hat, rung, order, cuts for
    every row) and ``rows_product`` for the requested rows, plus ``rows``.
    """
    A = np.asarray(A, dtype=np.float32)
    cls = classify(A, plan, metric)
    rows = np.arange(A.shape[0]) if rows is None else np.asarray(rows, dtype=np.int64)
    out = rows_product(A[rows], cls["rung"][rows], B, plan)
    out.update(cls)
    out["rows"] = rows
    return out


def head_aligned_rows(X, W, bias, head_dim: int = 64, L: int = 256, p: int = 8, rows=None):
    """The head-aligned SC compensator (scmp_vit README, its head-aligned
    compensator section; "Precision As You Need" Key design 4 runs the
    compensation layer W_b x + b_b as an SC linear): x (M x D) is split into
    heads of ``head_dim`` columns, head h is an SC linear of its own on
    columns [h head_dim, (h + 1) head_dim) of x and W (its own per-row
    scales on both operands, the one Sobol table, stream length L), the
    heads' outputs are summed and the bias is added.  Float64; restricted to
    the output rows ``rows`` (all when None).  Returns ``C`` and ``C_abs``
    (the sum of the absolute decode terms plus |bias|, for tolerances)."""
    X = np.asarray(X, dtype=np.float32)
    W = np.asarray(W, dtype=np.float32)
    bias = np.asarray(bias, dtype=np.float64)
    D = X.shape[1]
    rows = np.arange(X.shape[0]) if rows is None else np.asarray(rows, dtype=np.int64)
    C = np.zeros((len(rows), W.shape[0]), dtype=np.float64)
    C_abs = np.zeros_like(C)
    for h0 in range(0, D, head_dim):
        cols = slice(h0, min(D, h0 + head_dim))
        plan_h = OraclePlan(p=p, Lmax=2 ** p, D=cols.stop - cols.start, levels=(L,))
        r = rows_product(X[rows][:, cols], np.zeros(len(rows), dtype=np.int64), W[:, cols], plan_h)
        C += r["C"]
        C_abs += r["C_abs"]
    return {"C": C + bias[None, :], "C_abs": C_abs + np.abs(bias)[None, :]}


def head_rungs(Q_heads, plan: OraclePlan):
    """Per-head fixed mixed precision on QK (scmp_vit README, the
    mixed-precision flag table: QK levels, head fractions, head metric
    |Q_h|.amax) for one image: ``Q_heads`` (H, M, D).  The metric of head h
    is the largest |Q| over all of its rows and columns (float32); the heads
    are ranked by its normalised value exactly as rows are ranked in
    "Precision As You Need" Key design 2 (descending, ties by head index),
    and the plan's fractions, read as head fractions, cut that ranking into
    the ladder's rungs.  Returns ``metric`` (H,), ``g_hat``, ``rung`` (H,)
    and ``order``."""
    Q = np.asarray(Q_heads, dtype=np.float32)
    H = Q.shape[0]
    metric = np.abs(Q).reshape(H, -1).max(axis=1).astype(np.float32)
    g_hat = normalise_metric(metric)
    if plan.n_rungs > 1:
        rung, order = assign_rungs(g_hat, plan.n_rungs, plan.fractions)
    else:
        rung = np.zeros(H, dtype=np.int64)
        order = np.arange(H, dtype=np.int64)
    return {"metric": metric, "g_hat": g_hat, "rung": np.asarray(rung, dtype=np.int64), "order": order}


def head_mp_rows(Q_heads, K_heads, plan: OraclePlan, head: int, rows=None):
    """Scores Q_h K_h^T of head ``head`` of one image under per-head fixed
    mixed precision: every row of the head runs the head's rung from
    ``head_rungs`` ("Precision As You Need" Key design 3 with one length per
    head).  Restricted to the query rows ``rows`` (all when None).  Returns
    ``rows_product``'s dict plus ``head_rung`` and ``rows``."""
    Q = np.asarray(Q_heads, dtype=np.float32)
    cls = head_rungs(Q, plan)
    k = int(cls["rung"][head])
    rows = np.arange(Q.shape[1]) if rows is None else np.asarray(rows, dtype=np.int64)
    out = rows_product(Q[head][rows], np.full(len(rows), k, dtype=np.int64), np.asarray(K_heads)[head], plan)
    out["head_rung"] = k
    out["rows"] = rows
    return out
