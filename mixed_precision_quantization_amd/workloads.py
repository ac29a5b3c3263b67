"""Seeded synthetic workloads for the SC matmul.

This module only draws inputs and states the shapes and ladders of each
workload; it contains none of the method's arithmetic (no quantisation,
streams, counts or decode).  Both the HIP path's tests and the CPU oracle's
tests take their inputs from here.

The shapes stand in for DINOv2 ViT-L/14 at 224 px (257 tokens, width 1024,
16 heads of 64, MLP 4096) as the scmp_vit README describes it; ImageNet
images and model weights are not used.  Every array is drawn with
``numpy.random.default_rng(seed)`` in float64, in the order listed, and cast
to float32.
"""

from dataclasses import dataclass, field
from typing import Optional, Tuple

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str                     # "linear", "qk" or "av"
    G: int                        # batch x heads (1 for linear ops)
    M: int                        # rows of the row-side operand A
    N: int                        # rows of the weight-side operand B
    D: int                        # contraction length
    levels: Tuple[int, ...]       # stream-length ladder, longest first
    fractions: Optional[Tuple[float, ...]] = None
    chunk_d: int = 0
    n_bands: int = 1
    tilt: float = 0.0
    seed: int = 0
    a_dist: str = "normal"        # see draw()
    b_dist: str = "normal"
    extra: dict = field(default_factory=dict)
    mode: str = "bipolar"         # SC gate: "bipolar" (XNOR) or "unipolar" (AND)

    @property
    def metric(self) -> str:
        return "av" if self.kind == "av" else "linear"


# The five workloads (the fifth has two parts: fc2 with K-bands, and AV),
# per-query-row and per-head mixed precision on QK^T, the head-aligned
# compensator, the unipolar mode on AV and on the compensator, and
# range-based per-weight-group MP on fc1.
WORKLOADS = {
    "single_64": Workload(
        "single_64", "linear", 1, 64, 64, 64, (64,), seed=1001,
        a_dist="normal", b_dist="normal"),
    "vitl_qk": Workload(
        "vitl_qk", "qk", 128, 257, 257, 64, (128,), seed=1002,
        a_dist="normal", b_dist="normal"),
    "vitl_qkv_proj": Workload(
        "vitl_qkv_proj", "linear", 1, 32 * 257, 3072, 1024, (256,), seed=1003,
        a_dist="outlier", b_dist="weight"),
    "vitl_fc1_mp": Workload(
        "vitl_fc1_mp", "linear", 1, 64 * 257, 4096, 1024,
        (256, 192, 128, 96, 64), (0.1, 0.15, 0.2, 0.25, 0.3), seed=1004,
        a_dist="outlier", b_dist="weight"),
    "vitl_fc2_kband": Workload(
        "vitl_fc2_kband", "linear", 1, 64 * 257, 1024, 4096,
        (256, 192, 128, 64), None, chunk_d=64, n_bands=4, tilt=0.25, seed=1005,
        a_dist="gelu", b_dist="weight"),
    "vitl_av_mp": Workload(
        "vitl_av_mp", "av", 128, 257, 64, 257,
        (256, 128, 64), (0.333, 0.334, 0.333), seed=1006,
        a_dist="softmax", b_dist="normal"),
    # Per-query-row mixed precision on QK^T: each query row's length from
    # its ||Q_i||_inf within its head (the QK metric of "Precision As You
    # Need", Key design 2), on the same ladder and split as AV.
    "vitl_qk_mp": Workload(
        "vitl_qk_mp", "qk", 128, 257, 257, 64,
        (256, 128, 64), (0.333, 0.334, 0.333), seed=1007,
        a_dist="normal", b_dist="normal"),
    # The head-aligned SC compensator of one block (scmp_vit README): the
    # block's 64 x 257 tokens x (16 heads x 64), a 1024 x 1024 W_b and a
    # bias, every head at L = 256 (chunk_d = 64 gives each head its own
    # per-row scales on both operands).
    "vitl_comp_head_aligned": Workload(
        "vitl_comp_head_aligned", "linear", 1, 64 * 257, 1024, 1024,
        (256,), None, chunk_d=64, seed=1008,
        a_dist="outlier", b_dist="weight", extra={"bias": True}),
    # Per-head fixed mixed precision on QK^T (scmp_vit README, the
    # mixed-precision flag table): 8 images x 16 heads, each head's scores
    # at one length from its |Q_h|.amax rank within the image, on the same
    # ladder, with head fractions 1/4, 1/2, 1/4 (4, 8 and 4 heads).
    "vitl_qk_head_mp": Workload(
        "vitl_qk_head_mp", "qk", 128, 257, 257, 64,
        (256, 128, 64), (0.25, 0.5, 0.25), seed=1009,
        a_dist="head_scaled", b_dist="normal", extra={"heads": 16}),
    # The unipolar (AND) mode: attention probabilities are non-negative, so
    # AV is the natural unipolar product (V keeps its signs); same shapes,
    # draws and ladder as vitl_av_mp.
    "vitl_av_unipolar": Workload(
        "vitl_av_unipolar", "av", 128, 257, 64, 257,
        (256, 128, 64), (0.333, 0.334, 0.333), seed=1006,
        a_dist="softmax", b_dist="normal", mode="unipolar"),
    # The head-aligned compensator in the unipolar per-row mode (scmp_vit
    # README, SC compensation flags): same draws as vitl_comp_head_aligned.
    "vitl_comp_unipolar": Workload(
        "vitl_comp_unipolar", "linear", 1, 64 * 257, 1024, 1024,
        (256,), None, chunk_d=64, seed=1008,
        a_dist="outlier", b_dist="weight", extra={"bias": True}, mode="unipolar"),
    # Range-based per-weight-group MP on fc1 (scmp_vit README, the
    # mixed-precision flag table defaults: levels 256,128, threshold 0.3),
    # 128-row weight groups with spread amplitudes.
    "vitl_fc1_range": Workload(
        "vitl_fc1_range", "linear", 1, 64 * 257, 4096, 1024,
        (256, 128), None, seed=1011, a_dist="outlier", b_dist="weight_groups",
        extra={"range_mp": True, "range_threshold": 0.3, "range_group": 128}),
}


def shrink(w: Workload, G=None, M=None, N=None, D=None, seed=None) -> Workload:
    """A smaller workload with the same distributions, ladder and bands."""
    kw = dict(w.__dict__)
    for key, val in (("G", G), ("M", M), ("N", N), ("D", D), ("seed", seed)):
        if val is not None:
            kw[key] = val
    kw["name"] = w.name + "_small"
    return Workload(**kw)


def _gelu(z: np.ndarray) -> np.ndarray:
    from scipy.special import erf
    return 0.5 * z * (1.0 + erf(z / np.sqrt(2.0)))


def _softmax_rows(logits: np.ndarray) -> np.ndarray:
    m = logits.max(axis=-1, keepdims=True)
    e = np.exp(logits - m)
    return e / e.sum(axis=-1, keepdims=True)


def _draw(rng, dist: str, lead: tuple, rows: int, cols: int) -> np.ndarray:
    shape = lead + (rows, cols)
    if dist == "normal":
        return rng.standard_normal(shape)
    if dist == "weight":
        return rng.standard_normal(shape) * 0.02
    if dist == "outlier":
        x = rng.standard_normal(shape)
        n_out = int(round(0.01 * cols))
        chans = rng.choice(cols, size=n_out, replace=False)
        x[..., chans] *= 20.0
        return x
    if dist == "head_scaled":
        # Gaussian rows, each group (one image's head) scaled by its own
        # log-normal amplitude exp(0.5 z), so that heads differ in |Q|.amax.
        x = rng.standard_normal(shape)
        amp = np.exp(0.5 * rng.standard_normal(lead + (1, 1)))
        return x * amp
    if dist == "weight_groups":
        # 0.02 N(0, 1) weights, each group of 128 rows scaled by its own
        # log-normal amplitude exp(0.75 z), so that group ranges differ.
        x = rng.standard_normal(shape) * 0.02
        n_groups = -(-rows // 128)
        amp = np.exp(0.75 * rng.standard_normal(lead + (n_groups, 1)))
        return x * np.repeat(amp, 128, axis=-2)[..., :rows, :]
    if dist == "gelu":
        return _gelu(rng.standard_normal(shape))
    if dist == "softmax":
        return _softmax_rows(3.0 * rng.standard_normal(shape))
    raise ValueError(dist)


def draw(w: Workload):
    """Inputs of a workload as float32 arrays ``(A, B)``.

    A has shape (G, M, D) (or (M, D) when G == 1 and kind is linear) and is
    the row side; B has shape (G, N, D) (or (N, D)) and is the weight side.
    For "qk", A = Q and B = K.  For "av", A = softmax of scale-3 Gaussian
    logits (computed in float64) and B = V^T, where V (G, D, N) is drawn
    first as Gaussian and transposed.
    """
    rng = np.random.default_rng(w.seed)
    lead = () if (w.G == 1 and w.kind == "linear") else (w.G,)
    if w.kind == "av":
        A = _draw(rng, w.a_dist, lead, w.M, w.D)
        V = _draw(rng, w.b_dist, lead, w.D, w.N)
        B = np.swapaxes(V, -1, -2)
        return A.astype(np.float32), np.ascontiguousarray(B.astype(np.float32))
    A = _draw(rng, w.a_dist, lead, w.M, w.D)
    B = _draw(rng, w.b_dist, lead, w.N, w.D)
    return A.astype(np.float32), B.astype(np.float32)


def draw_bias(w: Workload) -> np.ndarray:
    """The bias of a workload with ``extra["bias"]``: float32 [G, N] (or [N]
    when G == 1), drawn as 0.02 N(0, 1) from its own seed (seed + 50000) so
    that A and B are the same draws as without it."""
    rng = np.random.default_rng(w.seed + 50000)
    shape = (w.N,) if w.G == 1 else (w.G, w.N)
    return (0.02 * rng.standard_normal(shape)).astype(np.float32)


def draw_v(w: Workload):
    """For "av" workloads: (A, V) with V of shape (G, D, N), untransposed."""
    if w.kind != "av":
        raise ValueError("only attention-times-value workloads have V")
    rng = np.random.default_rng(w.seed)
    A = _draw(rng, w.a_dist, (w.G,), w.M, w.D)
    V = _draw(rng, w.b_dist, (w.G,), w.D, w.N)
    return A.astype(np.float32), V.astype(np.float32)


def sample_rows(M: int, cuts, per_rung: int = 8, seed: int = 7) -> np.ndarray:
    """Positions in sorted order to check: for each rung, its first and last
    sorted position plus ``per_rung - 2`` seeded positions inside it."""
    rng = np.random.default_rng(seed)
    pos = set()
    for k in range(len(cuts) - 1):
        lo, hi = int(cuts[k]), int(cuts[k + 1])
        if hi <= lo:
            continue
        pos.update((lo, hi - 1))
        n = min(per_rung - 2, hi - lo)
        if n > 0:
            pos.update(int(v) for v in rng.choice(np.arange(lo, hi), size=n, replace=False))
    return np.asarray(sorted(pos), dtype=np.int64)


def tile_positions(M: int, cuts, tile: int = 128, seed: int = 7) -> np.ndarray:
    """Positions in sorted order that touch every row tile: for each rung,
    its first and last sorted position plus one seeded position inside each
    run of ``tile`` consecutive positions of the rung (the row tiles of the
    matrix-core kernels, which take a rung's positions ``tile`` at a
    time)."""
    rng = np.random.default_rng(seed)
    pos = set()
    for k in range(len(cuts) - 1):
        lo, hi = int(cuts[k]), int(cuts[k + 1])
        if hi <= lo:
            continue
        pos.update((lo, hi - 1))
        for t0 in range(lo, hi, tile):
            pos.add(int(rng.integers(t0, min(t0 + tile, hi))))
    return np.asarray(sorted(pos), dtype=np.int64)
