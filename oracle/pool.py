"""Run the CPU oracle over many output rows in a process pool (test
infrastructure, like the rest of this package: used by the GPU parity tests
and by the benchmark's CPU-baseline leg).

Workers are spawned (not forked) and import only NumPy and ``oracle``, so
they never touch the GPU or torch.  ``workers()`` is the pool size: one per
host core, at most 16.
"""

import multiprocessing as mp
import os
from concurrent.futures import ProcessPoolExecutor

import numpy as np

from . import matmul as _m


def workers() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _task(args):
    A_rows, rung_rows, B, plan_kw = args
    return _m.rows_product(A_rows, rung_rows, B, _m.OraclePlan(**plan_kw))


def pooled_rows_product(A_rows, rung_rows, B, plan_kw, n_workers=None):
    """rows_product over ``A_rows`` split across worker processes."""
    R = A_rows.shape[0]
    n = min(n_workers or workers(), max(R, 1))
    if n <= 1 or R <= 1:
        return _m.rows_product(A_rows, rung_rows, B, _m.OraclePlan(**plan_kw))
    parts = [p for p in np.array_split(np.arange(R), n) if p.size]
    ctx = mp.get_context("spawn")
    with ProcessPoolExecutor(max_workers=len(parts), mp_context=ctx) as ex:
        outs = list(ex.map(_task, [(A_rows[p], rung_rows[p], B, plan_kw) for p in parts]))
    merged = {}
    for key in ("x_a", "s_a", "counts", "band_counts", "L", "C", "C_abs"):
        merged[key] = np.concatenate([r[key] for r in outs], axis=0)
    for key in ("x_b", "s_b", "ladder"):
        merged[key] = outs[0][key]
    return merged


class OraclePool:
    """A reusable pool for many rows_product jobs (A_rows, rung_rows, B).
    ``run(jobs)`` splits each job's rows into pieces so that every worker
    has work, and returns, per job, the merged rows_product result."""

    def __init__(self, plan_kw, n_workers=None):
        self.plan_kw = plan_kw
        self.n = n_workers or workers()
        self.ex = ProcessPoolExecutor(max_workers=self.n, mp_context=mp.get_context("spawn"))

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.ex.shutdown()

    def run(self, jobs):
        total = sum(int(a.shape[0]) for a, _, _ in jobs)
        piece = max(1, -(-total // (2 * self.n)))
        tasks, owner = [], []
        for ji, (A_rows, rung_rows, B) in enumerate(jobs):
            for r0 in range(0, A_rows.shape[0], piece):
                tasks.append((A_rows[r0:r0 + piece], rung_rows[r0:r0 + piece], B, self.plan_kw))
                owner.append(ji)
        outs = list(self.ex.map(_task, tasks))
        merged = []
        for ji in range(len(jobs)):
            parts = [r for r, o_ in zip(outs, owner) if o_ == ji]
            m = {k: np.concatenate([r[k] for r in parts], axis=0)
                 for k in ("x_a", "s_a", "counts", "band_counts", "L", "C", "C_abs")}
            merged.append(m)
        return merged
