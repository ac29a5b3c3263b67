"""CPU oracle for the stochastic-computing (SC) bipolar XNOR matmul with
dynamic mixed precision.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import, call or execute anything in this package.  The HIP library never
calls it, and it shares no code with the HIP library (no kernels, headers,
helpers, tables or constant generators).  The only module both sides use is
the seeded input generator ``mixed_precision_quantization_amd.workloads``,
which holds none of the method's arithmetic.

It is plain, slow and written to be checked by eye against the pages:

* "Precision As You Need: Stochastic Computing Is a Dense Adaptive Quantizer"
  (paper notes), section "Key design 1" (fused quantisation and Sobol
  cumulative-table lookup, C-BSG, the bipolar XNOR decode equation),
  "Key design 2" (row metrics, thresholds, the length ladder) and
  "Key design 3" (early termination, cost proportional to the sum of row
  lengths);
* the scmp_vit README, section "Why it works" (per-row bipolar quantisation
  with scale = row abs-max / 127) and the mixed-precision flag table;
* the pull request "feat(mp): per-group (K-band) stream lengths on the
  contraction axis", sections "How the banding works", "Guards" and
  "Tooling";
* for the unipolar (AND) mode, "Precision As You Need" "Research background
  and motivation" and Key design 3, and the scmp_vit README's SC
  compensation driver flags (``unipolar.py``);
* for range-based per-weight-group MP, the scmp_vit README's
  mixed-precision flag table and the K-band pull request's "Guards"
  (``range_mp.py``).

Every stream is materialised bit by bit and every XNOR is counted; counts are
int64 and the decode is float64.  Floating point that decides an integer (the
quantiser, the normalised row metric) is done in float32, the precision the
GPU path uses, so that both sides take the same decision.

Parity status of each function is recorded in its docstring; every function
here is pinned by ``tests/test_oracle_pins.py`` (none is "parity unpinned").
"""

from .sobol import sobol_points
from .table import indicator_table, cumulative_table
from .quant import quantize, bipolar_level, QMAX
from .cbsg import (
    stream_a,
    conditional_stream_b,
    xnor_count,
    xnor_count_row,
)
from .mp import (
    row_metric,
    attention_row_metric,
    normalise_metric,
    sorted_order,
    rung_cuts,
    assign_rungs,
    thresholds,
    tilt_band_ladder,
    band_columns,
    budget_use,
    check_band_ladder,
)
from .decode import decode_terms, decode
from .unipolar import and_count, and_count_row, decode_unipolar, sign_of, unipolar_level
from .range_mp import range_levels, range_mp_rows
from .matmul import (
    OraclePlan,
    classify,
    head_aligned_rows,
    head_mp_rows,
    head_rungs,
    rows_product,
    sc_matmul_rows,
)

__all__ = [
    "sobol_points",
    "indicator_table",
    "cumulative_table",
    "quantize",
    "bipolar_level",
    "QMAX",
    "stream_a",
    "conditional_stream_b",
    "xnor_count",
    "xnor_count_row",
    "row_metric",
    "attention_row_metric",
    "normalise_metric",
    "sorted_order",
    "rung_cuts",
    "assign_rungs",
    "thresholds",
    "tilt_band_ladder",
    "band_columns",
    "budget_use",
    "check_band_ladder",
    "decode_terms",
    "decode",
    "OraclePlan",
    "classify",
    "rows_product",
    "sc_matmul_rows",
    "head_aligned_rows",
    "head_mp_rows",
    "head_rungs",
    "unipolar_level",
    "and_count",
    "and_count_row",
    "sign_of",
    "decode_unipolar",
    "range_levels",
    "range_mp_rows",
]
