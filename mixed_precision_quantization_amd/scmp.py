"""Thin ctypes binding of libscmp (include/scmp.h).

Argument marshalling only: every function below checks tensor dtypes,
devices and shapes, passes raw device pointers and the current HIP stream to
the C function of the same name, and raises ``ScmpError`` on a non-zero
status.  All arithmetic of the SC path runs in the library's HIP kernels.
PyTorch is used for device memory and streams.  There is no CPU fallback:
loading fails loudly when the library is missing.
"""

import ctypes
import os
from typing import Optional, Sequence

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libscmp.so")

SCMP_OK = 0
SCMP_ERR_ARG = 1
SCMP_ERR_CEILING = 2
SCMP_ERR_ISO_COMPUTE = 3
SCMP_ERR_UNSUPPORTED = 4
SCMP_ERR_PLAN_MISMATCH = 5
SCMP_ERR_NONFINITE = 6
SCMP_ERR_WORKSPACE = 7
SCMP_ERR_HIP = 8

SCMP_OP_LINEAR, SCMP_OP_QK, SCMP_OP_AV = 0, 1, 2
SCMP_MODE_BIPOLAR, SCMP_MODE_UNIPOLAR = 0, 1
SCMP_ALGO_AUTO, SCMP_ALGO_BITSERIAL, SCMP_ALGO_MFMA = 0, 1, 2
SCMP_ALGO_MFMA_PERSISTENT, SCMP_ALGO_MFMA_ONEPASS, SCMP_ALGO_GATHER, SCMP_ALGO_MFMA_QUARTER = 3, 4, 5, 6
SCMP_MAX_RUNGS = 8
SCMP_MAX_BANDS = 16

OPS = {"linear": SCMP_OP_LINEAR, "qk": SCMP_OP_QK, "av": SCMP_OP_AV}
MODES = {"bipolar": SCMP_MODE_BIPOLAR, "unipolar": SCMP_MODE_UNIPOLAR}
ALGOS = {"auto": SCMP_ALGO_AUTO, "bitserial": SCMP_ALGO_BITSERIAL, "mfma": SCMP_ALGO_MFMA,
         "mfma_persistent": SCMP_ALGO_MFMA_PERSISTENT, "mfma_onepass": SCMP_ALGO_MFMA_ONEPASS,
         "gather": SCMP_ALGO_GATHER, "mfma_quarter": SCMP_ALGO_MFMA_QUARTER}

EXPORTED = [
    "scmp_status_string", "scmp_last_error", "scmp_build_sobol_table", "scmp_table_destroy",
    "scmp_table_info", "scmp_table_export", "scmp_plan_create", "scmp_plan_destroy",
    "scmp_plan_query", "scmp_plan_band_lengths", "scmp_plan_band_columns", "scmp_plan_budget_use",
    "scmp_plan_row_cuts", "scmp_quantize_encode", "scmp_classify_rows", "scmp_matmul_workspace_bytes",
    "scmp_matmul", "scmp_matmul_noalloc", "scmp_matmul_bias", "scmp_matmul_group_rungs", "scmp_group_max", "scmp_range_classify",
    "scmp_gather_rows", "scmp_matmul_range", "scmp_matmul_issued_macs", "scmp_matmul_window_macs", "scmp_decode",
    "scmp_error_flags",
]


class ScmpError(RuntimeError):
    def __init__(self, func: str, status: int, detail: str):
        self.status = status
        super().__init__(f"{func}: {status_string(status)}: {detail}")


class PlanDesc(ctypes.Structure):
    _fields_ = [
        ("op", ctypes.c_int), ("p", ctypes.c_int), ("Lmax", ctypes.c_int), ("D", ctypes.c_int),
        ("chunk_d", ctypes.c_int), ("n_rungs", ctypes.c_int),
        ("levels", ctypes.POINTER(ctypes.c_int)), ("fractions", ctypes.POINTER(ctypes.c_double)),
        ("n_bands", ctypes.c_int), ("band_chunks", ctypes.POINTER(ctypes.c_int)),
        ("tilt", ctypes.c_double), ("band_L", ctypes.POINTER(ctypes.c_int)),
        ("table_chunk_d", ctypes.c_int), ("table_D", ctypes.c_int),
        ("ceiling", ctypes.c_int), ("range_mp", ctypes.c_int), ("mode", ctypes.c_int),
        ("range_threshold", ctypes.c_double), ("range_group", ctypes.c_int),
    ]


class PlanInfo(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int) for n in
                ("op", "p", "Lmax", "D", "chunk_d", "n_chunks", "n_rungs", "n_bands", "ceiling", "mode",
                 "range_mp", "range_group", "mfma_exact")]


_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libscmp.so (built by mixed_precision_quantization_amd.build)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -m mixed_precision_quantization_amd.build`; "
            "there is no fallback path")
    lib = ctypes.CDLL(path)
    vp, i, i64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
    sig = {
        "scmp_status_string": (ctypes.c_char_p, [i]),
        "scmp_last_error": (ctypes.c_char_p, []),
        "scmp_build_sobol_table": (i, [i, i, vp, ctypes.POINTER(vp)]),
        "scmp_table_destroy": (i, [vp]),
        "scmp_table_info": (i, [vp, ctypes.POINTER(i), ctypes.POINTER(i)]),
        "scmp_table_export": (i, [vp, vp, vp, vp, vp]),
        "scmp_plan_create": (i, [ctypes.POINTER(PlanDesc), ctypes.POINTER(vp)]),
        "scmp_plan_destroy": (i, [vp]),
        "scmp_plan_query": (i, [vp, ctypes.POINTER(PlanInfo)]),
        "scmp_plan_band_lengths": (i, [vp, ctypes.POINTER(i)]),
        "scmp_plan_band_columns": (i, [vp, ctypes.POINTER(i)]),
        "scmp_plan_budget_use": (i, [vp, ctypes.POINTER(ctypes.c_double)]),
        "scmp_plan_row_cuts": (i, [vp, i, ctypes.POINTER(i)]),
        "scmp_quantize_encode": (i, [vp, vp, vp, i, i, i, i64, i64, i64, vp, vp, vp, vp, vp]),
        "scmp_classify_rows": (i, [vp, vp, i, i, vp, vp, vp, vp, vp]),
        "scmp_matmul_workspace_bytes": (i, [vp, vp, i, i, i, i, ctypes.POINTER(ctypes.c_size_t)]),
        "scmp_matmul": (i, [vp, vp, i, i, i, i, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, vp, ctypes.c_size_t, vp]),
        "scmp_matmul_noalloc": (i, [vp, vp, i, i, i, i, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, vp]),
        "scmp_matmul_bias": (i, [vp, vp, i, i, i, i, vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, vp, ctypes.c_size_t,
                                 vp]),
        "scmp_matmul_group_rungs": (i, [vp, vp, i, i, i, i, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, vp,
                                        ctypes.c_size_t, vp]),
        "scmp_group_max": (i, [vp, i, i, vp, vp]),
        "scmp_range_classify": (i, [vp, vp, i, i, i64, vp, vp, vp, ctypes.POINTER(i), vp]),
        "scmp_gather_rows": (i, [vp, i, i, ctypes.c_size_t, vp, i, vp, vp]),
        "scmp_matmul_range": (i, [vp, vp, i, i, i, i, i, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, vp,
                                  ctypes.c_size_t, vp]),
        "scmp_matmul_issued_macs": (i, [vp, vp, i, i, i, i, vp, ctypes.c_size_t,
                                        ctypes.POINTER(ctypes.c_ulonglong), ctypes.POINTER(ctypes.c_ulonglong),
                                        vp]),
        "scmp_matmul_window_macs": (i, [vp, vp, i, i, i, i, vp, ctypes.c_size_t, ctypes.POINTER(ctypes.c_ulonglong),
                                        vp]),
        "scmp_decode": (i, [vp, i, i, i, vp, vp, vp, vp, vp, i64, i64, vp]),
        "scmp_error_flags": (i, [vp, ctypes.POINTER(i)]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().scmp_status_string(status).decode()


def _check(func: str, status: int):
    if status != SCMP_OK:
        raise ScmpError(func, status, load().scmp_last_error().decode())


def _stream(stream):
    if stream is None:
        if not torch.cuda.is_available():
            return None
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream) if hasattr(stream, "cuda_stream") else ctypes.c_void_p(stream)


def _ptr(t: Optional[torch.Tensor], dtype=None, name: str = "tensor"):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _need(t: Optional[torch.Tensor], numel: int, name: str):
    if t is not None and t.numel() < numel:
        raise ValueError(f"{name} holds {t.numel()} elements, needs {numel}")


# ------------------------------------------------------------------ table --

class Table:
    """Owner of a scmp_table_t."""

    def __init__(self, handle: int, p: int, Lmax: int):
        self.handle = ctypes.c_void_p(handle)
        self.p = p
        self.Lmax = Lmax

    @property
    def P(self) -> int:
        return 1 << self.p

    @property
    def words(self) -> int:
        return (self.Lmax + 31) // 32

    def close(self):
        if self.handle:
            load().scmp_table_destroy(self.handle)
            self.handle = ctypes.c_void_p(None)

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def scmp_build_sobol_table(p: int = 8, Lmax: int = 256, stream=None) -> Table:
    out = ctypes.c_void_p()
    _check("scmp_build_sobol_table", load().scmp_build_sobol_table(p, Lmax, _stream(stream), ctypes.byref(out)))
    return Table(out.value, p, Lmax)


def scmp_table_export(table: Table, stream=None):
    """(r uint16 [Lmax], K int32 view of uint32 [P+1][words], cum uint16 [P+1][Lmax+1])."""
    dev = torch.device("cuda")
    r = torch.empty(table.Lmax, dtype=torch.int16, device=dev)
    K = torch.empty((table.P + 1, table.words), dtype=torch.int32, device=dev)
    cum = torch.empty((table.P + 1, table.Lmax + 1), dtype=torch.int16, device=dev)
    _check("scmp_table_export", load().scmp_table_export(table.handle, _ptr(r), _ptr(K), _ptr(cum), _stream(stream)))
    return r, K, cum


# ------------------------------------------------------------------- plan --

class Plan:
    """Owner of a scmp_plan_t (host only)."""

    def __init__(self, handle: int):
        self.handle = ctypes.c_void_p(handle)
        info = PlanInfo()
        _check("scmp_plan_query", load().scmp_plan_query(self.handle, ctypes.byref(info)))
        for name, _ in PlanInfo._fields_:
            setattr(self, name, getattr(info, name))

    @property
    def unipolar(self) -> bool:
        return self.mode == MODES["unipolar"]

    def needs_packed(self, algo: str) -> bool:
        """Whether the contraction reads packed weight-side streams (the
        bit-serial kernel does)."""
        return algo == "bitserial"

    def band_lengths(self):
        buf = (ctypes.c_int * (self.n_bands * self.n_rungs))()
        _check("scmp_plan_band_lengths", load().scmp_plan_band_lengths(self.handle, buf))
        return [[buf[b * self.n_rungs + k] for k in range(self.n_rungs)] for b in range(self.n_bands)]

    def band_columns(self):
        buf = (ctypes.c_int * (self.n_bands + 1))()
        _check("scmp_plan_band_columns", load().scmp_plan_band_columns(self.handle, buf))
        return list(buf)

    def budget_use(self):
        buf = (ctypes.c_double * self.n_rungs)()
        _check("scmp_plan_budget_use", load().scmp_plan_budget_use(self.handle, buf))
        return list(buf)

    def row_cuts(self, M: int):
        buf = (ctypes.c_int * (self.n_rungs + 1))()
        _check("scmp_plan_row_cuts", load().scmp_plan_row_cuts(self.handle, M, buf))
        return list(buf)

    def close(self):
        if self.handle:
            load().scmp_plan_destroy(self.handle)
            self.handle = ctypes.c_void_p(None)

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def scmp_plan_create(op: str = "linear", p: int = 8, Lmax: int = 256, D: int = 64, chunk_d: int = 0,
                     levels: Sequence[int] = (256,), fractions: Optional[Sequence[float]] = None,
                     n_bands: int = 1, band_chunks: Optional[Sequence[int]] = None, tilt: float = 0.0,
                     band_L=None, table_chunk_d: int = 0, table_D: int = 0, ceiling: int = 0,
                     range_mp: bool = False, mode: str = "bipolar", range_threshold: float = 0.3,
                     range_group: int = 128) -> Plan:
    lv = (ctypes.c_int * len(levels))(*[int(v) for v in levels])
    fr = (ctypes.c_double * len(fractions))(*[float(v) for v in fractions]) if fractions else None
    bc = (ctypes.c_int * len(band_chunks))(*[int(v) for v in band_chunks]) if band_chunks else None
    bl = None
    if band_L is not None:
        flat = [int(v) for row in band_L for v in row]
        bl = (ctypes.c_int * len(flat))(*flat)
    desc = PlanDesc(OPS[op] if isinstance(op, str) else int(op), p, Lmax, D, chunk_d, len(levels), lv,
                    ctypes.cast(fr, ctypes.POINTER(ctypes.c_double)) if fr else None, n_bands,
                    ctypes.cast(bc, ctypes.POINTER(ctypes.c_int)) if bc else None, float(tilt),
                    ctypes.cast(bl, ctypes.POINTER(ctypes.c_int)) if bl else None,
                    table_chunk_d, table_D, ceiling, 1 if range_mp else 0,
                    MODES[mode] if isinstance(mode, str) else int(mode), float(range_threshold), int(range_group))
    out = ctypes.c_void_p()
    _check("scmp_plan_create", load().scmp_plan_create(ctypes.byref(desc), ctypes.byref(out)))
    return Plan(out.value)


# ------------------------------------------------------------ device calls --

def scmp_quantize_encode(table: Table, plan: Plan, X: torch.Tensor, q_out=None, scales_out=None,
                         metric_out=None, packed_out=None, want_metric: bool = True,
                         want_packed: bool = False, stream=None):
    """Quantise X ([G,] rows, cols; any strides, float32) per row or per chunk.

    Returns (q int8 [G, rows, cols], scales float [G, rows, n_chunks],
    metric float [G, rows] or None, packed int32 view [G, rows, cols, words]
    or None).
    """
    if X.dtype != torch.float32 or not X.is_cuda:
        raise ValueError("X must be a float32 device tensor")
    X3 = X if X.dim() == 3 else X.unsqueeze(0)
    G, rows, cols = X3.shape
    bs, rs, cs = X3.stride()
    dev = X.device
    if q_out is None:
        q_out = torch.empty((G, rows, cols), dtype=torch.int8, device=dev)
    if scales_out is None:
        scales_out = torch.empty((G, rows, plan.n_chunks), dtype=torch.float32, device=dev)
    if metric_out is None and want_metric:
        metric_out = torch.empty((G, rows), dtype=torch.float32, device=dev)
    if packed_out is None and want_packed:
        packed_out = torch.empty((G, rows, cols, table.words), dtype=torch.int32, device=dev)
    _need(q_out, G * rows * cols, "q_out")
    _need(scales_out, G * rows * plan.n_chunks, "scales_out")
    _need(metric_out, G * rows, "metric_out")
    _need(packed_out, G * rows * cols * table.words, "packed_out")
    st = load().scmp_quantize_encode(
        table.handle, plan.handle, ctypes.c_void_p(X3.data_ptr()), G, rows, cols, bs, rs, cs,
        _ptr(q_out, torch.int8, "q_out"), _ptr(scales_out, torch.float32, "scales_out"),
        _ptr(metric_out, torch.float32, "metric_out"), _ptr(packed_out, torch.int32, "packed_out"),
        _stream(stream))
    _check("scmp_quantize_encode", st)
    return q_out, scales_out, metric_out, packed_out


def scmp_classify_rows(plan: Plan, metric: torch.Tensor, ghat_out=None, rung_out=None, perm_out=None,
                       thresholds_out=None, stream=None):
    """Returns (ghat float [G,M], rung uint8 [G,M], perm int32 [G,M], thresholds float [G,K-1])."""
    m2 = metric if metric.dim() == 2 else metric.unsqueeze(0)
    G, M = m2.shape
    dev = metric.device
    if ghat_out is None:
        ghat_out = torch.empty((G, M), dtype=torch.float32, device=dev)
    if rung_out is None:
        rung_out = torch.empty((G, M), dtype=torch.uint8, device=dev)
    if perm_out is None:
        perm_out = torch.empty((G, M), dtype=torch.int32, device=dev)
    if thresholds_out is None and plan.n_rungs > 1:
        thresholds_out = torch.empty((G, plan.n_rungs - 1), dtype=torch.float32, device=dev)
    for t, n, name in ((ghat_out, G * M, "ghat_out"), (rung_out, G * M, "rung_out"), (perm_out, G * M, "perm_out"),
                       (thresholds_out, G * max(plan.n_rungs - 1, 0), "thresholds_out")):
        _need(t, n, name)
    st = load().scmp_classify_rows(
        plan.handle, _ptr(m2.contiguous(), torch.float32, "metric"), G, M,
        _ptr(ghat_out, torch.float32, "ghat_out"), _ptr(rung_out, torch.uint8, "rung_out"),
        _ptr(perm_out, torch.int32, "perm_out"), _ptr(thresholds_out, torch.float32, "thresholds_out"),
        _stream(stream))
    _check("scmp_classify_rows", st)
    return ghat_out, rung_out, perm_out, thresholds_out


def scmp_matmul_workspace_bytes(table: Table, plan: Plan, G: int, M: int, N: int, algo: str = "auto") -> int:
    out = ctypes.c_size_t(0)
    _check("scmp_matmul_workspace_bytes",
           load().scmp_matmul_workspace_bytes(table.handle, plan.handle, ALGOS[algo], G, M, N, ctypes.byref(out)))
    return int(out.value)


def scmp_matmul(table: Table, plan: Plan, qA, sA, qB, sB, permA=None, packedB=None, algo: str = "auto",
                counts_out=None, C_out=None, want_counts: bool = False, want_C: bool = True, workspace=None,
                bias=None, group_rung=None, stream=None):
    """SC product of encoded operands.  qA int8 [G, M, D], qB int8 [G, N, D].
    ``workspace``: uint8 device tensor of at least scmp_matmul_workspace_bytes
    (allocated here when None).  ``bias``: float [G, N] added to every row
    of C (scmp_matmul_bias), or None.  ``group_rung``: uint8 [G], one rung
    per group for all its rows (scmp_matmul_group_rungs; no permA), or None.

    Returns (counts int32 [G, M, N, n_bands] or None, C float [G, M, N] or None).
    """
    qA3 = qA if qA.dim() == 3 else qA.unsqueeze(0)
    qB3 = qB if qB.dim() == 3 else qB.unsqueeze(0)
    G, M, D = qA3.shape
    G2, N, D2 = qB3.shape
    if G2 != G or D2 != D:
        raise ValueError("qA and qB disagree on G or D")
    dev = qA.device
    if counts_out is None and want_counts:
        counts_out = torch.empty((G, M, N, plan.n_bands), dtype=torch.int32, device=dev)
    if C_out is None and want_C:
        C_out = torch.empty((G, M, N), dtype=torch.float32, device=dev)
    _need(sA, G * M * plan.n_chunks, "sA")
    _need(sB, G * N * plan.n_chunks, "sB")
    _need(permA, G * M, "permA")
    _need(packedB, G * N * D * table.words, "packedB")
    _need(counts_out, G * M * N * plan.n_bands, "counts_out")
    _need(C_out, G * M * N, "C_out")
    ws_need = scmp_matmul_workspace_bytes(table, plan, G, M, N, algo)
    if workspace is None:
        workspace = torch.empty(max(ws_need, 1), dtype=torch.uint8, device=dev)
    _need(workspace, ws_need, "workspace")
    head = (table.handle, plan.handle, ALGOS[algo], G, M, N,
            _ptr(qA3, torch.int8, "qA"), _ptr(sA, torch.float32, "sA"), _ptr(permA, torch.int32, "permA"),
            _ptr(qB3, torch.int8, "qB"), _ptr(packedB, torch.int32, "packedB"), _ptr(sB, torch.float32, "sB"))
    tail = (_ptr(counts_out, torch.int32, "counts_out"), _ptr(C_out, torch.float32, "C_out"),
            N, M * N, _ptr(workspace, torch.uint8, "workspace"), workspace.numel(), _stream(stream))
    if group_rung is not None:
        if bias is not None or permA is not None:
            raise ValueError("group_rung excludes bias and permA")
        _need(group_rung, G, "group_rung")
        head = head[:8] + head[9:] + (_ptr(group_rung, torch.uint8, "group_rung"),)
        _check("scmp_matmul_group_rungs", load().scmp_matmul_group_rungs(*head, *tail))
    elif bias is None:
        _check("scmp_matmul", load().scmp_matmul(*head, *tail))
    else:
        _need(bias, G * N, "bias")
        _check("scmp_matmul_bias", load().scmp_matmul_bias(*head, _ptr(bias, torch.float32, "bias"), *tail))
    return counts_out, C_out


NOALLOC_SCRATCH_BYTES = 64 << 20


def scmp_matmul_noalloc(table: Table, plan: Plan, qA, sA, qB, sB, permA=None, packedB=None, algo: str = "auto",
                        counts_out=None, C_out=None, stream=None):
    """scmp_matmul_noalloc: the product of scmp_matmul with the library's
    static scratch instead of a workspace.  The outputs must be given
    (counts_out int32 [G, M, N, n_bands] and / or C_out float [G, M, N]);
    nothing is allocated here or in the library."""
    qA3 = qA if qA.dim() == 3 else qA.unsqueeze(0)
    qB3 = qB if qB.dim() == 3 else qB.unsqueeze(0)
    G, M, D = qA3.shape
    G2, N, D2 = qB3.shape
    if G2 != G or D2 != D:
        raise ValueError("qA and qB disagree on G or D")
    if counts_out is None and C_out is None:
        raise ValueError("give counts_out and / or C_out")
    _need(sA, G * M * plan.n_chunks, "sA")
    _need(sB, G * N * plan.n_chunks, "sB")
    _need(permA, G * M, "permA")
    _need(packedB, G * N * D * table.words, "packedB")
    _need(counts_out, G * M * N * plan.n_bands, "counts_out")
    _need(C_out, G * M * N, "C_out")
    _check("scmp_matmul_noalloc", load().scmp_matmul_noalloc(
        table.handle, plan.handle, ALGOS[algo], G, M, N, _ptr(qA3, torch.int8, "qA"), _ptr(sA, torch.float32, "sA"),
        _ptr(permA, torch.int32, "permA"), _ptr(qB3, torch.int8, "qB"), _ptr(packedB, torch.int32, "packedB"),
        _ptr(sB, torch.float32, "sB"), _ptr(counts_out, torch.int32, "counts_out"),
        _ptr(C_out, torch.float32, "C_out"), N, M * N, _stream(stream)))
    return counts_out, C_out


def scmp_matmul_issued_macs(table: Table, plan: Plan, G: int, M: int, N: int, workspace, algo: str = "auto",
                            stream=None, split: bool = False):
    """MACs the last MFMA-path matmul with ``workspace`` issued on the matrix
    cores (synchronises); with ``split`` the pair (all, fp4 part)."""
    out = ctypes.c_ulonglong(0)
    fp4 = ctypes.c_ulonglong(0)
    _check("scmp_matmul_issued_macs",
           load().scmp_matmul_issued_macs(table.handle, plan.handle, ALGOS[algo], G, M, N,
                                          _ptr(workspace, torch.uint8, "workspace"), workspace.numel(),
                                          ctypes.byref(out), ctypes.byref(fp4), _stream(stream)))
    return (int(out.value), int(fp4.value)) if split else int(out.value)


def scmp_matmul_window_macs(table: Table, plan: Plan, G: int, M: int, N: int, workspace, algo: str = "auto",
                            stream=None) -> int:
    """MACs the exact count needed in the last MFMA-path matmul with
    ``workspace`` (per element and index the row's window, times N;
    synchronises)."""
    out = ctypes.c_ulonglong(0)
    _check("scmp_matmul_window_macs",
           load().scmp_matmul_window_macs(table.handle, plan.handle, ALGOS[algo], G, M, N,
                                          _ptr(workspace, torch.uint8, "workspace"), workspace.numel(),
                                          ctypes.byref(out), _stream(stream)))
    return int(out.value)


def scmp_decode(plan: Plan, counts, sA, sB, rung=None, C_out=None, stream=None):
    """Decode counts [G, M, N, 1] of a plan without chunk scales into C [G, M, N]."""
    c4 = counts if counts.dim() == 4 else counts.unsqueeze(0)
    G, M, N, _ = c4.shape
    if C_out is None:
        C_out = torch.empty((G, M, N), dtype=torch.float32, device=counts.device)
    _need(C_out, G * M * N, "C_out")
    st = load().scmp_decode(plan.handle, G, M, N, _ptr(c4, torch.int32, "counts"), _ptr(sA, torch.float32, "sA"),
                            _ptr(sB, torch.float32, "sB"), _ptr(rung, torch.uint8, "rung"),
                            _ptr(C_out, torch.float32, "C_out"), N, M * N, _stream(stream))
    _check("scmp_decode", st)
    return C_out


def scmp_group_max(values: torch.Tensor, out=None, stream=None) -> torch.Tensor:
    """out[g] = max of values[g, :] (float [G, M] -> float [G])."""
    v2 = values if values.dim() == 2 else values.unsqueeze(0)
    v2 = v2.contiguous()
    G, M = v2.shape
    if out is None:
        out = torch.empty(G, dtype=torch.float32, device=values.device)
    _need(out, G, "out")
    _check("scmp_group_max", load().scmp_group_max(_ptr(v2, torch.float32, "values"), G, M,
                                                    _ptr(out, torch.float32, "out"), _stream(stream)))
    return out


def scmp_range_classify(plan: Plan, W: torch.Tensor, stream=None):
    """Range-MP weight groups of W [N, D] (float32, unit column stride).
    Returns (norm float [n_groups], level uint8 [n_groups], cols int32 [N],
    (rows of level 0, rows of level 1)); synchronises."""
    if W.dim() != 2 or W.stride(1) != 1:
        raise ValueError("W must be 2-D with unit column stride")
    N, D = W.shape
    n_groups = -(-N // plan.range_group)
    norm = torch.empty(n_groups, dtype=torch.float32, device=W.device)
    level = torch.empty(n_groups, dtype=torch.uint8, device=W.device)
    cols = torch.empty(N, dtype=torch.int32, device=W.device)
    counts = (ctypes.c_int * 2)()
    _check("scmp_range_classify",
           load().scmp_range_classify(plan.handle, _ptr(W, torch.float32, "W") if W.is_contiguous()
                                      else ctypes.c_void_p(W.data_ptr()), N, D, W.stride(0),
                                      _ptr(norm, torch.float32, "norm"), _ptr(level, torch.uint8, "level"),
                                      _ptr(cols, torch.int32, "cols"), counts, _stream(stream)))
    return norm, level, cols, (counts[0], counts[1])


def scmp_gather_rows(src: torch.Tensor, idx: torch.Tensor, out=None, stream=None) -> torch.Tensor:
    """dst[g, i] = src[g, idx[i]] for src [G, n, ...] (or [n, ...]); ``out``
    (contiguous, same dtype) is allocated when None."""
    s3 = src if src.dim() >= 3 else src.unsqueeze(0)
    s3 = s3.contiguous()
    G, n_src = s3.shape[0], s3.shape[1]
    row_bytes = s3[0, 0].numel() * s3.element_size() if n_src else 0
    if out is None:
        out = torch.empty((G, idx.numel()) + tuple(s3.shape[2:]), dtype=src.dtype, device=src.device)
    if out.dtype != src.dtype or not out.is_contiguous() or out.numel() != G * idx.numel() * s3[0, 0].numel():
        raise ValueError("out must be contiguous, of src's dtype and of G x len(idx) rows")
    _check("scmp_gather_rows", load().scmp_gather_rows(ctypes.c_void_p(s3.data_ptr()), G, n_src, row_bytes,
                                                        _ptr(idx, torch.int32, "idx"), idx.numel(),
                                                        ctypes.c_void_p(out.data_ptr()), _stream(stream)))
    return out if (src.dim() >= 3 or out.dim() < 3) else out[0]


def scmp_matmul_range(table: Table, plan: Plan, level: int, qA, sA, qB, sB, cols, C_out, packedB=None,
                      algo: str = "auto", counts_out=None, workspace=None, stream=None):
    """One level of a range-MP product: every row of A at levels[level]
    against the compact weight rows qB [G, n, D] (sB [G, n, n_chunks]),
    compact column j written to C_out column cols[j] (C_out [G, M, N_total])."""
    qA3 = qA if qA.dim() == 3 else qA.unsqueeze(0)
    qB3 = qB if qB.dim() == 3 else qB.unsqueeze(0)
    G, M, D = qA3.shape
    n = qB3.shape[1]
    C3 = C_out if C_out.dim() == 3 else C_out.unsqueeze(0)
    _need(sA, G * M * plan.n_chunks, "sA")
    _need(sB, G * n * plan.n_chunks, "sB")
    _need(cols, n, "cols")
    _need(counts_out, G * M * n, "counts_out")
    ws_need = scmp_matmul_workspace_bytes(table, plan, G, M, n, algo)
    if workspace is None:
        workspace = torch.empty(max(ws_need, 1), dtype=torch.uint8, device=qA.device)
    _need(workspace, ws_need, "workspace")
    _check("scmp_matmul_range", load().scmp_matmul_range(
        table.handle, plan.handle, ALGOS[algo], int(level), G, M, n, _ptr(qA3, torch.int8, "qA"),
        _ptr(sA, torch.float32, "sA"), _ptr(qB3, torch.int8, "qB"), _ptr(packedB, torch.int32, "packedB"),
        _ptr(sB, torch.float32, "sB"), _ptr(cols, torch.int32, "cols"), _ptr(counts_out, torch.int32, "counts_out"),
        _ptr(C3, torch.float32, "C_out"), C3.shape[2], C3.shape[1] * C3.shape[2],
        _ptr(workspace, torch.uint8, "workspace"), workspace.numel(), _stream(stream)))
    return C_out


def scmp_error_flags(stream=None) -> int:
    """Synchronise and return (then clear) the device error flags; raises on NONFINITE."""
    flags = ctypes.c_int(0)
    st = load().scmp_error_flags(_stream(stream), ctypes.byref(flags))
    if st not in (SCMP_OK, SCMP_ERR_NONFINITE):
        _check("scmp_error_flags", st)
    return flags.value


# --------------------------------------------------------------- pipeline --

def sc_linear(table: Table, plan: Plan, A: torch.Tensor, B: torch.Tensor, algo: str = "auto",
              want_counts: bool = False, bias=None, stream=None):
    """The whole path for one product: encode both operands, classify rows,
    contract and decode (plus ``bias`` [G, N] when given).  Returns a dict of
    every intermediate (device)."""
    qA, sA, mA, _ = scmp_quantize_encode(table, plan, A, stream=stream)
    qB, sB, _, pB = scmp_quantize_encode(table, plan, B, want_metric=False,
                                         want_packed=plan.needs_packed(algo), stream=stream)
    ghat = rung = perm = thr = None
    if plan.n_rungs > 1:
        ghat, rung, perm, thr = scmp_classify_rows(plan, mA, stream=stream)
    counts, C = scmp_matmul(table, plan, qA, sA, qB, sB, permA=perm, packedB=pB, algo=algo,
                            want_counts=want_counts, bias=bias, stream=stream)
    return {"qA": qA, "sA": sA, "metric": mA, "qB": qB, "sB": sB, "packedB": pB, "ghat": ghat,
            "rung": rung, "perm": perm, "thresholds": thr, "counts": counts, "C": C}


def sc_qk_head_mp(table: Table, plan: Plan, Q: torch.Tensor, K: torch.Tensor, heads: int, algo: str = "auto",
                  want_counts: bool = False, stream=None):
    """Scores Q K^T with one stream length per head: Q [B*heads, M, D] and
    K [B*heads, N, D] (group g = image g // heads, head g % heads).  Each
    head's metric is |Q_h|.amax (the largest of its row metrics); per image
    the heads are ranked by it with the plan's levels and fractions (read as
    head fractions), and every score of a head runs at its rung."""
    qA, sA, mA, _ = scmp_quantize_encode(table, plan, Q, stream=stream)
    qB, sB, _, pB = scmp_quantize_encode(table, plan, K, want_metric=False,
                                         want_packed=plan.needs_packed(algo), stream=stream)
    G = qA.shape[0] if qA.dim() == 3 else 1
    if G % heads:
        raise ValueError("G must be a multiple of heads")
    head_metric = scmp_group_max(mA.reshape(G, -1), stream=stream)
    ghat = rung = perm = thr = None
    if plan.n_rungs > 1:
        ghat, rung, perm, thr = scmp_classify_rows(plan, head_metric.view(G // heads, heads), stream=stream)
        group_rung = rung.view(G)
    else:
        group_rung = torch.zeros(G, dtype=torch.uint8, device=qA.device)
    counts, C = scmp_matmul(table, plan, qA, sA, qB, sB, packedB=pB, algo=algo, want_counts=want_counts,
                            group_rung=group_rung, stream=stream)
    return {"qA": qA, "sA": sA, "metric": mA, "head_metric": head_metric, "qB": qB, "sB": sB, "packedB": pB,
            "ghat": ghat, "head_rung": group_rung, "perm": perm, "thresholds": thr, "counts": counts, "C": C}


def sc_linear_range(table: Table, plan: Plan, X: torch.Tensor, W: torch.Tensor, algo: str = "auto",
                    want_counts: bool = False, stream=None):
    """C = X W^T under range-based per-weight-group MP: W's groups are
    classified by normalised range (at load time, synchronising), W is
    quantised once and stored in level order, and each level's columns are
    contracted at that level's length into their place in C."""
    norm, level, cols, n_lv = scmp_range_classify(plan, W, stream=stream)
    qA, sA, mA, _ = scmp_quantize_encode(table, plan, X, stream=stream)
    qW, sW, _, pW = scmp_quantize_encode(table, plan, W, want_metric=False, want_packed=plan.needs_packed(algo),
                                         stream=stream)
    qB = scmp_gather_rows(qW, cols, stream=stream)
    sB = scmp_gather_rows(sW, cols, stream=stream)
    pB = scmp_gather_rows(pW, cols, stream=stream) if pW is not None else None
    G = qA.shape[0] if qA.dim() == 3 else 1
    M = qA.shape[-2]
    N = W.shape[0]
    C = torch.empty((G, M, N), dtype=torch.float32, device=X.device)
    counts = []
    off = 0
    for k in range(2):
        n = n_lv[k]
        cnt = torch.empty((G, M, n), dtype=torch.int32, device=X.device) if (want_counts and n) else None
        if n:
            scmp_matmul_range(table, plan, k, qA, sA, qB[:, off:off + n], sB[:, off:off + n], cols[off:off + n], C,
                              packedB=None if pB is None else pB[:, off:off + n], algo=algo, counts_out=cnt,
                              stream=stream)
        counts.append(cnt)
        off += n
    return {"qA": qA, "sA": sA, "qB": qB, "sB": sB, "norm": norm, "level": level, "cols": cols,
            "n_per_level": n_lv, "counts": counts, "C": C}
