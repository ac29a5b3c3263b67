"""Host-side tests of the C ABI: the library loads, exports every symbol the
header declares, and its plan logic (guards, K-band ladder, row cuts,
budget use) agrees with the oracle.  No device call is made here."""

import ctypes
import json
import os
import re
import subprocess

import numpy as np
import pytest

import oracle as o
from mixed_precision_quantization_amd import scmp
from mixed_precision_quantization_amd.workloads import WORKLOADS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "scmp.h")


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^(?:const char\*|int)\s+(scmp_\w+)\(", text, re.M)))


def test_header_declares_the_binding_functions():
    assert _declared() == sorted(scmp.EXPORTED)


def test_library_loads_and_exports_every_declared_symbol():
    lib = scmp.load()
    for name in _declared():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", scmp.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (scmp_\w+)", out))
    assert set(_declared()) <= exported


def test_status_strings():
    for code, name in [(0, "SCMP_OK"), (1, "SCMP_ERR_ARG"), (2, "SCMP_ERR_CEILING"),
                       (3, "SCMP_ERR_ISO_COMPUTE"), (4, "SCMP_ERR_UNSUPPORTED"),
                       (5, "SCMP_ERR_PLAN_MISMATCH"), (6, "SCMP_ERR_NONFINITE"), (8, "SCMP_ERR_HIP")]:
        assert scmp.status_string(code) == name


def _err(fn, code):
    with pytest.raises(scmp.ScmpError) as ei:
        fn()
    assert ei.value.status == code, str(ei.value)
    return str(ei.value)


# ------------------------------------------------------------------ guards --

def test_guard_kbands_rejected_on_qk_and_av():
    for op in ("qk", "av"):
        _err(lambda: scmp.scmp_plan_create(op, D=256, chunk_d=64, levels=(128, 64), n_bands=4, tilt=0.25),
             scmp.SCMP_ERR_UNSUPPORTED)


def test_guard_band_above_ceiling_rejected_at_startup():
    msg = _err(lambda: scmp.scmp_plan_create(D=4096, chunk_d=64, levels=(256, 192, 128, 64), n_bands=4, tilt=0.5),
               scmp.SCMP_ERR_CEILING)
    assert "ceiling" in msg
    _err(lambda: scmp.scmp_plan_create(D=64, levels=(128,), ceiling=96), scmp.SCMP_ERR_CEILING)


def test_guard_kbands_with_range_mp_raises():
    _err(lambda: scmp.scmp_plan_create(D=256, chunk_d=64, levels=(128, 64), n_bands=4, range_mp=True),
         scmp.SCMP_ERR_UNSUPPORTED)


def test_range_mp_plan_rules():
    plan = scmp.scmp_plan_create(D=256, levels=(256, 128), range_mp=True, range_threshold=0.3, range_group=64)
    assert plan.range_mp == 1 and plan.range_group == 64
    assert scmp.scmp_plan_create(D=256, levels=(256, 128), range_mp=True, range_group=0).range_group == 128
    _err(lambda: scmp.scmp_plan_create(op="qk", D=64, levels=(256, 128), range_mp=True), scmp.SCMP_ERR_UNSUPPORTED)
    _err(lambda: scmp.scmp_plan_create(D=64, levels=(256, 128, 64), range_mp=True), scmp.SCMP_ERR_ARG)
    _err(lambda: scmp.scmp_plan_create(D=64, levels=(256, 128), range_mp=True, range_threshold=-1.0),
         scmp.SCMP_ERR_ARG)
    _err(lambda: scmp.scmp_plan_create(D=64, levels=(256, 128), range_mp=True, range_group=-2), scmp.SCMP_ERR_ARG)
    lib = scmp.load()
    # Host-side checks of the range entry points, before any device work.
    n = (scmp.ctypes.c_int * 2)()
    bip = scmp.scmp_plan_create(D=64, levels=(256, 128))
    assert lib.scmp_range_classify(bip.handle, None, 4, 64, 64, None, None, None, n, None) == scmp.SCMP_ERR_ARG
    rp = scmp.scmp_plan_create(D=64, levels=(256, 128), range_mp=True)
    assert lib.scmp_range_classify(rp.handle, None, 4, 32, 64, None, None, None, n, None) == \
        scmp.SCMP_ERR_PLAN_MISMATCH
    assert lib.scmp_matmul_range(None, rp.handle, 0, 2, 1, 1, 1, *([None] * 8), 1, 1, None, 0,
                                 None) == scmp.SCMP_ERR_ARG
    assert lib.scmp_gather_rows(None, 1, 4, 16, None, 2, None, None) == scmp.SCMP_ERR_ARG
    assert lib.scmp_gather_rows(None, 1, 4, 16, None, 0, None, None) == scmp.SCMP_OK


def test_guard_table_priced_at_other_chunk_or_width():
    bl = [[128, 64]] * 4
    _err(lambda: scmp.scmp_plan_create(D=256, chunk_d=64, levels=(128, 64), n_bands=4, band_L=bl,
                                       table_chunk_d=32, table_D=256), scmp.SCMP_ERR_PLAN_MISMATCH)
    _err(lambda: scmp.scmp_plan_create(D=256, chunk_d=64, levels=(128, 64), n_bands=4, band_L=bl,
                                       table_chunk_d=64, table_D=512), scmp.SCMP_ERR_PLAN_MISMATCH)
    ok = scmp.scmp_plan_create(D=256, chunk_d=64, levels=(128, 64), n_bands=4, band_L=bl,
                               table_chunk_d=64, table_D=256)
    assert ok.band_lengths() == bl


def test_guard_iso_compute_overspend():
    bl = [[129, 64], [128, 64], [128, 64], [128, 64]]
    _err(lambda: scmp.scmp_plan_create(D=256, chunk_d=64, levels=(128, 64), n_bands=4, band_L=bl),
         scmp.SCMP_ERR_ISO_COMPUTE)
    under = [[127, 64], [128, 64], [128, 64], [128, 64]]
    plan = scmp.scmp_plan_create(D=256, chunk_d=64, levels=(128, 64), n_bands=4, band_L=under)
    use = plan.budget_use()
    assert use[1] == 1.0 and abs(use[0] - (127 + 3 * 128) / 512) < 1e-15


@pytest.mark.parametrize("kw", [
    dict(levels=(64, 128)),                      # not descending
    dict(levels=(0,)),                           # below 1
    dict(levels=(128, 64), fractions=(0.5, 0.6)),
    dict(levels=(128,), n_bands=2),              # bands without chunk_d
    dict(levels=(128,), chunk_d=-1),
    dict(levels=(128,), p=9),
    dict(levels=(128,), Lmax=300),
    dict(levels=(128,), D=0),
    dict(levels=(128,) * 9),
])
def test_plan_argument_errors(kw):
    args = dict(D=256)
    args.update(kw)
    _err(lambda: scmp.scmp_plan_create(**args), scmp.SCMP_ERR_ARG)


def test_chunk_d_must_be_a_multiple_of_32():
    _err(lambda: scmp.scmp_plan_create(D=256, chunk_d=24, levels=(128,)), scmp.SCMP_ERR_UNSUPPORTED)
    _err(lambda: scmp.scmp_plan_create(D=256, chunk_d=48, levels=(128,)), scmp.SCMP_ERR_UNSUPPORTED)


# ---------------------------------------------------- ladder and row cuts --

@pytest.mark.parametrize("tilt", [0.0, 0.1, 0.25, 1.0 / 3.0])
@pytest.mark.parametrize("levels", [(256, 192, 128, 64), (192, 160, 96, 48, 17), (255, 100, 3)])
@pytest.mark.parametrize("n_bands", [2, 3, 4, 8])
def test_band_ladder_matches_oracle(tilt, levels, n_bands):
    D = 64 * 8 * 3
    chunks = D // 64
    want = o.tilt_band_ladder(levels, n_bands, tilt, 256)
    if np.any(want > 256):
        # A tilted band above the ceiling: both sides reject it at startup.
        _err(lambda: scmp.scmp_plan_create(D=D, chunk_d=64, levels=levels, n_bands=n_bands, tilt=tilt),
             scmp.SCMP_ERR_CEILING)
        with pytest.raises(ValueError, match="ceiling"):
            o.check_band_ladder(want, o.band_columns(D, 64, [chunks // n_bands] * n_bands), levels, 256)
        return
    plan = scmp.scmp_plan_create(D=D, chunk_d=64, levels=levels, n_bands=n_bands, tilt=tilt)
    assert np.array_equal(np.asarray(plan.band_lengths()), want)
    cols = o.band_columns(D, 64, [chunks // n_bands] * n_bands)
    assert plan.band_columns() == cols.tolist()
    assert np.allclose(plan.budget_use(), o.budget_use(want, cols, levels), rtol=0, atol=1e-15)


def test_workload_fc2_ladder():
    w = WORKLOADS["vitl_fc2_kband"]
    plan = scmp.scmp_plan_create(D=w.D, chunk_d=w.chunk_d, levels=w.levels, n_bands=w.n_bands, tilt=w.tilt)
    L = np.asarray(plan.band_lengths())
    assert L[:, 0].tolist() == [256] * 4
    assert L[:, 1].tolist() == [144, 176, 208, 240]
    assert L[:, 2].tolist() == [96, 117, 139, 160]
    assert L[:, 3].tolist() == [48, 59, 69, 80]
    assert plan.budget_use() == [1.0] * 4


@pytest.mark.parametrize("M", [0, 1, 2, 5, 7, 86, 257, 1000, 16448, 16449])
@pytest.mark.parametrize("fr", [None, (0.1, 0.15, 0.2, 0.25, 0.3), (0.333, 0.334, 0.333), (0.5, 0.5), (1.0,)])
def test_row_cuts_match_oracle(M, fr):
    n = len(fr) if fr else 3
    levels = tuple(range(200, 200 - 10 * n, -10))
    plan = scmp.scmp_plan_create(D=64, levels=levels, fractions=fr)
    assert plan.row_cuts(M) == o.rung_cuts(M, n, fr).tolist()


def test_uneven_bands_with_ragged_last_chunk():
    plan = scmp.scmp_plan_create(D=150, chunk_d=64, levels=(128, 64), n_bands=2, band_chunks=(2, 1),
                                 band_L=[[120, 60], [128, 64]])
    assert plan.n_chunks == 3
    assert plan.band_columns() == o.band_columns(150, 64, [2, 1]).tolist()
    # the tilt needs equal widths
    _err(lambda: scmp.scmp_plan_create(D=150, chunk_d=64, levels=(128, 64), n_bands=2, band_chunks=(2, 1),
                                       tilt=0.2), scmp.SCMP_ERR_ARG)


def test_device_entry_points_reject_null_handles_without_touching_the_device():
    lib = scmp.load()
    assert lib.scmp_matmul(None, None, 0, 1, 1, 1, *([None] * 8), 1, 1, None, 0, None) == scmp.SCMP_ERR_ARG
    assert lib.scmp_quantize_encode(None, None, None, 1, 1, 1, 1, 1, 1, None, None, None, None,
                                    None) == scmp.SCMP_ERR_ARG
    assert lib.scmp_classify_rows(None, None, 1, 1, None, None, None, None, None) == scmp.SCMP_ERR_ARG
    assert lib.scmp_decode(None, 1, 1, 1, None, None, None, None, None, 1, 1, None) == scmp.SCMP_ERR_ARG
    out = ctypes.c_void_p()
    assert lib.scmp_build_sobol_table(9, 256, None, ctypes.byref(out)) == scmp.SCMP_ERR_ARG
    assert lib.scmp_build_sobol_table(8, 257, None, ctypes.byref(out)) == scmp.SCMP_ERR_ARG
    assert b"Lmax" in lib.scmp_last_error()
    plan = scmp.scmp_plan_create(D=64, chunk_d=0, levels=(128, 64))
    # shape checks before any launch: cols must equal D
    assert lib.scmp_decode(plan.handle, 1, 1, 1, None, None, None, None, None, 1, 1, None) == scmp.SCMP_ERR_ARG
    assert lib.scmp_matmul(None, plan.handle, 0, 1, 1, 1, *([None] * 8), 1, 1, None, 0, None) == scmp.SCMP_ERR_ARG
    size = ctypes.c_size_t(7)
    assert lib.scmp_matmul_workspace_bytes(None, plan.handle, 0, 1, 1, 1, ctypes.byref(size)) == scmp.SCMP_ERR_ARG


def test_plan_mode_is_recorded_and_checked():
    assert scmp.scmp_plan_create(D=64, levels=(128,)).mode == scmp.SCMP_MODE_BIPOLAR
    uni = scmp.scmp_plan_create(D=64, levels=(128, 64), mode="unipolar")
    assert uni.mode == scmp.SCMP_MODE_UNIPOLAR and uni.unipolar
    assert uni.needs_packed("bitserial") and not uni.needs_packed("auto") and not uni.needs_packed("mfma")
    _err(lambda: scmp.scmp_plan_create(D=64, levels=(128,), mode=7), scmp.SCMP_ERR_ARG)


def test_group_entry_points_check_arguments_on_the_host():
    lib = scmp.load()
    assert lib.scmp_matmul_group_rungs(None, None, 0, 1, 1, 1, *([None] * 6), None, None, 1, 1, None, 0,
                                       None) == scmp.SCMP_ERR_ARG
    assert b"group_rung" in lib.scmp_last_error()
    assert lib.scmp_group_max(None, 0, 5, None, None) == scmp.SCMP_OK        # nothing to do
    assert lib.scmp_group_max(None, -1, 5, None, None) == scmp.SCMP_ERR_ARG
    assert lib.scmp_group_max(None, 3, 0, None, None) == scmp.SCMP_ERR_ARG
    assert lib.scmp_group_max(None, 3, 4, None, None) == scmp.SCMP_ERR_ARG
    assert lib.scmp_matmul_bias(None, None, 0, 1, 1, 1, *([None] * 7), None, None, 1, 1, None, 0,
                                None) == scmp.SCMP_ERR_ARG


def test_bench_refuses_more_than_one_gpu():
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0 and "one GPU" in r.stderr


def test_bench_traffic_is_null_when_sources_differ(tmp_path, monkeypatch):
    import bench
    real = bench.sources_sha256()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))        # profiles/ under tmp_path
    monkeypatch.setattr(bench, "sources_sha256", lambda: real)
    (tmp_path / "profiles").mkdir()
    rec = {"workload": "w", "algo": "auto", "fetch_bytes_per_dispatch": 10, "write_bytes_per_dispatch": 5}
    for sha, expect in ((real, 30), ("0" * 64, None)):
        text = "summary\n```json\n" + json.dumps(dict(rec, sources_sha256=sha)) + "\n```\n"
        (tmp_path / "profiles" / "k_mfma_w.md").write_text(text)
        assert bench.profiled_traffic("w", "auto", 2) == expect
        assert bench.profiled_traffic("w", "gather", 2) is None


def test_matrix_core_exactness_limit():
    # The matrix-core forms sum each accumulation segment in float32; one
    # index adds at most L + 1, so counts stay exact integers only while
    # segment * (longest L + 1) < 2^24 (at L = 256: D <= 65280).
    assert scmp.scmp_plan_create(D=65280, levels=(256,)).mfma_exact == 1
    assert scmp.scmp_plan_create(D=65281, levels=(256,)).mfma_exact == 0
    assert scmp.scmp_plan_create(D=65281, levels=(128,)).mfma_exact == 1          # 65281 * 129 < 2^24
    assert scmp.scmp_plan_create(D=130055, levels=(128,)).mfma_exact == 1         # 130055 * 129 < 2^24
    assert scmp.scmp_plan_create(D=130056, levels=(128,)).mfma_exact == 0         # 130056 * 129 >= 2^24
    # With chunk scales each chunk is its own segment.
    assert scmp.scmp_plan_create(D=200000, chunk_d=64, levels=(256,)).mfma_exact == 1
    # The longest length of any band or rung sets the bound.
    assert scmp.scmp_plan_create(D=65281, levels=(256, 64), fractions=(0.5, 0.5)).mfma_exact == 0
    assert scmp.scmp_plan_create(D=65280, levels=(256, 64), fractions=(0.5, 0.5)).mfma_exact == 1
