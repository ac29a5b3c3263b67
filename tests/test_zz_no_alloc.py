"""scmp_matmul_noalloc, the allocation-free form of scmp_matmul (its scratch
is the library's static device array), against scmp_matmul with a caller
workspace on the same encoded inputs: counts bit-exact and C identical, on
two calls in a row, the second with smaller sizes (the array keeps the first
call's contents), for every launch form; sizes beyond the array's maximum
are rejected before any launch."""

import numpy as np
import pytest
import torch

from mixed_precision_quantization_amd import scmp

pytestmark = pytest.mark.gpu

PLANS = {
    "mp_rows": dict(D=256, levels=(256, 128, 64), fractions=(0.2, 0.3, 0.5)),
    "kband_chunks": dict(D=256, chunk_d=64, levels=(256, 192, 128, 64), n_bands=4, tilt=0.25),
}
FORMS = {"mp_rows": ("auto", "mfma_persistent", "mfma_onepass", "gather", "mfma_quarter"),
         "kband_chunks": ("auto", "mfma_onepass", "gather")}


@pytest.fixture(scope="module")
def table():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    t = scmp.scmp_build_sobol_table(8, 256)
    yield t
    t.close()


def _encode(table, plan, M, N, seed):
    rng = np.random.default_rng(seed)
    A = rng.standard_normal((M, plan.D)).astype(np.float32)
    A[:, 3] *= 20.0
    B = (0.02 * rng.standard_normal((N, plan.D))).astype(np.float32)
    qA, sA, mA, _ = scmp.scmp_quantize_encode(table, plan, torch.from_numpy(A).cuda())
    qB, sB, _, _ = scmp.scmp_quantize_encode(table, plan, torch.from_numpy(B).cuda(), want_metric=False)
    perm = None
    if plan.n_rungs > 1:
        _, _, perm, _ = scmp.scmp_classify_rows(plan, mA)
    return qA, sA, qB, sB, perm


@pytest.mark.parametrize("case,algo", [(c, a) for c in PLANS for a in FORMS[c]])
def test_noalloc_matches_workspace_call_on_two_calls(table, case, algo):
    plan = scmp.scmp_plan_create(**PLANS[case])
    for M, N, seed in ((700, 300, 1), (150, 70, 2)):
        print(f"  noalloc {case} algo={algo} M={M} N={N}", flush=True)
        qA, sA, qB, sB, perm = _encode(table, plan, M, N, seed)
        c_ref, C_ref = scmp.scmp_matmul(table, plan, qA, sA, qB, sB, permA=perm, algo=algo, want_counts=True)
        c_out = torch.full_like(c_ref, -7)
        C_out = torch.full_like(C_ref, float("nan"))
        scmp.scmp_matmul_noalloc(table, plan, qA, sA, qB, sB, permA=perm, algo=algo, counts_out=c_out,
                                 C_out=C_out)
        torch.cuda.synchronize()
        assert torch.equal(c_out, c_ref), "counts differ from scmp_matmul"
        assert torch.equal(C_out, C_ref), "C differs from scmp_matmul"


def test_noalloc_rejects_sizes_beyond_its_scratch(table):
    # A 16448 x 4096 x 1024 product needs about 84 MB of scratch; the call
    # must refuse before launching anything (the outputs stay untouched).
    plan = scmp.scmp_plan_create(D=1024, levels=(256,))
    M, N = 16448, 4096
    assert scmp.scmp_matmul_workspace_bytes(table, plan, 1, M, N) > scmp.NOALLOC_SCRATCH_BYTES
    qA = torch.zeros((1, M, 1024), dtype=torch.int8, device="cuda")
    qB = torch.zeros((1, N, 1024), dtype=torch.int8, device="cuda")
    sA = torch.zeros((1, M, 1), dtype=torch.float32, device="cuda")
    sB = torch.zeros((1, N, 1), dtype=torch.float32, device="cuda")
    C = torch.full((1, 4, N), 3.0, dtype=torch.float32, device="cuda").expand(1, 4, N)
    C_out = torch.full((1, M, N), 3.0, dtype=torch.float32, device="cuda")
    with pytest.raises(scmp.ScmpError) as ei:
        scmp.scmp_matmul_noalloc(table, plan, qA, sA, qB, sB, C_out=C_out)
    assert ei.value.status == scmp.SCMP_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((C_out[:, :4] == C).all())
