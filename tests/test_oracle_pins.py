"""Pins of the CPU oracle against what the pages and the mathematics fix.

Nothing here compares the oracle with itself: each test checks a closed
form, an invariant, a library special case, a hand-derived example or a
brute-force identity, chosen so that a dropped term, a wrong sign or index,
or swapped operands in the oracle fails at least one of them.
"""

import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle as o

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _table(p, L=None):
    P = 1 << p
    r = o.sobol_points(p, P if L is None else L)
    K = o.indicator_table(r, P)
    return r, K, o.cumulative_table(K)


# ---------------------------------------------------------------- Sobol ----

def _bitrev(v, p):
    out = 0
    for _ in range(p):
        out = (out << 1) | (v & 1)
        v >>= 1
    return out


@pytest.mark.parametrize("p", range(1, 11))
def test_sobol_recurrence_equals_bitreversed_gray_code(p):
    P = 1 << p
    r = o.sobol_points(p, P)
    closed = [_bitrev(l ^ (l >> 1), p) for l in range(P)]
    assert r.tolist() == closed


@pytest.mark.parametrize("p", range(1, 11))
def test_sobol_full_period_is_a_permutation(p):
    P = 1 << p
    assert sorted(o.sobol_points(p, P).tolist()) == list(range(P))


def test_sobol_matches_torch_unscrambled_engine():
    torch = pytest.importorskip("torch")
    from torch.quasirandom import SobolEngine

    pts = SobolEngine(1, scramble=False).draw(256).double().flatten() * 256
    assert pts.tolist() == [float(v) for v in o.sobol_points(8, 256)]


def test_sobol8_prefix_golden():
    g = json.load(open(os.path.join(GOLDEN, "sobol8_prefix.json")))
    assert o.sobol_points(8, 16).tolist() == g["r"]


# ---------------------------------------------------------------- table ----

@pytest.mark.parametrize("p", [2, 3, 4, 8])
def test_full_period_unipolar_count_is_b_plus_one(p):
    # K[b, l] = 1[r_l <= b]: over a full period the count of row b is b + 1.
    P = 1 << p
    _, K, cum = _table(p)
    for u in range(P + 1):
        assert cum[u, P] == u
    assert not K[0].any() and K[P].all()


@pytest.mark.parametrize("p", [3, 4, 8])
def test_prefix_truncation_at_powers_of_two(p):
    # The 2^k prefix of the Sobol table is a stratified coarser table:
    # cum[u][2^k] = ceil(u 2^k / P) for every level u.
    P = 1 << p
    _, _, cum = _table(p)
    for k in range(p + 1):
        L = 1 << k
        for u in range(P + 1):
            assert cum[u, L] == -((-u * L) // P)


def test_table_rows_are_nested():
    _, K, _ = _table(8)
    assert np.all(K[1:] >= K[:-1])


# ------------------------------------------------------------- quantiser ----

def test_quantiser_hand_example():
    # Row abs-max 4 -> s = 4/127; x/s = 31.75 x.  Values chosen far from
    # rounding ties: 4 -> 127, -2.1 -> -66.675 -> -67, 1 -> 31.75 -> 32,
    # 0 -> 0, -4 -> -127, 0.3 -> 9.525 -> 10, 0.02 -> 0.635 -> 1.
    X = np.array([[4.0, -2.1, 1.0, 0.0, -4.0, 0.3, 0.02]], dtype=np.float32)
    x, s = o.quantize(X, 8)
    assert abs(float(s[0, 0]) - 4.0 / 127.0) < 1e-8
    assert x[0].tolist() == [127, -67, 32, 0, -127, 10, 1]
    # Round half to even on an exact tie: amax 127 -> s = 1, 2.5 -> 2, 3.5 -> 4.
    x2, s2 = o.quantize(np.array([[127.0, 2.5, 3.5, -2.5]], dtype=np.float32), 8)
    assert s2[0, 0] == 1.0 and x2[0].tolist() == [127, 2, 4, -2]


def test_quantiser_invariants():
    rng = np.random.default_rng(0)
    X = (rng.standard_normal((50, 37)) * rng.uniform(0.01, 100, (50, 1))).astype(np.float32)
    X[3] = 0.0
    x, s = o.quantize(X, 8)
    assert x.min() >= -127 and x.max() <= 127
    assert np.all(x[3] == 0) and s[3, 0] == 0
    for i in range(50):
        if i == 3:
            continue
        j = int(np.argmax(np.abs(X[i])))
        assert abs(x[i, j]) == 127
        err = np.abs(X[i].astype(np.float64) - s[i, 0] * x[i])
        assert err.max() <= 0.5 * float(s[i, 0]) * (1 + 1e-5)
    xn, sn = o.quantize(-X, 8)
    assert np.array_equal(xn, -x) and np.array_equal(sn, s)


def test_quantiser_matches_torch_cpu_rounding():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(1)
    X = rng.standard_normal((20, 64)).astype(np.float32)
    x, s = o.quantize(X, 8)
    t = torch.from_numpy(X)
    ts = t.abs().amax(dim=1, keepdim=True) / 127.0
    tx = torch.clamp(torch.round(t / ts), -127, 127).to(torch.int64)
    assert np.array_equal(ts.numpy()[:, 0], s[:, 0])
    assert np.array_equal(tx.numpy(), x)


def test_chunked_quantiser_is_per_chunk():
    rng = np.random.default_rng(2)
    X = rng.standard_normal((7, 150)).astype(np.float32)
    x, s = o.quantize(X, 8, chunk_d=64)
    assert s.shape == (7, 3)
    for c, (c0, c1) in enumerate([(0, 64), (64, 128), (128, 150)]):
        xc, sc = o.quantize(X[:, c0:c1], 8)
        assert np.array_equal(x[:, c0:c1], xc) and np.array_equal(s[:, c], sc[:, 0])


@pytest.mark.parametrize("p", [3, 4, 8])
def test_level_map(p):
    q = (1 << (p - 1)) - 1
    P = 1 << p
    u = [int(o.bipolar_level(x, p)) for x in range(-q, q + 1)]
    assert u[0] == 0 and u[q] == P // 2 and u[-1] == P
    for x, ux in zip(range(-q, q + 1), u):
        exact = Fraction(P * (x + q), 2 * q)
        assert abs(ux - exact) < Fraction(1, 2)      # round, never a tie
        assert int(o.bipolar_level(-x, p)) == P - ux
    assert all(b > a for a, b in zip(u, u[1:]))


def test_level_map_values_at_p8():
    assert [int(o.bipolar_level(x, 8)) for x in (-127, -1, 0, 1, 2, 64, 127)] == \
        [0, 127, 128, 129, 130, 193, 256]


# ------------------------------------------------------------ C-BSG count ---

def _closed_form(cum, ua, ub, L):
    n1 = int(cum[ua, L])
    n0 = L - n1
    return int(cum[ub, n1]) + n0 - int(cum[ub, n0])


@pytest.mark.parametrize("p", [2, 3, 4])
def test_count_equals_closed_form_exhaustive(p):
    # Under the counter reading B emits K[u_B][0..n1) where A is 1 and
    # K[u_B][0..n0) where A is 0, so XNOR count = cum[u_B][n1] + n0 - cum[u_B][n0].
    P = 1 << p
    _, K, cum = _table(p)
    for L in range(1, P + 1):
        for ua in range(P + 1):
            for ub in range(P + 1):
                assert o.xnor_count(K, K, ua, ub, L) == _closed_form(cum, ua, ub, L)


def test_count_equals_closed_form_p8_workload_lengths():
    rng = np.random.default_rng(3)
    _, K, cum = _table(8)
    for L in (48, 59, 64, 69, 80, 96, 117, 128, 139, 144, 160, 176, 192, 208, 240, 256):
        for ua, ub in rng.integers(0, 257, size=(40, 2)):
            assert o.xnor_count(K, K, int(ua), int(ub), L) == _closed_form(cum, int(ua), int(ub), L)


def test_vectorised_row_count_matches_per_triple_count():
    rng = np.random.default_rng(4)
    _, K, _ = _table(8)
    D, N = 9, 5
    ua = rng.integers(0, 257, D)
    ub = rng.integers(0, 257, (N, D))
    Ld = rng.integers(1, 257, D)
    per_d = o.xnor_count_row(K, ua, ub, Ld, col_block=2)
    for j in range(N):
        for d in range(D):
            assert per_d[j, d] == o.xnor_count(K, K, ua[d], ub[j, d], int(Ld[d]))


def _shift_table(p, t):
    P = 1 << p
    r = o.sobol_points(p, P)
    return o.indicator_table(np.roll(r, -t), P)


@pytest.mark.parametrize("p", [2, 3, 4])
def test_cbsg_unbiased_over_b_offsets(p):
    # Offsetting B's counter sequence by t over a full period: the summed
    # count is n1 u_B + n0 (P - u_B) exactly, i.e. the conditional
    # probability that B emits 1 equals its marginal u_B / P.
    P = 1 << p
    _, K, cum = _table(p)
    shifted = [_shift_table(p, t) for t in range(P)]
    for L in range(1, P + 1):
        for ua in range(P + 1):
            n1 = int(cum[ua, L])
            n0 = L - n1
            for ub in range(P + 1):
                total = sum(o.xnor_count(K, Kt, ua, ub, L) for Kt in shifted)
                assert total == n1 * ub + n0 * (P - ub)


@pytest.mark.parametrize("p", [2, 3])
def test_cbsg_unbiased_over_both_offsets(p):
    # Offsetting A as well: sum_s sum_t count = L [u_A u_B + (P-u_A)(P-u_B)],
    # so E[(2/L) count - 1] = (2u_A/P - 1)(2u_B/P - 1).
    P = 1 << p
    shifted = [_shift_table(p, t) for t in range(P)]
    for L in range(1, P + 1):
        for ua in range(P + 1):
            for ub in range(P + 1):
                total = sum(o.xnor_count(Ks, Kt, ua, ub, L) for Ks in shifted for Kt in shifted)
                assert total == L * (ua * ub + (P - ua) * (P - ub))
                mean = Fraction(2, L) * Fraction(total, P * P) - 1
                assert mean == Fraction(2 * ua - P, P) * Fraction(2 * ub - P, P)


@pytest.mark.parametrize("D", [1, 2, 3])
def test_cbsg_unbiased_is_additive_over_contraction(D):
    p, P = 3, 8
    shifted = [_shift_table(p, t) for t in range(P)]
    _, K, cum = _table(p)
    rng = np.random.default_rng(5 + D)
    for _ in range(30):
        ua = rng.integers(0, P + 1, D)
        ub = rng.integers(0, P + 1, D)
        L = int(rng.integers(1, P + 1))
        total = sum(o.xnor_count(K, Kt, ua, ub, L) for Kt in shifted)
        expect = 0
        for d in range(D):
            n1 = int(cum[ua[d], L])
            expect += n1 * int(ub[d]) + (L - n1) * (P - int(ub[d]))
        assert total == expect


@pytest.mark.parametrize("p,n_bad", [(2, 36), (3, 392), (4, 3600)])
def test_negative_control_shared_index_generator_is_biased(p, n_bad):
    # A generator whose two streams read the same random numbers at the same
    # index (one shared offset s, b_l = K_s[u_B][l]) is maximally correlated:
    # summed over the P offset pairs it does not reach the unbiased total
    # L [u_A u_B + (P-u_A)(P-u_B)] unless min(u) = 0 or max(u) = P.  This
    # guards the identity tests above against being vacuous.
    P = 1 << p
    shifted = [_shift_table(p, t) for t in range(P)]
    bad = 0
    for L in range(1, P + 1):
        for ua in range(P + 1):
            for ub in range(P + 1):
                total = 0
                for Ks in shifted:
                    a = Ks[ua, :L]
                    b = Ks[ub, :L]
                    total += int(np.sum(1 - (a ^ b)))
                if P * total != L * (ua * ub + (P - ua) * (P - ub)):
                    bad += 1
                # The same shared offsets with the conditional generator
                # meet the identity (A offset s, B counters offset t).
    assert bad == n_bad


def test_exact_zero_operand_gives_half_count():
    # x_A = 0 (u = P/2): for even L the count is exactly L/2 for every u_B.
    _, K, cum = _table(8)
    for L in range(2, 257, 2):
        for ub in range(0, 257, 7):
            assert o.xnor_count(K, K, 128, ub, L) == L // 2


def test_exact_full_scale_operand():
    # x_A = +-127: A's stream is all ones / all zeros; at L = 256 the count
    # is u_B (resp. 256 - u_B) and the unit decode (2/L) count - 1 is exactly
    # the bipolar value of B (resp. its negative).
    _, K, cum = _table(8)
    for ub in range(257):
        c = o.xnor_count(K, K, 256, ub, 256)
        assert c == ub
        assert Fraction(2 * c, 256) - 1 == Fraction(2 * ub - 256, 256)
        assert o.xnor_count(K, K, 0, ub, 256) == 256 - ub
    for L in (48, 100, 192):
        for ub in range(0, 257, 5):
            assert o.xnor_count(K, K, 256, ub, L) == cum[ub, L]


def test_exact_stratified_products():
    # When 2^j divides n1 and n0 and P / 2^j divides u_B, the 2^j-aligned
    # Sobol blocks are exactly stratified and count * P = n1 u_B + n0 (P - u_B).
    P = 256
    _, K, cum = _table(8)
    hits = 0
    for L in (64, 128, 192, 256):
        for ua in range(P + 1):
            n1 = int(cum[ua, L])
            n0 = L - n1
            j = 0
            while j < 8 and n1 % (1 << (j + 1)) == 0 and n0 % (1 << (j + 1)) == 0:
                j += 1
            step = P >> j
            for ub in range(0, P + 1, step):
                c = o.xnor_count(K, K, ua, ub, L)
                assert c * P == n1 * ub + n0 * (P - ub)
                hits += 1
    assert hits > 500


def test_worked_example_p3_golden():
    g = json.load(open(os.path.join(GOLDEN, "worked_example_p3.json")))
    p = g["p"]
    r, K, cum = _table(p)
    assert r.tolist() == g["sobol_r"]
    for xs, u in g["level_of_x"].items():
        assert int(o.bipolar_level(int(xs), p)) == u
    a = o.stream_a(K, g["u_a"], g["L"])
    b = o.conditional_stream_b(K, a, g["u_b"])
    assert a.tolist() == g["stream_a"] and b.tolist() == g["stream_b"]
    assert (1 - (a ^ b)).tolist() == g["xnor"]
    assert o.xnor_count(K, K, g["u_a"], g["u_b"], g["L"]) == g["count"]
    by_t = [o.xnor_count(K, _shift_table(p, t), g["u_a"], g["u_b"], g["L"]) for t in range(8)]
    assert by_t == g["counts_by_b_offset"] and sum(by_t) == g["sum_over_b_offsets"]
    mean = 2.0 / g["L"] * (sum(by_t) / 8.0) - 1.0
    assert mean == g["mean_decoded_over_offsets"]


# --------------------------------------------------------------- decode ----

def test_decode_single_chunk_is_the_printed_equation():
    # C = s_A s_B q^2 [ (2/L) count - D ] for one chunk of width D.
    rng = np.random.default_rng(6)
    counts = rng.integers(0, 64 * 64, (3, 4, 1))
    sA = rng.uniform(0.1, 1, (3, 1))
    sB = rng.uniform(0.1, 1, (4, 1))
    L = np.full((3, 1), 64)
    C, _ = o.decode(counts, sA, sB, L, np.array([64]), 127)
    for i in range(3):
        for j in range(4):
            want = sA[i, 0] * sB[j, 0] * 127 ** 2 * (2.0 / 64 * counts[i, j, 0] - 64)
            assert math.isclose(C[i, j], want, rel_tol=1e-12, abs_tol=1e-9)


def test_decode_full_scale_row_is_exact_product_of_levels():
    # Row of +127 at L = 256: every term is (2 u_B / 256 - 1), exact.
    plan = o.OraclePlan(p=8, Lmax=256, D=16, levels=(256,))
    rng = np.random.default_rng(7)
    A = np.full((1, 16), 3.0, dtype=np.float32)
    B = rng.standard_normal((5, 16)).astype(np.float32)
    out = o.sc_matmul_rows(A, B, plan)
    ub = o.bipolar_level(out["x_b"], 8)
    want = np.float64(out["s_a"][0, 0]) * out["s_b"][:, 0].astype(np.float64) * 127 ** 2 * ((2.0 * ub / 256 - 1).sum(axis=1))
    assert np.allclose(out["C"][0], want, rtol=1e-12)


def test_sc_error_falls_with_stream_length_and_norm_ratio_is_near_one():
    rng = np.random.default_rng(8)
    A = rng.standard_normal((6, 64)).astype(np.float32)
    B = rng.standard_normal((40, 64)).astype(np.float32)
    ref = A.astype(np.float64) @ B.astype(np.float64).T
    errs = []
    for L in (16, 64, 256):
        out = o.sc_matmul_rows(A, B, o.OraclePlan(D=64, levels=(L,)))
        errs.append(np.linalg.norm(out["C"] - ref) / np.linalg.norm(ref))
        if L == 256:
            ratio = np.linalg.norm(out["C"]) / np.linalg.norm(ref)
            assert 0.97 < ratio < 1.03
    assert errs[0] > errs[1] > errs[2]
    assert errs[2] < 0.1


# ------------------------------------------- head-aligned compensator ----

def test_head_aligned_zero_weights_give_the_bias():
    # W = 0 quantises to zero scales, so every head's decode term is 0.
    rng = np.random.default_rng(31)
    X = rng.standard_normal((5, 192)).astype(np.float32)
    b = rng.standard_normal(7)
    out = o.head_aligned_rows(X, np.zeros((7, 192), np.float32), b, head_dim=64, L=256)
    assert np.array_equal(out["C"], np.broadcast_to(b, (5, 7)))


def test_head_aligned_full_scale_heads_are_exact():
    # Each head of each x row holds one positive value (a different one per
    # head), so x quantises to +127 on every column with that head's own
    # scale, and at L = 256 every term is (2 u_B / 256 - 1) exactly: the
    # output is the sum over heads of s^A_h s^B_jh 127^2 sum_d (2 u_B / 256 - 1)
    # with W quantised per row over each head's columns, plus the bias.
    rng = np.random.default_rng(32)
    hd, H, N = 16, 3, 6
    X = np.repeat(np.array([[1.0, 5.0, 0.25], [2.0, 0.5, 3.0]], np.float32), hd, axis=1)
    W = rng.standard_normal((N, H * hd)).astype(np.float32)
    b = rng.standard_normal(N)
    out = o.head_aligned_rows(X, W, b, head_dim=hd, L=256)
    want = np.tile(b, (2, 1)).astype(np.float64)
    for h in range(H):
        cols = slice(h * hd, (h + 1) * hd)
        xa, sa = o.quantize(X[:, cols], 8)
        xb, sb = o.quantize(W[:, cols], 8)
        assert np.all(xa == 127)
        ub = o.bipolar_level(xb, 8)
        term = (2.0 * ub / 256 - 1).sum(axis=1)
        want += np.float64(sa[:, :1]) * sb[:, 0].astype(np.float64)[None, :] * 127 ** 2 * term[None, :]
    assert np.allclose(out["C"], want, rtol=1e-12, atol=1e-12)


def test_head_aligned_tracks_the_float_product():
    rng = np.random.default_rng(33)
    X = rng.standard_normal((4, 256)).astype(np.float32)
    W = (0.02 * rng.standard_normal((24, 256))).astype(np.float32)
    b = 0.02 * rng.standard_normal(24)
    ref = X.astype(np.float64) @ W.astype(np.float64).T + b
    out = o.head_aligned_rows(X, W, b, head_dim=64, L=256)
    assert np.linalg.norm(out["C"] - ref) / np.linalg.norm(ref) < 0.1


def test_head_rungs_follow_head_amplitude_and_fractions():
    # Head h of the image is a unit-variance block scaled by amp[h]; with
    # the amplitudes far apart the |Q_h|.amax ranking is the amplitude
    # ranking, and fractions (0.25, 0.5, 0.25) of 8 heads give 2 / 4 / 2.
    rng = np.random.default_rng(41)
    amp = np.array([3.0, 0.1, 9.0, 1.0, 0.3, 27.0, 0.03, 0.9], np.float32)
    Q = (rng.uniform(-1, 1, (8, 5, 16)) * amp[:, None, None]).astype(np.float32)
    Q[:, 0, 0] = amp                                 # pin each head's amax
    plan = o.OraclePlan(D=16, levels=(256, 128, 64), fractions=(0.25, 0.5, 0.25))
    cls = o.head_rungs(Q, plan)
    assert np.array_equal(cls["metric"], amp)
    assert cls["order"].tolist() == [5, 2, 0, 3, 7, 4, 1, 6]
    want = np.empty(8, np.int64)
    want[[5, 2]] = 0
    want[[0, 3, 7, 4]] = 1
    want[[1, 6]] = 2
    assert np.array_equal(cls["rung"], want)


def test_head_rungs_ties_go_to_the_lower_head_index():
    Q = np.ones((4, 3, 8), np.float32)
    plan = o.OraclePlan(D=8, levels=(256, 64), fractions=(0.5, 0.5))
    assert o.head_rungs(Q, plan)["rung"].tolist() == [0, 0, 1, 1]


def test_head_mp_rows_is_the_fixed_length_product_at_the_head_rung():
    # Every row of a head runs the head's length: the same counts as the
    # single-length plan at that level, and the counts of a head at L = 64
    # stay within 64 D while differing from the L = 256 product.
    rng = np.random.default_rng(42)
    H, M, N, D = 4, 6, 5, 32
    amp = np.array([1.0, 4.0, 0.25, 2.0], np.float32)
    Q = (rng.standard_normal((H, M, D)) * amp[:, None, None]).astype(np.float32)
    Kt = rng.standard_normal((H, N, D)).astype(np.float32)
    plan = o.OraclePlan(D=D, levels=(256, 64), fractions=(0.5, 0.5))
    rungs = o.head_rungs(Q, plan)["rung"]
    assert rungs.tolist() == [1, 0, 1, 0]
    for h in range(H):
        L = plan.levels[rungs[h]]
        got = o.head_mp_rows(Q, Kt, plan, h)
        ref = o.rows_product(Q[h], np.zeros(M, np.int64), Kt[h], o.OraclePlan(D=D, levels=(L,)))
        assert got["head_rung"] == rungs[h]
        assert np.array_equal(got["counts"], ref["counts"])
        assert np.array_equal(got["C"], ref["C"])
        assert got["counts"].max() <= L * D
    long = o.rows_product(Q[0], np.zeros(M, np.int64), Kt[0], o.OraclePlan(D=D, levels=(256,)))
    assert not np.array_equal(o.head_mp_rows(Q, Kt, plan, 0)["counts"], long["counts"])


# --------------------------------------------------- unipolar (AND) mode --

def test_unipolar_level_values_and_symmetry():
    # round(256 |x| / 127): 0 -> 0, 1 -> 2 (2.016), 63 -> 127 (126.99),
    # 64 -> 129 (129.01), 127 -> 256; magnitude only; monotone in |x|.
    x = np.array([0, 1, -1, 63, 64, -64, 127, -127])
    assert o.unipolar_level(x, 8).tolist() == [0, 2, 2, 127, 129, 129, 256, 256]
    allx = np.arange(0, 128)
    u = o.unipolar_level(allx, 8)
    assert np.all(np.diff(u) >= 2) and np.all(np.diff(u) <= 3)
    # No ties: 2 P |x| is never an odd multiple of q, and u is the nearest level.
    assert np.all(np.abs(256 * allx - 127 * u) * 2 < 127)
    for p in (2, 3, 4, 8):
        q, P = o.QMAX(p), 1 << p
        assert o.unipolar_level(q, p) == P and o.unipolar_level(-q, p) == P and o.unipolar_level(0, p) == 0


def _and_closed_form(cum, ua, ub, L):
    # Under AND only A's ones count, and there B emits K[u_B][0..n1).
    return int(cum[ub, int(cum[ua, L])])


@pytest.mark.parametrize("p", [2, 3, 4])
def test_and_count_equals_closed_form_exhaustive(p):
    P = 1 << p
    _, K, cum = _table(p)
    for L in range(1, P + 1):
        for ua in range(P + 1):
            for ub in range(P + 1):
                assert o.and_count(K, K, ua, ub, L) == _and_closed_form(cum, ua, ub, L)


def test_and_count_special_levels_p8():
    # Level 0 emits no ones (count 0 on either side); level P emits all ones,
    # so A at P makes the count B's ones in its L-prefix and B at P makes it
    # A's ones; the count never exceeds either operand's ones.
    rng = np.random.default_rng(61)
    _, K, cum = _table(8)
    for L in (1, 33, 64, 97, 128, 200, 256):
        for u in rng.integers(0, 257, 12):
            u = int(u)
            assert o.and_count(K, K, 0, u, L) == 0 and o.and_count(K, K, u, 0, L) == 0
            assert o.and_count(K, K, 256, u, L) == cum[u, L]
            assert o.and_count(K, K, u, 256, L) == cum[u, L]
        for ua, ub in rng.integers(0, 257, (20, 2)):
            c = o.and_count(K, K, int(ua), int(ub), L)
            assert c <= min(cum[int(ua), L], cum[int(ub), L])


def test_and_count_full_period_power_of_two_is_within_one_of_the_product():
    # At L = P the row at level 2^k emits exactly 2^k ones, and B's prefix
    # of 2^k Sobol points is stratified: count = ceil(u_B 2^k / P), within 1
    # of the exact product u_A u_B / P.
    _, K, _ = _table(8)
    for k in range(9):
        ua = 1 << k
        for ub in range(257):
            c = o.and_count(K, K, ua, ub, 256)
            assert c == -(-ub * ua // 256)
            assert 0 <= c - ua * ub / 256 < 1


def test_vectorised_and_row_count_matches_per_triple_count():
    rng = np.random.default_rng(62)
    _, K, _ = _table(8)
    D, N = 9, 5
    ua = rng.integers(0, 257, D)
    ub = rng.integers(0, 257, (N, D))
    Ls = rng.integers(1, 257, D)
    got = o.and_count_row(K, ua, ub, Ls)
    for j in range(N):
        for d in range(D):
            assert got[j, d] == o.and_count(K, K, int(ua[d]), int(ub[j, d]), int(Ls[d]))


def test_unipolar_full_scale_rows_are_exact_products():
    # Entries in {0, +-127} are levels 0 and P, whose streams are all zeros
    # or all ones, so every count is exact and the decode equals the float
    # product up to the float32 rounding of the two scales (3/127, 0.5/127).
    rng = np.random.default_rng(63)
    vals = np.array([0.0, 1.0, -1.0], np.float32)
    A = vals[rng.integers(0, 3, (4, 40))] * np.float32(3.0)
    B = vals[rng.integers(0, 3, (6, 40))] * np.float32(0.5)
    A[:, 0], B[:, 0] = 3.0, 0.5                       # every row has full scale
    for L in (64, 97, 256):
        plan = o.OraclePlan(D=40, levels=(L,), mode="unipolar")
        out = o.rows_product(A, np.zeros(4, np.int64), B, plan)
        want = A.astype(np.float64) @ B.astype(np.float64).T
        assert np.allclose(out["C"], want, rtol=3e-7, atol=1e-12)
        assert np.all(out["counts"] % L == 0)          # each index adds 0 or +-L


def test_unipolar_signs_and_zero_rows():
    rng = np.random.default_rng(64)
    A = rng.standard_normal((5, 48)).astype(np.float32)
    B = rng.standard_normal((7, 48)).astype(np.float32)
    plan = o.OraclePlan(D=48, levels=(128,), mode="unipolar")
    r = o.rows_product(A, np.zeros(5, np.int64), B, plan)
    neg = o.rows_product(-A, np.zeros(5, np.int64), B, plan)
    assert np.array_equal(neg["counts"], -r["counts"])
    assert np.array_equal(neg["C"], -r["C"])
    Bn = B.copy()
    Bn[2] = -Bn[2]
    flip = o.rows_product(A, np.zeros(5, np.int64), Bn, plan)
    assert np.array_equal(flip["counts"][:, 2], -r["counts"][:, 2])
    assert np.array_equal(np.delete(flip["counts"], 2, axis=1), np.delete(r["counts"], 2, axis=1))
    zero = o.rows_product(np.zeros((2, 48), np.float32), np.zeros(2, np.int64), B, plan)
    assert not zero["counts"].any() and not zero["C"].any()
    # The bipolar mode on the same inputs counts differently.
    bip = o.rows_product(A, np.zeros(5, np.int64), B, o.OraclePlan(D=48, levels=(128,)))
    assert not np.array_equal(bip["counts"], r["counts"])


def test_unipolar_nonnegative_rows_track_the_float_product():
    # Softmax rows times Gaussian columns: the error falls as L grows.
    rng = np.random.default_rng(65)
    z = 3.0 * rng.standard_normal((6, 64))
    A = (np.exp(z - z.max(1, keepdims=True)) / np.exp(z - z.max(1, keepdims=True)).sum(1, keepdims=True))
    A = A.astype(np.float32)
    B = rng.standard_normal((20, 64)).astype(np.float32)
    ref = A.astype(np.float64) @ B.astype(np.float64).T
    errs = []
    for L in (32, 256):
        out = o.rows_product(A, np.zeros(6, np.int64), B, o.OraclePlan(D=64, levels=(L,), mode="unipolar"))
        errs.append(np.linalg.norm(out["C"] - ref) / np.linalg.norm(ref))
    assert errs[1] < errs[0] and errs[1] < 0.1


# ------------------------------------------------ range-based weight MP --

def test_range_levels_hand_example():
    # Three groups of two rows: ranges 4.0, 1.0 and 0.5 (the last group is
    # one row, ragged); normalised 1, 0.25, 0.125; threshold 0.3 puts the
    # last two low, 0.2 only the last, 0 none, anything above 1 all.
    W = np.array([[1.0, -3.0], [0.5, 0.0],
                  [2.0, 2.5], [1.5, 2.0],
                  [-0.25, 0.25]], np.float32)
    r = o.range_levels(W, 2, 0.3)
    assert r["range"].tolist() == [4.0, 1.0, 0.5]
    assert r["norm"].tolist() == [1.0, 0.25, 0.125]
    assert r["level"].tolist() == [0, 1, 1]
    assert o.range_levels(W, 2, 0.2)["level"].tolist() == [0, 0, 1]
    assert o.range_levels(W, 2, 0.0)["level"].tolist() == [0, 0, 0]
    assert o.range_levels(W, 2, 1.01)["level"].tolist() == [1, 1, 1]
    assert o.range_levels(np.zeros((4, 3), np.float32), 2, 0.3)["level"].tolist() == [1, 1]


def test_range_levels_monotone_in_threshold_and_scale_free():
    rng = np.random.default_rng(81)
    W = (rng.standard_normal((1000, 16)) * np.exp(rng.standard_normal((1000, 1)))).astype(np.float32)
    prev = o.range_levels(W, 64, 0.0)["level"]
    for t in (0.1, 0.3, 0.5, 0.9):
        cur = o.range_levels(W, 64, t)["level"]
        assert np.all(cur >= prev)
        prev = cur
    assert np.array_equal(o.range_levels(4 * W, 64, 0.3)["level"], o.range_levels(W, 64, 0.3)["level"])


def test_range_mp_columns_run_at_their_group_length():
    # Columns of a high group equal the uniform product at L_high and those
    # of a low group the uniform product at L_low; threshold 0 is the
    # uniform plan at L_high.
    rng = np.random.default_rng(82)
    A = rng.standard_normal((5, 32)).astype(np.float32)
    W = (rng.standard_normal((12, 32)) * np.repeat([1.0, 0.1, 2.0], 4)[:, None]).astype(np.float32)
    out = o.range_mp_rows(A, W, (256, 64), 0.3, 4)
    assert out["level"].tolist() == [0, 1, 0]
    assert out["L_col"].tolist() == [256] * 4 + [64] * 4 + [256] * 4
    for L, cols in ((256, [0, 1, 2, 3, 8, 9, 10, 11]), (64, [4, 5, 6, 7])):
        ref = o.rows_product(A, np.zeros(5, np.int64), W[cols], o.OraclePlan(D=32, levels=(L,)))
        assert np.array_equal(out["counts"][:, cols], ref["counts"])
        assert np.array_equal(out["C"][:, cols], ref["C"])
    uni = o.rows_product(A, np.zeros(5, np.int64), W, o.OraclePlan(D=32, levels=(256,)))
    assert np.array_equal(o.range_mp_rows(A, W, (256, 64), 0.0, 4)["C"], uni["C"])
    assert not np.array_equal(out["C"], uni["C"])


# ---------------------------------------------------- mixed precision ----

def test_rung_cuts_workload_fractions():
    cuts = o.rung_cuts(16448, 5, (0.1, 0.15, 0.2, 0.25, 0.3))
    sizes = np.diff(cuts)
    for s, f in zip(sizes, (0.1, 0.15, 0.2, 0.25, 0.3)):
        assert abs(s - f * 16448) <= 1
    assert sizes.sum() == 16448
    ladder = (256, 192, 128, 96, 64)
    L_eff = sum(int(s) * L for s, L in zip(sizes, ladder)) / 16448
    assert abs(L_eff - 123.20) < 0.01
    assert np.diff(o.rung_cuts(257, 3, (0.333, 0.334, 0.333))).tolist() == [86, 85, 86]
    assert np.diff(o.rung_cuts(16448, 4, None)).tolist() == [4112] * 4


def test_rungs_respect_metric_order_and_ties():
    rng = np.random.default_rng(9)
    g = rng.uniform(0, 5, 300).astype(np.float32)
    g[10:20] = g[5]                                 # a block of ties
    gh = o.normalise_metric(g)
    rung, order = o.assign_rungs(gh, 4, (0.1, 0.2, 0.3, 0.4))
    for k in range(3):
        assert gh[rung == k].min() >= gh[rung == k + 1].max()
    pos = {int(r): i for i, r in enumerate(order)}
    tied = sorted([5] + list(range(10, 20)))
    assert [pos[i] for i in tied] == sorted(pos[i] for i in tied)  # index order
    assert sorted(order.tolist()) == list(range(300))


def test_rungs_invariant_under_power_of_two_rescale_and_order_pins_largest():
    rng = np.random.default_rng(10)
    g = rng.uniform(0, 1, 200).astype(np.float32)
    r1, _ = o.assign_rungs(o.normalise_metric(g), 3)
    r2, _ = o.assign_rungs(o.normalise_metric(g * np.float32(8.0)), 3)
    assert np.array_equal(r1, r2)
    assert r1[int(np.argmax(g))] == 0 and r1[int(np.argmin(g))] == 2
    assert np.all(o.normalise_metric(np.zeros(5, np.float32)) == 0)


def test_thresholds_descend_and_separate_rungs():
    rng = np.random.default_rng(11)
    gh = o.normalise_metric(rng.uniform(0, 1, 100).astype(np.float32))
    rung, order = o.assign_rungs(gh, 4)
    tau = o.thresholds(gh, order, o.rung_cuts(100, 4))
    assert np.all(np.diff(tau) <= 0)
    for k in range(1, 4):
        assert gh[rung < k].min() >= tau[k - 1] >= gh[rung >= k].max()


def test_attention_metric_equals_row_max_for_probabilities():
    rng = np.random.default_rng(12)
    lg = 3 * rng.standard_normal((9, 31))
    A = np.exp(lg - lg.max(1, keepdims=True))
    A = (A / A.sum(1, keepdims=True)).astype(np.float32)
    assert np.array_equal(o.attention_row_metric(A), o.row_metric(A))


# ------------------------------------------------------------- K-bands ----

def test_tilt_zero_reproduces_parent_ladder():
    lad = o.tilt_band_ladder((256, 192, 128, 64), 4, 0.0, 256)
    assert np.all(lad == np.array([256, 192, 128, 64])[None, :])


def test_tilted_ladder_identity_ceiling_and_rounding():
    levels = (256, 192, 128, 64)
    lad = o.tilt_band_ladder(levels, 4, 0.25, 256)
    assert lad[:, 0].tolist() == [256] * 4                 # at the ceiling: untilted
    cols = o.band_columns(4096, 64, [16] * 4)
    use = o.check_band_ladder(lad, cols, levels, 256)
    assert np.all(use == 1.0)                               # exact, never overspent
    for k, Lk in enumerate(levels[1:], start=1):
        col = lad[:, k]
        assert col.sum() == 4 * Lk and np.all(np.diff(col) > 0)
        raw = [Lk * (1 + 0.25 * (2 * b - 3) / 3) for b in range(4)]
        # Brute force: among vectors with entries floor(raw) or floor(raw)+1
        # summing to 4 L_k, the chosen one is closest to raw (ties to the
        # lower band getting the unit).
        best = None
        for mask in range(16):
            v = [math.floor(raw[b]) + ((mask >> b) & 1) for b in range(4)]
            if sum(v) != 4 * Lk:
                continue
            dist = sum(abs(v[b] - raw[b]) for b in range(4))
            key = (round(dist, 12), [-((mask >> b) & 1) for b in range(4)])
            if best is None or key < best[0]:
                best = (key, v)
        assert col.tolist() == best[1]


def test_ceiling_guard_fires():
    levels = (256, 192, 128, 64)
    lad = o.tilt_band_ladder(levels, 4, 0.5, 256)
    cols = o.band_columns(4096, 64, [16] * 4)
    with pytest.raises(ValueError, match="ceiling"):
        o.check_band_ladder(lad, cols, levels, 256)
    over = o.tilt_band_ladder(levels, 4, 0.0, 256)
    over[0, 2] += 1
    with pytest.raises(ValueError, match="overspent"):
        o.check_band_ladder(over, cols, levels, 256)


def test_band_columns_with_ragged_last_chunk():
    cols = o.band_columns(150, 64, [2, 1])
    assert cols.tolist() == [0, 128, 150]
    with pytest.raises(ValueError):
        o.band_columns(150, 64, [1, 1])


def _kband_inputs():
    rng = np.random.default_rng(13)
    A = rng.standard_normal((6, 256)).astype(np.float32)
    B = (0.02 * rng.standard_normal((7, 256))).astype(np.float32)
    return A, B


def test_kband_parent_equivalence_and_non_degeneracy():
    A, B = _kband_inputs()
    common = dict(p=8, Lmax=256, D=256, chunk_d=64, levels=(192, 128, 64))
    parent = o.sc_matmul_rows(A, B, o.OraclePlan(**common))
    flat = o.sc_matmul_rows(A, B, o.OraclePlan(n_bands=4, tilt=0.0, **common))
    tilted = o.sc_matmul_rows(A, B, o.OraclePlan(n_bands=4, tilt=0.25, **common))
    assert np.array_equal(parent["counts"], flat["counts"])
    assert np.array_equal(parent["C"], flat["C"])
    assert np.array_equal(flat["band_counts"].sum(axis=2), parent["band_counts"][:, :, 0])
    rel = np.linalg.norm(tilted["C"] - parent["C"]) / np.linalg.norm(parent["C"])
    assert rel > 1e-4


def test_kband_hand_example_p3_golden():
    # A two-band product worked out by hand (tests/golden/kband_hand_p3.json,
    # K-band pull request "How the banding works"): band 0 runs L = 8 and
    # band 1 runs L = 4; swapping the two lengths changes the band counts
    # and the decoded value, so a reversed band -> length mapping fails.
    g = json.load(open(os.path.join(GOLDEN, "kband_hand_p3.json")))
    p = g["p"]
    A = np.asarray([g["A_row"]], dtype=np.float32)
    B = np.asarray([g["B_row"]], dtype=np.float32)

    def run(band_L):
        plan = o.OraclePlan(p=p, Lmax=1 << p, D=g["D"], chunk_d=g["chunk_d"], levels=tuple(g["levels"]),
                            n_bands=len(g["band_chunks"]), band_chunks=tuple(g["band_chunks"]),
                            band_L=np.asarray(band_L))
        return o.rows_product(A, np.zeros(1, dtype=np.int64), B, plan)

    r = run(g["band_L"])
    assert r["x_a"][0].tolist() == g["x_a"] and r["s_a"][0].tolist() == g["s_a"]
    assert r["x_b"][0].tolist() == g["x_b"] and r["s_b"][0].tolist() == g["s_b"]
    assert o.bipolar_level(r["x_a"][0], p).tolist() == g["u_a"]
    assert o.bipolar_level(r["x_b"][0], p).tolist() == g["u_b"]
    assert r["counts"][0, 0].tolist() == g["counts_per_chunk"]
    assert r["band_counts"][0, 0].tolist() == g["band_counts"]
    assert r["L"][0].tolist() == g["L_per_chunk"]
    assert r["C"][0, 0] == g["C"]
    rev = run(g["reversed_band_L"])
    assert rev["band_counts"][0, 0].tolist() == g["reversed_band_counts"]
    assert rev["C"][0, 0] == g["reversed_C"]


# Band layouts written out by hand: band columns, the band owning each
# 64-column chunk, and L[b][k] for the ladder (the tilt-0.25 values are the
# straight-line tilt of 192 / 128 / 64 over four bands, K-band pull request
# "Tooling"; the ragged case is an explicit table within budget).
_KBAND_CASES = {
    "tilt_equal_bands": dict(
        D=256, levels=(192, 128, 64), n_bands=4, band_chunks=None, tilt=0.25, band_L=None,
        cols=[(0, 64), (64, 128), (128, 192), (192, 256)], owner=[0, 1, 2, 3],
        L=[[144, 96, 48], [176, 117, 59], [208, 139, 69], [240, 160, 80]]),
    "ragged_uneven_bands": dict(
        D=150, levels=(128, 96, 60), n_bands=2, band_chunks=(2, 1), tilt=0.0,
        band_L=[[120, 90, 40], [128, 96, 64]],
        cols=[(0, 128), (128, 150)], owner=[0, 0, 1],
        L=[[120, 90, 40], [128, 96, 64]]),
}


@pytest.mark.parametrize("case", sorted(_KBAND_CASES))
def test_kband_each_band_is_the_uniform_product_over_its_own_columns(case):
    # K-band pull request, "How the banding works": band b of the
    # contraction axis runs rung k at L[b][k], and the band partial sums add.
    # Each band's partial count must equal a uniform-length product over
    # exactly that band's columns at its own L[b][k] (the uniform product is
    # pinned by the closed-form and unbiasedness pins above), every chunk
    # must carry its owner band's length, and the mirrored table (band b at
    # the lengths of band B-1-b) must give different counts.
    c = _KBAND_CASES[case]
    rng = np.random.default_rng(17)
    D = c["D"]
    A = rng.standard_normal((9, D)).astype(np.float32)
    A[:, 5] *= 20.0
    B = (0.02 * rng.standard_normal((7, D))).astype(np.float32)
    common = dict(D=D, chunk_d=64, levels=c["levels"], n_bands=c["n_bands"], band_chunks=c["band_chunks"])
    plan = o.OraclePlan(tilt=c["tilt"], band_L=None if c["band_L"] is None else np.asarray(c["band_L"]), **common)
    out = o.sc_matmul_rows(A, B, plan)
    assert plan.ladder().tolist() == c["L"]
    cols, owner = plan.bands()
    assert [(int(cols[b]), int(cols[b + 1])) for b in range(c["n_bands"])] == c["cols"]
    assert owner.tolist() == c["owner"]
    mirrored = o.sc_matmul_rows(A, B, o.OraclePlan(band_L=np.asarray(c["L"])[::-1].copy(), **common))
    assert set(out["rung"].tolist()) == {0, 1, 2}
    for i in range(A.shape[0]):
        k = int(out["rung"][i])
        assert out["L"][i].tolist() == [c["L"][b][k] for b in c["owner"]]
        for b, (c0, c1) in enumerate(c["cols"]):
            uni = o.rows_product(A[i:i + 1, c0:c1], np.zeros(1, dtype=np.int64), B[:, c0:c1],
                                 o.OraclePlan(D=c1 - c0, chunk_d=64, levels=(c["L"][b][k],)))
            assert np.array_equal(out["band_counts"][i, :, b], uni["counts"][0].sum(axis=1)), (i, b)
    assert not np.array_equal(out["band_counts"], mirrored["band_counts"])


def test_mp_rows_use_their_rung_length():
    # Each row's count equals a uniform-L run at that row's rung length.
    A, B = _kband_inputs()
    plan = o.OraclePlan(D=256, levels=(192, 96, 40), fractions=(0.3, 0.3, 0.4))
    out = o.sc_matmul_rows(A, B, plan)
    for i in range(A.shape[0]):
        L = plan.levels[out["rung"][i]]
        uni = o.sc_matmul_rows(A[i:i + 1], B, o.OraclePlan(D=256, levels=(L,)))
        assert np.array_equal(out["counts"][i], uni["counts"][0])
