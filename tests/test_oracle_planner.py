"""Pins for the oracle's offline planner (CPU only)."""
import itertools

import numpy as np
import pytest

from oracle import planner, quant
from oracle.recurrence import delta_update

GRID4 = (1.0, 0.875, 0.75, 0.625)


def test_lifetime_closed_form_for_constant_gate():
    # alpha = sigmoid(mu) constant: sum_j alpha^j = 1 / (1 - alpha) = 1 + e^mu.
    for mu in (-1.0, 0.0, 4.0, 7.0):
        alpha = 1.0 / (1.0 + np.exp(-mu))
        L = planner.lifetime_weight(np.log(alpha))
        assert L == pytest.approx(1.0 + np.exp(mu), rel=1e-12)
    assert planner.lifetime_weight(np.log(1 / (1 + np.exp(-4.0)))) == pytest.approx(55.598150033, rel=1e-9)


def test_lifetime_equals_truncated_series():
    for lbar in (-0.5, -0.05, -0.002):
        j = np.arange(200000)
        assert planner.lifetime_weight(lbar) == pytest.approx(np.sum(np.exp(j * lbar)), rel=1e-9)


def test_lifetime_of_unit_gate_is_finite():
    assert np.isfinite(planner.lifetime_weight(0.0))
    assert planner.lifetime_weight(0.0) == pytest.approx(1.0 / (1.0 - np.exp(-(2.0 ** -20))))


def test_unit_log_retention_layouts():
    a_gdn = np.array([[0.9, 0.99]])
    assert np.allclose(planner.unit_log_retention(a_gdn, "gdn", "head", 4), np.log([0.9, 0.99]))
    assert np.allclose(planner.unit_log_retention(a_gdn, "gdn", "row", 3),
                       np.log([0.9, 0.9, 0.9, 0.99, 0.99, 0.99]))
    a_kda = np.array([[[0.5, 0.8], [0.9, 0.7]]])
    assert np.allclose(planner.unit_log_retention(a_kda, "kda", "row", 2), np.log([0.5, 0.8, 0.9, 0.7]))
    assert np.allclose(planner.unit_log_retention(a_kda, "kda", "head", 2),
                       [np.log([0.5, 0.8]).mean(), np.log([0.9, 0.7]).mean()])


def _brute_alloc(cost, widths, budget_milli):
    U = cost.shape[0]
    best = None
    for combo in itertools.product(range(len(widths)), repeat=U):
        bits = sum(widths[j] for j in combo)
        if 1000 * bits > budget_milli * U:
            continue
        c = sum(cost[u, j] for u, j in enumerate(combo))
        key = (c, bits)
        if best is None or key < best[0]:
            best = (key, combo)
    return np.array(best[1])


@pytest.mark.parametrize("seed,U,budget", [(0, 5, 6000), (1, 8, 6000), (2, 7, 5000), (3, 8, 7250), (4, 6, 4000)])
def test_allocation_equals_brute_force(seed, U, budget):
    g = np.random.default_rng(seed)
    widths = (4, 6, 8)
    # distortion falls with width; lifetime weights spread over two decades
    D = np.sort(g.uniform(0.01, 1.0, size=(U, 3)), axis=1)[:, ::-1] * g.uniform(1, 100, size=(U, 1))
    got = planner.allocate(D, widths, budget)
    ref = _brute_alloc(D, widths, budget)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("seed,U,budget", [(5, 6, 4000), (6, 6, 3500), (7, 5, 5000)])
def test_allocation_with_five_widths_equals_brute_force(seed, U, budget):
    g = np.random.default_rng(seed)
    widths = (2, 3, 4, 6, 8)
    D = np.sort(g.uniform(0.01, 1.0, size=(U, 5)), axis=1)[:, ::-1] * g.uniform(1, 100, size=(U, 1))
    got = planner.allocate(D, widths, budget)
    assert np.array_equal(got, _brute_alloc(D, widths, budget))
    bits = np.asarray(widths)[got]
    assert bits.sum() * 1000 <= budget * U and len(set(bits)) > 1     # the 4-bit budget mixes widths


def test_allocation_ties_prefer_fewer_bits():
    cost = np.zeros((4, 3))                        # distortion already zero at every width
    assert np.array_equal(planner.allocate(cost, (4, 6, 8), 8000), [0, 0, 0, 0])
    cost = np.tile([[2.0, 1.0, 1.0]], (3, 1))      # 6 and 8 bits equally good
    assert np.array_equal(planner.allocate(cost, (4, 6, 8), 8000), [1, 1, 1])


def test_allocation_respects_budget_exactly():
    g = np.random.default_rng(5)
    U = 300
    D = np.sort(g.uniform(0.01, 1.0, size=(U, 3)), axis=1)[:, ::-1]
    ch = planner.allocate(D, (4, 6, 8), 6000)
    bits = np.asarray((4, 6, 8))[ch]
    assert bits.sum() <= 6 * U
    assert bits.sum() >= 6 * U - 2                 # a strictly decreasing cost uses the budget


def test_pivots_are_top_lifetime_units():
    g = np.random.default_rng(6)
    L = g.uniform(1, 1000, 50)
    D4 = g.uniform(0, 1, 50)
    n = planner.pivot_count(10000, 50)             # 1% of 50 -> 1
    assert n == 1 and planner.pivot_count(10000, 1152) == 12 and planner.pivot_count(5000, 4096) == 21
    assert planner.pivot_count(0, 10) == 0 and planner.pivot_count(10000, 100) == 1
    piv = planner.select_pivots(L, D4, 5)
    assert set(piv.tolist()) == set(np.argsort(-L)[:5].tolist())
    # equal lifetimes: the larger distortion wins, then the lower index
    piv = planner.select_pivots(np.ones(4), np.array([0.1, 0.5, 0.5, 0.2]), 2)
    assert piv.tolist() == [1, 2]


def test_impact_score_is_the_readout_sensitivity():
    """a_i is the factor by which row i of a state error reaches the next readout.

    Perturbing the state by E and running the same token gives
    delta y = y(S + E) - y(S) = sum_i a_i E_i. ; w_i = mean over tokens of a_i^2.
    """
    g = np.random.default_rng(7)
    dk, dv, T = 6, 5, 40
    q = g.standard_normal((T, dk)); q /= np.linalg.norm(q, axis=1, keepdims=True)
    k = g.standard_normal((T, dk)); k /= np.linalg.norm(k, axis=1, keepdims=True)
    v = g.standard_normal((T, dv))
    beta = g.uniform(0, 1, T)
    alpha = g.uniform(0.5, 1.0, dk)
    S = g.standard_normal((1, dk, dv))
    a2 = np.zeros((T, dk))
    for t in range(T):
        for i in range(dk):
            E = np.zeros_like(S)
            E[0, i, 0] = 1.0
            _, y0 = delta_update(S, q[t][None], k[t][None], v[t][None], alpha[None], beta[t:t + 1])
            _, y1 = delta_update(S + E, q[t][None], k[t][None], v[t][None], alpha[None], beta[t:t + 1])
            a2[t, i] = (y1[0, 0] - y0[0, 0]) ** 2
    w = planner.impact_from_traces(q, k, beta, alpha)
    assert np.allclose(w, a2.mean(axis=0), rtol=1e-9, atol=1e-12)


def test_impact_expectation_without_write():
    # beta = 0, q uniform on the sphere: E[a_i^2] = alpha_i^2 / d_k.
    g = np.random.default_rng(8)
    dk, T = 16, 200000
    q = g.standard_normal((T, dk)); q /= np.linalg.norm(q, axis=1, keepdims=True)
    alpha = g.uniform(0.3, 1.0, dk)
    w = planner.impact_from_traces(q, q, np.zeros(T), alpha)
    assert np.allclose(w, alpha ** 2 / dk, rtol=0.02)


def test_distortion_properties():
    g = np.random.default_rng(9)
    S, dk, dv = 3, 8, 8
    snap = g.standard_normal((S, dk, dv))
    w = g.uniform(0.5, 2.0, dk)
    Dh = planner.head_distortion(snap, w, (4, 6, 8), GRID4, "head")
    Dr = planner.head_distortion(snap, w, (4, 6, 8), GRID4, "row")
    assert Dh.shape == (1, 3) and Dr.shape == (dk, 3)
    assert np.allclose(Dh[0], Dr.sum(axis=0), rtol=1e-12)
    assert Dh[0, 0] > Dh[0, 1] > Dh[0, 2] > 0
    Z = planner.head_distortion(np.zeros((S, dk, dv)), w, (4, 6, 8), GRID4, "head")
    assert np.all(Z == 0)


def test_calibration_snapshot_from_zero_single_token():
    g = np.random.default_rng(10)
    q = g.standard_normal((2, 1, 4)); k = g.standard_normal((2, 1, 4)); v = g.standard_normal((2, 1, 3))
    beta = np.array([[0.5], [0.25]])
    snap = planner.calib_snapshots(q, k, v, beta, 0.9)
    assert np.allclose(snap, beta[:, 0, None, None] * k[:, 0, :, None] * v[:, 0, None, :], atol=1e-15)


def test_make_plan_small_end_to_end():
    g = np.random.default_rng(11)
    L_, H, dk, dv = 1, 6, 8, 8
    alpha = 1 / (1 + np.exp(-g.normal(4, 1, (L_, H))))

    def traces(l, h):
        r = np.random.default_rng(100 + h)
        q = r.standard_normal((2, 16, dk)); q /= np.linalg.norm(q, axis=-1, keepdims=True)
        k = r.standard_normal((2, 16, dk)); k /= np.linalg.norm(k, axis=-1, keepdims=True)
        return q, k, r.standard_normal((2, 16, dv)), r.uniform(0, 1, (2, 16))

    w = g.uniform(0.5, 2, (L_, H, dk))
    p = planner.make_plan("gdn", "head", L_, H, dk, dv, (4, 6, 8), 6000, 200000, GRID4, alpha, traces, w)
    assert len(p.pivot_units) == 2                         # ceil(0.2 * 6)
    assert set(p.pivot_units.tolist()) == set(np.argsort(-alpha[0])[:2].tolist())
    rest = [u for u in range(H) if u not in p.pivot_units]
    assert np.sum(p.unit_bits[rest]) <= 6 * len(rest)
    ref = _brute_alloc(p.L[rest, None] * p.D[rest], (4, 6, 8), 6000)
    assert np.array_equal(p.unit_bits[rest], np.asarray((4, 6, 8))[ref])
    assert np.all(p.bits[0, p.pivot_units] == 16) and np.all(p.pivot[0, p.pivot_units])


# ---------------------------------------------------------------- distortion and calibration snapshots
#
# hyper.ai summary, 方法 (Method), the Lifetime-Aware Bit Allocation paragraph: the planner estimates each
# unit's reconstruction distortion at every candidate width on calibration states.  Reading taken: D_u(b) is
# the mean over the segment-final calibration states of the unweighted squared error of the unit's entries,
# with every row of the state quantized at width b by the step's own quantizer and no row kept as a pivot.

from fractions import Fraction as Fr
from math import isqrt

GRID4_EXACT = (Fr(1), Fr(7, 8), Fr(3, 4), Fr(5, 8))


def _ulp16(x: Fr) -> Fr:
    """Spacing of binary16 values around a positive x in the normal range (11 significant bits)."""
    e = 0
    while x >= Fr(2) ** (e + 1):
        e += 1
    while x < Fr(2) ** e:
        e -= 1
    return Fr(2) ** (max(e, -14) - 10)


def _f16_exact(x: Fr) -> Fr:
    """binary16 value nearest to a positive rational x (ties to even), clamped to [2^-14, 65504] first."""
    x = min(max(x, Fr(1, 2 ** 14)), Fr(65504))
    ulp = _ulp16(x)
    n, rem = divmod(x, ulp)
    n = int(n)
    if rem > ulp / 2 or (rem == ulp / 2 and n % 2 == 1):
        n += 1
    return min(n * ulp, Fr(65504))


def _f16_sqrt_exact(x: Fr) -> Fr:
    """binary16 value nearest to sqrt(x) for a positive rational x, by comparing squares (exact)."""
    num, den = x.numerator, x.denominator
    s = Fr(isqrt(num * den), den)              # s <= sqrt(x) < s + 1/den
    lo = min(max(s, Fr(1, 2 ** 14)), Fr(65504))
    ulp = _ulp16(lo)
    n = int(lo // ulp)
    while ((n + 1) * ulp) ** 2 <= x:           # largest multiple of ulp whose square is <= x
        n += 1
    while n > 0 and (n * ulp) ** 2 > x:
        n -= 1
    mid = (n + Fr(1, 2)) * ulp
    if mid * mid < x or (mid * mid == x and n % 2 == 1):
        n += 1
    return min(max(n * ulp, Fr(1, 2 ** 14)), Fr(65504))


def _exact_state_error(X, w, b):
    """Squared error per entry of the dual-axis quantizer at width b, in exact rational arithmetic: the row
    factors from binary16(sqrt(m / w)), every candidate scale binary16(gamma c0), the codes of each candidate
    found by trying every code in [-qmax, qmax], the candidate with the smallest impact-weighted error (first
    on ties).  X is a list of rows of Fractions, w a list of Fractions."""
    dk, dv = len(X), len(X[0])
    qm = 2 ** (b - 1) - 1
    r = []
    for i in range(dk):
        m = max(abs(x) for x in X[i])
        r.append(Fr(1) if m == 0 else _f16_sqrt_exact(m / w[i]))
    err = [[Fr(0)] * dv for _ in range(dk)]
    for j in range(dv):
        c0 = max(abs(X[i][j]) / (r[i] * qm) for i in range(dk))
        if c0 == 0:
            continue
        best = None
        for g in GRID4_EXACT:
            c = _f16_exact(g * c0)
            e = [min((X[i][j] - r[i] * c * q for q in range(-qm, qm + 1)), key=abs) for i in range(dk)]
            F = sum(w[i] * e[i] * e[i] for i in range(dk))
            if best is None or F < best[0]:
                best = (F, e)
        for i in range(dk):
            err[i][j] = best[1][i] ** 2
    return err


def test_distortion_worked_example_2x2():
    """Hand-worked 2x2 state, one calibration snapshot, w = (1, 1/4), grid {1, 7/8, 3/4, 5/8}.

    X = [[4, 1], [9/4, -3/4]].  Row factors r = sqrt(m / w): r0 = sqrt(4 / 1) = 2, r1 = sqrt((9/4) / (1/4)) = 3
    (binary16-exact).  t = X / r = [[2, 1/2], [3/4, -1/4]].
    Width 2 (qmax 1): c0 = (2, 1/2).
      column 0, t = (2, 3/4):
        c = 2:    z = (1, 3/8)   Q = (1, 0)  X^ = (4, 0)       err = (0, 9/4)     F = 81/64
        c = 7/4:  z = (8/7, 3/7) Q = (1, 0)  X^ = (7/2, 0)     err = (1/2, 9/4)   F = 97/64
        c = 3/2:  z = (4/3, 1/2) Q = (1, 0)  (the tie rounds to even)  err = (1, 9/4)  F = 145/64
        c = 5/4:  z = (8/5, 3/5) Q = (1, 1)  X^ = (5/2, 15/4)  err = (3/2, -3/2)  F = 45/16
        -> c = 2, squared errors (0, 81/16)
      column 1, t = (1/2, -1/4):
        c = 1/2:  z = (1, -1/2)    Q = (1, 0)   err = (0, -3/4)      F = 9/64
        c = 7/16: z = (8/7, -4/7)  Q = (1, -1)  X^ = (7/8, -21/16)  err = (1/8, 9/16)  F = 97/1024
        c = 3/8:  z = (4/3, -2/3)  Q = (1, -1)  err = (1/4, 3/8)     F = 100/1024
        c = 5/16: z = (8/5, -4/5)  Q = (1, -1)  err = (3/8, 3/16)    F = 153/1024
        -> c = 7/16, squared errors (1/64, 81/256)
      D_row = (1/64, 81/16 + 81/256) = (1/64, 1377/256);  D_head = 1381/256.
      (Weighting the distortion by w would give D_head = 1/64 + 1377/1024 = 1393/1024.)
    Width 4 (qmax 7): c0 = (2/7, 1/14); binary16(2/7) = 1170 * 2^-12 = 585/2048, binary16(1/14) = 585/8192,
      binary16(7/8 * 2/7) = 1/4; both columns keep gamma = 1 (F = 431665/2^24 against 1/4, and
      23981/2^23 against 1/64), codes [[7, 7], [3, -4]]:
      column 0 errors (4 - 2 * 7 * 585/2048, 9/4 - 3 * 3 * 585/2048) = (1/1024, -3/2048);
      D_row = (17/2^24, 239805/2^21), D_head = 1918457/2^24.
    Widths 6 and 8 (qmax 31, 127): values from the exact brute force below, D_head = 6272657/2^30 and
      92177/2^28, D_row = (17/2^30, 49005/2^23) and (17/2^28, 45/2^17).
    """
    X = np.array([[[4.0, 1.0], [2.25, -0.75]]])
    w = np.array([1.0, 0.25])
    expect_head = {2: Fr(1381, 256), 4: Fr(1918457, 2 ** 24), 6: Fr(6272657, 2 ** 30), 8: Fr(92177, 2 ** 28)}
    expect_row = {2: (Fr(1, 64), Fr(1377, 256)), 4: (Fr(17, 2 ** 24), Fr(239805, 2 ** 21)),
                  6: (Fr(17, 2 ** 30), Fr(49005, 2 ** 23)), 8: (Fr(17, 2 ** 28), Fr(45, 2 ** 17))}
    widths = (2, 4, 6, 8)
    Dh = planner.head_distortion(X, w, widths, GRID4, "head")
    Dr = planner.head_distortion(X, w, widths, GRID4, "row")
    for k, b in enumerate(widths):
        assert Dh[0, k] == pytest.approx(float(expect_head[b]), rel=1e-12), b
        assert Dr[:, k] == pytest.approx([float(v) for v in expect_row[b]], rel=1e-12, abs=1e-300), b
    # the exact brute force reproduces the hand-worked values
    Xf = [[Fr(4), Fr(1)], [Fr(9, 4), Fr(-3, 4)]]
    for b in widths:
        e = _exact_state_error(Xf, [Fr(1), Fr(1, 4)], b)
        assert sum(map(sum, e)) == expect_head[b]
        assert (sum(e[0]), sum(e[1])) == expect_row[b]


def _dyadic_state(seed, n, dk, dv, den=16, span=48):
    g = np.random.default_rng(seed)
    return g.integers(-span, span + 1, size=(n, dk, dv)) / den


@pytest.mark.parametrize("seed", [0, 1])
def test_distortion_equals_exact_brute_force_4x4(seed):
    """Two 4x4 calibration snapshots (dyadic entries, a zero column in one of them), w non-uniform: D_u(b) at
    widths 2, 4, 6 and 8 for head and row units equals the mean over the snapshots of the exact squared errors
    of the brute-force quantizer."""
    S = _dyadic_state(40 + seed, 2, 4, 4)
    S[1, :, 2] = 0.0
    w = np.array([1.0, 0.25, 2.0, 0.5625])
    widths = (2, 4, 6, 8)
    Dh = planner.head_distortion(S, w, widths, GRID4, "head")
    Dr = planner.head_distortion(S, w, widths, GRID4, "row")
    wf = [Fr(x) for x in w.tolist()]
    for k, b in enumerate(widths):
        per_row = [Fr(0)] * 4
        for s in range(2):
            Xf = [[Fr(x) for x in row] for row in S[s].tolist()]
            e = _exact_state_error(Xf, wf, b)
            for i in range(4):
                per_row[i] += sum(e[i]) / 2
        assert Dh[0, k] == pytest.approx(float(sum(per_row)), rel=1e-12), b
        assert Dr[:, k] == pytest.approx([float(v) for v in per_row], rel=1e-12, abs=1e-300), b
    assert np.all(np.diff(Dh[0]) < 0)


def test_calibration_snapshot_three_tokens():
    """Three tokens from the zero state, beta = 1/2, k = (1, 0), (0, 1), (3/5, 4/5), v = (2, 4), (4, 2), (1, 1).

    GDN, alpha = 1/2:
      token 1: X = (1/2) k v^T                                      = [[1, 2], [0, 0]]
      token 2: D X = [[1/2, 1], [0, 0]], k^T D X = (0, 0), e = (4, 2) -> [[1/2, 1], [2, 1]]
      token 3: D X = [[1/4, 1/2], [1, 1/2]], k^T D X = (0.95, 0.7), e = (0.05, 0.3)
               X = D X + (1/2) k e^T                                 = [[0.265, 0.59], [1.02, 0.62]]
    KDA, alpha = (1/2, 1): tokens 1-2 as above (row 1 is still zero after token 1), then
      token 3: D X = [[1/4, 1/2], [2, 1]], k^T D X = (1.75, 1.1), e = (-0.75, -0.1)
               X = [[0.025, 0.47], [1.7, 0.96]]
    (Dropping the last token leaves [[1/2, 1], [2, 1]]; restarting from zero at every token gives
    (1/2) k3 v3^T = [[0.3, 0.3], [0.4, 0.4]].)"""
    k = np.array([[[1.0, 0.0], [0.0, 1.0], [0.6, 0.8]]])
    v = np.array([[[2.0, 4.0], [4.0, 2.0], [1.0, 1.0]]])
    q = np.ones_like(k)
    beta = np.full((1, 3), 0.5)
    gdn = planner.calib_snapshots(q, k, v, beta, 0.5)
    assert gdn.shape == (1, 2, 2)
    assert np.allclose(gdn[0], [[0.265, 0.59], [1.02, 0.62]], rtol=0, atol=1e-14)
    kda = planner.calib_snapshots(q, k, v, beta, np.array([0.5, 1.0]))
    assert np.allclose(kda[0], [[0.025, 0.47], [1.7, 0.96]], rtol=0, atol=1e-14)
    # two segments are independent: the second segment's state does not see the first's tokens
    both = planner.calib_snapshots(np.concatenate([q, q]), np.concatenate([k, k[:, ::-1]]),
                                   np.concatenate([v, v]), np.concatenate([beta, beta]), 0.5)
    assert np.allclose(both[0], gdn[0], rtol=0, atol=1e-14)
    assert not np.allclose(both[1], gdn[0])
