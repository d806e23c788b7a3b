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
