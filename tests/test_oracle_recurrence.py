"""Pins for the oracle's gated delta update and readout (CPU only).

Each check is a property fixed by the mathematics of the update
X = D S + beta k (v^T - k^T D S), y = X^T q (rcap.io post, decode-step
pseudocode), not a retyping of the oracle's own expression.
"""
import numpy as np
import pytest

from oracle.recurrence import delta_update, run_unquantized


def _unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _rand(seed, N=5, dk=8, dv=6):
    g = np.random.default_rng(seed)
    S = g.standard_normal((N, dk, dv))
    q = _unit(g.standard_normal((N, dk)))
    k = _unit(g.standard_normal((N, dk)))
    v = g.standard_normal((N, dv))
    return g, S, q, k, v


def test_write_property_unit_gate():
    # alpha = 1, beta = 1, |k| = 1: the updated state maps k exactly onto v.
    g, S, q, k, v = _rand(1)
    X, _ = delta_update(S, q, k, v, np.ones(5), np.ones(5))
    assert np.max(np.abs(np.einsum("nij,ni->nj", X, k) - v)) < 1e-12


def test_matrix_form_of_update():
    # The same update as a linear map on S: X = (I - beta k k^T) D S + beta k v^T.
    g, S, q, k, v = _rand(2)
    alpha = g.uniform(0.5, 1.0, size=(5, 8))
    beta = g.uniform(0.1, 0.9, size=5)
    X, _ = delta_update(S, q, k, v, alpha, beta)
    for n in range(5):
        P = np.eye(8) - beta[n] * np.outer(k[n], k[n])
        ref = P @ np.diag(alpha[n]) @ S[n] + beta[n] * np.outer(k[n], v[n])
        assert np.allclose(X[n], ref, rtol=0, atol=1e-12)


def test_readout_is_transposed_state_times_query():
    # y = X^T q: a basis query e_i reads key row i of the updated state.
    g, S, q, k, v = _rand(3)
    beta = np.full(5, 0.3)
    alpha = np.full(5, 0.9)
    for i in range(8):
        e = np.zeros((5, 8))
        e[:, i] = 1.0
        X, y = delta_update(S, e, k, v, alpha, beta)
        assert np.allclose(y, X[:, i, :], atol=1e-14)


def test_gate_scales_key_rows_kda():
    # beta = 0: the step is the transition alone, D = diag(alpha) scales key rows (not value columns).
    g, S, q, k, v = _rand(4)
    alpha = g.uniform(0.1, 1.0, size=(5, 8))
    X, _ = delta_update(S, q, k, v, alpha, np.zeros(5))
    assert np.array_equal(X, alpha[:, :, None] * S)


def test_gdn_equals_kda_with_equal_rows():
    g, S, q, k, v = _rand(5)
    a = g.uniform(0.5, 1.0, size=5)
    b = g.uniform(0.0, 1.0, size=5)
    X1, y1 = delta_update(S, q, k, v, a, b)
    X2, y2 = delta_update(S, q, k, v, np.repeat(a[:, None], 8, 1), b)
    assert np.array_equal(X1, X2) and np.array_equal(y1, y2)


def test_zero_write_strength_is_pure_decay_over_steps():
    # beta = 0 over T steps: S_T = (prod_t D_t) S_0.
    g, S, q, k, v = _rand(6)
    T = 7
    alpha = g.uniform(0.8, 1.0, size=(T, 5, 8))
    qs = _unit(g.standard_normal((T, 5, 8)))
    ks = _unit(g.standard_normal((T, 5, 8)))
    vs = g.standard_normal((T, 5, 6))
    ST, _ = run_unquantized(S, qs, ks, vs, alpha, np.zeros((T, 5)))
    assert np.allclose(ST, np.prod(alpha, axis=0)[:, :, None] * S, rtol=1e-13, atol=0)


def test_orthonormal_keys_are_all_recalled():
    # alpha = beta = 1 and orthonormal keys written in sequence: every key recalls its value.
    g = np.random.default_rng(7)
    dk, dv, T = 8, 5, 6
    Qm, _ = np.linalg.qr(g.standard_normal((dk, dk)))
    ks = Qm[:, :T].T[:, None, :]                 # [T, 1, dk]
    vs = g.standard_normal((T, 1, dv))
    S0 = g.standard_normal((1, dk, dv))
    ST, _ = run_unquantized(S0, ks, ks, vs, np.ones((T, 1)), np.ones((T, 1)))
    for t in range(T):
        assert np.allclose(ST[0].T @ ks[t, 0], vs[t, 0], atol=1e-12)


def test_first_step_from_zero_is_rank_one():
    # From S = 0 the update is beta k v^T and the readout beta (k.q) v.
    g, S, q, k, v = _rand(8)
    beta = g.uniform(0, 1, 5)
    X, y = delta_update(np.zeros_like(S), q, k, v, g.uniform(0.5, 1, 5), beta)
    assert np.allclose(X, beta[:, None, None] * k[:, :, None] * v[:, None, :], atol=1e-15)
    assert np.allclose(y, (beta * np.sum(k * q, 1))[:, None] * v, atol=1e-15)
