"""Pins for the oracle's packed decode step (CPU only)."""
import numpy as np

from oracle import quant
from oracle.step import int8_step, packed_step, run_packed
from workloads import configs, gen

GRID4 = (1.0, 0.875, 0.75, 0.625)


def _tiny_rows(N, dk, w):
    return quant.RowPlan(bits=np.full((N, dk), 6), pivot=np.zeros((N, dk), bool), w=w)


def test_first_step_from_zero_state_reads_out_exactly():
    # Zero packed state (r = c = 1, Q = 0): X = beta k v^T and the readout, taken before
    # requantization, is exactly beta (k.q) v.
    wl = configs.TINY
    q, k, v, beta = gen.eval_inputs(wl, 1, 1, 1)
    N = wl.n_heads
    q, k, v, beta = q[0, 0, 0], k[0, 0, 0], v[0, 0, 0], beta[0, 0, 0]
    alpha = gen.unit_gates(wl)[0]
    w = gen.impact_scores(wl)[0].astype(np.float64)
    P0 = quant.Packed(Q=np.zeros((N, 16, 16), np.int64), r=np.ones((N, 16)), c=np.ones((N, 16)),
                      V=np.zeros((N, 16, 16)))
    rows = _tiny_rows(N, 16, w)
    P1, y, X = packed_step(P0, rows, q, k, v, alpha, beta, GRID4)
    kq = np.sum(k.astype(np.float64) * q, axis=1)
    assert np.allclose(y, (beta * kq)[:, None] * v, rtol=1e-14, atol=1e-15)
    S1 = quant.dequantize(P1, rows)
    step = P1.r[:, :, None] * P1.c[:, None, :]
    assert np.all(np.abs(S1 - X) <= step / 2 * (1 + 1e-12))


def test_readout_precedes_requantization():
    g = np.random.default_rng(3)
    N, dk, dv = 3, 16, 16
    w = g.uniform(0.5, 2, (N, dk))
    rows = _tiny_rows(N, dk, w)
    P = quant.quantize(g.standard_normal((N, dk, dv)), rows, GRID4)
    q = g.standard_normal((N, dk)); q /= np.linalg.norm(q, axis=1, keepdims=True)
    k = g.standard_normal((N, dk)); k /= np.linalg.norm(k, axis=1, keepdims=True)
    v = g.standard_normal((N, dv))
    P2, y, X = packed_step(P, rows, q, k, v, np.full(N, 0.97), np.full(N, 0.5), GRID4)
    assert np.allclose(y, np.einsum("nij,ni->nj", X, q), rtol=0, atol=1e-13)
    y_req = np.einsum("nij,ni->nj", quant.dequantize(P2, rows), q)
    assert not np.allclose(y, y_req, rtol=0, atol=1e-9)


def test_packed_run_error_shrinks_with_width():
    # Over 64 steps the readout error against the unquantized run falls about 4x per two extra
    # bits (the quantization step halves per bit).
    from oracle.recurrence import run_unquantized
    wl = configs.TINY
    T = 64
    q, k, v, beta = [x[:, 0, 0] for x in gen.eval_inputs(wl, T, 1, 1)]
    alpha = np.broadcast_to(gen.unit_gates(wl)[0], (T, wl.n_heads))
    w = gen.impact_scores(wl)[0].astype(np.float64)
    _, yf = run_unquantized(np.zeros((wl.n_heads, 16, 16)), q, k, v, alpha, beta)
    err = []
    for b in (4, 6, 8):
        rows = quant.RowPlan(bits=np.full((wl.n_heads, 16), b), pivot=np.zeros((wl.n_heads, 16), bool), w=w)
        P0 = quant.quantize(np.zeros((wl.n_heads, 16, 16)), rows, GRID4)
        _, ys = run_packed(P0, rows, q, k, v, alpha, beta, GRID4)
        err.append(np.linalg.norm(ys - yf) / np.linalg.norm(yf))
    assert err[0] > err[1] > err[2]
    assert 2.5 < err[0] / err[1] < 8 and 2.5 < err[1] / err[2] < 8


def test_int8_step_first_step():
    g = np.random.default_rng(5)
    N, dk, dv = 2, 8, 8
    Q = np.zeros((N, dk, dv), np.int64)
    s = np.ones((N, dk))
    q = g.standard_normal((N, dk)); k = g.standard_normal((N, dk)); v = g.standard_normal((N, dv))
    beta = np.array([0.5, 0.25])
    Q2, s2, y, X = int8_step(Q, s, q, k, v, np.array([0.9, 0.8]), beta)
    assert np.allclose(y, (beta * np.sum(k * q, 1))[:, None] * v)
    assert np.all(np.abs(s2[:, :, None] * Q2 - X) <= s2[:, :, None] / 2 * (1 + 1e-12))
