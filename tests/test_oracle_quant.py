"""Pins for the oracle's binary16 rounding and dual-axis quantizer (CPU only)."""
import itertools

import numpy as np
import pytest

from oracle import quant
from oracle.numerics import fp16_round

GRID4 = (1.0, 0.875, 0.75, 0.625)


# ---------------------------------------------------------------- binary16

def test_fp16_matches_library_conversion():
    g = np.random.default_rng(0)
    x = np.concatenate([g.standard_normal(20000) * s for s in (1e-6, 1e-3, 1, 1e3, 3e4)])
    ref = np.clip(x, -65504, 65504).astype(np.float16).astype(np.float64)
    assert np.array_equal(fp16_round(x), ref)


def test_fp16_ties_to_even_and_saturation():
    one = 1.0
    ulp = 2.0 ** -10
    assert fp16_round(one + ulp / 2) == one                       # tie -> even (1.0)
    assert fp16_round(one + 3 * ulp / 2) == one + 2 * ulp         # tie -> even (1 + 2 ulp)
    assert fp16_round(one + ulp / 2 + 2.0 ** -40) == one + ulp    # just above the tie -> up
    assert fp16_round(65519.0) == 65504.0 and fp16_round(1e9) == 65504.0
    assert fp16_round(-1e9) == -65504.0
    assert fp16_round(2.0 ** -24 * 0.75) == 2.0 ** -24            # subnormal spacing


# ---------------------------------------------------------------- helpers

def _rows(N, dk, bits, w=None, pivot=None, seed=0):
    g = np.random.default_rng(seed)
    if w is None:
        w = g.uniform(0.5, 2.0, size=(N, dk))
    b = np.broadcast_to(np.asarray(bits), (N, dk)).copy()
    p = np.zeros((N, dk), bool) if pivot is None else np.broadcast_to(pivot, (N, dk)).copy()
    return quant.RowPlan(bits=b, pivot=p, w=np.asarray(w, np.float64))


def _state(seed, N=4, dk=16, dv=12, scale=1.0):
    return np.random.default_rng(seed).standard_normal((N, dk, dv)) * scale


# ---------------------------------------------------------------- properties

@pytest.mark.parametrize("bits", [2, 3, 4, 6, 8])
def test_half_step_bound_and_clipping(bits):
    X = _state(1)
    rows = _rows(4, 16, bits, seed=1)
    P, D = quant.quantize(X, rows, GRID4, diag=True)
    step = P.r[:, :, None] * P.c[:, None, :]
    err = np.abs(X - quant.dequantize(P, rows))
    qmax = 2 ** (bits - 1) - 1
    assert np.all(np.abs(P.Q) <= qmax)
    clipped = np.abs(D.z) > qmax + 0.5
    assert np.all(err[~clipped] <= step[~clipped] / 2 * (1 + 1e-12))
    assert np.allclose(err[clipped], np.abs(X[clipped]) - qmax * step[clipped], rtol=1e-12)


def test_unit_grid_never_clips():
    X = _state(2)
    rows = _rows(4, 16, 4, seed=2)
    P, D = quant.quantize(X, rows, (1.0,), diag=True)
    step = P.r[:, :, None] * P.c[:, None, :]
    err = np.abs(X - quant.dequantize(P, rows))
    assert np.all(err <= step / 2 * (1 + 1e-12))


def _brute_force_fit(X, rows, r, grid):
    """For each column: every candidate scale and every code vector; returns best F per candidate."""
    N, dk, dv = X.shape
    qmax = rows.qmax
    c0 = quant.column_base(X, rows, r)
    out = np.zeros((len(grid), N, dv))
    for n in range(N):
        levels = [np.arange(-qmax[n, i], qmax[n, i] + 1) for i in range(dk)]
        allQ = np.array(list(itertools.product(*levels)))          # [M, dk]
        for j in range(dv):
            for g, gam in enumerate(grid):
                c = fp16_round(np.clip(gam * c0[n, j], 2 ** -14, 65504))
                err = X[n, :, j][None, :] - r[n][None, :] * c * allQ
                F = np.sum(rows.w[n][None, :] * err * err, axis=1)
                out[g, n, j] = F.min()
    return out


@pytest.mark.parametrize("dk,dv,bits", [(2, 2, 6), (4, 4, 4), (4, 4, 3), (4, 4, 2)])
def test_column_fit_equals_brute_force(dk, dv, bits):
    X = _state(3, N=3, dk=dk, dv=dv)
    rows = _rows(3, dk, bits, seed=3)
    P, D = quant.quantize(X, rows, GRID4, diag=True)
    brute = _brute_force_fit(X, rows, P.r, GRID4)
    # nearest rounding plus clamp is each candidate's optimum ...
    assert np.allclose(D.F, brute, rtol=1e-12, atol=1e-300)
    # ... and the chosen candidate is the brute-force argmin (first on ties)
    assert np.array_equal(D.g, np.argmin(brute, axis=0))
    best = np.min(brute, axis=0)
    F_chosen = quant.fit_objective(X, rows, P.r, P.c, P.Q.astype(float))
    assert np.allclose(F_chosen, best, rtol=1e-12)


def test_rank_one_closed_form():
    # X = beta k v^T with exact (unrounded) scales: z_ij = sign(k_i v_j) qmax sqrt(|k_i| w_i / max_l |k_l| w_l)
    g = np.random.default_rng(4)
    dk, dv, qmax = 16, 16, 31
    k = g.standard_normal(dk)
    k /= np.linalg.norm(k)
    v = g.choice([-1.0, 1.0], dv) * g.uniform(0.5, 2.0, dv)   # keeps every scale inside the clamp range
    beta = 0.37
    w = g.uniform(0.5, 2.0, dk)
    X = (beta * np.outer(k, v))[None]
    rows = quant.RowPlan(bits=np.full((1, dk), 6), pivot=np.zeros((1, dk), bool), w=w[None])
    P, D = quant.quantize(X, rows, GRID4, scale_fp16=False, diag=True)
    ref = np.sign(np.outer(k, v)) * qmax * np.sqrt(np.abs(k) * w / np.max(np.abs(k) * w))[:, None]
    # z with the chosen scale is the closed form divided by the chosen gamma
    gam = np.asarray(GRID4)[D.g[0]]
    assert np.allclose(D.z[0] * gam[None, :], ref, rtol=1e-12, atol=1e-12)
    # every column has the same |z| pattern, so every column picks the same candidate
    assert len(set(D.g[0].tolist())) == 1


def test_impact_and_magnitude_invariances():
    X = _state(5, N=3, dk=10, dv=9)
    rows = _rows(3, 10, 6, seed=5)
    P = quant.quantize(X, rows, GRID4)
    rows4 = quant.RowPlan(bits=rows.bits, pivot=rows.pivot, w=4 * rows.w)
    P4 = quant.quantize(X, rows4, GRID4)
    assert np.array_equal(P4.r, P.r / 2) and np.array_equal(P4.c, P.c * 2)
    assert np.array_equal(P4.Q, P.Q)
    PX = quant.quantize(4 * X, rows, GRID4)
    assert np.array_equal(PX.r, P.r * 2) and np.array_equal(PX.c, P.c * 2)
    assert np.array_equal(PX.Q, P.Q)


def test_permutation_equivariance():
    X = _state(6, N=2, dk=12, dv=10)
    g = np.random.default_rng(6)
    bits = g.choice([4, 6, 8], size=(2, 12))
    rows = quant.RowPlan(bits=bits, pivot=np.zeros((2, 12), bool), w=g.uniform(0.5, 2, (2, 12)))
    P = quant.quantize(X, rows, GRID4)
    pr = g.permutation(12)
    pc = g.permutation(10)
    rows_p = quant.RowPlan(bits=bits[:, pr], pivot=rows.pivot[:, pr], w=rows.w[:, pr])
    Pp = quant.quantize(X[:, pr][:, :, pc], rows_p, GRID4)
    assert np.array_equal(Pp.Q, P.Q[:, pr][:, :, pc])
    assert np.array_equal(Pp.r, P.r[:, pr]) and np.array_equal(Pp.c, P.c[:, pc])


def test_pivot_rows_are_fp16_and_excluded():
    X = _state(7, N=2, dk=8, dv=6)
    piv = np.zeros((2, 8), bool)
    piv[:, [1, 5]] = True
    rows = _rows(2, 8, 4, pivot=piv, seed=7)
    X_big = X.copy()
    X_big[:, [1, 5]] *= 1e4                       # pivot rows cannot influence the code rows
    P = quant.quantize(X, rows, GRID4)
    Pb = quant.quantize(X_big, rows, GRID4)
    assert np.array_equal(P.Q, Pb.Q) and np.array_equal(P.c, Pb.c)
    assert np.array_equal(P.r, Pb.r)
    assert np.array_equal(Pb.V[:, [1, 5]], fp16_round(X_big[:, [1, 5]]))
    assert np.all(Pb.Q[:, [1, 5]] == 0) and np.all(Pb.r[:, [1, 5]] == 1.0)
    S = quant.dequantize(Pb, rows)
    assert np.array_equal(S[:, [1, 5]], fp16_round(X_big[:, [1, 5]]))


def test_zero_rows_and_columns():
    X = _state(8, N=1, dk=6, dv=5)
    X[0, 2, :] = 0
    X[0, :, 3] = 0
    rows = _rows(1, 6, 6, seed=8)
    P = quant.quantize(X, rows, GRID4)
    assert P.r[0, 2] == 1.0 and P.c[0, 3] == 1.0
    assert np.all(P.Q[0, 2] == 0) and np.all(P.Q[0, :, 3] == 0)
    Z = quant.quantize(np.zeros((1, 6, 5)), rows, GRID4)
    assert np.all(Z.Q == 0) and np.all(Z.r == 1) and np.all(Z.c == 1)


def test_worked_example_fit_values():
    """Hand-worked 2x1 column, 4-bit (qmax 7), grid {1, 7/8, 3/4, 5/8}.

    w = (1, 4), X = (49, 9/4).  Row factors: r0 = sqrt(49/1) = 7, r1 = sqrt((9/4)/4) = 3/4,
    both exact in binary16.  t = X / r = (7, 3).  c0 = max(7/7, 3/7) = 1.
    Candidates: c = 1, 7/8, 3/4, 5/8 (all exact in binary16).
      c = 1:   z = (7, 3)        Q = (7, 3)  err_X = (0, 0)            -> F = 0
    so c = 1 wins.  Now w = (1, 1/4): r1 = sqrt(9) = 3, t = (7, 3/4), c0 = 1.
      c = 1:   z = (7, 0.75)     Q = (7, 1)  err_X = (0, 3*(0.75-1)=-0.75)   F = (1/4)(0.5625) = 0.140625
      c = 7/8: z = (8, 6/7)      Q = (7, 1)  err_X = (49-42.875=6.125, 3*(0.75-0.875)=-0.375)
                                             F = 37.515625 + (1/4)(0.140625) = 37.55078125
      c = 3/4: z = (9.33, 1)     Q = (7, 1)  err_X = (49-36.75=12.25, 0)   F = 150.0625
      c = 5/8: z = (11.2, 1.2)   Q = (7, 1)  err_X = (49-30.625=18.375, 3*(0.75-0.625)=0.375)
                                             F = 337.640625 + 0.03515625 = 337.67578125
    so c = 1 again, with F = 0.140625.  An unweighted objective would give 0.5625 there.
    """
    X = np.array([[[49.0], [2.25]]])
    rows = quant.RowPlan(bits=np.full((1, 2), 4), pivot=np.zeros((1, 2), bool), w=np.array([[1.0, 4.0]]))
    P, D = quant.quantize(X, rows, GRID4, diag=True)
    assert np.array_equal(P.r[0], [7.0, 0.75]) and P.c[0, 0] == 1.0
    assert np.array_equal(P.Q[0, :, 0], [7, 3]) and D.F[0, 0, 0] == 0.0
    rows2 = quant.RowPlan(bits=rows.bits, pivot=rows.pivot, w=np.array([[1.0, 0.25]]))
    P2, D2 = quant.quantize(X, rows2, GRID4, diag=True)
    assert np.array_equal(P2.r[0], [7.0, 3.0])
    assert np.array_equal(D2.F[:, 0, 0], [0.140625, 37.55078125, 150.0625, 337.67578125])
    assert D2.g[0, 0] == 0 and np.array_equal(P2.Q[0, :, 0], [7, 1])


def test_int8_comparator_matches_library_per_channel_quantization():
    torch = pytest.importorskip("torch")
    X = _state(9, N=3, dk=8, dv=64, scale=3.0).astype(np.float32).astype(np.float64)
    Q, s = quant.int8_row_quantize(X)
    diffs = 0
    for n in range(3):
        t = torch.tensor(X[n], dtype=torch.float32)
        qt = torch.quantize_per_channel(t, torch.tensor(s[n]), torch.zeros(8, dtype=torch.long),
                                        axis=0, dtype=torch.qint8)
        ref = np.clip(qt.int_repr().numpy().astype(np.int64), -127, 127)
        assert np.max(np.abs(ref - Q[n])) <= 1          # the library divides in float32
        diffs += int(np.sum(ref != Q[n]))
    assert diffs <= 2


# ---------------------------------------------------------------- per-row absmax quantizer (ablation)

@pytest.mark.parametrize("bits", [2, 3, 4, 6, 8])
def test_row_absmax_matches_library_fake_quantization(bits):
    """Per-row absmax codes = the library's per-channel symmetric quantization with the same
    (binary16-rounded) scales; the library divides in float32, so codes may differ by one
    level where the quotient sits at a half-integer."""
    torch = pytest.importorskip("torch")
    X = _state(21 + bits, N=4, dk=16, dv=48, scale=2.0).astype(np.float32).astype(np.float64)
    rows = _rows(4, 16, bits)
    P = quant.quantize(X, rows, GRID4, mode="row_absmax")
    qm = 2 ** (bits - 1) - 1
    assert np.all(P.c == 1.0)
    diffs = 0
    for n in range(4):
        t = torch.tensor(X[n], dtype=torch.float32)
        ref = torch.fake_quantize_per_channel_affine(t, torch.tensor(P.r[n], dtype=torch.float32),
                                                     torch.zeros(16, dtype=torch.int32), 0, -qm, qm)
        Qref = np.rint(ref.numpy().astype(np.float64) / P.r[n][:, None])
        assert np.max(np.abs(Qref - P.Q[n])) <= 1
        diffs += int(np.sum(Qref != P.Q[n]))
    assert diffs <= 2


def test_row_absmax_half_step_bound_zero_rows_and_pivots():
    X = _state(31, N=3, dk=8, dv=16, scale=4.0)
    X[0, 2] = 0.0
    rows = _rows(3, 8, 6)
    rows.pivot[:, 5] = True
    rows.bits[:, 5] = 16
    P = quant.quantize(X, rows, GRID4, mode="row_absmax")
    Xh = quant.dequantize(P, rows)
    code = ~rows.pivot
    err = np.abs(X - Xh)
    # the scale covers the row without clipping (half-step bound everywhere) and uses the full
    # range: the row's largest entry takes the extreme code
    assert np.all((err <= P.r[:, :, None] / 2 + 1e-12)[code])
    imax = np.argmax(np.abs(X), axis=2)
    top = np.abs(np.take_along_axis(P.Q, imax[:, :, None], axis=2)[:, :, 0])
    live = code & (np.max(np.abs(X), axis=2) > 0)
    assert np.all(top[live] == rows.qmax[live])
    assert P.r[0, 2] == 1.0 and np.all(P.Q[0, 2] == 0)
    assert np.all(P.r[:, 5] == 1.0) and np.array_equal(P.V[:, 5], fp16_round(X[:, 5]))
    with pytest.raises(ValueError):
        quant.quantize(X, rows, GRID4, mode="row_max")
