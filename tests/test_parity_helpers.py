"""CPU checks of the GPU tests' comparison helpers (no GPU).

The tie-aware comparison must accept the oracle's own result, reject planted
mistakes, and its float32 error bound for the update must hold for a float32
evaluation of the update done the way the library does it (column sums of the
signed codes), and for one that sums codes stored with an offset and takes the
offset's sum off afterwards when the bound is told the offset.
"""
import numpy as np

from oracle import quant
from oracle.step import packed_step

from _parity import compare_step, step_error_bound


def _case(seed=0, N=6, dk=32, dv=48, kda=True):
    g = np.random.default_rng(seed)
    bits = g.choice([4, 6, 8], size=(N, dk))
    piv = np.zeros((N, dk), bool)
    piv[:, [3, 17]] = True
    bits = np.where(piv, 16, bits)
    rows = quant.RowPlan(bits=bits, pivot=piv, w=g.uniform(0.5, 2.0, (N, dk)))
    S = 2.0 * g.standard_normal((N, dk, dv))
    P = quant.quantize(S, rows, (1.0, 0.875, 0.75, 0.625))
    q = g.standard_normal((N, dk))
    k = g.standard_normal((N, dk))
    q /= np.linalg.norm(q, axis=1, keepdims=True)
    k /= np.linalg.norm(k, axis=1, keepdims=True)
    v = g.standard_normal((N, dv))
    a = 1 / (1 + np.exp(-g.normal(3, 1.5, (N, dk) if kda else N)))
    b = 1 / (1 + np.exp(-g.standard_normal(N)))
    return rows, P, q, k, v, a, b


def _update_float32(P, rows, k, v, a, b, bias):
    """X in float32 arithmetic, column sums over offset codes (Q + bias) as the library forms them."""
    f = np.float32
    N, dk, dv = P.Q.shape
    a2 = np.broadcast_to(a[:, None] if a.ndim == 1 else a, (N, dk)).astype(f)
    X = np.zeros((N, dk, dv), f)
    for n in range(N):
        piv = rows.pivot[n]
        A = np.where(piv, f(0), a2[n] * P.r[n].astype(f)).astype(f)
        Ak = (A * k[n].astype(f)).astype(f)
        ak = np.where(piv, a2[n] * k[n].astype(f), f(0)).astype(f)
        off = np.where(piv, 0, bias).astype(f)
        su = np.zeros(dv, f)
        sp = np.zeros(dv, f)
        for i in range(dk):
            su = (su + Ak[i] * (P.Q[n, i].astype(f) + off[i])).astype(f)
            sp = (sp + ak[i] * P.V[n, i].astype(f)).astype(f)
        kb = f(0)
        for i in range(dk):
            kb = f(kb + f(Ak[i] * off[i]))
        c = P.c[n].astype(f)
        u = (c * (su - kb) + sp).astype(f)
        e = (v[n].astype(f) - u).astype(f)
        for i in range(dk):
            ds = (P.V[n, i].astype(f) * a2[n, i]) if piv[i] else c * (A[i] * P.Q[n, i].astype(f))
            X[n, i] = (ds + f(b[n] * k[n, i]) * e).astype(f)
    return X.astype(np.float64)


def test_error_bound_covers_float32_update():
    for seed, kda in [(0, True), (1, False), (2, True)]:
        rows, P, q, k, v, a, b = _case(seed, kda=kda)
        _, _, X = packed_step(P, rows, q, k, v, a, b, (1.0, 0.875, 0.75, 0.625))
        for off in (0.0, 128.0):
            X32 = _update_float32(P, rows, k, v, a, b, off)
            bound = step_error_bound(P, rows, k, v, a, b, bias=off)
            err = np.abs(X32 - X)
            assert np.all(err <= bound)
            # the bound is a bound, but not a vacuous one: well under the entries' own size
            assert np.median(bound / np.maximum(np.abs(X), 1e-30)) < 1e-3


def test_compare_accepts_oracle_and_rejects_planted_mistakes():
    grid = (1.0, 0.875, 0.75, 0.625)
    rows, P, q, k, v, a, b = _case(3)
    P2, y, X = packed_step(P, rows, q, k, v, a, b, grid)
    xe = step_error_bound(P, rows, k, v, a, b)
    assert compare_step(X, y, rows, grid, y.copy(), P2, P2, x_err=xe).ok()

    def planted(**kw):
        Pg = quant.Packed(Q=P2.Q.copy(), r=P2.r.copy(), c=P2.c.copy(), V=P2.V.copy())
        yg = y.copy()
        if "code" in kw:
            n, i, j = np.argwhere(~rows.pivot[:, :, None] & (np.abs(P2.Q) < 3))[0]
            Pg.Q[n, i, j] += 2
        if "pivot" in kw:
            Pg.V[0, 3, 5] = Pg.V[0, 3, 5] * 1.01 + 0.01
        if "r" in kw:
            Pg.r[1, 0] *= 1.5
        if "c" in kw:
            Pg.c[2, 7] *= 1.3
        if "y" in kw:
            yg *= 1.001
        return compare_step(X, y, rows, grid, yg, Pg, P2, x_err=xe)

    for what in ["code", "pivot", "r", "c", "y"]:
        assert not planted(**{what: True}).ok(), what


def test_compare_in_row_absmax_mode():
    grid = (1.0, 0.875, 0.75, 0.625)
    rows, P, q, k, v, a, b = _case(4)
    P2, y, X = packed_step(P, rows, q, k, v, a, b, grid, mode="row_absmax")
    assert np.all(P2.c == 1.0)
    assert compare_step(X, y, rows, grid, y.copy(), P2, P2, mode="row_absmax").ok()
    bad = quant.Packed(Q=P2.Q, r=P2.r, c=P2.c.copy(), V=P2.V)
    bad.c[0, 3] = 0.875
    assert not compare_step(X, y, rows, grid, y.copy(), bad, P2, mode="row_absmax").ok()
    # the dual-axis comparison rejects a row-absmax result (different row factors)
    assert not compare_step(X, y, rows, grid, y.copy(), P2, P2).ok()


def test_binary16_neighbours_at_the_top_of_the_range():
    """Adjacent binary16 values are accepted as a rounding tie only when the pre-rounding value sits at
    their midpoint; at 65504, whose upper neighbour is infinity, the gap is the one below (32)."""
    from _parity import _fp16_neighbours_tie, _spacing16
    assert _spacing16(np.array([65504.0]))[0] == 32.0
    assert _spacing16(np.array([1.0]))[0] == 2.0 ** -10
    assert _spacing16(np.array([65472.0]))[0] == 32.0
    got, want = np.array([65504.0]), np.array([65472.0])
    assert _fp16_neighbours_tie(np.array([65488.0]), got, want, 1e-5)[0]
    assert not _fp16_neighbours_tie(np.array([65500.0]), got, want, 1e-5)[0]
    # not neighbours: the largest value against one far below it
    assert not _fp16_neighbours_tie(np.array([32768.0]), np.array([65504.0]), np.array([1024.0]), 1.0)[0]
