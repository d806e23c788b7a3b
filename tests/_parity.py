"""Test helpers: canonical packed format <-> oracle Packed, and the tie-aware comparison.

The comparison accepts a different result from the library only where the
oracle's own float64 value sits at a rounding boundary (a "tie" within the
library's float32 arithmetic):
  * a binary16 row factor or column scale one step away from the oracle's, when
    the oracle's pre-rounding value lies within `scale_tie` (relative) of the
    boundary between the two;
  * a binary16 pivot value that is the rounding of some real within the forward
    error bound of a float32 evaluation of the update (`x_err`, from
    `step_error_bound`; without it, `pivot_tie` times the row's largest magnitude);
  * a column-scale candidate other than the oracle's choice, when its objective
    (evaluated by the oracle) is within `fit_tie` (relative) of the minimum;
  * a code one level away from the oracle's code for the library's scales, when
    the oracle's pre-rounding value lies within `code_tie` of a half-integer, on
    at most `max_code_ties` of the code entries.
Everything else must match exactly.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from oracle import quant
from oracle.numerics import fp16_bits, fp16_from_bits, fp16_round


def to_canonical(P: quant.Packed, rows: quant.RowPlan):
    piv = np.asarray(rows.pivot)
    codes = P.Q.astype(np.int64)
    vbits = fp16_bits(P.V).astype(np.int64)
    vbits = np.where(vbits >= 32768, vbits - 65536, vbits)
    codes = np.where(piv[:, :, None], vbits, codes).astype(np.int16)
    r = fp16_bits(P.r).view(np.int16)
    c = fp16_bits(P.c).view(np.int16)
    return codes, r, c


def from_canonical(codes, r, c, rows: quant.RowPlan) -> quant.Packed:
    piv = np.asarray(rows.pivot)
    codes = np.asarray(codes)
    V = fp16_from_bits(codes.view(np.uint16))
    Q = np.where(piv[:, :, None], 0, codes.astype(np.int64))
    V = np.where(piv[:, :, None], V, 0.0)
    return quant.Packed(Q=Q, r=fp16_from_bits(np.asarray(r).view(np.uint16)),
                        c=fp16_from_bits(np.asarray(c).view(np.uint16)), V=V)


def step_error_bound(P0: quant.Packed, rows: quant.RowPlan, k, v, alpha, beta, bias=0.0):
    """Per-entry bound on |X_float32 - X| for X = D S + beta k (v^T - k^T D S).

    Whatever the summation order, a float32 evaluation that adds n terms errs by at most
    gamma_n = n u / (1 - n u) times the sum of the terms' magnitudes (u = 2^-24).  The sum
    counted here covers every term the library adds: alpha_i S_ij, and beta k_i times
    |v_j| + sum_m |alpha_m k_m| (|S_mj| + bias r_m c_j).  The library sums signed codes
    (bias 0); an evaluation that summed codes stored with an offset of `bias` levels would
    carry the extra term.  n is d_k plus a margin for the few products and sums around the
    column reduction.
    """
    S = quant.dequantize(P0, rows)
    N, dk, dv = S.shape
    a = np.asarray(alpha, np.float64)
    a = a[:, None] if a.ndim == 1 else a                      # [N, dk]
    k = np.asarray(k, np.float64)
    b = np.asarray(beta, np.float64)[:, None]
    code = (~np.asarray(rows.pivot)).astype(np.float64)       # [N, dk]
    off = bias * code[:, :, None] * P0.r[:, :, None] * P0.c[:, None, :]
    col = np.abs(np.asarray(v, np.float64)) + np.einsum('nm,nmj->nj', np.abs(a * k), np.abs(S) + off)
    M = np.abs(a[:, :, None] * S) + np.abs(b * k)[:, :, None] * col[:, None, :]
    n = dk + 16
    u = 2.0 ** -24
    return (n * u / (1 - n * u)) * M


def _spacing16(x):
    """Gap from |x| (a binary16 value) to its binary16 neighbour above; at the largest finite value, 65504,
    the gap below (32), since above it lies infinity."""
    h = np.abs(np.asarray(x, np.float64)).astype(np.float16)
    top = h == np.float16(65504)
    up = np.spacing(np.where(top, np.float16(0), h))
    return np.where(top, 32.0, up.astype(np.float64))


def _fp16_neighbours_tie(pre, got, want, tol):
    """got != want are adjacent binary16 values and pre is within tol (relative) of their midpoint."""
    adjacent = np.abs(got - want) <= np.maximum(_spacing16(got), _spacing16(want)) * 1.0001
    mid = 0.5 * (got + want)
    return adjacent & (np.abs(pre - mid) <= tol * np.abs(pre) + 1e-300)


@dataclass
class Report:
    n_states: int = 0
    y_rel: float = 0.0
    r_ties: int = 0
    c_ties: int = 0
    fit_ties: int = 0
    pivot_ties: int = 0
    code_ties: int = 0
    code_entries: int = 0
    xhat_rel_clean: float = 0.0
    xhat_rel_all: float = 0.0
    failures: list = field(default_factory=list)

    def ok(self):
        return not self.failures


def compare_step(X, y_ref, rows: quant.RowPlan, grid, y_gpu, P_gpu: quant.Packed, P_ref: quant.Packed,
                 y_tol=1e-4, scale_tie=1e-5, fit_tie=1e-5, code_tie=1e-3, max_code_ties=1e-3,
                 xhat_tol=1e-4, pivot_tie=2e-6, x_err=None, mode="dual_axis") -> Report:
    """X, y_ref: the oracle's float state and readout for the step; P_ref its packed result;
    x_err: optional per-entry bound on the library's float32 error in X (step_error_bound);
    mode: the plan's quantizer (quant.MODES)."""
    R = Report(n_states=X.shape[0])
    piv = np.asarray(rows.pivot)
    code_row = ~piv
    # readout
    R.y_rel = float(np.linalg.norm(y_gpu - y_ref) / max(np.linalg.norm(y_ref), 1e-300))
    if not R.y_rel <= y_tol:
        R.failures.append(f"y relative L2 {R.y_rel:.3e} > {y_tol}")
    # row factors
    r_pre, r_ref = quant.row_factors(X, rows) if mode == "dual_axis" else quant.row_absmax_factors(X, rows)
    r_pre_c = np.clip(r_pre, 2.0 ** -14, 65504)
    bad_r = P_gpu.r != r_ref
    tie_r = bad_r & code_row & _fp16_neighbours_tie(r_pre_c, P_gpu.r, r_ref, scale_tie)
    R.r_ties = int(tie_r.sum())
    if np.any(bad_r & ~tie_r):
        i = np.argwhere(bad_r & ~tie_r)[0]
        R.failures.append(f"row factor mismatch at {tuple(i)}: gpu {P_gpu.r[tuple(i)]} oracle {r_ref[tuple(i)]}")
    if mode == "row_absmax":
        # no column fit: every column scale stays 1
        if np.any(P_gpu.c != 1.0):
            n, j = np.argwhere(P_gpu.c != 1.0)[0]
            R.failures.append(f"column scale at state {n} col {j} is {P_gpu.c[n, j]}, not 1")
    else:
        # column scales: a candidate of the grid built on the library's row factors
        c0 = quant.column_base(X, rows, P_gpu.r)
        cands = quant.candidate_scales(c0, grid)
        F = np.stack([quant.fit_objective(X, rows, P_gpu.r, cands[g], quant.codes_for(X, rows, P_gpu.r, cands[g])[0])
                      for g in range(len(grid))])
        Fmin = F.min(axis=0)
        pre = np.stack([np.clip(g * c0, 2.0 ** -14, 65504) for g in grid])
        match = np.zeros((len(grid),) + c0.shape, bool)
        for g in range(len(grid)):
            exact = P_gpu.c == cands[g]
            tie = _fp16_neighbours_tie(pre[g], P_gpu.c, cands[g], scale_tie)
            match[g] = exact | tie
            R.c_ties += int((tie & ~exact).sum())
        near_opt = F <= Fmin[None] * (1 + fit_tie) + 1e-300
        ok_col = np.any(match & near_opt, axis=0) | ((c0 == 0) & (P_gpu.c == 1.0))
        best = np.argmin(F, axis=0)
        chose_other = ~np.take_along_axis(match, best[None], 0)[0] & ok_col & (c0 > 0)
        R.fit_ties = int(chose_other.sum())
        if not np.all(ok_col):
            n, j = np.argwhere(~ok_col)[0]
            R.failures.append(f"column scale at state {n} col {j}: gpu {P_gpu.c[n, j]} candidates "
                              f"{cands[:, n, j]} F {F[:, n, j]}")
    # codes for the library's scales
    Qo, z = quant.codes_for(X, rows, P_gpu.r, P_gpu.c)
    dQ = (P_gpu.Q - Qo) * code_row[:, :, None]
    frac = np.abs(np.abs(z - np.floor(z)) - 0.5)
    qm = rows.qmax[:, :, None]
    near = (frac <= code_tie) & (np.abs(z) <= qm + 0.5 + code_tie)
    R.code_entries = int(code_row.sum() * X.shape[2])
    bad_q = dQ != 0
    R.code_ties = int((bad_q & near).sum())
    if np.any(np.abs(dQ) > 1) or np.any(bad_q & ~near):
        idx = np.argwhere((np.abs(dQ) > 1) | (bad_q & ~near))[0]
        R.failures.append(f"code mismatch at {tuple(idx)}: gpu {P_gpu.Q[tuple(idx)]} oracle {Qo[tuple(idx)]} "
                          f"z {z[tuple(idx)]}")
    if R.code_entries and R.code_ties > max_code_ties * R.code_entries:
        R.failures.append(f"{R.code_ties} code ties exceed {max_code_ties:.1e} of {R.code_entries}")
    # pivot rows
    if np.any(piv):
        want = fp16_round(X)
        bad_v = (P_gpu.V != want) & piv[:, :, None]
        if x_err is None:
            # a pivot entry is a float32 sum of terms of the row's magnitude: its absolute error
            # scales with the row maximum, not with the entry (small entries come from cancellation)
            x_err = pivot_tie * np.max(np.abs(X), axis=2, keepdims=True)
        d = x_err + scale_tie * np.abs(X)
        # binary16 rounding is monotone: the roundings of [X - d, X + d] are exactly the values between
        # the roundings of its ends
        tie_v = bad_v & (P_gpu.V >= fp16_round(X - d)) & (P_gpu.V <= fp16_round(X + d))
        R.pivot_ties = int(tie_v.sum())
        if np.any(bad_v & ~tie_v):
            idx = np.argwhere(bad_v & ~tie_v)[0]
            R.failures.append(f"pivot value mismatch at {tuple(idx)}: gpu {P_gpu.V[tuple(idx)]} want {want[tuple(idx)]}")
    # dequantized state
    Xg = quant.dequantize(P_gpu, rows)
    Xr = quant.dequantize(P_ref, rows)
    denom = max(np.linalg.norm(Xr), 1e-300)
    R.xhat_rel_all = float(np.linalg.norm(Xg - Xr) / denom)
    clean = np.ones(X.shape[0], bool)
    clean &= ~np.any(bad_r, axis=1)
    clean &= ~np.any(P_gpu.c != P_ref.c, axis=1)
    if np.any(clean):
        num = np.linalg.norm((Xg - Xr)[clean] * ~(bad_q[clean]))
        R.xhat_rel_clean = float(num / max(np.linalg.norm(Xr[clean]), 1e-300))
        if not R.xhat_rel_clean <= xhat_tol:
            R.failures.append(f"dequantized state relative L2 {R.xhat_rel_clean:.3e} > {xhat_tol}")
    return R
