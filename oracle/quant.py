"""Key-row-aware dual-axis quantizer and dequantizer (oracle; test infrastructure).

Sources
-------
* hyper.ai summary, 方法 (Method), the paragraph on Key-Row-Aware Dual-Axis
  Fitting: the updated state is stored as row factor x column factor x a
  low-bit integer; each key row's factor uses its current magnitude and its
  impact on the readout with square-root scaling; given the row factors, the
  column scales are fitted by minimising the impact-weighted reconstruction
  error; every scaled entry then goes to the nearest representable level at
  its unit's precision.  The first paragraph of the same section fixes the
  quantizer as symmetric and uniform.
* rcap.io post, decode-step pseudocode: after the update, the row factors are
  the square root of each row's magnitude over the square root of its impact
  score, the column scales come from an impact-weighted least-squares fit given
  those row factors, the codes are the state divided by the product of the two
  scales and rounded at each unit's width, and the next step reconstructs the
  state from codes, row factors, column scales and the binary16 pivots.  In
  this module's notation: r_i = binary16(sqrt(m_i / w_i)), then the weighted
  grid fit for c_j, then Q_ij = clamp(rint(X_ij / (r_i c_j))).
* hyper.ai summary, 方法, the Lifetime-Aware Bit Allocation paragraph: the
  riskiest units are kept in FP16 as sparse pivots.

Readings taken where the pages are open
---------------------------------------
* row magnitude = the row's absolute maximum of the float state X.
* row factor r_i = sqrt(m_i / w_i), w_i the calibrated row-impact score.
* fit weight = w_i (the expected squared weighting factor of the row, which is
  what the impact score is defined as); the column fit minimises
  F_j(c) = sum_i w_i (X_ij - r_i c Q_ij(c))^2 over a fixed candidate grid
  c = gamma * c0_j with c0_j = max_i |X_ij| / (r_i qmax_i), gamma in the grid;
  exact ties go to the earliest candidate.
* codes are symmetric: Q in [-qmax, qmax], qmax = 2^(b-1) - 1, round half to
  even, then clamp.
* row factors and column scales are stored as binary16, clamped to
  [2^-14, 65504] before rounding, and the codes are computed with the stored
  values.  A zero row gets r = 1; a column whose non-pivot entries are all zero
  gets c = 1 and zero codes.
* pivot rows are stored as binary16 values of X (saturating) and take no part
  in the row factors, the column base or the fit.

Second quantizer, for the ablations (rcap.io post, the paragraph on the
ablation: temporal allocation alone, i.e. the allocation and pivots with a
plain quantizer instead of the dual-axis fit): symmetric per-row absmax,
r_i = binary16(m_i / qmax_i), every column scale 1, the same rounding and
clamp.  Reading: "plain" is the per-row absmax scale of the uniform baseline,
with the scale stored in binary16 like the dual-axis factors.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .numerics import FP16_MAX, FP16_MIN_NORMAL, fp16_round, fp32_round


@dataclass
class RowPlan:
    """Per-row quantization plan for a batch of states (canonical row order).

    bits  int   [N, d_k]  code width of each key row (ignored on pivot rows)
    pivot bool  [N, d_k]  row kept as binary16 values
    w     float [N, d_k]  row-impact score
    """
    bits: np.ndarray
    pivot: np.ndarray
    w: np.ndarray

    @property
    def qmax(self) -> np.ndarray:
        return (2.0 ** (np.asarray(self.bits, np.float64) - 1.0)) - 1.0


@dataclass
class Packed:
    """A quantized state batch.

    Q [N, d_k, d_v] int64 codes (0 on pivot rows); r [N, d_k] row factors
    (binary16 values; 1 on pivot rows); c [N, d_v] column scales (binary16
    values); V [N, d_k, d_v] binary16 values on pivot rows, 0 elsewhere.
    """
    Q: np.ndarray
    r: np.ndarray
    c: np.ndarray
    V: np.ndarray


def _scale_round(x, scale_fp16: bool):
    x = np.clip(x, FP16_MIN_NORMAL, FP16_MAX)
    return fp16_round(x) if scale_fp16 else x


def dequantize(P: Packed, rows: RowPlan) -> np.ndarray:
    """S_ij = r_i c_j Q_ij on code rows; the binary16 value on pivot rows."""
    S = P.r[:, :, None] * P.c[:, None, :] * P.Q
    return np.where(np.asarray(rows.pivot)[:, :, None], P.V, S)


def row_factors(X, rows: RowPlan, scale_fp16: bool = True):
    """Row absmax m_i and factor r_i = sqrt(m_i / w_i).  Returns (r_pre, r_stored)."""
    m = np.max(np.abs(X), axis=2)
    r_pre = np.sqrt(m / np.asarray(rows.w, np.float64))
    r = _scale_round(r_pre, scale_fp16)
    r = np.where(m > 0, r, 1.0)
    r = np.where(rows.pivot, 1.0, r)
    return r_pre, r


def column_base(X, rows: RowPlan, r):
    """c0_j = max over non-pivot rows of |X_ij| / (r_i qmax_i)."""
    ratio = np.abs(X) / (r[:, :, None] * rows.qmax[:, :, None])
    ratio = np.where(np.asarray(rows.pivot)[:, :, None], 0.0, ratio)
    return np.max(ratio, axis=1)


def candidate_scales(c0, grid, scale_fp16: bool = True):
    """Stored candidate scales [G, N, d_v]: round(clamp(gamma_g * c0))."""
    return np.stack([_scale_round(g * c0, scale_fp16) for g in grid])


def codes_for(X, rows: RowPlan, r, c):
    """Codes for given stored scales: clamp(rint(X / (r c))).  Returns (Q, z) with z the pre-rounding value."""
    z = X / (r[:, :, None] * c[:, None, :])
    qm = rows.qmax[:, :, None]
    Q = np.clip(np.rint(z), -qm, qm)
    Q = np.where(np.asarray(rows.pivot)[:, :, None], 0.0, Q)
    return Q, z


def fit_objective(X, rows: RowPlan, r, c, Q):
    """F_j = sum over non-pivot rows of w_i (X_ij - r_i c_j Q_ij)^2  -> [N, d_v]."""
    err = X - r[:, :, None] * c[:, None, :] * Q
    term = np.asarray(rows.w, np.float64)[:, :, None] * err * err
    term = np.where(np.asarray(rows.pivot)[:, :, None], 0.0, term)
    return np.sum(term, axis=1)


@dataclass
class QuantDiag:
    """Intermediate values kept for the tie-aware comparison of another implementation."""
    r_pre: np.ndarray     # [N, d_k] sqrt(m / w) before binary16 rounding
    c0: np.ndarray        # [N, d_v]
    cands: np.ndarray     # [G, N, d_v] stored candidate scales
    F: np.ndarray         # [G, N, d_v] objective of each candidate
    g: np.ndarray         # [N, d_v] chosen candidate index (-1 for an all-zero column)
    z: np.ndarray         # [N, d_k, d_v] pre-rounding code values with the chosen scales


MODES = ("dual_axis", "row_absmax")


def row_absmax_factors(X, rows: RowPlan, scale_fp16: bool = True):
    """Per-row absmax factors r_i = m_i / qmax_i.  Returns (r_pre, r_stored); zero and pivot rows get 1."""
    m = np.max(np.abs(X), axis=2)
    r_pre = m / rows.qmax
    r = _scale_round(r_pre, scale_fp16)
    r = np.where(m > 0, r, 1.0)
    r = np.where(rows.pivot, 1.0, r)
    return r_pre, r


def _quantize_row_absmax(X, rows: RowPlan, scale_fp16: bool, diag: bool):
    N, d_k, d_v = X.shape
    r_pre, r = row_absmax_factors(X, rows, scale_fp16)
    c = np.ones((N, d_v))
    Q, z = codes_for(X, rows, r, c)
    piv = np.asarray(rows.pivot)[:, :, None]
    V = np.where(piv, fp16_round(X) if scale_fp16 else X, 0.0)
    P = Packed(Q=Q.astype(np.int64), r=r, c=c, V=V)
    if not diag:
        return P
    F = fit_objective(X, rows, r, c, Q)[None]
    return P, QuantDiag(r_pre=r_pre, c0=c, cands=c[None], F=F, g=np.zeros((N, d_v), np.int64), z=z)


def quantize(X, rows: RowPlan, grid, scale_fp16: bool = True, diag: bool = False, mode: str = "dual_axis"):
    """Quantization of float states X [N, d_k, d_v] (dual-axis fit, or per-row absmax when
    mode == "row_absmax", which ignores the grid).  Returns Packed (and QuantDiag)."""
    X = np.asarray(X, dtype=np.float64)
    if mode == "row_absmax":
        return _quantize_row_absmax(X, rows, scale_fp16, diag)
    if mode != "dual_axis":
        raise ValueError(f"unknown quantizer {mode!r}")
    N, d_k, d_v = X.shape
    r_pre, r = row_factors(X, rows, scale_fp16)
    c0 = column_base(X, rows, r)
    cands = candidate_scales(c0, grid, scale_fp16)
    F = np.empty((len(grid), N, d_v))
    Qs = []
    for g in range(len(grid)):
        Qg, _ = codes_for(X, rows, r, cands[g])
        F[g] = fit_objective(X, rows, r, cands[g], Qg)
        Qs.append(Qg)
    best = np.zeros((N, d_v), dtype=np.int64)
    for g in range(1, len(grid)):           # strict improvement only: ties keep the earlier candidate
        better = F[g] < F[best, np.arange(N)[:, None], np.arange(d_v)[None, :]]
        best = np.where(better, g, best)
    zero_col = c0 == 0
    c = np.take_along_axis(cands, best[None], axis=0)[0]
    c = np.where(zero_col, 1.0, c)
    Q = np.take_along_axis(np.stack(Qs), best[None, :, None, :].repeat(d_k, axis=2), axis=0)[0]
    Q = np.where(zero_col[:, None, :], 0.0, Q)
    piv = np.asarray(rows.pivot)[:, :, None]
    V = np.where(piv, fp16_round(X) if scale_fp16 else X, 0.0)
    P = Packed(Q=Q.astype(np.int64), r=r, c=c, V=V)
    if not diag:
        return P
    _, z = codes_for(X, rows, r, c)
    g_out = np.where(zero_col, -1, best)
    return P, QuantDiag(r_pre=r_pre, c0=c0, cands=cands, F=F, g=g_out, z=z)


# ----------------------------------------------------------------------------
# Uniform INT8 per-row comparator (the baseline the pages compare against).

def int8_row_quantize(X):
    """Symmetric per-row INT8: s_i = max_j |X_ij| / 127 stored as binary32, Q = clamp(rint(X / s_i)).

    A zero row gets s = 1.  Returns (Q int64 [N, d_k, d_v], s float64 [N, d_k]).
    """
    X = np.asarray(X, dtype=np.float64)
    m = np.max(np.abs(X), axis=2)
    s = fp32_round(m / 127.0)
    s = np.where(m > 0, s, 1.0)
    Q = np.clip(np.rint(X / s[:, :, None]), -127, 127)
    return Q.astype(np.int64), s


def int8_row_dequantize(Q, s):
    return s[:, :, None] * Q
