"""Offline planner: lifetime-aware bit allocation, FP16 pivots, impact scores (oracle; test infrastructure).

Sources
-------
* hyper.ai summary, 方法 (Method), Lifetime-Aware Bit Allocation paragraph: for
  every state unit, estimate the reconstruction distortion at each candidate
  width and the mean log retention; the error retention after j updates is
  approximated by an exponential, which gives a lifetime weight standing for
  how long an error persists; under an average-bit budget, pick each unit's
  width from the candidate set to minimise the lifetime-weighted distortion;
  the riskiest units stay in FP16 as sparse pivots.
* Same section, the spatial paragraph: the row-impact score is the expectation
  over calibration tokens of the squared weighting factor that the transition
  and the query give each key row's error in the next readout.
* rcap.io post, "Temporal" paragraph: a unit is a head (Qwen / GDN) or a key
  row (KDA); the post's limitations list calls the lifetime weight a gate-only
  approximation.  Same post: allocation and pivots run offline on calibration
  text (32 segments); here seeded synthetic traces stand in for it.

Readings taken
--------------
* mean log retention l_u = mean over the unit's gate values of ln(alpha); the
  synthetic gates are constant per unit, so l_u = ln(alpha_u) (rows of a head
  unit are averaged).
* lifetime weight L_u = sum_{j>=0} exp(j l_u) = 1 / (1 - exp(l_u)), with
  l_u clamped to <= -2^-20.
* distortion D_u(b) = mean over calibration snapshots (the state at the end of
  each segment, unquantized recurrence from zero) of the summed squared error
  of the unit's entries when the whole state is quantized by the dual-axis
  quantizer with every row at width b and no pivots (the plan's quantizer:
  dual-axis, or per-row absmax for the ablation of the fit).
* pivots: ceil(ppm * U / 1e6) units ranked by L desc, then D(smallest width)
  desc, then unit index asc.  Pivots sit outside the budget.
* allocation: exact dynamic programme over the non-pivot units in index order,
  minimising sum_u L_u D_u(b_u) subject to sum_u b_u <= budget * U'.  Ties:
  fewer excess bits win, and within a unit the narrower width wins.
* impact score w_i = mean over calibration tokens of a_i^2 with
  a = D (I - beta k k^T) q, the factor by which row i of an error in the state
  before the token reaches that token's readout.
"""
from __future__ import annotations

from dataclasses import dataclass
from math import gcd
from typing import Callable

import numpy as np

from . import quant
from .recurrence import delta_update

HEAD, ROW = "head", "row"


def lifetime_weight(lbar):
    """L = 1 / (1 - exp(l)) with l clamped to <= -2^-20 (the sum of exp(j l) over j >= 0)."""
    l = np.minimum(np.asarray(lbar, np.float64), -(2.0 ** -20))
    return 1.0 / (1.0 - np.exp(l))


def unit_log_retention(alpha_unit, form: str, unit: str, d_k: int) -> np.ndarray:
    """Mean log retention per allocation unit, flattened in (layer, head[, row]) order."""
    la = np.log(np.asarray(alpha_unit, np.float64))
    if form == "gdn":                      # [L, H]
        if unit == HEAD:
            return la.reshape(-1)
        return np.repeat(la[:, :, None], d_k, axis=2).reshape(-1)
    if unit == HEAD:                       # [L, H, d_k]
        return la.mean(axis=2).reshape(-1)
    return la.reshape(-1)


def calib_snapshots(q, k, v, beta, alpha_head) -> np.ndarray:
    """Unquantized recurrence from zero over each segment; returns the segment-final states [S, d_k, d_v].

    q, k [S, T, d_k]; v [S, T, d_v]; beta [S, T]; alpha_head scalar (GDN) or [d_k] (KDA).
    """
    n_seg, T, d_k = q.shape
    d_v = v.shape[2]
    a = np.asarray(alpha_head, np.float64)
    alpha = np.full(n_seg, float(a)) if a.ndim == 0 else np.broadcast_to(a, (n_seg, d_k))
    S = np.zeros((n_seg, d_k, d_v))
    for t in range(T):
        S, _ = delta_update(S, q[:, t], k[:, t], v[:, t], alpha, beta[:, t])
    return S


def head_distortion(snap, w_head, widths, grid, unit: str, mode: str = "dual_axis") -> np.ndarray:
    """D(b) for the units of one head: [1, nb] (head unit) or [d_k, nb] (row units), with the plan's quantizer."""
    n_seg, d_k, _ = snap.shape
    out = []
    for b in widths:
        rows = quant.RowPlan(bits=np.full((n_seg, d_k), b), pivot=np.zeros((n_seg, d_k), bool),
                             w=np.broadcast_to(np.asarray(w_head, np.float64), (n_seg, d_k)))
        P = quant.quantize(snap, rows, grid, mode=mode)
        err = snap - quant.dequantize(P, rows)
        e2 = np.sum(err * err, axis=2)            # [S, d_k] per-row squared error
        out.append(e2.sum(axis=1).mean()[None] if unit == HEAD else e2.mean(axis=0))
    return np.stack(out, axis=-1)


def impact_from_traces(q, k, beta, alpha_head) -> np.ndarray:
    """w_i = mean over tokens of (alpha_i (q_i - beta k_i k.q))^2  -> [d_k]."""
    q = np.asarray(q, np.float64).reshape(-1, q.shape[-1])
    k = np.asarray(k, np.float64).reshape(-1, k.shape[-1])
    b = np.asarray(beta, np.float64).reshape(-1)
    kq = np.sum(k * q, axis=1)
    a = np.asarray(alpha_head, np.float64) * (q - b[:, None] * k * kq[:, None])
    return np.mean(a * a, axis=0)


def pivot_count(pivot_ppm: int, n_units: int) -> int:
    return (pivot_ppm * n_units + 999_999) // 1_000_000


def select_pivots(L, D_min, count: int) -> np.ndarray:
    """Indices of the `count` riskiest units: L desc, then D(smallest width) desc, then index asc."""
    idx = np.arange(len(L))
    order = np.lexsort((idx, -np.asarray(D_min), -np.asarray(L)))
    return np.sort(order[:count])


def allocate(cost, widths, budget_milli: int) -> np.ndarray:
    """Exact DP.  cost [U', nb] (widths ascending).  Returns the chosen width index per unit."""
    cost = np.asarray(cost, np.float64)
    U, nb = cost.shape
    w = list(widths)
    if U == 0:
        return np.zeros(0, np.int64)
    step = 0
    for b in w[1:]:
        step = gcd(step, b - w[0])
    step = max(step, 1)
    ex = [(b - w[0]) // step for b in w]
    num = budget_milli * U - 1000 * w[0] * U
    if num < 0:
        raise ValueError("budget below the narrowest width")
    E = min(num // (1000 * step), ex[-1] * U)
    INF = np.inf
    best = np.full(E + 1, INF)
    best[0] = 0.0
    choice = np.zeros((U, E + 1), np.int8)
    for u in range(U):
        nxt = np.full(E + 1, INF)
        ch = np.zeros(E + 1, np.int8)
        for j in range(nb):
            e = ex[j]
            cand = np.full(E + 1, INF)
            if e <= E:
                cand[e:] = best[: E + 1 - e] + cost[u, j]
            better = cand < nxt
            nxt = np.where(better, cand, nxt)
            ch = np.where(better, j, ch)
        best = nxt
        choice[u] = ch
    x = int(np.argmin(best))               # the first minimum: fewest excess bits among equal cost
    out = np.zeros(U, np.int64)
    for u in range(U - 1, -1, -1):
        j = int(choice[u, x])
        out[u] = j
        x -= ex[j]
    return out


@dataclass
class Plan:
    """Planner output (canonical order).

    lbar, L [U]; D [U, nb]; pivot_units [P] (unit indices); unit_bits [U]
    (16 for a pivot unit); bits, pivot, w [L, H, d_k] per key row.
    """
    lbar: np.ndarray
    L: np.ndarray
    D: np.ndarray
    pivot_units: np.ndarray
    unit_bits: np.ndarray
    bits: np.ndarray
    pivot: np.ndarray
    w: np.ndarray


def make_plan(form: str, unit: str, n_layers: int, n_heads: int, d_k: int, d_v: int,
              widths, budget_milli: int, pivot_ppm: int, grid, alpha_unit,
              traces: Callable, impact=None, mode: str = "dual_axis") -> Plan:
    """Full planner.  traces(l, h) -> (q, k, v, beta) arrays of shape [S, T, ...]; mode = the quantizer
    whose distortion the allocation weighs (quant.MODES)."""
    widths = tuple(sorted(widths))
    lbar = unit_log_retention(alpha_unit, form, unit, d_k)
    L = lifetime_weight(lbar)
    per = 1 if unit == HEAD else d_k
    U = n_layers * n_heads * per
    D = np.zeros((U, len(widths)))
    w_all = np.zeros((n_layers, n_heads, d_k))
    for l in range(n_layers):
        for h in range(n_heads):
            q, k, v, beta = traces(l, h)
            a_h = alpha_unit[l, h]
            if impact is None:
                w_all[l, h] = impact_from_traces(q, k, beta, a_h)
            else:
                w_all[l, h] = impact[l, h]
            snap = calib_snapshots(q, k, v, beta, a_h)
            u0 = (l * n_heads + h) * per
            D[u0:u0 + per] = head_distortion(snap, w_all[l, h], widths, grid, unit, mode)
    piv = select_pivots(L, D[:, 0], pivot_count(pivot_ppm, U))
    is_piv = np.zeros(U, bool)
    is_piv[piv] = True
    rest = np.nonzero(~is_piv)[0]
    choice = allocate(L[rest, None] * D[rest], widths, budget_milli)
    unit_bits = np.full(U, 16, np.int64)
    unit_bits[rest] = np.asarray(widths)[choice]
    if unit == HEAD:
        bits = np.repeat(unit_bits.reshape(n_layers, n_heads)[:, :, None], d_k, axis=2)
        pivot = np.repeat(is_piv.reshape(n_layers, n_heads)[:, :, None], d_k, axis=2)
    else:
        bits = unit_bits.reshape(n_layers, n_heads, d_k)
        pivot = is_piv.reshape(n_layers, n_heads, d_k)
    bits = np.where(pivot, 16, bits)
    return Plan(lbar=lbar, L=L, D=D, pivot_units=piv, unit_bits=unit_bits, bits=bits,
                pivot=pivot, w=w_all)
