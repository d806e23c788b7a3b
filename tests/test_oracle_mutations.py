"""Planted mistakes in the oracle must be caught by its pins (CPU only).

Each case swaps one oracle function for a plausibly wrong variant (a dropped
term, a wrong sign, a transposed operand, a wrong formula) and runs a pin that
must then fail.  The oracle itself is never modified on disk.
"""
import numpy as np
import pytest

import oracle.planner as planner
import oracle.quant as quant
import oracle.recurrence as recurrence
import test_oracle_planner as tp
import test_oracle_quant as tq
import test_oracle_recurrence as tr

_orig_update = recurrence.delta_update


def _update_sign_flip(S, q, k, v, alpha, beta):
    d = recurrence.gate_rows(alpha, S.shape[1])
    DS = d[:, :, None] * S
    kDS = np.einsum("ni,nij->nj", k, DS)
    X = DS - beta[:, None, None] * k[:, :, None] * (v - kDS)[:, None, :]
    return X, np.einsum("nij,ni->nj", X, q)


def _update_gate_after_delta(S, q, k, v, alpha, beta):
    d = recurrence.gate_rows(alpha, S.shape[1])
    kS = np.einsum("ni,nij->nj", k, S)
    X = d[:, :, None] * (S + beta[:, None, None] * k[:, :, None] * (v - kS)[:, None, :])
    return X, np.einsum("nij,ni->nj", X, q)


def _update_readout_before_update(S, q, k, v, alpha, beta):
    X, _ = _orig_update(S, q, k, v, alpha, beta)
    d = recurrence.gate_rows(alpha, S.shape[1])
    return X, np.einsum("nij,ni->nj", d[:, :, None] * S, q)


def _row_factors_times_w(X, rows, scale_fp16=True):
    m = np.max(np.abs(X), axis=2)
    r_pre = np.sqrt(m * rows.w)
    r = quant._scale_round(r_pre, scale_fp16)
    return r_pre, np.where(rows.pivot, 1.0, np.where(m > 0, r, 1.0))


def _objective_unweighted(X, rows, r, c, Q):
    err = X - r[:, :, None] * c[:, None, :] * Q
    return np.sum(np.where(rows.pivot[:, :, None], 0.0, err * err), axis=1)


def _codes_truncated(X, rows, r, c):
    z = X / (r[:, :, None] * c[:, None, :])
    qm = rows.qmax[:, :, None]
    return np.where(rows.pivot[:, :, None], 0.0, np.clip(np.trunc(z), -qm, qm)), z


def _column_base_without_qmax(X, rows, r):
    ratio = np.abs(X) / r[:, :, None]
    return np.max(np.where(rows.pivot[:, :, None], 0.0, ratio), axis=1)


def _lifetime_linear(lbar):
    return 1.0 / (1.0 - np.minimum(np.asarray(lbar, np.float64), -(2.0 ** -20)))


def _impact_without_gate(q, k, beta, alpha_head):
    q = np.asarray(q, np.float64).reshape(-1, q.shape[-1])
    k = np.asarray(k, np.float64).reshape(-1, k.shape[-1])
    b = np.asarray(beta, np.float64).reshape(-1)
    a = q - b[:, None] * k * np.sum(k * q, 1)[:, None]
    return np.mean(a * a, axis=0)


def _row_absmax_power_of_two(X, rows, scale_fp16=True):
    m = np.max(np.abs(X), axis=2)
    r_pre = m / (2.0 ** (np.asarray(rows.bits, np.float64) - 1.0))
    r = quant._scale_round(r_pre, scale_fp16)
    return r_pre, np.where(rows.pivot, 1.0, np.where(m > 0, r, 1.0))


def _row_absmax_half_range(X, rows, scale_fp16=True):
    m = np.max(np.abs(X), axis=2)
    r_pre = 2.0 * m / rows.qmax
    r = quant._scale_round(r_pre, scale_fp16)
    return r_pre, np.where(rows.pivot, 1.0, np.where(m > 0, r, 1.0))


def _allocate_widest_first(cost, widths, budget_milli):
    return np.full(cost.shape[0], len(widths) - 1)


_orig_head_distortion = planner.head_distortion


def _distortion_weighted(snap, w_head, widths, grid, unit, mode="dual_axis"):
    """Squared errors weighted by the impact score (the fit's objective instead of the plain reconstruction)."""
    n_seg, d_k, _ = snap.shape
    out = []
    for b in widths:
        rows = quant.RowPlan(bits=np.full((n_seg, d_k), b), pivot=np.zeros((n_seg, d_k), bool),
                             w=np.broadcast_to(np.asarray(w_head, np.float64), (n_seg, d_k)))
        err = snap - quant.dequantize(quant.quantize(snap, rows, grid, mode=mode), rows)
        e2 = np.sum(err * err, axis=2) * np.asarray(w_head, np.float64)[None, :]
        out.append(e2.sum(axis=1).mean()[None] if unit == "head" else e2.mean(axis=0))
    return np.stack(out, axis=-1)


def _distortion_first_row_pivot(snap, w_head, widths, grid, unit, mode="dual_axis"):
    """The first key row treated as a pivot (excluded from the quantizer) while distortion is measured."""
    n_seg, d_k, _ = snap.shape
    piv = np.zeros((n_seg, d_k), bool)
    piv[:, 0] = True
    out = []
    for b in widths:
        rows = quant.RowPlan(bits=np.full((n_seg, d_k), b), pivot=piv,
                             w=np.broadcast_to(np.asarray(w_head, np.float64), (n_seg, d_k)))
        err = snap - quant.dequantize(quant.quantize(snap, rows, grid, mode=mode), rows)
        e2 = np.sum(err * err, axis=2)
        out.append(e2.sum(axis=1).mean()[None] if unit == "head" else e2.mean(axis=0))
    return np.stack(out, axis=-1)


def _distortion_next_width(snap, w_head, widths, grid, unit, mode="dual_axis"):
    """Each column measured at the next wider candidate width (an index off by one)."""
    ws = list(widths)
    shifted = [ws[min(i + 1, len(ws) - 1)] for i in range(len(ws))]
    return _orig_head_distortion(snap, w_head, shifted, grid, unit, mode)


def _snapshots_drop_last_token(q, k, v, beta, alpha_head):
    return _orig_snapshots(q[:, :-1], k[:, :-1], v[:, :-1], beta[:, :-1], alpha_head)


def _snapshots_reset_per_token(q, k, v, beta, alpha_head):
    """Each token starts again from the zero state (the recurrence is not carried)."""
    return _orig_snapshots(q[:, -1:], k[:, -1:], v[:, -1:], beta[:, -1:], alpha_head)


_orig_snapshots = planner.calib_snapshots


CASES = [
    ("update sign", [(recurrence, "delta_update", _update_sign_flip), (tr, "delta_update", _update_sign_flip)],
     tr.test_write_property_unit_gate),
    ("gate after delta", [(recurrence, "delta_update", _update_gate_after_delta),
                          (tr, "delta_update", _update_gate_after_delta)], tr.test_matrix_form_of_update),
    ("readout of old state", [(recurrence, "delta_update", _update_readout_before_update),
                              (tr, "delta_update", _update_readout_before_update)],
     tr.test_readout_is_transposed_state_times_query),
    ("row factor sqrt(m w)", [(quant, "row_factors", _row_factors_times_w)],
     tq.test_impact_and_magnitude_invariances),
    ("unweighted fit", [(quant, "fit_objective", _objective_unweighted)], tq.test_worked_example_fit_values),
    ("truncating codes", [(quant, "codes_for", _codes_truncated)],
     lambda: tq.test_column_fit_equals_brute_force(4, 4, 4)),
    ("column base without qmax", [(quant, "column_base", _column_base_without_qmax)],
     tq.test_rank_one_closed_form),
    ("row absmax over 2^(b-1)", [(quant, "row_absmax_factors", _row_absmax_power_of_two)],
     tq.test_row_absmax_half_step_bound_zero_rows_and_pivots),
    ("row absmax at half range", [(quant, "row_absmax_factors", _row_absmax_half_range)],
     tq.test_row_absmax_half_step_bound_zero_rows_and_pivots),
    ("linear lifetime", [(planner, "lifetime_weight", _lifetime_linear)],
     tp.test_lifetime_closed_form_for_constant_gate),
    ("impact without gate", [(planner, "impact_from_traces", _impact_without_gate)],
     tp.test_impact_score_is_the_readout_sensitivity),
    ("allocation ignores budget", [(planner, "allocate", _allocate_widest_first)],
     lambda: tp.test_allocation_equals_brute_force(1, 8, 6000)),
    ("distortion weighted by impact", [(planner, "head_distortion", _distortion_weighted)],
     tp.test_distortion_worked_example_2x2),
    ("distortion with a pivot row excluded", [(planner, "head_distortion", _distortion_first_row_pivot)],
     tp.test_distortion_worked_example_2x2),
    ("distortion at the next width", [(planner, "head_distortion", _distortion_next_width)],
     lambda: tp.test_distortion_equals_exact_brute_force_4x4(0)),
    ("snapshot drops the last token", [(planner, "calib_snapshots", _snapshots_drop_last_token)],
     tp.test_calibration_snapshot_three_tokens),
    ("snapshot restarts per token", [(planner, "calib_snapshots", _snapshots_reset_per_token)],
     tp.test_calibration_snapshot_three_tokens),
]


@pytest.mark.parametrize("name,patches,pin", CASES, ids=[c[0] for c in CASES])
def test_planted_mistake_is_caught(monkeypatch, name, patches, pin):
    pin()                                      # the pin passes on the real oracle
    for mod, attr, fn in patches:
        monkeypatch.setattr(mod, attr, fn)
    with pytest.raises(AssertionError):
        pin()
