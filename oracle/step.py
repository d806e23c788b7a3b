"""One packed decode step (oracle; test infrastructure).

rcap.io post, decode-step pseudocode, taken in its order: unpack the stored
state, apply the gated delta update, emit the readout before requantizing,
recompute row factors and column scales, and quantize back at each unit's
width.  The hyper.ai summary (方法 / Method, last paragraph) describes the same
sequence: chunked state reconstruction, delta update and readout, then the
dual-axis fit and packed write-back that keep the state compressed between
tokens.
"""
from __future__ import annotations

import numpy as np

from . import quant
from .recurrence import delta_update


def packed_step(P: quant.Packed, rows: quant.RowPlan, q, k, v, alpha, beta, grid,
                scale_fp16: bool = True, diag: bool = False, mode: str = "dual_axis"):
    """Returns (Packed', y [N, d_v], X [N, d_k, d_v]) and the quantizer diagnostics if diag;
    mode selects the quantizer (quant.MODES)."""
    S = quant.dequantize(P, rows)
    X, y = delta_update(S, q, k, v, alpha, beta)
    out = quant.quantize(X, rows, grid, scale_fp16=scale_fp16, diag=diag, mode=mode)
    if diag:
        P2, D = out
        return P2, y, X, D
    return out, y, X


def run_packed(P: quant.Packed, rows: quant.RowPlan, q, k, v, alpha, beta, grid):
    """T free-running packed steps.  Inputs carry a leading step axis.  Returns (P_T, y [T, N, d_v])."""
    ys = []
    for t in range(q.shape[0]):
        P, y, _ = packed_step(P, rows, q[t], k[t], v[t], alpha[t], beta[t], grid)
        ys.append(y)
    return P, np.stack(ys)


def int8_step(Q, s, q, k, v, alpha, beta):
    """One step of the uniform INT8 per-row comparator.  Returns (Q', s', y, X)."""
    S = quant.int8_row_dequantize(Q, s)
    X, y = delta_update(S, q, k, v, alpha, beta)
    Q2, s2 = quant.int8_row_quantize(X)
    return Q2, s2, y, X
