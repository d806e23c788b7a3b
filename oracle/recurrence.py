"""Gated delta-rule update and readout (oracle; test infrastructure).

Follows the rcap.io post's decode-step pseudocode: the reconstructed state
S_prev is multiplied by the transition D_t, the delta correction
beta_t * k_t (v_t^T - k_t^T D_t S_prev) is added, and the readout
y_t = X^T q_t is taken from the updated float state before requantization.
The same post's "Temporal" paragraph and the hyper.ai summary (方法 / Method)
give the gate: one retention value per head for Gated DeltaNet (GDN) and one
per key row for Kimi Delta Attention (KDA), so D = alpha * I or diag(alpha).

Reading taken: the readout carries no 1/sqrt(d_k) factor, output gate or norm
(those belong to the surrounding model, not to the state step).
"""
from __future__ import annotations

import numpy as np


def gate_rows(alpha, d_k: int) -> np.ndarray:
    """Per-key-row retention for a batch: alpha [N] (GDN) or [N, d_k] (KDA) -> [N, d_k]."""
    a = np.asarray(alpha, dtype=np.float64)
    if a.ndim == 1:
        return np.repeat(a[:, None], d_k, axis=1)
    return a


def delta_update(S, q, k, v, alpha, beta):
    """One unquantized step for a batch of states.

    S [N, d_k, d_v]; q, k [N, d_k]; v [N, d_v]; alpha [N] or [N, d_k]; beta [N].
    Returns (X [N, d_k, d_v], y [N, d_v]) with
        X = D S + beta k (v^T - k^T D S),   y = X^T q.
    """
    S = np.asarray(S, dtype=np.float64)
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    beta = np.asarray(beta, dtype=np.float64)
    d = gate_rows(alpha, S.shape[1])
    DS = d[:, :, None] * S                          # transition D_t S_prev
    kDS = np.einsum("ni,nij->nj", k, DS)            # k^T D S  (a row over value columns)
    X = DS + beta[:, None, None] * k[:, :, None] * (v - kDS)[:, None, :]
    y = np.einsum("nij,ni->nj", X, q)               # readout from the float state
    return X, y


def run_unquantized(S0, q, k, v, alpha, beta):
    """T unquantized steps.  q, k [T, N, d_k]; v [T, N, d_v]; alpha [T, N(, d_k)]; beta [T, N].

    Returns (S_T, y [T, N, d_v]).
    """
    S = np.asarray(S0, dtype=np.float64)
    ys = []
    for t in range(q.shape[0]):
        S, y = delta_update(S, q[t], k[t], v[t], alpha[t], beta[t])
        ys.append(y)
    return S, np.stack(ys)
