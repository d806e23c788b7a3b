"""Seeded synthetic inputs for the quantized gated-delta state step.

This module is shared by the oracle side (tests, the CPU baseline) and the GPU
side (tests, the benchmark).  It draws random numbers and nothing else: no step
of the method is computed here.

Two kinds of generators:

* NumPy ``PCG64`` streams keyed by ``SeedSequence([workload id, stream])`` for
  gates, impact scores, decode-step inputs, warm-up tokens, slot maps and ridge
  positions (host side, moderate sizes).
* A counter-based Philox-4x32-10 generator (Salmon, Moraes, Dror and Shaw,
  "Parallel random numbers: as easy as 1, 2, 3", SC'11) for the planner's
  calibration traces.  The C++ planner carries its own implementation of the
  same published generator so that it can draw traces for any (layer, head)
  without receiving them; the two are compared bit for bit in the tests.

Streams: 0 gates, 1 impact scores, 3 warm-up tokens, 4 decode inputs,
5 slot map, 6 ridge positions.  Calibration traces use Philox with key
``calib_seed(workload)``.
"""
from __future__ import annotations

import numpy as np

from .configs import GDN, KDA, Workload

S_GATE, S_IMPACT, S_WARMUP, S_EVAL, S_SLOTS, S_RIDGE = 0, 1, 3, 4, 5, 6


def rng(w: Workload, stream: int, sub: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([w.cid, stream, sub])))


def _sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def unit_gates(w: Workload) -> np.ndarray:
    """Retention gate alpha, constant over steps and requests.

    GDN: one value per (layer, head) -> float32 [L, H].
    KDA: one value per (layer, head, key row) -> float32 [L, H, d_k].
    """
    g = rng(w, S_GATE)
    shape = (w.n_layers, w.n_heads) if w.form == GDN else (w.n_layers, w.n_heads, w.d_k)
    mu = g.normal(w.gate_mu, w.gate_sigma, size=shape)
    return _sigmoid(mu).astype(np.float32)


def impact_scores(w: Workload) -> np.ndarray:
    """Row-impact scores drawn directly, float32 [L, H, d_k]."""
    g = rng(w, S_IMPACT)
    shape = (w.n_layers, w.n_heads, w.d_k)
    kind = w.impact[0]
    if kind == "uniform":
        x = g.uniform(w.impact[1], w.impact[2], size=shape)
    elif kind == "lognormal":
        x = g.lognormal(w.impact[1], w.impact[2], size=shape)
    elif kind == "pareto":
        # classical Pareto with x_m = 1: NumPy's pareto() draws the Lomax form
        x = 1.0 + g.pareto(w.impact[1], size=shape)
    else:
        raise ValueError(kind)
    return x.astype(np.float32)


def _unit_norm(x: np.ndarray) -> np.ndarray:
    n = np.sqrt(np.sum(x.astype(np.float64) ** 2, axis=-1, keepdims=True))
    return (x / n).astype(np.float32)


def token_inputs(g: np.random.Generator, lead: tuple, d_k: int, d_v: int):
    """q, k unit-norm N(0,1) directions; v ~ N(0,1); beta = sigmoid(N(0,1))."""
    q = _unit_norm(g.standard_normal(lead + (d_k,)))
    k = _unit_norm(g.standard_normal(lead + (d_k,)))
    v = g.standard_normal(lead + (d_v,)).astype(np.float32)
    beta = _sigmoid(g.standard_normal(lead)).astype(np.float32)
    return q, k, v, beta


def step_gate(w: Workload, alpha_unit: np.ndarray, n_steps: int, n_layers: int, batch: int,
              layer0: int = 0) -> np.ndarray:
    """Per-step gate arrays [T, n_layers, batch, H] (GDN) or [T, n_layers, batch, H, d_k] (KDA).

    The synthetic gates are constant per unit, so every step and request sees
    the unit's value.
    """
    a = alpha_unit[layer0:layer0 + n_layers]
    if w.form == GDN:
        a = a[None, :, None, :]
        return np.broadcast_to(a, (n_steps, n_layers, batch, w.n_heads)).astype(np.float32)
    a = a[None, :, None, :, :]
    return np.broadcast_to(a, (n_steps, n_layers, batch, w.n_heads, w.d_k)).astype(np.float32)


def eval_inputs(w: Workload, n_steps: int, n_layers: int, batch: int, sub: int = 0):
    """Decode inputs for n_steps steps: q, k [T, nL, B, H, d_k], v [T, nL, B, H, d_v], beta [T, nL, B, H]."""
    g = rng(w, S_EVAL, sub)
    q, k, v, beta = token_inputs(g, (n_steps, n_layers, batch, w.n_heads), w.d_k, w.d_v)
    if w.ridge_cols:
        cols = ridge_positions(w)[1]                      # [L, H, ridge_cols]
        for h in range(w.n_heads):
            v[:, :, :, h, cols[0, h]] *= np.float32(w.ridge_scale)
    return q, k, v, beta


def warmup_inputs(w: Workload, n_steps: int, n_layers: int, batch: int, sub: int = 0):
    g = rng(w, S_WARMUP, sub)
    return token_inputs(g, (n_steps, n_layers, batch, w.n_heads), w.d_k, w.d_v)


def slot_map(w: Workload) -> np.ndarray:
    """Random request -> slot map over a pool with spare slots: perm(n_slots)[:batch]."""
    g = rng(w, S_SLOTS)
    return g.permutation(w.n_slots)[: w.batch].astype(np.int32)


def ridge_positions(w: Workload):
    """Per (layer, head): ridge_rows key rows and ridge_cols value columns (sorted indices)."""
    g = rng(w, S_RIDGE)
    rows = np.zeros((w.n_layers, w.n_heads, w.ridge_rows), np.int64)
    cols = np.zeros((w.n_layers, w.n_heads, w.ridge_cols), np.int64)
    for l in range(w.n_layers):
        for h in range(w.n_heads):
            rows[l, h] = np.sort(g.choice(w.d_k, w.ridge_rows, replace=False))
            cols[l, h] = np.sort(g.choice(w.d_v, w.ridge_cols, replace=False))
    return rows, cols


def random_state(g: np.random.Generator, lead: tuple, d_k: int, d_v: int, scale: float = 1.0):
    """A dense fp32 state with N(0, scale^2) entries (used where no warm-up is wanted)."""
    return (g.standard_normal(lead + (d_k, d_v)) * scale).astype(np.float32)


# ----------------------------------------------------------------------------
# Philox-4x32-10 (counter-based) for calibration traces.

_PHILOX_M0 = np.uint64(0xD2511F53)
_PHILOX_M1 = np.uint64(0xCD9E8D57)
_PHILOX_W0 = np.uint32(0x9E3779B9)
_PHILOX_W1 = np.uint32(0xBB67AE85)
_MASK32 = np.uint64(0xFFFFFFFF)


def philox4x32(ctr: np.ndarray, key: tuple) -> np.ndarray:
    """Philox-4x32 with 10 rounds.  ctr: uint32 [..., 4]; key: two uint32.  Returns uint32 [..., 4]."""
    c = ctr.astype(np.uint64)
    c0, c1, c2, c3 = c[..., 0], c[..., 1], c[..., 2], c[..., 3]
    k0 = np.uint32(key[0])
    k1 = np.uint32(key[1])
    for _ in range(10):
        p0 = _PHILOX_M0 * c0
        p1 = _PHILOX_M1 * c2
        hi0, lo0 = p0 >> np.uint64(32), p0 & _MASK32
        hi1, lo1 = p1 >> np.uint64(32), p1 & _MASK32
        c0 = hi1 ^ c1 ^ np.uint64(k0)
        c1 = lo1
        c2 = hi0 ^ c3 ^ np.uint64(k1)
        c3 = lo0
        k0 = np.uint32((int(k0) + int(_PHILOX_W0)) & 0xFFFFFFFF)
        k1 = np.uint32((int(k1) + int(_PHILOX_W1)) & 0xFFFFFFFF)
    return np.stack([c0, c1, c2, c3], axis=-1).astype(np.uint32)


def calib_seed(w: Workload) -> int:
    return 0x5EED0000 + 7919 * w.cid


def calib_normals(seed: int, layer: int, head: int, n_seg: int, seg_len: int, n: int) -> np.ndarray:
    """n standard normals per (segment, token): float64 [n_seg, seg_len, n].

    Counter = (block, token, segment, layer << 16 | head), key = (seed lo, seed hi).
    Each block yields four uint32 -> two Box-Muller pairs -> four normals.
    Uniform u = (x + 0.5) * 2^-32; z0 = sqrt(-2 ln u0) cos(2 pi u1), z1 = ... sin(...).
    """
    n_blk = (n + 3) // 4
    b, t, s = np.meshgrid(np.arange(n_blk), np.arange(seg_len), np.arange(n_seg), indexing="ij")
    ctr = np.stack([b, t, s, np.full_like(b, (layer << 16) | head)], axis=-1).astype(np.uint32)
    x = philox4x32(ctr, (seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF))   # [n_blk, T, S, 4]
    u = (x.astype(np.float64) + 0.5) * 2.0 ** -32
    r0 = np.sqrt(-2.0 * np.log(u[..., 0]))
    r1 = np.sqrt(-2.0 * np.log(u[..., 2]))
    th0 = 2.0 * np.pi * u[..., 1]
    th1 = 2.0 * np.pi * u[..., 3]
    z = np.stack([r0 * np.cos(th0), r0 * np.sin(th0), r1 * np.cos(th1), r1 * np.sin(th1)], axis=-1)
    z = z.transpose(2, 1, 0, 3).reshape(n_seg, seg_len, n_blk * 4)
    return z[..., :n]


def calib_traces(seed: int, layer: int, head: int, n_seg: int, seg_len: int, d_k: int, d_v: int):
    """Calibration tokens for one (layer, head): q, k [S, T, d_k], v [S, T, d_v], beta [S, T] (float32).

    Normal index order per token: q (d_k), k (d_k), v (d_v), the beta logit (1).
    q and k are scaled to unit L2 norm (sequential sum of squares in float64).
    """
    z = calib_normals(seed, layer, head, n_seg, seg_len, 2 * d_k + d_v + 1)
    q = z[..., :d_k]
    k = z[..., d_k:2 * d_k]
    v = z[..., 2 * d_k:2 * d_k + d_v]
    bl = z[..., 2 * d_k + d_v]
    qn = np.sqrt(np.cumsum(q * q, axis=-1)[..., -1:])
    kn = np.sqrt(np.cumsum(k * k, axis=-1)[..., -1:])
    beta = 1.0 / (1.0 + np.exp(-bl))
    return ((q / qn).astype(np.float32), (k / kn).astype(np.float32),
            v.astype(np.float32), beta.astype(np.float32))
