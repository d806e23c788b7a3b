#!/usr/bin/env python3
"""Experiments on one MI355X beyond the throughput line of bench.py; each prints one JSON line.

  python experiments.py ablation [--workload gdn-decode-32h-128] [--steps 256]
      Readout drift of the packed recurrence against the float32 trajectory from the same
      warmed-up state and inputs, for the method and its ablations (rcap.io post, the ablation
      paragraph): spatial fit only (uniform widths, no pivots), temporal allocation only (the
      allocation and pivots with a per-row absmax quantizer), no pivots, the fit without the
      row-impact weighting (w = 1), the fit with the workload's synthetic impact draws instead of
      the calibrated scores, the uniform per-row absmax baseline, and the candidate-grid sweep.
  python experiments.py lifetime [--steps 256]
      Spearman correlation between each head's gate half-life and the state error it accumulates
      under uniform 6-bit per-row absmax quantization (rcap.io post, "Temporal" paragraph), on the
      serving pool's 36 x 32 heads, next to the same statistic for the method's 6-bit plan.
  python experiments.py overlap
      The two-stream arrangement against a stand-in for the model's per-layer compute (a bf16
      GEMM on the main stream): fit + pack of layer l on the second stream overlaps the GEMM of
      layer l + 1 (hyper.ai summary, 方法, the second-stream arrangement).

Inputs are seeded synthetic tensors of the workloads' shapes (workloads/); nothing is read from
disk.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class Workbench:
    """A workload on the GPU: gates, the float32 reference state and trajectory inputs."""

    def __init__(self, wl, batch=None, seed=0):
        import numpy as np
        import torch
        import quantized_delta_rule_02_amd as sq
        from workloads import gen
        self.np, self.torch, self.sq, self.gen = np, torch, sq, gen
        self.wl = wl
        self.dev = torch.device("cuda:0")
        self.L, self.H, self.dk, self.dv = wl.n_layers, wl.n_heads, wl.d_k, wl.d_v
        self.B = wl.batch if batch is None else batch
        self.N = self.L * self.B * self.H
        self.form = sq.SQ_FORM_GDN if wl.form == "gdn" else sq.SQ_FORM_KDA
        self.unit = sq.SQ_UNIT_HEAD if wl.unit == "head" else sq.SQ_UNIT_ROW
        self.gates = gen.unit_gates(wl)
        g = torch.tensor(self.gates, device=self.dev)
        if self.form == sq.SQ_FORM_GDN:
            self.gate = g[:, None, :].expand(self.L, self.B, self.H).contiguous().reshape(-1)
        else:
            self.gate = g[:, None].expand(self.L, self.B, self.H, self.dk).contiguous().reshape(-1)
        self.ident = torch.arange(self.B, dtype=torch.int32, device=self.dev)
        self.tg = torch.Generator(device=self.dev)
        self.seed = seed
        self.y = torch.empty(self.N * self.dv, device=self.dev)

    def inputs(self, t):
        torch = self.torch
        self.tg.manual_seed(self.seed * 1_000_003 + t)
        n = self.N
        q = torch.randn(n, self.dk, device=self.dev, generator=self.tg)
        k = torch.randn(n, self.dk, device=self.dev, generator=self.tg)
        q = (q / q.norm(dim=1, keepdim=True)).reshape(-1)
        k = (k / k.norm(dim=1, keepdim=True)).reshape(-1)
        v = torch.randn(n * self.dv, device=self.dev, generator=self.tg)
        if self.wl.ridge_cols:
            cols = self.np.asarray(self.gen.ridge_positions(self.wl)[1])
            v = v.view(n, self.dv)
            v[:, cols] *= self.wl.ridge_scale
            v = v.reshape(-1)
        beta = torch.sigmoid(torch.randn(n, device=self.dev, generator=self.tg))
        return q.contiguous(), k.contiguous(), v.contiguous(), beta

    def fp32_step(self, S, t, y):
        q, k, v, beta = self.inputs(t)
        self.sq.sq_fp32_step(self.form, self.H, self.dk, self.dv, self.B, 0, self.L, self.B, self.ident, S,
                             q, k, v, self.gate, beta, y)

    def warm_state(self, steps):
        S = self.torch.zeros(self.N * self.dk * self.dv, device=self.dev)
        for t in range(steps):
            self.fp32_step(S, 10_000_000 + t, self.y)
        return S

    def plan(self, **over):
        """Library plan; by default the row-impact scores are estimated from the calibration traces
        (the method's calibration), not the workload's synthetic draws."""
        kw = dict(form=self.form, unit=self.unit, n_layers=self.L, n_heads=self.H, d_k=self.dk, d_v=self.dv,
                  widths=self.wl.widths, budget_milli=self.wl.budget_milli, pivot_ppm=self.wl.pivot_ppm,
                  grid=self.wl.grid, gate=self.gates, impact=None,
                  calib_seed=self.gen.calib_seed(self.wl), calib_segments=self.wl.calib_segments,
                  calib_len=self.wl.calib_len)
        kw.update(over)
        return self.sq.sq_plan_create(**kw)

    def pool(self, plan, S):
        mem = self.torch.empty(self.sq.sq_pool_bytes(plan, self.B), dtype=self.torch.uint8, device=self.dev)
        pool = self.sq.sq_pool_create(plan, mem, self.B)
        self.sq.sq_pack(pool, 0, self.L, self.B, self.ident, S)
        return pool, mem


def _rel(a, b):
    return float((a - b).double().norm() / b.double().norm().clamp_min(1e-300))


def ablation(args):
    import numpy as np
    from workloads import configs
    wl = configs.BY_NAME[args.workload]
    wb = Workbench(wl)
    torch, sq = wb.torch, wb.sq
    t0 = time.perf_counter()
    S0 = wb.warm_state(wl.warmup_steps)
    log(f"warm-up {wl.warmup_steps} float32 steps: {time.perf_counter() - t0:.1f} s")
    full = wb.plan()
    ub = sq.sq_plan_units(full)["unit_bits"]
    nominal = wl.budget_milli // 1000
    uniform = np.full_like(ub, nominal if nominal in wl.widths else min(wl.widths))
    variants = {
        "stepquant": full,
        "spatial_only": wb.plan(unit_bits=uniform, pivot_ppm=0),
        "temporal_only": wb.plan(quantizer=sq.SQ_QUANT_ROW_ABSMAX),
        "no_pivots": wb.plan(pivot_ppm=0),
        "unweighted_fit": wb.plan(impact=np.ones_like(wb.gen.impact_scores(wl))),
        "synthetic_impact": wb.plan(impact=wb.gen.impact_scores(wl)),
        "uniform_row_absmax": wb.plan(unit_bits=uniform, pivot_ppm=0, quantizer=sq.SQ_QUANT_ROW_ABSMAX),
        "grid_1": wb.plan(unit_bits=ub, grid=(1.0,)),
        "grid_2": wb.plan(unit_bits=ub, grid=(1.0, 0.875)),
        "grid_8": wb.plan(unit_bits=ub, grid=(1.0, 0.9375, 0.875, 0.8125, 0.75, 0.6875, 0.625, 0.5625)),
    }
    pools = {name: wb.pool(p, S0) for name, p in variants.items()}
    S = S0.clone()
    y_ref = torch.empty_like(wb.y)
    y = torch.empty_like(wb.y)
    acc = {name: [] for name in variants}
    for t in range(args.steps):
        q, k, v, beta = wb.inputs(t)
        sq.sq_fp32_step(wb.form, wb.H, wb.dk, wb.dv, wb.B, 0, wb.L, wb.B, wb.ident, S, q, k, v, wb.gate, beta, y_ref)
        for name, (pool, _) in pools.items():
            sq.sq_state_step(pool, 0, wb.L, wb.B, wb.ident, q, k, v, wb.gate, beta, y)
            acc[name].append(_rel(y, y_ref))
    torch.cuda.synchronize()
    Xh = torch.empty_like(S)
    out = {}
    for name, (pool, _) in pools.items():
        sq.sq_unpack(pool, 0, wb.L, wb.B, wb.ident, Xh)
        e = acc[name]
        d = variants[name].desc
        out[name] = {"y_rel_mean": float(np.mean(e)), "y_rel_last": e[-1], "y_rel_max": float(np.max(e)),
                     "state_rel_last": _rel(Xh, S), "stored_bits_per_entry": round(d["stored_bits_per_entry"], 4),
                     "pivot_units": d["n_pivot_units"]}
    print(json.dumps({"experiment": "ablation", "workload": wl.name, "steps": args.steps,
                      "budget_bits": wl.budget_milli / 1000, "metric": "relative L2 of y against the float32 "
                      "trajectory (all states of the step), and of the dequantized state after the last step",
                      "variants": out}), flush=True)


def lifetime(args):
    import numpy as np
    from scipy.stats import spearmanr
    from workloads import configs
    wl = configs.SERVING_6
    wb = Workbench(wl, batch=args.batch, seed=1)
    torch, sq = wb.torch, wb.sq
    S0 = wb.warm_state(wl.warmup_steps)
    U = wb.L * wb.H
    plans = {"uniform_int6_row_absmax": wb.plan(unit_bits=np.full(U, 6, np.int32), pivot_ppm=0,
                                                quantizer=sq.SQ_QUANT_ROW_ABSMAX),
             "uniform6_dual_axis": wb.plan(unit_bits=np.full(U, 6, np.int32), pivot_ppm=0),
             "stepquant_6bit": wb.plan()}
    pools = {name: wb.pool(p, S0) for name, p in plans.items()}
    S = S0.clone()
    y = torch.empty_like(wb.y)
    for t in range(args.steps):
        q, k, v, beta = wb.inputs(t)
        sq.sq_fp32_step(wb.form, wb.H, wb.dk, wb.dv, wb.B, 0, wb.L, wb.B, wb.ident, S, q, k, v, wb.gate, beta, y)
        for pool, _ in pools.values():
            sq.sq_state_step(pool, 0, wb.L, wb.B, wb.ident, q, k, v, wb.gate, beta, y)
    torch.cuda.synchronize()
    alpha = wb.gates.reshape(-1).astype(np.float64)                  # [L * H]
    half_life = np.log(0.5) / np.log(alpha)
    Sr = S.view(wb.L, wb.B, wb.H, wb.dk * wb.dv).double()
    out = {}
    Xh = torch.empty_like(S)
    for name, (pool, _) in pools.items():
        sq.sq_unpack(pool, 0, wb.L, wb.B, wb.ident, Xh)
        Xr = Xh.view(wb.L, wb.B, wb.H, wb.dk * wb.dv).double()
        err = ((Xr - Sr).norm(dim=3) / Sr.norm(dim=3).clamp_min(1e-300)).mean(dim=1).reshape(-1).cpu().numpy()
        rho = spearmanr(half_life, err)
        out[name] = {"spearman_rho": float(rho.correlation), "p_value": float(rho.pvalue),
                     "mean_state_rel_err": float(err.mean()), "max_state_rel_err": float(err.max())}
    print(json.dumps({"experiment": "lifetime", "workload": wl.name, "heads": U, "requests": wb.B,
                      "steps": args.steps, "metric": "Spearman rho between gate half-life ln(1/2)/ln(alpha) and "
                      "the head's relative state error after the steps, averaged over requests",
                      "results": out}), flush=True)


def overlap(args):
    import torch
    import quantized_delta_rule_02_amd as sq
    from workloads import configs
    wl = configs.SERVING_6
    wb = Workbench(wl)
    dev = wb.dev
    L, B, H = wb.L, wb.B, wb.H
    per = B * H
    plan = wb.plan()
    S0 = torch.randn(wb.N * wb.dk * wb.dv, device=dev)
    pool, mem = wb.pool(plan, S0)
    del S0
    q, k, v, beta = wb.inputs(0)
    y = torch.empty(wb.N * wb.dv, device=dev)
    slots = wb.ident
    dk, dv = wb.dk, wb.dv
    # stand-in for the model's per-layer compute: activations [B, K] x weights [K, N] in bf16
    K, Nn = args.gemm_k, args.gemm_n
    A = torch.randn(B, K, device=dev, dtype=torch.bfloat16)
    Ws = [torch.randn(K, Nn, device=dev, dtype=torch.bfloat16) for _ in range(2)]
    C = torch.empty(B, Nn, device=dev, dtype=torch.bfloat16)
    aux = torch.cuda.Stream()

    def gemm(l):
        torch.matmul(A, Ws[l % 2], out=C)

    def layer_call(l, flags, s_aux):
        a0, a1 = l * per, (l + 1) * per
        sq.sq_state_step(pool, l, 1, B, slots, q[a0 * dk:a1 * dk], k[a0 * dk:a1 * dk], v[a0 * dv:a1 * dv],
                         wb.gate[a0:a1], beta[a0:a1], y[a0 * dv:a1 * dv], stream_aux=s_aux, flags=flags)

    def run_gemm_only():
        for l in range(L):
            gemm(l)

    def run_step_only():
        sq.sq_state_step(pool, 0, L, B, slots, q, k, v, wb.gate, beta, y)

    def run_sequential():
        for l in range(L):
            gemm(l)
            layer_call(l, 0, None)

    def run_overlapped():
        for l in range(L):
            gemm(l)
            layer_call(l, sq.SQ_STEP_SPLIT | sq.SQ_STEP_NO_JOIN, aux)
        torch.cuda.current_stream().wait_stream(aux)

    def timed(fn, reps=args.reps):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    res = {"gemm_only_ms": timed(run_gemm_only), "step_fused_ms": timed(run_step_only),
           "sequential_ms": timed(run_sequential), "split_overlapped_ms": timed(run_overlapped)}
    res["hidden_ms"] = res["sequential_ms"] - res["split_overlapped_ms"]
    res["overlapped_over_sum"] = res["split_overlapped_ms"] / (res["gemm_only_ms"] + res["step_fused_ms"])
    print(json.dumps({"experiment": "overlap", "workload": wl.name, "layers": L, "requests": B,
                      "model_compute": f"bf16 GEMM [{B} x {K}] x [{K} x {Nn}] per layer "
                                       f"({2 * B * K * Nn / 1e9:.1f} GFLOP)",
                      "results": res}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    a = sub.add_parser("ablation")
    a.add_argument("--workload", default="gdn-decode-32h-128")
    a.add_argument("--steps", type=int, default=256)
    b = sub.add_parser("lifetime")
    b.add_argument("--steps", type=int, default=256)
    b.add_argument("--batch", type=int, default=8)
    c = sub.add_parser("overlap")
    c.add_argument("--gemm-k", type=int, default=5120)
    c.add_argument("--gemm-n", type=int, default=24576)
    c.add_argument("--reps", type=int, default=10)
    args = ap.parse_args()
    {"ablation": ablation, "lifetime": lifetime, "overlap": overlap}[args.cmd](args)


if __name__ == "__main__":
    main()
