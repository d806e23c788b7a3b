#!/usr/bin/env python3
"""Throughput of the quantized gated-delta state step on one MI355X.

Workload (default): the serving-scale pool -- 256 concurrent requests x 36
linear-attention layers x 32 GDN heads x 128x128 states, per-head widths from
{4, 6, 8} at a 6.0-bit average budget with 1% FP16 pivot heads, requests mapped
at random onto a pool with 25% spare slots.  One step updates every layer of
every request once (one library call, 294,912 state updates).  Inputs are
seeded synthetic tensors already resident in HBM; the initial state is a
512-step float32 warm-up packed by the library.

Prints one JSON line (metric, value, roofline of the step kernel, and the
float64 CPU oracle timed on a bounded sample of the same workload).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "pmc_state_step_serving6.txt")
KERNEL_SRC = os.path.join(ROOT, "quantized_delta_rule_02_amd", "csrc", "kernels.hip")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="serving-36l-32h-256req-6bit")
    ap.add_argument("--state-warmup", type=int, default=512, help="float32 warm-up steps before packing")
    ap.add_argument("--split", action="store_true", help="time the two-stream arrangement")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--extras", action="store_true", help="also time the 4-bit pool and the copy reference")
    return ap.parse_args()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic_bytes(plan, batch, sq):
    """Bytes the step must move per call: packed codes + scales read and written, q/k/v/gate/beta read, y written."""
    import numpy as np
    d = plan.desc
    L, H, dk, dv = d["n_layers"], d["n_heads"], d["d_k"], d["d_v"]
    row_bits, _ = sq.sq_plan_rows(plan)
    code_bits = row_bits.astype(np.int64).sum(axis=2) * dv              # [L, H]
    state_bytes = code_bits // 8 + 2 * (dk + dv)                         # codes + binary16 scales
    gate = 4 * (dk if d["form"] == 1 else 1)
    io = 4 * (2 * dk + 2 * dv + 1) + gate                                # q, k, v, y, beta, gate
    return int(batch * (2 * state_bytes.sum() + L * H * io))


def traffic_per_launch():
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it matches this kernel source."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    for line in open(TRAFFIC_FILE):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    sha = hashlib.sha256(open(KERNEL_SRC, "rb").read()).hexdigest()
    if kv.get("kernel_source_sha256") != sha:
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(wl, seconds, seed=7):
    """The float64 oracle on a sample of the workload's states, timed on the host."""
    import numpy as np
    from oracle import quant
    from oracle.step import packed_step
    from workloads import gen

    g = np.random.default_rng(seed)
    n = 64
    gates = gen.unit_gates(wl)
    imp = gen.impact_scores(wl)
    lh = g.integers(0, wl.n_layers * wl.n_heads, size=n)
    alpha = gates.reshape(-1)[lh].astype(np.float64)
    w = imp.reshape(-1, wl.d_k)[lh].astype(np.float64)
    rows = quant.RowPlan(bits=np.full((n, wl.d_k), 6), pivot=np.zeros((n, wl.d_k), bool), w=w)
    X = g.standard_normal((n, wl.d_k, wl.d_v))
    P = quant.quantize(X, rows, wl.grid)
    q, k, v, beta = [a[0, 0, 0] for a in gen.eval_inputs(wl.scaled(n_layers=1, n_heads=n), 1, 1, 1)]
    done = 0
    t0 = time.perf_counter()
    while True:
        P, _, _ = packed_step(P, rows, q, k, v, alpha, beta, wl.grid)
        done += n
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    return {"value": done / el, "unit": "state-updates/s", "cores": 1, "kind": "oracle",
            "sample": f"{done} state updates ({n} sampled (layer, head) states of the workload, 6-bit rows, "
                      f"steps repeated for {el:.1f} s) by the float64 NumPy oracle in one host thread"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the step has no cross-GPU exchange "
              f"and each GPU's share is the single-GPU workload", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import quantized_delta_rule_02_amd as sq
    from workloads import configs, gen

    wl = configs.BY_NAME[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    L, H, dk, dv, B = wl.n_layers, wl.n_heads, wl.d_k, wl.d_v, wl.batch
    form = sq.SQ_FORM_GDN if wl.form == "gdn" else sq.SQ_FORM_KDA
    unit = sq.SQ_UNIT_HEAD if wl.unit == "head" else sq.SQ_UNIT_ROW

    t0 = time.perf_counter()
    plan = sq.sq_plan_create(form=form, unit=unit, n_layers=L, n_heads=H, d_k=dk, d_v=dv, widths=wl.widths,
                             budget_milli=wl.budget_milli, pivot_ppm=wl.pivot_ppm, grid=wl.grid,
                             gate=gen.unit_gates(wl), impact=gen.impact_scores(wl), calib_seed=gen.calib_seed(wl),
                             calib_segments=wl.calib_segments, calib_len=wl.calib_len)
    log(f"plan: {time.perf_counter() - t0:.1f} s  {plan.desc}")
    pool_mem = torch.empty(sq.sq_pool_bytes(plan, wl.n_slots), dtype=torch.uint8, device=dev)
    pool = sq.sq_pool_create(plan, pool_mem, wl.n_slots)
    slots = torch.tensor(gen.slot_map(wl), dtype=torch.int32, device=dev)

    gate_unit = torch.tensor(gen.unit_gates(wl), device=dev)
    if form == sq.SQ_FORM_GDN:
        gate = gate_unit[:, None, :].expand(L, B, H).contiguous().reshape(-1)
    else:
        gate = gate_unit[:, None].expand(L, B, H, dk).contiguous().reshape(-1)
    gen_t = torch.Generator(device=dev)

    def inputs(seed):
        gen_t.manual_seed(seed)
        n = L * B * H
        q = torch.randn(n, dk, device=dev, generator=gen_t)
        k = torch.randn(n, dk, device=dev, generator=gen_t)
        q = (q / q.norm(dim=1, keepdim=True)).reshape(-1).contiguous()
        k = (k / k.norm(dim=1, keepdim=True)).reshape(-1).contiguous()
        v = torch.randn(n * dv, device=dev, generator=gen_t)
        beta = torch.sigmoid(torch.randn(n, device=dev, generator=gen_t))
        return q, k, v, beta

    # initial state: float32 warm-up of every (layer, request, head) state, then packed by the library
    t0 = time.perf_counter()
    n_states = L * B * H
    S = torch.zeros(n_states * dk * dv, dtype=torch.float32, device=dev)
    ident = torch.arange(B, dtype=torch.int32, device=dev)
    y = torch.empty(n_states * dv, dtype=torch.float32, device=dev)
    for t in range(args.state_warmup):
        q, k, v, beta = inputs(10_000 + t)
        sq.sq_fp32_step(form, H, dk, dv, B, 0, L, B, ident, S, q, k, v, gate, beta, y)
    sq.sq_pack(pool, 0, L, B, slots, S)
    torch.cuda.synchronize()
    del S
    torch.cuda.empty_cache()
    log(f"state warm-up ({args.state_warmup} fp32 steps) + pack: {time.perf_counter() - t0:.1f} s")

    batches = [inputs(s) for s in (1, 2)]
    aux = torch.cuda.Stream() if args.split else None
    flags = sq.SQ_STEP_SPLIT if args.split else 0

    def step(i):
        q, k, v, beta = batches[i % len(batches)]
        sq.sq_state_step(pool, 0, L, B, slots, q, k, v, gate, beta, y, stream_aux=aux, flags=flags)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    ev0.record()
    for i in range(args.steps):
        step(i)
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms = ev0.elapsed_time(ev1) / args.steps
    per_step = L * B * H
    value = per_step / (ms / 1e3)

    alg = algorithmic_bytes(plan, B, sq)
    achieved = alg / (ms / 1e3) / 1e9
    traffic = traffic_per_launch()
    desc = plan.desc
    out = {
        "metric": "state-updates/s (req·head·step) + achieved HBM GB/s, 6-bit packed state",
        "value": value,
        "unit": "state-updates/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "requests": B, "slots": wl.n_slots, "layers": L, "heads": H,
                   "d_k": dk, "d_v": dv, "form": wl.form, "budget_bits": wl.budget_milli / 1000,
                   "pivot_units": desc["n_pivot_units"], "grid": list(wl.grid),
                   "arrangement": "split2" if args.split else "fused1",
                   "state_updates_per_step": per_step,
                   "compression_vs_fp32": round(desc["compression_vs_fp32"], 4),
                   "stored_bits_per_entry": round(desc["stored_bits_per_entry"], 4)},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS,
                     "traffic": None if traffic is None else traffic,
                     "algorithmic_bytes_per_launch": alg, "kernel": "k_state<128,128,step>",
                     "launch_ms": ms},
        "wall_s_timed": wall,
    }
    if args.extras:
        src = torch.empty(4 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        sq.sq_copy(src, dst)
        torch.cuda.synchronize()
        ev0.record()
        for _ in range(5):
            sq.sq_copy(src, dst)
        ev1.record()
        torch.cuda.synchronize()
        cms = ev0.elapsed_time(ev1) / 5
        out["copy_reference"] = {"bytes_moved": 2 * src.numel(), "ms": cms, "GBps": 2 * src.numel() / cms / 1e6}
        del src, dst
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
    print(json.dumps(out), flush=True)
    pool.close()
    plan.close()


if __name__ == "__main__":
    main()
