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
# fp32 vector peak of the MI355X: 256 CUs x 2.4 GHz x 256 flops per CU and clock (128 FMA lanes)
ALU_PEAK_TFLOPS = 256 * 2.4e9 * 256 / 1e12
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "pmc_state_step_serving6.txt")
VALU_FILE = os.path.join(ROOT, "profiles", "pmc_state_step_serving6_valu.txt")
PROFILED_WORKLOAD = "serving-36l-32h-256req-6bit"     # the workload the counter summaries were taken on
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
    ap.add_argument("--summarize", metavar="DB", nargs="+",
                    help="print per-kernel launch durations and counters from rocprofv3 result databases "
                         "(no GPU is used)")
    ap.add_argument("--launches", default="last:20",
                    help="with --summarize: which launches of each kernel, first:N or last:N")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the comparators (INT8 per-row, FP32), the split arrangement, the candidate-grid "
                         "sweep, the 4-bit budgets, the copy reference, the dual-axis outlier pool and the "
                         "cache-resident decode pools")
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


def per_state_bytes(dk, dv, form, state_bytes):
    gate = 4 * (dk if form == 1 else 1)
    return 2 * state_bytes + 4 * (2 * dk + 2 * dv + 1) + gate


def int8_group_order(dk, dv):
    """Row-major index of each byte of one INT8 comparator state, in the library's group-interleaved order
    (16 / cpl rows x cpl columns per lane and group, cpl = max(1, dv / 64))."""
    import numpy as np
    cpl = max(1, dv // 64)
    lpr, gr = dv // cpl, 16 // cpl
    return np.arange(dk * dv).reshape(dk // gr, gr, lpr, cpl).transpose(0, 2, 1, 3).reshape(-1)


def int8_states(S, n, dk, dv, chunk=4096):
    """Uniform INT8 per-row states of the float states S [n][dk][dv]: group-interleaved codes and row scales."""
    import torch
    order = torch.as_tensor(int8_group_order(dk, dv), device=S.device)
    codes = torch.empty(n, dk * dv, dtype=torch.int8, device=S.device)
    scales = torch.empty(n, dk, dtype=torch.float32, device=S.device)
    Sv = S.view(n, dk, dv)
    for i0 in range(0, n, chunk):
        blk = Sv[i0:i0 + chunk]
        sc = (blk.abs().amax(dim=2) / 127.0).clamp_min(1e-30)
        scales[i0:i0 + chunk] = sc
        q = torch.clamp(torch.round(blk / sc[:, :, None]), -127, 127).to(torch.int8)
        codes[i0:i0 + chunk] = q.reshape(-1, dk * dv)[:, order]
    return codes.reshape(-1), scales.reshape(-1)


def time_calls(fn, n, warm=2):
    """Mean milliseconds per call over n calls on torch's current stream (HIP events)."""
    import torch
    for _ in range(warm):
        fn()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(n):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n


def _profile_value(path, key):
    """A figure from a committed rocprofv3 summary, if the summary matches this kernel source."""
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    sha = hashlib.sha256(open(KERNEL_SRC, "rb").read()).hexdigest()
    if kv.get("kernel_source_sha256") != sha:
        return None
    try:
        return float(kv[key])
    except (KeyError, ValueError):
        return None


def traffic_per_launch():
    """HBM bytes per launch (FETCH_SIZE and WRITE_SIZE, calibrated on the copy kernel)."""
    return _profile_value(TRAFFIC_FILE, "hbm_bytes_per_launch")


def algorithmic_flops(n_states, dk, dv, n_grid):
    """Arithmetic the step must do per call: (12 + 5 G) d_k d_v flops per state update -- the two column
    sums (4), the rank-one update (2), dequantization (1), and the requantization with G candidates
    (5 + 5 G)."""
    return n_states * (12 + 5 * n_grid) * dk * dv


def _oracle_rows(wl, n, g):
    """Row plans of n (layer, head) states with the workload's structure: per-unit code widths drawn from its
    candidate set around its average-bit budget (a quarter each at the narrowest and widest width for a
    6-bit budget with {4, 6, 8}, every unit at the narrowest width for a budget at that width), the
    workload's pivot fraction (at least one pivot unit in the sample when the workload has pivots) and
    its drawn impact scores."""
    import numpy as np
    from oracle import quant
    from workloads import gen
    imp = gen.impact_scores(wl)
    lh = g.integers(0, wl.n_layers * wl.n_heads, size=n)
    w = imp.reshape(-1, wl.d_k)[lh].astype(np.float64)
    widths = np.asarray(sorted(wl.widths))
    per = 1 if wl.unit == "head" else wl.d_k
    units = n * per
    b = wl.budget_milli / 1000.0
    if b <= widths[0]:
        bits = np.full(units, widths[0])
    else:
        lo, mid, hi = widths[0], widths[len(widths) // 2], widths[-1]
        bits = g.choice([lo, mid, hi], size=units, p=[0.25, 0.5, 0.25])
    pivot = np.zeros(units, bool)
    if wl.pivot_ppm > 0:
        n_piv = max(1, -(-wl.pivot_ppm * units // 1_000_000))
        pivot[g.choice(units, size=n_piv, replace=False)] = True
    bits = np.where(pivot, 16, bits)
    if per == 1:
        bits = np.repeat(bits[:, None], wl.d_k, axis=1)
        pivot = np.repeat(pivot[:, None], wl.d_k, axis=1)
    else:
        bits = bits.reshape(n, wl.d_k)
        pivot = pivot.reshape(n, wl.d_k)
    return quant.RowPlan(bits=bits, pivot=pivot, w=w), lh


def _oracle_sample(wl, seed, n=64):
    """A seeded sample of the workload's states (oracle-quantized, with its widths and pivots) and one step's
    inputs."""
    import numpy as np
    from oracle import quant
    from workloads import gen

    g = np.random.default_rng(seed)
    gates = gen.unit_gates(wl)
    rows, lh = _oracle_rows(wl, n, g)
    alpha = (gates.reshape(-1)[lh] if wl.form == "gdn" else gates.reshape(-1, wl.d_k)[lh]).astype(np.float64)
    P = quant.quantize(g.standard_normal((n, wl.d_k, wl.d_v)), rows, wl.grid)
    q, k, v, beta = [a[0, 0, 0] for a in gen.eval_inputs(wl.scaled(n_layers=1, n_heads=n), 1, 1, 1)]
    return P, rows, q, k, v, alpha, beta


def _oracle_run(args):
    """Oracle steps over a sample of n states until `seconds` have passed (or `max_steps` steps are done);
    returns (state updates, elapsed s)."""
    wl_name, seed, seconds, n = args[:4]
    max_steps = args[4] if len(args) > 4 else None
    from threadpoolctl import threadpool_limits
    from oracle.step import packed_step
    from workloads import configs
    wl = configs.BY_NAME[wl_name]
    P, rows, q, k, v, alpha, beta = _oracle_sample(wl, seed, n)
    done, steps, t0 = 0, 0, time.perf_counter()
    with threadpool_limits(1):
        while True:
            P, _, _ = packed_step(P, rows, q, k, v, alpha, beta, wl.grid)
            done += P.Q.shape[0]
            steps += 1
            el = time.perf_counter() - t0
            if (max_steps is not None and steps >= max_steps) or (max_steps is None and el >= seconds):
                return done, el


# A one-GPU job on the GPU machine gets a share of 16 host cores (its process guard counts on that share),
# whatever the affinity mask shows; the oracle uses every core of that share.
HOST_CORE_SHARE = 16


def _host_cores():
    visible = len(os.sched_getaffinity(0))
    return max(1, min(visible, HOST_CORE_SHARE)), visible


def cpu_baseline(wl, seconds):
    """The float64 oracle on a bounded sample of the workload's states (its widths, pivots and impact scores),
    timed on the host: one thread for a third of the time, then one process per core of the host share for
    the rest; plus the smaller configurations, whose whole state set goes through the oracle."""
    import multiprocessing as mp
    from workloads import configs
    n1, t1 = _oracle_run((wl.name, 7, seconds / 3, 64))
    cores, visible = _host_cores()
    with mp.get_context("fork").Pool(cores) as pool:
        res = pool.map(_oracle_run, [(wl.name, 100 + i, 2 * seconds / 3, 64) for i in range(cores)])
        done = sum(r[0] for r in res)
        wall = max(r[1] for r in res)
        # configurations 0-2: every state of a step, split over the processes, steps repeated for a few
        # seconds (the tiny workload: all 64 steps of its 2 states)
        others = {}
        for ow, secs in ((configs.TINY, 0.0), (configs.GDN_DECODE, 3.0), (configs.KDA_DECODE, 3.0)):
            n_states = ow.states_per_step
            if n_states <= cores:
                upd, el = _oracle_run((ow.name, 200, 0.0, n_states, ow.steps))
                others[ow.name] = {"state_updates_per_s": upd / el, "states": n_states, "steps": ow.steps,
                                   "processes": 1}
                continue
            chunk = -(-n_states // cores)
            parts = [(ow.name, 300 + i, secs, min(chunk, n_states - i * chunk)) for i in range(cores)
                     if i * chunk < n_states]
            rr = pool.map(_oracle_run, parts)
            el = max(x[1] for x in rr)
            upd = sum(x[0] for x in rr)
            others[ow.name] = {"state_updates_per_s": upd / el, "states": n_states,
                               "steps": round(upd / n_states, 2), "processes": len(parts)}
    return {"value": done / wall, "unit": "state-updates/s", "cores": cores, "kind": "oracle",
            "cores_visible": visible, "single_thread": n1 / t1,
            "sample": f"{done} state updates over {cores} processes (each 64 sampled (layer, head) states of the "
                      f"workload with its widths {{4, 6, 8}} around the 6-bit budget and its pivot heads, steps "
                      f"repeated for {2 * seconds / 3:.0f} s) plus {n1} in one thread, by the float64 NumPy "
                      f"oracle, BLAS limited to one thread per process",
            "other_configs": others}


def small_pools(sq, torch, dev, n_steps=256, per_graph=32):
    """The decode workloads whose pools fit in the 256 MB last-level cache (GDN: 64 requests x 32 heads;
    KDA: 128 requests x 32 heads; 128x128 states, 6.0-bit budget): a step is a few microseconds of work,
    so launches matter.  Time per step over n_steps steps launched one by one, and replayed from a HIP
    graph holding per_graph steps (the graph is replayed n_steps / per_graph times)."""
    import numpy as np
    from workloads import configs, gen
    out = {}
    for wl in (configs.GDN_DECODE, configs.KDA_DECODE):
        L, H, dk, dv, B = wl.n_layers, wl.n_heads, wl.d_k, wl.d_v, wl.batch
        n = L * B * H
        form = sq.SQ_FORM_GDN if wl.form == "gdn" else sq.SQ_FORM_KDA
        unit = sq.SQ_UNIT_HEAD if wl.unit == "head" else sq.SQ_UNIT_ROW
        plan = sq.sq_plan_create(form=form, unit=unit, n_layers=L, n_heads=H, d_k=dk, d_v=dv, widths=wl.widths,
                                 budget_milli=wl.budget_milli, pivot_ppm=wl.pivot_ppm, grid=wl.grid,
                                 gate=gen.unit_gates(wl), impact=gen.impact_scores(wl),
                                 calib_seed=gen.calib_seed(wl), calib_segments=wl.calib_segments,
                                 calib_len=wl.calib_len)
        mem = torch.zeros(sq.sq_pool_bytes(plan, wl.n_slots), dtype=torch.uint8, device=dev)
        pool = sq.sq_pool_create(plan, mem, wl.n_slots)
        slots = torch.tensor(gen.slot_map(wl), dtype=torch.int32, device=dev)
        g = torch.Generator(device=dev)
        g.manual_seed(43)
        sq.sq_pack(pool, 0, L, B, slots, torch.randn(n * dk * dv, device=dev, generator=g))
        q = torch.randn(n, dk, device=dev, generator=g)
        k = torch.randn(n, dk, device=dev, generator=g)
        q = (q / q.norm(dim=1, keepdim=True)).reshape(-1).contiguous()
        k = (k / k.norm(dim=1, keepdim=True)).reshape(-1).contiguous()
        v = torch.randn(n * dv, device=dev, generator=g)
        beta = torch.sigmoid(torch.randn(n, device=dev, generator=g))
        gt = torch.tensor(gen.unit_gates(wl), device=dev)
        gate = (gt[:, None, :].expand(L, B, H) if form == sq.SQ_FORM_GDN
                else gt[:, None].expand(L, B, H, dk)).contiguous().reshape(-1)
        y = torch.empty(n * dv, device=dev)

        def step():
            sq.sq_state_step(pool, 0, L, B, slots, q, k, v, gate, beta, y)

        eager_ms = time_calls(step, n_steps)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=side):
            for _ in range(per_graph):
                step()
        torch.cuda.current_stream().wait_stream(side)
        reps = max(1, n_steps // per_graph)
        graph_ms = time_calls(graph.replay, reps) / per_graph
        alg = algorithmic_bytes(plan, B, sq)
        out[wl.name] = {"states_per_step": n, "eager_us_per_step": eager_ms * 1e3,
                        "graph_us_per_step": graph_ms * 1e3,
                        "state_updates_per_s_graph": n / (graph_ms / 1e3),
                        "effective_GBps_graph": alg / (graph_ms / 1e3) / 1e9,
                        "pool_MB": round(sq.sq_pool_bytes(plan, wl.n_slots) / 1e6, 1)}
        del graph
        pool.close()
        plan.close()
        del mem
    torch.cuda.empty_cache()
    return out


def outlier_comparison(sq, torch, dev, steps):
    """The dual-axis outlier pool (KDA, 128x256 states, 1024 requests x 32 heads, per-row widths at a 4.0-bit
    budget with FP16 pivot rows) against the uniform INT8 per-row and FP32 states on the same state and inputs.
    The state is Gaussian with each head's ridge rows and columns scaled as in the workload's warm-up; the v of
    each step carries the ridge columns."""
    import numpy as np
    from workloads import configs, gen
    wl = configs.OUTLIER
    L, H, dk, dv, B = wl.n_layers, wl.n_heads, wl.d_k, wl.d_v, wl.batch
    n = L * B * H
    t0 = time.perf_counter()
    plan = sq.sq_plan_create(form=sq.SQ_FORM_KDA, unit=sq.SQ_UNIT_ROW, n_layers=L, n_heads=H, d_k=dk, d_v=dv,
                             widths=wl.widths, budget_milli=wl.budget_milli, pivot_ppm=wl.pivot_ppm, grid=wl.grid,
                             gate=gen.unit_gates(wl), impact=gen.impact_scores(wl), calib_seed=gen.calib_seed(wl),
                             calib_segments=wl.calib_segments, calib_len=wl.calib_len)
    log(f"outlier plan: {time.perf_counter() - t0:.1f} s")
    mem = torch.empty(sq.sq_pool_bytes(plan, wl.n_slots), dtype=torch.uint8, device=dev)
    pool = sq.sq_pool_create(plan, mem, wl.n_slots)
    slots = torch.tensor(gen.slot_map(wl), dtype=torch.int32, device=dev)
    ident = torch.arange(B, dtype=torch.int32, device=dev)
    rows, cols = gen.ridge_positions(wl)                                 # [L, H, r], [L, H, c]
    rscale = torch.ones(H, dk, device=dev)
    cscale = torch.ones(H, dv, device=dev)
    for h in range(H):
        rscale[h, torch.as_tensor(rows[0, h], device=dev)] = wl.ridge_scale
        cscale[h, torch.as_tensor(cols[0, h], device=dev)] = wl.ridge_scale
    g = torch.Generator(device=dev)
    g.manual_seed(41)
    S = torch.randn(B, H, dk, dv, device=dev, generator=g)
    S *= rscale[None, :, :, None]
    S *= cscale[None, :, None, :]
    S = S.reshape(-1)
    sq.sq_pack(pool, 0, L, B, slots, S)
    q = torch.randn(n, dk, device=dev, generator=g)
    k = torch.randn(n, dk, device=dev, generator=g)
    q = (q / q.norm(dim=1, keepdim=True)).reshape(-1).contiguous()
    k = (k / k.norm(dim=1, keepdim=True)).reshape(-1).contiguous()
    v = (torch.randn(B, H, dv, device=dev, generator=g) * cscale[None]).reshape(-1).contiguous()
    beta = torch.sigmoid(torch.randn(n, device=dev, generator=g))
    gate = torch.tensor(gen.unit_gates(wl), device=dev)[:, None].expand(L, B, H, dk).contiguous().reshape(-1)
    y = torch.empty(n * dv, device=dev)
    ms_q = time_calls(lambda: sq.sq_state_step(pool, 0, L, B, slots, q, k, v, gate, beta, y), steps)
    alg = algorithmic_bytes(plan, B, sq)
    out = {"workload": wl.name, "states_per_step": n,
           "packed_4bit": {"ms": ms_q, "state_updates_per_s": n / (ms_q / 1e3), "GBps": alg / (ms_q / 1e3) / 1e9,
                           "algorithmic_bytes_per_launch": alg,
                           "compression_vs_fp32": round(plan.desc["compression_vs_fp32"], 4)}}
    pool.close()
    plan.close()
    del mem
    codes8, scales8 = int8_states(S, n, dk, dv)
    ms8 = time_calls(lambda: sq.sq_int8_step(sq.SQ_FORM_KDA, H, dk, dv, B, 0, L, B, ident, codes8, scales8, q, k, v,
                                             gate, beta, y), steps)
    by8 = per_state_bytes(dk, dv, 1, dk * dv + 4 * dk)
    out["int8_row"] = {"ms": ms8, "state_updates_per_s": n / (ms8 / 1e3), "GBps": n * by8 / (ms8 / 1e3) / 1e9,
                       "state_bytes": dk * dv + 4 * dk}
    del codes8, scales8
    ms32 = time_calls(lambda: sq.sq_fp32_step(sq.SQ_FORM_KDA, H, dk, dv, B, 0, L, B, ident, S, q, k, v, gate, beta,
                                              y), steps)
    by32 = per_state_bytes(dk, dv, 1, 4 * dk * dv)
    out["fp32"] = {"ms": ms32, "state_updates_per_s": n / (ms32 / 1e3), "GBps": n * by32 / (ms32 / 1e3) / 1e9,
                   "state_bytes": 4 * dk * dv}
    del S
    torch.cuda.empty_cache()
    return out


def valu_ceiling(sq, torch, dev):
    """FMA issue rate of the library's probe (independent chains, vector-register operands) with residency
    capped at 4 waves per SIMD (the step's: 128 VGPRs) and at 8, in wave-instructions per CU per clock at
    the nominal 2.4 GHz, the unit of the step's own rate beside it."""
    res = {}
    buf = torch.empty(65536 * 256, dtype=torch.float32, device=dev)     # 65,536 workgroups of 4 waves
    for w in (4, 8):
        try:
            sq.sq_valu_probe(w, buf)
        except sq.StepQError as e:
            res[f"waves_per_simd_{w}"] = {"error": str(e)}
            continue
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(3):
            n_fma, fit = sq.sq_valu_probe(w, buf)
        e1.record()
        torch.cuda.synchronize()
        t = e0.elapsed_time(e1) / 3
        res[f"waves_per_simd_{w}"] = {"fma_per_cu_per_clock": n_fma / (t / 1e3) / (256 * 2.4e9),
                                      "resident_workgroups_per_cu": fit, "ms": t}
    del buf
    return res


def summarize(paths, which):
    """Per-kernel figures from rocprofv3 result databases (sqlite): mean / min / max duration of the chosen
    launches of each kernel and the mean of each collected counter over the same launches."""
    import sqlite3
    mode, n = which.split(":")
    n = int(n)
    for path in paths:
        con = sqlite3.connect(path)
        cur = con.cursor()
        kcols = [r[1] for r in cur.execute("PRAGMA table_info(kernels)")]
        ki = {c: i for i, c in enumerate(kcols)}
        name_c = next(c for c in ("kernel_name", "name") if c in ki)
        disp_c = next(c for c in ("dispatch_id", "id") if c in ki)
        launches = {}
        for r in cur.execute("SELECT * FROM kernels ORDER BY start"):
            launches.setdefault(str(r[ki[name_c]]), []).append((r[ki[disp_c]], r[ki["end"]] - r[ki["start"]]))
        counters = {}
        try:
            ccols = [r[1] for r in cur.execute("PRAGMA table_info(counters_collection)")]
            ci = {c: i for i, c in enumerate(ccols)}
            cname = next(c for c in ("counter_name", "name") if c in ci)
            cval = next(c for c in ("value", "counter_value") if c in ci)
            for r in cur.execute("SELECT * FROM counters_collection"):
                key = (r[ci["dispatch_id"]], r[ci[cname]])
                counters[key] = counters.get(key, 0.0) + float(r[ci[cval]])
        except Exception:
            pass
        cnames = sorted({k[1] for k in counters})
        print(f"# {path}: {mode} {n} launches of each kernel")
        print(f"{'kernel':44s} {'calls':>6s} {'used':>5s} {'avg_us':>10s} {'min_us':>10s} {'max_us':>10s}"
              + "".join(f" {c:>18s}" for c in cnames))
        for name, ls in sorted(launches.items()):
            sel = ls[:n] if mode == "first" else ls[-n:]
            d = [x[1] / 1000.0 for x in sel]
            row = f"{name[:44]:44s} {len(ls):6d} {len(sel):5d} {sum(d) / len(d):10.1f} {min(d):10.1f} {max(d):10.1f}"
            for c in cnames:
                vals = [counters[(x[0], c)] for x in sel if (x[0], c) in counters]
                row += f" {sum(vals) / len(vals):18.6g}" if vals else f" {'-':>18s}"
            print(row)


def main():
    args = parse()
    if args.summarize:
        summarize(args.summarize, args.launches)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the step has no cross-GPU exchange "
              f"and each GPU's share is the single-GPU workload", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    from workloads import configs, gen

    wl = configs.BY_NAME[args.workload]
    # the oracle runs first, in forked host processes, before anything initializes the GPU
    cpu = None if args.no_cpu_baseline else cpu_baseline(wl, args.cpu_seconds)
    if cpu is not None:
        log(f"cpu baseline: {cpu['value']:.0f} state-updates/s on {cpu['cores']} cores")
    import torch

    import quantized_delta_rule_02_amd as sq
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
    log(f"state warm-up ({args.state_warmup} fp32 steps) + pack: {time.perf_counter() - t0:.1f} s")

    batches = [inputs(s) for s in (1, 2)]
    extras = {}
    if not args.no_extras:
        # the same update on other state formats, same inputs: float32 states and uniform INT8 per-row states
        q1, k1, v1, b1 = batches[0]
        ms32 = time_calls(lambda: sq.sq_fp32_step(form, H, dk, dv, B, 0, L, B, ident, S, q1, k1, v1, gate, b1, y),
                          args.steps)
        by32 = per_state_bytes(dk, dv, form, 4 * dk * dv)
        extras["fp32_step"] = {"ms": ms32, "state_updates_per_s": n_states / (ms32 / 1e3),
                               "GBps": n_states * by32 / (ms32 / 1e3) / 1e9, "state_bytes": 4 * dk * dv}
        codes8, scales8 = int8_states(S, n_states, dk, dv, chunk=8192)
        ms8 = time_calls(lambda: sq.sq_int8_step(form, H, dk, dv, B, 0, L, B, ident, codes8, scales8, q1, k1, v1,
                                                 gate, b1, y), args.steps)
        by8 = per_state_bytes(dk, dv, form, dk * dv + 4 * dk)
        extras["int8_step"] = {"ms": ms8, "state_updates_per_s": n_states / (ms8 / 1e3),
                               "GBps": n_states * by8 / (ms8 / 1e3) / 1e9, "state_bytes": dk * dv + 4 * dk}
        del codes8, scales8
    del S
    torch.cuda.empty_cache()
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
    flops = algorithmic_flops(per_step, dk, dv, len(wl.grid))
    tflops = flops / (ms / 1e3) / 1e12
    profiled = wl.name == PROFILED_WORKLOAD
    traffic = traffic_per_launch() if profiled else None
    valu_per_wave = _profile_value(VALU_FILE, "valu_per_wave") if profiled else None
    waves = per_step * 4                                  # four wave64 per 128x128 state
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
        # HBM roofline of the step kernel (the benchmark spec's measure); the kernel itself is bound by VALU
        # issue (the exact column fit), reported beside it
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS,
                     "traffic": None if traffic is None else traffic,
                     "algorithmic_bytes_per_launch": alg, "kernel": "k_state<128,128,step>",
                     "launch_ms": ms,
                     "valu": {"achieved": tflops, "peak": ALU_PEAK_TFLOPS, "unit": "TFLOP/s",
                              "frac": tflops / ALU_PEAK_TFLOPS, "algorithmic_flops_per_launch": flops,
                              "instructions_per_launch": None if valu_per_wave is None else valu_per_wave * waves,
                              "wave_instructions_per_cu_per_clock":
                                  None if valu_per_wave is None else valu_per_wave * waves / (ms / 1e3) / (256 * 2.4e9),
                              "issue_peak": 2.0,
                              "fma_probe": valu_ceiling(sq, torch, dev)}},
        "wall_s_timed": wall,
    }
    if not args.no_extras:
        q1, k1, v1, b1 = batches[0]
        # two-stream arrangement: readout kernel on the main stream, fit + pack on a second stream
        aux2 = torch.cuda.Stream()
        mss = time_calls(lambda: sq.sq_state_step(pool, 0, L, B, slots, q1, k1, v1, gate, b1, y, stream_aux=aux2,
                                                  flags=sq.SQ_STEP_SPLIT), args.steps)
        # time to y: the main stream's part of a split call (the readout kernels), the fit + pack of the call
        # left running on the second stream; the next call starts after it, so calls never overlap
        cur = torch.cuda.current_stream()
        t_y = 0.0
        for i in range(args.warmup + args.steps):
            a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a0.record(cur)
            sq.sq_state_step(pool, 0, L, B, slots, q1, k1, v1, gate, b1, y, stream_aux=aux2,
                             flags=sq.SQ_STEP_SPLIT | sq.SQ_STEP_NO_JOIN)
            a1.record(cur)
            cur.wait_stream(aux2)
            torch.cuda.synchronize()
            if i >= args.warmup:
                t_y += a0.elapsed_time(a1)
        # the same two kernels per layer on one stream: readout (A) and fit + pack (B) never overlap, so the
        # sum is their cost without the streams' competition for the CUs
        ms1 = time_calls(lambda: sq.sq_state_step(pool, 0, L, B, slots, q1, k1, v1, gate, b1, y,
                                                  flags=sq.SQ_STEP_SPLIT), args.steps)
        extras["split2"] = {"ms": mss, "state_updates_per_s": per_step / (mss / 1e3),
                            "time_to_y_ms": t_y / args.steps, "one_stream_ms": ms1}
        # candidate-grid sweep on the same packed pool (the grid does not change the layout)
        units = sq.sq_plan_units(plan)["unit_bits"]
        sweep = {}
        grids = {1: (1.0,), 2: (1.0, 0.875), 4: tuple(wl.grid),
                 8: (1.0, 0.9375, 0.875, 0.8125, 0.75, 0.6875, 0.625, 0.5625)}
        for G, grid in grids.items():
            if G == len(wl.grid):
                sweep[str(G)] = ms
                continue
            pg = sq.sq_plan_create(form=form, unit=unit, n_layers=L, n_heads=H, d_k=dk, d_v=dv, widths=wl.widths,
                                   budget_milli=wl.budget_milli, pivot_ppm=wl.pivot_ppm, grid=grid,
                                   gate=gen.unit_gates(wl), impact=gen.impact_scores(wl), unit_bits=units)
            poolg = sq.sq_pool_create(pg, pool_mem, wl.n_slots)
            sweep[str(G)] = time_calls(lambda: sq.sq_state_step(poolg, 0, L, B, slots, q1, k1, v1, gate, b1, y),
                                       args.steps)
            poolg.close()
            pg.close()
        extras["grid_sweep_ms"] = sweep
        # 4.0-bit budget: with widths {4, 6, 8} every non-pivot unit takes 4 bits; same pivots
        p4 = sq.sq_plan_create(form=form, unit=unit, n_layers=L, n_heads=H, d_k=dk, d_v=dv, widths=wl.widths,
                               budget_milli=4000, pivot_ppm=wl.pivot_ppm, grid=wl.grid, gate=gen.unit_gates(wl),
                               impact=gen.impact_scores(wl), unit_bits=np.where(units == 16, 16, 4).astype(np.int32))
        mem4 = torch.empty(sq.sq_pool_bytes(p4, wl.n_slots), dtype=torch.uint8, device=dev)
        pool4 = sq.sq_pool_create(p4, mem4, wl.n_slots)
        Xr = torch.randn(B * H * dk * dv, device=dev)
        for layer in range(L):
            sq.sq_pack(pool4, layer, 1, B, slots, Xr)
        del Xr
        ms4 = time_calls(lambda: sq.sq_state_step(pool4, 0, L, B, slots, q1, k1, v1, gate, b1, y), args.steps)
        alg4 = algorithmic_bytes(p4, B, sq)
        extras["budget_4bit"] = {"ms": ms4, "state_updates_per_s": per_step / (ms4 / 1e3),
                                 "GBps": alg4 / (ms4 / 1e3) / 1e9, "algorithmic_bytes_per_launch": alg4,
                                 "compression_vs_fp32": round(p4.desc["compression_vs_fp32"], 4)}
        pool4.close()
        p4.close()
        del mem4
        # 4.0-bit budget over {2, 3, 4, 6, 8}: the planner mixes widths (calibrated like the main plan)
        wm = configs.SERVING_4_MIXED
        pm = sq.sq_plan_create(form=form, unit=unit, n_layers=L, n_heads=H, d_k=dk, d_v=dv, widths=wm.widths,
                               budget_milli=wm.budget_milli, pivot_ppm=wm.pivot_ppm, grid=wm.grid,
                               gate=gen.unit_gates(wm), impact=gen.impact_scores(wm), calib_seed=gen.calib_seed(wm),
                               calib_segments=wm.calib_segments, calib_len=wm.calib_len)
        memm = torch.empty(sq.sq_pool_bytes(pm, wl.n_slots), dtype=torch.uint8, device=dev)
        poolm = sq.sq_pool_create(pm, memm, wl.n_slots)
        Xr = torch.randn(B * H * dk * dv, device=dev)
        for layer in range(L):
            sq.sq_pack(poolm, layer, 1, B, slots, Xr)
        del Xr
        msm = time_calls(lambda: sq.sq_state_step(poolm, 0, L, B, slots, q1, k1, v1, gate, b1, y), args.steps)
        algm = algorithmic_bytes(pm, B, sq)
        widths_used = {str(int(w)): int(c) for w, c in zip(*np.unique(sq.sq_plan_units(pm)["unit_bits"],
                                                                     return_counts=True))}
        extras["budget_4bit_mixed_widths"] = {"ms": msm, "state_updates_per_s": per_step / (msm / 1e3),
                                              "GBps": algm / (msm / 1e3) / 1e9, "algorithmic_bytes_per_launch": algm,
                                              "compression_vs_fp32": round(pm.desc["compression_vs_fp32"], 4),
                                              "units_per_width": widths_used}
        poolm.close()
        pm.close()
        del memm
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
        extras["copy_reference"] = {"bytes_moved": 2 * src.numel(), "ms": cms,
                                    "GBps": 2 * src.numel() / cms / 1e6}
        del src, dst
        torch.cuda.empty_cache()
        extras["outlier_dual_axis"] = outlier_comparison(sq, torch, dev, args.steps)
        extras["small_pools"] = small_pools(sq, torch, dev)
        out["extras"] = extras
    if cpu is not None:
        out["cpu_baseline"] = cpu
    print(json.dumps(out), flush=True)
    pool.close()
    plan.close()


if __name__ == "__main__":
    main()
