"""GPU parity at the workloads' full sizes, in the launch configuration the benchmark times.

The whole pool (every layer and request of the workload, random request -> slot
map over the workload's slots) is stepped by one library call.  A few sampled
(layer, request) pairs enter the pool from the oracle's quantizer (sq_import)
and are compared with the oracle's step on the same inputs; the rest of the
pool holds library-packed random states that only have to be processed.
"""
import numpy as np
import pytest

import quantized_delta_rule_02_amd as sq
from oracle import quant
from oracle.step import int8_step, packed_step
from workloads import configs, gen

from _parity import compare_step, from_canonical, step_error_bound, to_canonical

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


def _allocation(wl, seed):
    """A seeded allocation for the whole workload: pivots by the planner's count, the rest
    drawn from the candidate widths with the budget's mean (or all narrowest at a 4-bit budget)."""
    from oracle.planner import pivot_count
    g = np.random.default_rng(seed)
    U = wl.n_units
    bits = np.full(U, min(wl.widths), np.int32)
    if len(wl.widths) > 3:
        bits = g.choice(np.asarray(wl.widths, np.int32), size=U)
    elif wl.budget_milli > 1000 * min(wl.widths):
        bits = g.choice(np.asarray(wl.widths, np.int32), size=U, p=[0.25, 0.5, 0.25])
    piv = g.choice(U, pivot_count(wl.pivot_ppm, U), replace=False)
    bits[piv] = 16
    return bits


FULL = [("gdn", configs.GDN_DECODE), ("kda", configs.KDA_DECODE), ("serving6", configs.SERVING_6),
        ("serving4", configs.SERVING_4), ("serving4-mixed", configs.SERVING_4_MIXED),
        ("outlier", configs.OUTLIER), ("outlier-mixed", configs.OUTLIER_MIXED)]


@pytest.mark.parametrize("name,wl", FULL, ids=[c[0] for c in FULL])
def test_full_pool_step_sampled(dev, name, wl):
    import torch
    L, H, dk, dv, B = wl.n_layers, wl.n_heads, wl.d_k, wl.d_v, wl.batch
    say(f"full-size {name}: {L} layers x {B} requests x {H} heads, {dk}x{dv}")
    gates = gen.unit_gates(wl)
    imp = gen.impact_scores(wl)
    ub = _allocation(wl, 11)
    plan = sq.sq_plan_create(form=0 if wl.form == "gdn" else 1, unit=0 if wl.unit == "head" else 1, n_layers=L,
                             n_heads=H, d_k=dk, d_v=dv, widths=wl.widths, budget_milli=wl.budget_milli,
                             pivot_ppm=wl.pivot_ppm, grid=wl.grid, gate=gates, impact=imp, unit_bits=ub)
    row_bits, w = sq.sq_plan_rows(plan)
    mem = torch.zeros(sq.sq_pool_bytes(plan, wl.n_slots), dtype=torch.uint8, device=dev)
    pool = sq.sq_pool_create(plan, mem, wl.n_slots)
    slot_map = gen.slot_map(wl) if wl.n_slots > B else np.random.default_rng(5).permutation(B).astype(np.int32)
    slots = torch.tensor(slot_map, dtype=torch.int32, device=dev)
    # every state: library-packed random float state, one layer at a time
    tg = torch.Generator(device=dev)
    tg.manual_seed(7)
    for l in range(L):
        X = torch.randn(B * H * dk * dv, device=dev, generator=tg)
        sq.sq_pack(pool, l, 1, B, slots, X)
    del X
    # sampled (layer, request) pairs from the oracle's quantizer
    g = np.random.default_rng(3)
    picks = [(int(g.integers(L)), int(g.integers(B))) for _ in range(4)]
    picks = sorted(set(picks))
    rows_of = {}
    P0 = {}
    for (l, b) in picks:
        bits = row_bits[l]
        rows = quant.RowPlan(bits=bits, pivot=bits == 16, w=w[l].astype(np.float64))
        Xh = g.standard_normal((H, dk, dv)) * 2.0
        P = quant.quantize(Xh, rows, wl.grid)
        codes, r, c = to_canonical(P, rows)
        s1 = slots[b:b + 1]
        t = lambda a: torch.tensor(np.ascontiguousarray(a), device=dev)
        sq.sq_import(pool, l, 1, 1, s1, t(codes), t(r), t(c))
        rows_of[(l, b)] = rows
        P0[(l, b)] = P
    # inputs for the whole workload, on the device
    n = L * B * H
    q = torch.randn(n, dk, device=dev, generator=tg)
    k = torch.randn(n, dk, device=dev, generator=tg)
    q = (q / q.norm(dim=1, keepdim=True)).contiguous()
    k = (k / k.norm(dim=1, keepdim=True)).contiguous()
    v = torch.randn(n, dv, device=dev, generator=tg)
    beta = torch.sigmoid(torch.randn(n, device=dev, generator=tg))
    gt = torch.tensor(gates, device=dev)
    gate = (gt[:, None, :].expand(L, B, H) if wl.form == "gdn" else gt[:, None].expand(L, B, H, dk)).contiguous()
    y = torch.zeros(n, dv, device=dev)
    say(f"full-size {name}: stepping {n} states in one call")
    sq.sq_state_step(pool, 0, L, B, slots, q, k, v, gate, beta, y)
    torch.cuda.synchronize()
    worst = None
    for (l, b) in picks:
        s1 = slots[b:b + 1]
        codes = torch.zeros(H * dk * dv, dtype=torch.int16, device=dev)
        r = torch.zeros(H * dk, dtype=torch.int16, device=dev)
        c = torch.zeros(H * dv, dtype=torch.int16, device=dev)
        sq.sq_export(pool, l, 1, 1, s1, codes, r, c)
        torch.cuda.synchronize()
        rows = rows_of[(l, b)]
        Pg = from_canonical(codes.cpu().numpy().reshape(H, dk, dv), r.cpu().numpy().reshape(H, dk),
                            c.cpu().numpy().reshape(H, dv), rows)
        i0 = (l * B + b) * H
        sl = slice(i0, i0 + H)
        qh, kh, vh = q[sl].cpu().numpy(), k[sl].cpu().numpy(), v[sl].cpu().numpy()
        bh = beta[sl].cpu().numpy()
        ah = gate.reshape(n, -1)[sl].cpu().numpy().astype(np.float64)
        ah = ah[:, 0] if wl.form == "gdn" else ah
        P2, yo, Xo = packed_step(P0[(l, b)], rows, qh, kh, vh, ah, bh, wl.grid)
        R = compare_step(Xo, yo, rows, wl.grid, y[sl].cpu().numpy().astype(np.float64), Pg, P2,
                         x_err=step_error_bound(P0[(l, b)], rows, kh, vh, ah, bh))
        assert R.ok(), f"layer {l} request {b}: {R.failures}"
        if worst is None or R.y_rel > worst.y_rel:
            worst = R
    say(f"full-size {name}: {picks} {worst}")
    pool.close()
    plan.close()


def test_int8_comparator_full_outlier_pool(dev):
    """The uniform INT8 per-row comparator over the whole outlier pool, sampled against the oracle."""
    import torch
    wl = configs.OUTLIER
    H, dk, dv, B = wl.n_heads, wl.d_k, wl.d_v, wl.batch
    n = B * H
    say(f"int8 full-size: {n} states {dk}x{dv}")
    tg = torch.Generator(device=dev)
    tg.manual_seed(9)
    S = torch.randn(n, dk, dv, device=dev, generator=tg) * 2
    m = S.abs().amax(dim=2, keepdim=True)
    scales = (m / 127).squeeze(2).contiguous()
    codes_rm = torch.clamp(torch.round(S / (m / 127)), -127, 127).to(torch.int8).reshape(n, dk * dv)
    from _rig import int8_group_order
    order = torch.as_tensor(int8_group_order(dk, dv), device=dev)
    codes = codes_rm[:, order].contiguous()         # the library's group-interleaved order
    del codes_rm
    q = torch.randn(n, dk, device=dev, generator=tg)
    k = torch.randn(n, dk, device=dev, generator=tg)
    q = (q / q.norm(dim=1, keepdim=True)).contiguous()
    k = (k / k.norm(dim=1, keepdim=True)).contiguous()
    v = torch.randn(n, dv, device=dev, generator=tg)
    beta = torch.sigmoid(torch.randn(n, device=dev, generator=tg))
    gate = torch.tensor(gen.unit_gates(wl)[0], device=dev)[None].expand(B, H, dk).contiguous()
    slots = torch.arange(B, dtype=torch.int32, device=dev)
    pick = [0, 517, B - 1]
    def rowmajor(c):
        out = torch.empty_like(c)
        out[:, order] = c
        return out.reshape(-1, dk, dv)

    before = {b: (rowmajor(codes[b * H:(b + 1) * H]).cpu().numpy().astype(np.int64),
                  scales[b * H:(b + 1) * H].cpu().numpy().astype(np.float64)) for b in pick}
    y = torch.zeros(n, dv, device=dev)
    sq.sq_int8_step(1, H, dk, dv, B, 0, 1, B, slots, codes, scales, q, k, v, gate, beta, y)
    torch.cuda.synchronize()
    for b in pick:
        sl = slice(b * H, (b + 1) * H)
        Q0, s0 = before[b]
        Q1, s1, yo, X = int8_step(Q0, s0, q[sl].cpu().numpy(), k[sl].cpu().numpy(), v[sl].cpu().numpy(),
                                  gate[b].cpu().numpy().astype(np.float64), beta[sl].cpu().numpy())
        yg = y[sl].cpu().numpy()
        assert np.linalg.norm(yg - yo) / np.linalg.norm(yo) < 1e-5
        sg = scales[sl].cpu().numpy().astype(np.float64)
        assert np.allclose(sg, s1, rtol=1e-5)
        z = X / sg[:, :, None]
        Qz = np.clip(np.rint(z), -127, 127)
        dq = rowmajor(codes[sl]).cpu().numpy().astype(np.int64) - Qz
        near = np.abs(np.abs(z - np.floor(z)) - 0.5) < 1e-3
        assert np.all(np.abs(dq) <= 1) and np.all((dq == 0) | near)
