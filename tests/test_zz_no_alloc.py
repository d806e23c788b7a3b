"""The allocation-free split step (sq_state_step_split_static) through the C ABI.

It runs the split arrangement's two kernels on one stream with the library's
fixed per-GPU scratch, so its readout and pool bytes must equal those of
sq_state_step with SQ_STEP_SPLIT (which allocates its scratch per pool) bit for
bit: two calls in a row, the second over fewer layers and requests, then the
largest call the fixed scratch takes, and a call one request above it, which is
refused before anything is enqueued.
"""
import numpy as np
import pytest

import quantized_delta_rule_02_amd as sq
from workloads import configs, gen

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


def _plan(wl, n_layers, unit_bits):
    return sq.sq_plan_create(form=0 if wl.form == "gdn" else 1, unit=0 if wl.unit == "head" else 1,
                             n_layers=n_layers, n_heads=wl.n_heads, d_k=wl.d_k, d_v=wl.d_v, widths=wl.widths,
                             budget_milli=wl.budget_milli, pivot_ppm=wl.pivot_ppm, grid=wl.grid,
                             gate=gen.unit_gates(wl)[:n_layers], impact=gen.impact_scores(wl)[:n_layers],
                             unit_bits=unit_bits)


def _inputs(torch, wl, n_layers, batch, seed):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    n = n_layers * batch * wl.n_heads
    r = lambda m: torch.randn(m, device="cuda", generator=g)
    k = r(n * wl.d_k).view(n, wl.d_k)
    k = (k / k.norm(dim=1, keepdim=True)).reshape(-1)
    n_gate = n * (wl.d_k if wl.form == "kda" else 1)
    gate = torch.rand(n_gate, device="cuda", generator=g) * 0.2 + 0.8
    beta = torch.rand(n, device="cuda", generator=g)
    return r(n * wl.d_k), k, r(n * wl.d_v), gate, beta


def test_split_static_equals_split_on_two_calls():
    import torch
    wl = configs.SERVING_6
    nL, n_slots = 3, 10
    say(f"split_static vs split: {nL} layers, {n_slots} slots, {wl.n_heads} heads {wl.d_k}x{wl.d_v}")
    g = np.random.default_rng(21)
    ub = g.choice(np.asarray(wl.widths, np.int32), size=nL * wl.n_heads).astype(np.int32)
    ub[g.choice(ub.size, 2, replace=False)] = 16
    plan = _plan(wl, nL, ub)
    nbytes = sq.sq_pool_bytes(plan, n_slots)
    mem_a = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    pool_a = sq.sq_pool_create(plan, mem_a, n_slots)
    all_slots = torch.arange(n_slots, dtype=torch.int32, device="cuda")
    tg = torch.Generator(device="cuda")
    tg.manual_seed(4)
    X = torch.randn(nL * n_slots * wl.n_heads * wl.d_k * wl.d_v, device="cuda", generator=tg) * 2.0
    sq.sq_pack(pool_a, 0, nL, n_slots, all_slots, X)
    torch.cuda.synchronize()
    mem_b = mem_a.clone()
    pool_b = sq.sq_pool_create(plan, mem_b, n_slots)
    calls = [(0, 3, 8, 5), (1, 1, 3, 6)]       # (layer0, n_layers, batch, seed): the second is smaller
    for layer0, n_layers, batch, seed in calls:
        say(f"call layers [{layer0}, {layer0 + n_layers}) x {batch} requests")
        slots = torch.tensor(g.permutation(n_slots)[:batch].astype(np.int32), device="cuda")
        q, k, v, gate, beta = _inputs(torch, wl, n_layers, batch, seed)
        n_y = n_layers * batch * wl.n_heads * wl.d_v
        y_a = torch.full((n_y,), float("nan"), device="cuda")
        y_b = torch.full((n_y,), float("nan"), device="cuda")
        sq.sq_state_step(pool_a, layer0, n_layers, batch, slots, q, k, v, gate, beta, y_a, flags=sq.SQ_STEP_SPLIT)
        sq.sq_state_step_split_static(pool_b, layer0, n_layers, batch, slots, q, k, v, gate, beta, y_b)
        torch.cuda.synchronize()
        assert torch.isfinite(y_a).all()
        assert torch.equal(y_a, y_b)
        assert torch.equal(mem_a, mem_b)
    pool_a.close()
    pool_b.close()
    plan.close()


def test_split_static_at_and_above_its_limit():
    """The largest call the fixed scratch holds (n_layers * batch * H * d_v equal to the limit) runs and
    equals the allocating split step; one request more is refused with SQ_ERR_ARG, nothing touched."""
    import torch
    wl = configs.GDN_DECODE
    per_req = wl.n_heads * wl.d_v
    b_max = sq.SQ_SPLIT_STATIC_MAX_FLOATS // per_req
    assert b_max * per_req == sq.SQ_SPLIT_STATIC_MAX_FLOATS
    n_slots = b_max + 1
    say(f"split_static limit: {b_max} requests x {wl.n_heads} heads, {n_slots} slots")
    ub = np.full(wl.n_heads, min(wl.widths), np.int32)
    ub[0] = 16
    plan = _plan(wl, 1, ub)
    nbytes = sq.sq_pool_bytes(plan, n_slots)
    mem_a = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    pool_a = sq.sq_pool_create(plan, mem_a, n_slots)
    slots = torch.arange(n_slots, dtype=torch.int32, device="cuda")
    tg = torch.Generator(device="cuda")
    tg.manual_seed(9)
    X = torch.randn(n_slots * wl.n_heads * wl.d_k * wl.d_v, device="cuda", generator=tg)
    sq.sq_pack(pool_a, 0, 1, n_slots, slots, X)
    del X
    torch.cuda.synchronize()
    mem_b = mem_a.clone()
    pool_b = sq.sq_pool_create(plan, mem_b, n_slots)
    q, k, v, gate, beta = _inputs(torch, wl, 1, n_slots, 12)
    y_a = torch.zeros(n_slots * per_req, device="cuda")
    y_b = torch.zeros(n_slots * per_req, device="cuda")
    sq.sq_state_step(pool_a, 0, 1, b_max, slots, q, k, v, gate, beta, y_a, flags=sq.SQ_STEP_SPLIT)
    sq.sq_state_step_split_static(pool_b, 0, 1, b_max, slots, q, k, v, gate, beta, y_b)
    torch.cuda.synchronize()
    assert torch.equal(y_a, y_b)
    assert torch.equal(mem_a, mem_b)
    y_b.fill_(7.0)
    with pytest.raises(sq.StepQError) as err:
        sq.sq_state_step_split_static(pool_b, 0, 1, n_slots, slots, q, k, v, gate, beta, y_b)
    assert err.value.status == -1 and "above the fixed" in str(err.value)
    torch.cuda.synchronize()
    assert bool((y_b == 7.0).all())
    assert torch.equal(mem_a, mem_b)
    pool_a.close()
    pool_b.close()
    plan.close()
