"""The C-ABI library on the CPU: exports, the C++ planner against the oracle planner,
the built-in calibration generator, argument validation and plan serialization.
No device calls are made here."""
import ctypes
import json
import os
import subprocess
from dataclasses import replace

import numpy as np
import pytest

import quantized_delta_rule_02_amd as sq
from quantized_delta_rule_02_amd import _lib
from oracle import planner as oplanner
from oracle import quant as oquant
from workloads import configs, gen

HERE = os.path.dirname(os.path.abspath(__file__))


def test_library_exports_every_declared_function():
    lib = _lib.load()
    names = _lib.header_functions()
    assert len(names) >= 20
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True, text=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    assert set(names) <= exported


def test_header_constants_match_the_binding():
    """Every numeric #define SQ_* in include/stepq.h has the same value in the Python binding."""
    import re
    found = 0
    for line in open(_lib.HEADER):
        m = re.match(r"#define\s+(SQ_\w+)\s+(.*?)\s*(/\*.*)?$", line)
        if not m or not hasattr(_lib, m.group(1)):
            continue
        expr = re.sub(r"(\d+)(ll|u)\b", r"\1", m.group(2))
        assert re.fullmatch(r"[-0-9 <()]+", expr), line
        assert eval(expr) == getattr(_lib, m.group(1)), line
        found += 1
    assert found >= 12 and _lib.SQ_SPLIT_STATIC_MAX_FLOATS == 8 << 20


def test_alternative_names_are_the_same_calls():
    """sq_plan_info is sq_plan_describe; sq_pool_bind / sq_pool_release validate like sq_pool_create /
    sq_pool_destroy (host checks only, no device memory)."""
    wl = configs.GDN_DECODE
    plan = sq.sq_plan_create(**_plan_kw(wl, 1))
    assert sq.sq_plan_info(plan) == sq.sq_plan_describe(plan)
    lib = _lib.load()
    out = ctypes.c_void_p()
    assert lib.sq_pool_bind(plan.handle, None, 16, 1, ctypes.byref(out)) == -1 and not out.value
    lib.sq_pool_release(None)          # a NULL pool is ignored
    plan.close()


def test_supported_shapes_cover_the_workloads():
    shapes = set(sq.sq_supported_shapes())
    for w in configs.ALL:
        assert (w.d_k, w.d_v) in shapes


def _plan_kw(wl, n_layers):
    return dict(form=0 if wl.form == "gdn" else 1, unit=0 if wl.unit == "head" else 1, n_layers=n_layers,
                n_heads=wl.n_heads, d_k=wl.d_k, d_v=wl.d_v, widths=wl.widths, budget_milli=wl.budget_milli,
                pivot_ppm=wl.pivot_ppm, grid=wl.grid, gate=gen.unit_gates(wl)[:n_layers])


def test_calibration_generator_matches_numpy_generator():
    seed = gen.calib_seed(configs.KDA_DECODE)
    for (l, h) in ((0, 0), (3, 17)):
        a = sq.sq_calib_generate(seed, l, h, 3, 7, 128, 128)
        b = gen.calib_traces(seed, l, h, 3, 7, 128, 128)
        for x, y in zip(a, b):
            assert x.shape == y.shape
            # same Philox stream; transcendental functions may differ in the last bit
            assert np.max(np.abs(x - y)) <= 2e-7 * max(1.0, np.max(np.abs(y)))
            assert np.mean(x == y) > 0.99


CASES = [("tiny", configs.TINY, 1, 2, 16, 0), ("gdn", configs.GDN_DECODE, 1, 2, 24, 0),
         ("kda", configs.KDA_DECODE, 1, 2, 16, 0), ("serving", configs.SERVING_6, 2, 1, 16, 0),
         ("outlier", configs.OUTLIER, 1, 1, 12, 0), ("gdn-row-absmax", configs.GDN_DECODE, 1, 2, 24, 1),
         ("kda-row-absmax", configs.KDA_DECODE, 1, 2, 16, 1),
         ("serving4-mixed", configs.SERVING_4_MIXED, 2, 1, 16, 0), ("outlier-mixed", configs.OUTLIER_MIXED, 1, 1, 12, 0),
         ("kda64", configs.KDA_64, 1, 2, 16, 0),
         # the workloads' full calibration (32 segments of 512 tokens) on two heads
         ("gdn-2h-full-calibration", replace(configs.GDN_DECODE, n_heads=2), 1, 32, 512, 0),
         ("kda-2h-full-calibration", replace(configs.KDA_DECODE, n_heads=2), 1, 32, 512, 0)]


@pytest.mark.parametrize("name,wl,nL,S,T,qz", CASES, ids=[c[0] for c in CASES])
def test_cpp_planner_matches_oracle_planner(name, wl, nL, S, T, qz):
    seed = gen.calib_seed(wl)
    tr = {(l, h): gen.calib_traces(seed, l, h, S, T, wl.d_k, wl.d_v) for l in range(nL) for h in range(wl.n_heads)}
    stack = lambda i: np.stack([np.stack([tr[(l, h)][i] for h in range(wl.n_heads)]) for l in range(nL)])
    calib = tuple(stack(i) for i in range(4))
    imp = gen.impact_scores(wl)[:nL]
    p = sq.sq_plan_create(**_plan_kw(wl, nL), impact=imp, calib=calib, calib_segments=S, calib_len=T,
                          n_threads=4, quantizer=qz)
    assert p.desc["quantizer"] == qz
    u = sq.sq_plan_units(p)
    o = oplanner.make_plan(wl.form, wl.unit, nL, wl.n_heads, wl.d_k, wl.d_v, wl.widths, wl.budget_milli,
                           wl.pivot_ppm, wl.grid, gen.unit_gates(wl)[:nL], lambda l, h: tr[(l, h)], impact=imp,
                           mode=oquant.MODES[qz])
    assert np.allclose(u["lbar"], o.lbar, rtol=1e-12, atol=0)
    assert np.allclose(u["lifetime"], o.L, rtol=1e-12, atol=0)
    assert np.allclose(u["distortion"], o.D, rtol=1e-9, atol=1e-300)
    piv_c = np.nonzero(u["unit_bits"] == 16)[0]
    assert np.array_equal(piv_c, o.pivot_units)
    same = np.mean(u["unit_bits"] == o.unit_bits)
    if same < 1.0:
        # only a near-tie of the objective may separate the two allocations
        rest = np.nonzero(o.unit_bits != 16)[0]
        cost = o.L[rest, None] * o.D[rest]
        idx = lambda bits: np.searchsorted(np.asarray(wl.widths), bits[rest])
        obj_c = np.sum(np.take_along_axis(cost, idx(u["unit_bits"])[:, None], 1))
        obj_o = np.sum(np.take_along_axis(cost, idx(o.unit_bits)[:, None], 1))
        assert abs(obj_c - obj_o) <= 1e-9 * abs(obj_o)
        assert np.sum(u["unit_bits"][rest]) * 1000 <= wl.budget_milli * len(rest)
    rb, w = sq.sq_plan_rows(p)
    assert np.array_equal(rb, np.where(o.pivot, 16, o.bits))
    assert np.allclose(w, imp)


def test_planner_estimates_impact_like_the_oracle():
    wl = configs.GDN_DECODE
    S, T = 2, 16
    seed = gen.calib_seed(wl)
    tr = {(0, h): gen.calib_traces(seed, 0, h, S, T, wl.d_k, wl.d_v) for h in range(wl.n_heads)}
    calib = tuple(np.stack([tr[(0, h)][i] for h in range(wl.n_heads)])[None] for i in range(4))
    p = sq.sq_plan_create(**_plan_kw(wl, 1), calib=calib, calib_segments=S, calib_len=T)
    _, w = sq.sq_plan_rows(p)
    for h in (0, 5, 31):
        q, k, v, b = tr[(0, h)]
        ref = oplanner.impact_from_traces(q, k, b, gen.unit_gates(wl)[0, h])
        assert np.allclose(w[0, h], ref, rtol=1e-6)


def test_builtin_generator_plan_equals_supplied_traces():
    wl = configs.GDN_DECODE
    S, T = 2, 8
    seed = gen.calib_seed(wl)
    imp = gen.impact_scores(wl)[:1]
    p1 = sq.sq_plan_create(**_plan_kw(wl, 1), impact=imp, calib_seed=seed, calib_segments=S, calib_len=T)
    tr = [sq.sq_calib_generate(seed, 0, h, S, T, wl.d_k, wl.d_v) for h in range(wl.n_heads)]
    calib = tuple(np.stack([t[i] for t in tr])[None] for i in range(4))
    p2 = sq.sq_plan_create(**_plan_kw(wl, 1), impact=imp, calib=calib, calib_segments=S, calib_len=T)
    assert np.array_equal(sq.sq_plan_units(p1)["unit_bits"], sq.sq_plan_units(p2)["unit_bits"])
    assert np.array_equal(sq.sq_plan_units(p1)["distortion"], sq.sq_plan_units(p2)["distortion"])


def test_fixed_allocation_and_layout_accounting_match_the_pages():
    """Serving pool at a 6-bit average with 1% FP16 pivot heads: the pages report 5.03x and 6.3 bits."""
    figs = json.load(open(os.path.join(HERE, "golden", "pages_figures.json")))
    wl = configs.SERVING_6
    U = wl.n_units
    n_piv = oplanner.pivot_count(wl.pivot_ppm, U)
    bits = np.full(U, 6, np.int32)
    bits[:n_piv] = 16
    p = sq.sq_plan_create(**_plan_kw(wl, wl.n_layers), impact=gen.impact_scores(wl), unit_bits=bits)
    d = p.desc
    assert d["n_pivot_units"] == 12
    assert abs(d["compression_vs_fp32"] - figs["compression_6bit"]["value"]) <= 0.01 * figs["compression_6bit"]["value"]
    assert abs(d["stored_bits_per_entry"] - figs["effective_bits_6bit"]["value"]) <= 0.1
    # record sizes: 16 groups of 8 rows x 128 columns x 6 bits, two binary16 vectors, 256-byte padding
    assert d["slot_bytes"] == 1140 * 12800 + 12 * 33280


def test_argument_validation_status_codes():
    wl = configs.GDN_DECODE
    kw = _plan_kw(wl, 1)
    kw.update(impact=gen.impact_scores(wl)[:1], unit_bits=np.full(32, 6, np.int32))
    for bad, status in ((dict(form=2), -1), (dict(unit=5), -1), (dict(d_k=96, impact=None), -3), (dict(widths=(4, 5)), -3),
                        (dict(widths=(4, 4)), -1), (dict(grid=[]), None), (dict(pivot_ppm=-1), -1),
                        (dict(quantizer=2), -1)):
        args = dict(kw)
        args.update(bad)
        if status is None:
            with pytest.raises(ValueError):
                sq.sq_plan_create(**args)
            continue
        with pytest.raises(sq.StepQError) as e:
            sq.sq_plan_create(**args)
        assert e.value.status == status, bad
    g = gen.unit_gates(wl)[:1].copy()
    g[0, 3] = 1.5
    with pytest.raises(sq.StepQError):
        sq.sq_plan_create(**dict(kw, gate=g))
    ub = np.full(32, 6, np.int32)
    ub[2] = 5
    with pytest.raises(sq.StepQError):
        sq.sq_plan_create(**dict(kw, unit_bits=ub))
    lib = _lib.load()
    # calls that fail validation before touching the device
    assert lib.sq_state_step(None, 0, 1, 1, None, None, None, None, None, None, None, None, None, 0) == -1
    assert lib.sq_pack(None, 0, 1, 1, None, None, None) == -1
    assert lib.sq_copy(None, None, 16, None) == -1
    n_fma, fit = ctypes.c_uint64(0), ctypes.c_int32(0)
    assert lib.sq_valu_probe(4, 1, None, ctypes.byref(n_fma), ctypes.byref(fit), None) == -1
    for waves, blocks in ((0, 1), (9, 1), (4, 0)):
        assert lib.sq_valu_probe(waves, blocks, ctypes.c_void_p(0x10000), ctypes.byref(n_fma), ctypes.byref(fit),
                                 None) == -1
    assert lib.sq_int8_step(0, 32, 96, 128, 4, 0, 1, 1, None, None, None, None, None, None, None, None, None,
                            None) == -3
    # comparator state arrays: INT8 codes 16-byte aligned (one access per lane and group), FP32 states
    # aligned for one access per lane and row (never dereferenced here)
    fake = ctypes.c_void_p(0x10000)
    odd = ctypes.c_void_p(0x10001)
    assert lib.sq_int8_step(0, 32, 128, 128, 4, 0, 1, 1, fake, odd, fake, fake, fake, fake, fake, fake, fake,
                            None) == -1
    assert lib.sq_int8_step(0, 32, 128, 128, 4, 0, 1, 1, fake, ctypes.c_void_p(0x10008), fake, fake, fake, fake,
                            fake, fake, fake, None) == -1
    assert lib.sq_fp32_step(0, 32, 128, 128, 4, 0, 1, 1, fake, ctypes.c_void_p(0x10004), fake, fake, fake, fake,
                            fake, fake, None) == -1
    assert lib.sq_plan_create(None, ctypes.byref(ctypes.c_void_p())) == -1
    assert sq.StepQError(-1, "x").status == -1


@pytest.mark.parametrize("qz", [0, 1])
def test_plan_save_load_roundtrip(qz):
    wl = configs.KDA_DECODE
    p = sq.sq_plan_create(**_plan_kw(wl, 1), impact=gen.impact_scores(wl)[:1], calib_seed=3, calib_segments=1,
                          calib_len=8, quantizer=qz)
    blob = sq.sq_plan_save(p)
    q = sq.sq_plan_load(blob)
    assert q.desc == p.desc
    for key in ("lbar", "lifetime", "distortion", "unit_bits"):
        assert np.array_equal(sq.sq_plan_units(p)[key], sq.sq_plan_units(q)[key])
    assert sq.sq_plan_save(q) == blob
    bad = bytearray(blob)
    bad[20] ^= 0xFF
    with pytest.raises(sq.StepQError):
        sq.sq_plan_load(bytes(bad[:-3]))
    with pytest.raises(sq.StepQError):
        sq.sq_plan_load(b"not a plan")
