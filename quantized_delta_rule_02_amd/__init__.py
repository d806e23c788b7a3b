"""Python binding of libstepq (the MI355X quantized gated-delta state step).

Thin marshalling over the C ABI in include/stepq.h: every function here has the
name of the C call it wraps, converts its arguments (numpy arrays for host
data, torch CUDA tensors for device data, torch streams) and raises StepQError
on a negative status.  All computation runs in the library's HIP kernels and
C++ runtime; there is no Python or CPU fallback.
"""
from __future__ import annotations

import ctypes
from ctypes import POINTER, byref, c_double, c_float, c_int32, c_size_t, c_uint64, c_void_p

import numpy as np

from . import _lib
from ._lib import (SQ_FORM_GDN, SQ_FORM_KDA, SQ_PIVOT_BITS, SQ_QUANT_DUAL_AXIS, SQ_QUANT_ROW_ABSMAX,
                   SQ_SPLIT_STATIC_MAX_FLOATS, SQ_STEP_NO_JOIN, SQ_STEP_SPLIT, SQ_STEP_VALIDATE, SQ_UNIT_HEAD,
                   SQ_UNIT_ROW)

__all__ = [
    "StepQError", "Plan", "Pool", "sq_plan_create", "sq_plan_describe", "sq_plan_info", "sq_pool_bind", "sq_pool_release", "sq_plan_units", "sq_plan_rows",
    "sq_plan_save", "sq_plan_load", "sq_calib_generate", "sq_pool_bytes", "sq_pool_create", "sq_state_step", "sq_state_step_split_static",
    "sq_pack", "sq_unpack", "sq_export", "sq_import", "sq_int8_step", "sq_fp32_step", "sq_copy", "sq_valu_probe",
    "sq_supported_shapes", "SQ_FORM_GDN", "SQ_FORM_KDA", "SQ_UNIT_HEAD", "SQ_UNIT_ROW", "SQ_STEP_SPLIT",
    "SQ_STEP_VALIDATE", "SQ_STEP_NO_JOIN", "SQ_SPLIT_STATIC_MAX_FLOATS", "SQ_PIVOT_BITS", "SQ_QUANT_DUAL_AXIS", "SQ_QUANT_ROW_ABSMAX",
]


class StepQError(RuntimeError):
    def __init__(self, status: int, where: str):
        lib = _lib.load()
        self.status = status
        msg = lib.sq_last_error().decode()
        super().__init__(f"{where}: {lib.sq_status_str(status).decode()} ({status}): {msg}")


def _check(status: int, where: str):
    if status != 0:
        raise StepQError(status, where)


def _fptr(a, dtype=np.float32, ctype=c_float):
    if a is None:
        return None, None
    arr = np.ascontiguousarray(a, dtype=dtype)
    return arr, arr.ctypes.data_as(POINTER(ctype))


# ---------------------------------------------------------------- plan

class Plan:
    """Owns an sq_plan handle (host memory)."""

    def __init__(self, handle: int):
        self.handle = c_void_p(handle)
        self.desc = sq_plan_describe(self)

    def close(self):
        if self.handle and self.handle.value:
            _lib.load().sq_plan_destroy(self.handle)
            self.handle = c_void_p(None)

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def sq_plan_create(*, form, unit, n_layers, n_heads, d_k, d_v, widths, budget_milli, pivot_ppm, grid, gate,
                   impact=None, unit_bits=None, calib=None, calib_seed=0, calib_segments=32, calib_len=512,
                   n_threads=0, quantizer=SQ_QUANT_DUAL_AXIS) -> Plan:
    """Run the offline planner.  gate/impact/unit_bits/calib are host arrays (calib = (q, k, v, beta))."""
    lib = _lib.load()
    cfg = _lib.SqPlanCfg()
    cfg.form, cfg.unit = int(form), int(unit)
    cfg.n_layers, cfg.n_heads, cfg.d_k, cfg.d_v = int(n_layers), int(n_heads), int(d_k), int(d_v)
    widths = list(widths)
    if not 1 <= len(widths) <= _lib.SQ_MAX_WIDTHS:
        raise ValueError(f"between 1 and {_lib.SQ_MAX_WIDTHS} candidate widths")
    cfg.n_widths = len(widths)
    for i, b in enumerate(widths):
        cfg.widths[i] = int(b)
    cfg.budget_milli, cfg.pivot_ppm = int(budget_milli), int(pivot_ppm)
    grid = list(grid)
    if not 1 <= len(grid) <= _lib.SQ_MAX_GRID:
        raise ValueError("between 1 and 8 grid candidates")
    cfg.n_grid = len(grid)
    for i, g in enumerate(grid):
        cfg.grid[i] = float(g)
    keep = []
    n_gate = n_layers * n_heads * (d_k if form == SQ_FORM_KDA else 1)
    g_arr, cfg.gate = _fptr(gate)
    if g_arr.size != n_gate:
        raise ValueError(f"gate has {g_arr.size} values, expected {n_gate}")
    keep.append(g_arr)
    if impact is not None:
        i_arr, cfg.impact = _fptr(impact)
        if i_arr.size != n_layers * n_heads * d_k:
            raise ValueError("impact must have L * H * d_k values")
        keep.append(i_arr)
    if unit_bits is not None:
        u_arr, cfg.unit_bits = _fptr(unit_bits, np.int32, c_int32)
        n_units = n_layers * n_heads * (d_k if unit == SQ_UNIT_ROW else 1)
        if u_arr.size != n_units:
            raise ValueError(f"unit_bits has {u_arr.size} values, expected {n_units}")
        keep.append(u_arr)
    if calib is not None:
        q, k, v, b = calib
        nt = n_layers * n_heads * calib_segments * calib_len
        arrs = []
        for a, per in ((q, d_k), (k, d_k), (v, d_v), (b, 1)):
            arr, _ = _fptr(a)
            if arr.size != nt * per:
                raise ValueError("calibration trace size does not match L * H * segments * len")
            arrs.append(arr)
        keep.extend(arrs)
        cfg.calib_q = arrs[0].ctypes.data_as(POINTER(c_float))
        cfg.calib_k = arrs[1].ctypes.data_as(POINTER(c_float))
        cfg.calib_v = arrs[2].ctypes.data_as(POINTER(c_float))
        cfg.calib_beta = arrs[3].ctypes.data_as(POINTER(c_float))
    cfg.calib_seed = int(calib_seed)
    cfg.calib_segments, cfg.calib_len, cfg.n_threads = int(calib_segments), int(calib_len), int(n_threads)
    cfg.quantizer = int(quantizer)
    out = c_void_p()
    _check(lib.sq_plan_create(byref(cfg), byref(out)), "sq_plan_create")
    return Plan(out.value)


def sq_plan_describe(plan: Plan, _entry="sq_plan_describe") -> dict:
    d = _lib.SqPlanDesc()
    _check(getattr(_lib.load(), _entry)(plan.handle, byref(d)), _entry)
    out = {name: getattr(d, name) for name, _ in d._fields_}
    out["widths"] = [int(d.widths[i]) for i in range(d.n_widths)]
    return out


def sq_plan_info(plan: Plan) -> dict:
    """sq_plan_describe under its other name (the C ABI exports both)."""
    return sq_plan_describe(plan, _entry="sq_plan_info")


def sq_plan_units(plan: Plan) -> dict:
    d = plan.desc
    U = d["n_units"]
    nw = len(d["widths"])
    lbar = np.zeros(U, np.float64)
    L = np.zeros(U, np.float64)
    D = np.zeros((U, nw), np.float64)
    ub = np.zeros(U, np.int32)
    _check(_lib.load().sq_plan_units(plan.handle, lbar.ctypes.data_as(POINTER(c_double)),
                                     L.ctypes.data_as(POINTER(c_double)), D.ctypes.data_as(POINTER(c_double)),
                                     ub.ctypes.data_as(POINTER(c_int32))), "sq_plan_units")
    return {"lbar": lbar, "lifetime": L, "distortion": D, "unit_bits": ub}


def sq_plan_rows(plan: Plan):
    d = plan.desc
    n = d["n_layers"] * d["n_heads"] * d["d_k"]
    rb = np.zeros(n, np.int32)
    w = np.zeros(n, np.float32)
    _check(_lib.load().sq_plan_rows(plan.handle, rb.ctypes.data_as(POINTER(c_int32)),
                                    w.ctypes.data_as(POINTER(c_float))), "sq_plan_rows")
    shape = (d["n_layers"], d["n_heads"], d["d_k"])
    return rb.reshape(shape), w.reshape(shape)


def sq_plan_save(plan: Plan) -> bytes:
    lib = _lib.load()
    n = c_size_t(0)
    _check(lib.sq_plan_save(plan.handle, None, byref(n)), "sq_plan_save")
    buf = ctypes.create_string_buffer(n.value)
    _check(lib.sq_plan_save(plan.handle, buf, byref(n)), "sq_plan_save")
    return buf.raw[: n.value]


def sq_plan_load(data: bytes) -> Plan:
    out = c_void_p()
    buf = ctypes.create_string_buffer(bytes(data), len(data))
    _check(_lib.load().sq_plan_load(buf, len(data), byref(out)), "sq_plan_load")
    return Plan(out.value)


def sq_calib_generate(seed, layer, head, n_seg, seg_len, d_k, d_v):
    q = np.zeros((n_seg, seg_len, d_k), np.float32)
    k = np.zeros_like(q)
    v = np.zeros((n_seg, seg_len, d_v), np.float32)
    b = np.zeros((n_seg, seg_len), np.float32)
    P = POINTER(c_float)
    _check(_lib.load().sq_calib_generate(int(seed), layer, head, n_seg, seg_len, d_k, d_v, q.ctypes.data_as(P),
                                         k.ctypes.data_as(P), v.ctypes.data_as(P), b.ctypes.data_as(P)),
           "sq_calib_generate")
    return q, k, v, b


def sq_supported_shapes():
    lib = _lib.load()
    n = lib.sq_supported_shapes(None, 0)
    buf = (c_int32 * (2 * n))()
    lib.sq_supported_shapes(buf, n)
    return [(buf[2 * i], buf[2 * i + 1]) for i in range(n)]


# ---------------------------------------------------------------- device helpers

def _dev(t, dtype, numel, name):
    """Device pointer of a contiguous CUDA tensor with at least numel elements of dtype."""
    import torch
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.numel() < numel:
        raise ValueError(f"{name} has {t.numel()} elements, needs {numel}")
    return c_void_p(t.data_ptr())


def _stream(s):
    import torch
    if s is None:
        s = torch.cuda.current_stream()
    return c_void_p(s.cuda_stream if hasattr(s, "cuda_stream") else int(s))


class Pool:
    """An sq_pool bound to caller-owned device memory (the tensor is kept alive here)."""

    def __init__(self, handle: int, plan: Plan, memory, n_slots: int):
        self.handle = c_void_p(handle)
        self.plan = plan
        self.memory = memory
        self.n_slots = n_slots
        d = plan.desc
        self.L, self.H, self.d_k, self.d_v, self.form = d["n_layers"], d["n_heads"], d["d_k"], d["d_v"], d["form"]

    def close(self):
        if self.handle and self.handle.value:
            _lib.load().sq_pool_destroy(self.handle)
            self.handle = c_void_p(None)

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def sq_pool_bytes(plan: Plan, n_slots: int) -> int:
    n = c_size_t(0)
    _check(_lib.load().sq_pool_bytes(plan.handle, n_slots, byref(n)), "sq_pool_bytes")
    return n.value


def sq_pool_create(plan: Plan, memory, n_slots: int, _entry="sq_pool_create") -> Pool:
    """memory: a uint8 CUDA tensor of at least sq_pool_bytes(plan, n_slots) bytes."""
    import torch
    nbytes = sq_pool_bytes(plan, n_slots)
    ptr = _dev(memory, torch.uint8, nbytes, "pool memory")
    out = c_void_p()
    _check(getattr(_lib.load(), _entry)(plan.handle, ptr, memory.numel(), n_slots, byref(out)), _entry)
    return Pool(out.value, plan, memory, n_slots)


def sq_pool_bind(plan: Plan, memory, n_slots: int) -> Pool:
    """sq_pool_create under its other name (the C ABI exports both): binds caller-owned memory."""
    return sq_pool_create(plan, memory, n_slots, _entry="sq_pool_bind")


def sq_pool_release(pool: Pool) -> None:
    """Release a pool's device tables (the C ABI's sq_pool_release); the caller's memory stays."""
    if pool.handle and pool.handle.value:
        _lib.load().sq_pool_release(pool.handle)
        pool.handle = c_void_p(None)


def sq_state_step(pool: Pool, layer0, n_layers, batch, slots, q, k, v, gate, beta, y,
                  stream_main=None, stream_aux=None, flags=0):
    import torch
    n = n_layers * batch * pool.H
    f = torch.float32
    n_gate = n * (pool.d_k if pool.form == SQ_FORM_KDA else 1)
    aux = _stream(stream_aux) if stream_aux is not None else None
    _check(_lib.load().sq_state_step(
        pool.handle, layer0, n_layers, batch, _dev(slots, torch.int32, batch, "slots"),
        _dev(q, f, n * pool.d_k, "q"), _dev(k, f, n * pool.d_k, "k"), _dev(v, f, n * pool.d_v, "v"),
        _dev(gate, f, n_gate, "gate"), _dev(beta, f, n, "beta"), _dev(y, f, n * pool.d_v, "y"),
        _stream(stream_main), aux, int(flags)), "sq_state_step")


def sq_state_step_split_static(pool: Pool, layer0, n_layers, batch, slots, q, k, v, gate, beta, y, stream=None):
    """The split step with the library's fixed per-GPU scratch (no device allocation)."""
    import torch
    n = n_layers * batch * pool.H
    f = torch.float32
    n_gate = n * (pool.d_k if pool.form == SQ_FORM_KDA else 1)
    _check(_lib.load().sq_state_step_split_static(
        pool.handle, layer0, n_layers, batch, _dev(slots, torch.int32, batch, "slots"),
        _dev(q, f, n * pool.d_k, "q"), _dev(k, f, n * pool.d_k, "k"), _dev(v, f, n * pool.d_v, "v"),
        _dev(gate, f, n_gate, "gate"), _dev(beta, f, n, "beta"), _dev(y, f, n * pool.d_v, "y"),
        _stream(stream)), "sq_state_step_split_static")


def sq_pack(pool: Pool, layer0, n_layers, batch, slots, X, stream=None):
    import torch
    n = n_layers * batch * pool.H * pool.d_k * pool.d_v
    _check(_lib.load().sq_pack(pool.handle, layer0, n_layers, batch, _dev(slots, torch.int32, batch, "slots"),
                               _dev(X, torch.float32, n, "X"), _stream(stream)), "sq_pack")


def sq_unpack(pool: Pool, layer0, n_layers, batch, slots, X, stream=None):
    import torch
    n = n_layers * batch * pool.H * pool.d_k * pool.d_v
    _check(_lib.load().sq_unpack(pool.handle, layer0, n_layers, batch, _dev(slots, torch.int32, batch, "slots"),
                                 _dev(X, torch.float32, n, "X"), _stream(stream)), "sq_unpack")


def sq_export(pool: Pool, layer0, n_layers, batch, slots, codes, r, c, stream=None):
    import torch
    n = n_layers * batch * pool.H
    _check(_lib.load().sq_export(pool.handle, layer0, n_layers, batch, _dev(slots, torch.int32, batch, "slots"),
                                 _dev(codes, torch.int16, n * pool.d_k * pool.d_v, "codes"),
                                 _dev(r, torch.int16, n * pool.d_k, "r"), _dev(c, torch.int16, n * pool.d_v, "c"),
                                 _stream(stream)), "sq_export")


def sq_import(pool: Pool, layer0, n_layers, batch, slots, codes, r, c, stream=None):
    import torch
    n = n_layers * batch * pool.H
    _check(_lib.load().sq_import(pool.handle, layer0, n_layers, batch, _dev(slots, torch.int32, batch, "slots"),
                                 _dev(codes, torch.int16, n * pool.d_k * pool.d_v, "codes"),
                                 _dev(r, torch.int16, n * pool.d_k, "r"), _dev(c, torch.int16, n * pool.d_v, "c"),
                                 _stream(stream)), "sq_import")


def sq_int8_step(form, n_heads, d_k, d_v, n_slots, layer0, n_layers, batch, slots, codes, scales,
                 q, k, v, gate, beta, y, stream=None):
    import torch
    n = n_layers * batch * n_heads
    n_states = (layer0 + n_layers) * n_slots * n_heads
    f = torch.float32
    _check(_lib.load().sq_int8_step(
        form, n_heads, d_k, d_v, n_slots, layer0, n_layers, batch, _dev(slots, torch.int32, batch, "slots"),
        _dev(codes, torch.int8, n_states * d_k * d_v, "codes"), _dev(scales, f, n_states * d_k, "scales"),
        _dev(q, f, n * d_k, "q"), _dev(k, f, n * d_k, "k"), _dev(v, f, n * d_v, "v"),
        _dev(gate, f, n * (d_k if form == SQ_FORM_KDA else 1), "gate"), _dev(beta, f, n, "beta"),
        _dev(y, f, n * d_v, "y"), _stream(stream)), "sq_int8_step")


def sq_fp32_step(form, n_heads, d_k, d_v, n_slots, layer0, n_layers, batch, slots, S, q, k, v, gate, beta, y,
                 stream=None):
    import torch
    n = n_layers * batch * n_heads
    n_states = (layer0 + n_layers) * n_slots * n_heads
    f = torch.float32
    _check(_lib.load().sq_fp32_step(
        form, n_heads, d_k, d_v, n_slots, layer0, n_layers, batch, _dev(slots, torch.int32, batch, "slots"),
        _dev(S, f, n_states * d_k * d_v, "S"), _dev(q, f, n * d_k, "q"), _dev(k, f, n * d_k, "k"),
        _dev(v, f, n * d_v, "v"), _dev(gate, f, n * (d_k if form == SQ_FORM_KDA else 1), "gate"),
        _dev(beta, f, n, "beta"), _dev(y, f, n * d_v, "y"), _stream(stream)), "sq_fp32_step")


def sq_copy(src, dst, n_bytes=None, stream=None):
    import torch
    nb = src.numel() * src.element_size() if n_bytes is None else int(n_bytes)
    if src.numel() * src.element_size() < nb or dst.numel() * dst.element_size() < nb:
        raise ValueError("copy larger than the tensors")
    _check(_lib.load().sq_copy(c_void_p(src.data_ptr()), c_void_p(dst.data_ptr()), nb, _stream(stream)), "sq_copy")


def sq_valu_probe(waves_per_simd, out, stream=None):
    """Launch the FMA issue-rate probe over out.numel() // 256 workgroups (out: float32 on the GPU).
    Returns (wave-level FMA instructions issued, workgroups resident per CU)."""
    import torch
    n_blocks = out.numel() // 256
    if out.dtype != torch.float32 or not out.is_cuda or n_blocks < 1:
        raise ValueError("out must be a float32 GPU tensor of at least 256 elements")
    n = c_uint64(0)
    fit = c_int32(0)
    _check(_lib.load().sq_valu_probe(int(waves_per_simd), n_blocks, c_void_p(out.data_ptr()), byref(n), byref(fit),
                                     _stream(stream)), "sq_valu_probe")
    return n.value, fit.value
