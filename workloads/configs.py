"""The five synthetic workloads of the quantized gated-delta state step.

Each workload fixes a state shape, a pool (requests and slots), the gate form,
the quantization plan inputs (candidate widths, average-bit budget, pivot
fraction, impact-score distribution) and the number of decode steps.  The
shapes follow the serving setting the STEPQuant pages describe: GDN heads with
a scalar gate per head (Qwen-style), KDA heads with a per-key-row gate
(Kimi-style), a serving pool of many concurrent requests, and a dual-axis
outlier case.  Nothing here performs any of the method's arithmetic.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Tuple


GDN = "gdn"
KDA = "kda"
UNIT_HEAD = "head"
UNIT_ROW = "row"


@dataclass(frozen=True)
class Workload:
    cid: int                 # stream id for the seeded generators
    name: str
    form: str                # GDN (scalar gate per head) or KDA (gate per key row)
    n_layers: int
    n_heads: int
    d_k: int
    d_v: int
    batch: int               # concurrent requests
    n_slots: int             # pool slots (>= batch); extra slots stay idle
    steps: int               # decode steps of the workload
    unit: str                # allocation unit: a head or a key row
    widths: Tuple[int, ...]  # candidate code widths
    budget_milli: int        # average bits x 1000 over non-pivot units
    pivot_ppm: int           # pivot fraction in parts per million of units
    gate_mu: float           # alpha = sigmoid(N(gate_mu, gate_sigma))
    gate_sigma: float
    impact: Tuple            # ('uniform', lo, hi) | ('lognormal', mu, sigma) | ('pareto', shape)
    warmup_steps: int        # fp32 warm-up steps from zero before packing (0: zero state)
    ridge_rows: int = 0      # rows scaled x ridge_scale in the warm-up state
    ridge_cols: int = 0      # columns scaled x ridge_scale (also applied to v each step)
    ridge_scale: float = 1.0
    grid: Tuple[float, ...] = (1.0, 0.875, 0.75, 0.625)
    calib_segments: int = 32
    calib_len: int = 512

    @property
    def states_per_step(self) -> int:
        return self.n_layers * self.batch * self.n_heads

    @property
    def n_units(self) -> int:
        per = 1 if self.unit == UNIT_HEAD else self.d_k
        return self.n_layers * self.n_heads * per

    def scaled(self, **kw) -> "Workload":
        """A copy with some fields replaced (used for reduced-size test cases)."""
        return replace(self, **kw)


# Config 0: tiny reference (parity config that the oracle runs whole).
TINY = Workload(
    cid=0, name="tiny-gdn-16", form=GDN, n_layers=1, n_heads=2, d_k=16, d_v=16,
    batch=1, n_slots=1, steps=64, unit=UNIT_HEAD, widths=(6,), budget_milli=6000,
    pivot_ppm=0, gate_mu=4.0, gate_sigma=1.0, impact=("uniform", 0.5, 2.0),
    warmup_steps=0)

# Config 1: GDN-shaped decode, per-head widths, one pivot head.
GDN_DECODE = Workload(
    cid=1, name="gdn-decode-32h-128", form=GDN, n_layers=1, n_heads=32, d_k=128, d_v=128,
    batch=64, n_slots=64, steps=256, unit=UNIT_HEAD, widths=(4, 6, 8), budget_milli=6000,
    pivot_ppm=10000, gate_mu=4.0, gate_sigma=1.0, impact=("lognormal", 0.0, 0.5),
    warmup_steps=512)

# Config 2: KDA-shaped decode, per-row widths, pivot rows.
KDA_DECODE = Workload(
    cid=2, name="kda-decode-32h-128", form=KDA, n_layers=1, n_heads=32, d_k=128, d_v=128,
    batch=128, n_slots=128, steps=256, unit=UNIT_ROW, widths=(4, 6, 8), budget_milli=6000,
    pivot_ppm=5000, gate_mu=3.0, gate_sigma=1.5, impact=("lognormal", 0.0, 0.5),
    warmup_steps=512)

# Config 3: serving-scale pool, 36 layers x 32 heads x 256 requests (6-bit and 4-bit budgets).
SERVING_6 = Workload(
    cid=3, name="serving-36l-32h-256req-6bit", form=GDN, n_layers=36, n_heads=32, d_k=128,
    d_v=128, batch=256, n_slots=320, steps=256, unit=UNIT_HEAD, widths=(4, 6, 8),
    budget_milli=6000, pivot_ppm=10000, gate_mu=4.0, gate_sigma=1.0,
    impact=("lognormal", 0.0, 0.5), warmup_steps=512)
SERVING_4 = replace(SERVING_6, name="serving-36l-32h-256req-4bit", budget_milli=4000)

# Config 4: dual-axis outlier stress, KDA, d_v = 256, 4-bit budget with pivot rows.
OUTLIER = Workload(
    cid=4, name="outlier-kda-32h-128x256", form=KDA, n_layers=1, n_heads=32, d_k=128,
    d_v=256, batch=1024, n_slots=1024, steps=256, unit=UNIT_ROW, widths=(4, 6, 8),
    budget_milli=4000, pivot_ppm=5000, gate_mu=3.0, gate_sigma=1.5,
    impact=("pareto", 1.5), warmup_steps=512, ridge_rows=3, ridge_cols=6, ridge_scale=20.0)

# Candidate widths extended to {2, 3, 4, 6, 8}, so that a 4.0-bit budget mixes widths (the
# pages list no candidate set; with {4, 6, 8} a 4-bit budget leaves every unit at 4 bits).
SERVING_4_MIXED = replace(SERVING_4, name="serving-36l-32h-256req-4bit-mixed", widths=(2, 3, 4, 6, 8))
OUTLIER_MIXED = replace(OUTLIER, name="outlier-kda-32h-128x256-mixed", widths=(2, 3, 4, 6, 8))

# The 64x64 state shape (one wave per state in the library): test cases only.
GDN_64 = replace(GDN_DECODE, name="gdn-decode-32h-64", d_k=64, d_v=64)
KDA_64 = replace(KDA_DECODE, name="kda-decode-32h-64", d_k=64, d_v=64)

ALL = (TINY, GDN_DECODE, KDA_DECODE, SERVING_6, SERVING_4, OUTLIER)
EXTENDED = (SERVING_4_MIXED, OUTLIER_MIXED, GDN_64, KDA_64)
BY_NAME = {w.name: w for w in ALL + EXTENDED}
