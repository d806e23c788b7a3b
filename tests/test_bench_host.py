"""CPU checks of bench.py's roofline figures (no GPU).

The algorithmic bytes per launch of the serving pool come from the plan's per-row widths; here they
are held against a closed form from the plan's unit counts (the allocation spends the 6.0-bit budget
exactly over the non-pivot heads, pivot heads hold binary16 values) and against the pool's record
size, which the library lays out independently.  The flops and peaks are the figures the JSON line
states; a summary whose kernel checksum does not match the source yields no figure.
"""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import quantized_delta_rule_02_amd as sq  # noqa: E402
from workloads import configs, gen  # noqa: E402


def _serving_plan():
    wl = configs.BY_NAME["serving-36l-32h-256req-6bit"]
    plan = sq.sq_plan_create(form=0, unit=0, n_layers=wl.n_layers, n_heads=wl.n_heads, d_k=wl.d_k, d_v=wl.d_v,
                             widths=wl.widths, budget_milli=wl.budget_milli, pivot_ppm=wl.pivot_ppm, grid=wl.grid,
                             gate=gen.unit_gates(wl), impact=gen.impact_scores(wl), calib_seed=gen.calib_seed(wl),
                             calib_segments=2, calib_len=16)
    return wl, plan


def test_algorithmic_bytes_of_the_serving_pool():
    wl, plan = _serving_plan()
    d = plan.desc
    dk, dv, U, piv = d["d_k"], d["d_v"], d["n_units"], d["n_pivot_units"]
    io = 4 * (2 * dk + 2 * dv + 1) + 4                        # q, k, v, y, beta and the head's gate
    state = ((U - piv) * 6 + piv * 16) * dk * dv // 8 + U * 2 * (dk + dv)
    want = wl.batch * (2 * state + U * io)
    assert bench.algorithmic_bytes(plan, wl.batch, sq) == want == 8_281_915_392
    # the pool's per-slot record (codes and scales of every layer and head) has the same size
    assert d["slot_bytes"] == state
    plan.close()


def test_flops_and_peaks():
    n = 36 * 32 * 256
    assert n == 294_912
    assert bench.algorithmic_flops(n, 128, 128, 4) == n * (12 + 5 * 4) * 128 * 128 == 154_618_822_656
    assert abs(bench.ALU_PEAK_TFLOPS - 157.2864) < 1e-9
    assert bench.HBM_PEAK_GBPS == 8000.0


def test_counter_summary_needs_the_matching_kernel_source(tmp_path):
    f = tmp_path / "summary.txt"
    f.write_text("# header: not a figure\nhbm_bytes_per_launch: 123\nkernel_source_sha256: 00\n")
    assert bench._profile_value(str(f), "hbm_bytes_per_launch") is None
    import hashlib
    sha = hashlib.sha256(open(bench.KERNEL_SRC, "rb").read()).hexdigest()
    f.write_text(f"hbm_bytes_per_launch: 123\nkernel_source_sha256: {sha}\n")
    assert bench._profile_value(str(f), "hbm_bytes_per_launch") == 123.0
    assert bench._profile_value(str(f), "missing") is None
    assert bench._profile_value(str(tmp_path / "absent.txt"), "hbm_bytes_per_launch") is None


def test_summarize_reads_a_rocprofv3_database(tmp_path, capsys):
    """bench.py --summarize: durations and counters of the chosen launches of each kernel, from a database
    laid out like rocprofv3's (a kernels view with name, dispatch, start and end; counters per dispatch)."""
    import sqlite3
    import bench
    db = str(tmp_path / "run_results.db")
    con = sqlite3.connect(db)
    con.execute("CREATE TABLE kernels (dispatch_id INTEGER, kernel_name TEXT, start INTEGER, end INTEGER)")
    con.execute("CREATE TABLE counters_collection (dispatch_id INTEGER, counter_name TEXT, value REAL)")
    for i in range(5):   # k_state: 1000, 2000, ... ns; one other kernel
        con.execute("INSERT INTO kernels VALUES (?, 'sq::k_state<128, 128, 0, 4, false>', ?, ?)",
                    (i, 10 * i * 1000, 10 * i * 1000 + 1000 * (i + 1)))
        con.execute("INSERT INTO counters_collection VALUES (?, 'SQ_WAVES', ?)", (i, 100.0 * (i + 1)))
    con.execute("INSERT INTO kernels VALUES (9, 'sq::k_copy', 0, 500)")
    con.commit()
    con.close()
    bench.summarize([db], "last:2")
    out = capsys.readouterr().out.splitlines()
    row = next(l for l in out if l.startswith("sq::k_state"))
    f = row.split()
    # last two launches: 4 and 5 us, SQ_WAVES 400 and 500
    assert "4.5" in f and "4.0" in f and "5.0" in f and "450" in f
    bench.summarize([db], "first:1")
    row = next(l for l in capsys.readouterr().out.splitlines() if l.startswith("sq::k_state"))
    assert "1.0" in row.split() and "100" in row.split()
