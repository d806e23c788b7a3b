"""The seeded input generators (CPU only)."""
import numpy as np

from workloads import configs, gen


def test_philox_known_answers():
    # Known-answer vectors published with the Random123 library for Philox-4x32-10.
    def run(ctr, key):
        return [int(x) for x in gen.philox4x32(np.array(ctr, np.uint32), key)]
    assert run([0, 0, 0, 0], (0, 0)) == [0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8]
    assert run([0xFFFFFFFF] * 4, (0xFFFFFFFF, 0xFFFFFFFF)) == [0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD]
    assert run([0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344], (0xA4093822, 0x299F31D0)) == \
        [0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1]


def test_calibration_traces_shape_and_normalisation():
    q, k, v, b = gen.calib_traces(gen.calib_seed(configs.TINY), 0, 1, 3, 5, 16, 16)
    assert q.shape == (3, 5, 16) and v.shape == (3, 5, 16) and b.shape == (3, 5)
    assert np.allclose(np.linalg.norm(q, axis=-1), 1, atol=1e-6)
    assert np.allclose(np.linalg.norm(k, axis=-1), 1, atol=1e-6)
    assert np.all((b > 0) & (b < 1))
    q2, _, _, _ = gen.calib_traces(gen.calib_seed(configs.TINY), 0, 1, 3, 5, 16, 16)
    assert np.array_equal(q, q2)
    z = gen.calib_normals(123, 2, 3, 4, 256, 64)
    assert abs(z.mean()) < 0.02 and abs(z.std() - 1) < 0.02


def test_gates_and_impacts_match_the_workload_recipes():
    a = gen.unit_gates(configs.GDN_DECODE)
    assert a.shape == (1, 32) and np.all((a > 0.5) & (a < 1))
    a = gen.unit_gates(configs.KDA_DECODE)
    assert a.shape == (1, 32, 128)
    w = gen.impact_scores(configs.TINY)
    assert np.all((w >= 0.5) & (w <= 2.0))
    w = gen.impact_scores(configs.OUTLIER)
    assert np.all(w >= 1.0)
    s = gen.slot_map(configs.SERVING_6)
    assert len(np.unique(s)) == 256 and s.max() < 320


def test_unit_counts():
    assert configs.SERVING_6.states_per_step == 256 * 36 * 32
    assert configs.KDA_DECODE.n_units == 32 * 128
    assert configs.SERVING_6.n_units == 36 * 32
