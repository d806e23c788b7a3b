"""CPU check of the residual identity the GPU column fit evaluates (no GPU).

The fit needs, per candidate scale c and entry, the rounding residual of the
clamped symmetric quantizer, e = y - min(rint(y), qmax) for y = |X| / (r c) >= 0
(STEPQuant's dual-axis quantizer; hyper.ai summary, 方法, the per-column scale
fit over a candidate grid).  The kernel does not form the code: with
a = y + 1/2 - qmax it takes max(a, fract(a)) - 1/2, fract being the GPU's
v_fract_f32 (x - floor(x), kept below 1).  This test restates that formula in
float32 and holds it against the plain definition in float64 over every width's
range, the clip boundary and the exact half-way points, where either rounding
direction leaves the same |e|.
"""
import numpy as np
import pytest

ONE_MINUS = np.float32(np.nextafter(np.float32(1.0), np.float32(0.0)))


def fract32(x):
    x = np.asarray(x, np.float32)
    return np.minimum(x - np.floor(x), ONE_MINUS).astype(np.float32)


def kernel_residual(y, qmax, can_clip=True):
    """|residual| as the fit computes it: a in float32 (one rounding), then fract and max."""
    a = (np.asarray(y, np.float64) + (0.5 - qmax)).astype(np.float32)
    f = fract32(a)
    e2 = np.maximum(a, f) if can_clip else f
    return np.abs(e2.astype(np.float64) - 0.5), a


def true_residual(y, qmax):
    return np.abs(y - np.minimum(np.rint(y), qmax))


@pytest.mark.parametrize("bits", [2, 3, 4, 6, 8])
def test_residual_matches_the_clamped_rounding(bits):
    qmax = 2 ** (bits - 1) - 1
    g = np.random.default_rng(bits)
    hi = qmax / 0.5625 + 3.0                       # past the smallest grid factor's largest quotient
    y = np.concatenate([
        np.linspace(0.0, hi, 200_001),
        g.uniform(0.0, hi, 200_000),
        np.arange(0, 2 * qmax + 3) + 0.5,          # half-way points, inside and beyond the range
        np.arange(0, 2 * qmax + 3, dtype=np.float64),
        qmax + 0.5 + np.array([-1e-6, -1e-9, 0.0, 1e-9, 1e-6]),
    ])
    y = y.astype(np.float32).astype(np.float64)   # the kernel's y is a float32 quotient
    got, a = kernel_residual(y, qmax)
    want = true_residual(y, qmax)
    # a carries one float32 rounding at its own magnitude; everything else is exact
    tol = np.maximum(np.abs(a.astype(np.float64)), 1.0) * 2.0 ** -24 + 1e-12
    assert np.all(np.abs(got - want) <= tol), np.max(np.abs(got - want) - tol)
    # the clipped entries are exactly the ones past qmax + 1/2
    clip = y > qmax + 0.5
    assert np.all(a[clip] >= 1.0) and np.all(a[~clip] <= 1.0)


@pytest.mark.parametrize("bits", [2, 3, 4, 6, 8])
def test_first_candidate_needs_no_clamp(bits):
    """gamma = 1: c is the binary16 rounding of c0 = max |X| / (r qmax), at most 2^-11 below it while
    c0 <= 65504, so y <= qmax (1 + 2^-11) < qmax + 1/2 and the fract alone is the residual.  (Above
    65504 the stored scale is clamped and the kernel uses the clamping form for gamma = 1 as well.)"""
    qmax = 2 ** (bits - 1) - 1
    ymax = qmax * (1.0 + 2.0 ** -11)
    assert ymax < qmax + 0.5
    y = np.linspace(0.0, ymax, 100_001).astype(np.float32).astype(np.float64)
    got, a = kernel_residual(y, qmax, can_clip=False)
    tol = np.maximum(np.abs(a.astype(np.float64)), 1.0) * 2.0 ** -24 + 1e-12
    assert np.all(np.abs(got - true_residual(y, qmax)) <= tol)


def test_a_planted_sign_slip_is_caught():
    """The same check fails for a plausible slip: shifting by +qmax instead of -qmax keeps the
    fract (qmax is an integer) but loses the clip."""
    qmax = 31
    y = np.linspace(0.0, 60.0, 10_001)
    a = (y + (0.5 + qmax)).astype(np.float32)
    slipped = np.abs(np.maximum(a, fract32(a)).astype(np.float64) - 0.5)
    assert not np.allclose(slipped, true_residual(y, qmax), atol=1e-4)
