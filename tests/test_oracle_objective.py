"""Pins of the oracle's objective gradients and of its exp.

The oracle writes exp out (Cody-Waite reduction, degree-13 Taylor polynomial)
so that a device implementation of the same operations can match it bit for
bit.  These tests tie it to things outside the oracle: the platform's libm /
numpy exp (a special case that reduces to a library routine), exact values
at m = 0, the saturation of the logistic probability, exact scaling by
power-of-two weights, and the derivatives checked by finite differences of
the loss itself."""
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle
from histogram_gradient_boosted_amd import synth


def ulp_diff(a, b):
    a = np.asarray(a)
    b = np.asarray(b)
    return np.abs(a.astype(np.float64) - b.astype(np.float64)) / np.spacing(np.abs(b))


def test_exp_within_one_ulp_of_libm():
    rng = np.random.default_rng(11)
    x = np.concatenate([rng.uniform(-708, 709.7, 100_000), rng.uniform(-1, 1, 100_000),
                        rng.normal(0, 8, 100_000)])
    got = oracle.exp(x)
    ref = np.exp(x)
    assert ulp_diff(got, ref).max() <= 1.0
    # most results are the correctly rounded ones
    assert (got == ref).mean() > 0.85


def test_exp_against_decimal_at_hand_points():
    """exp at points where an exact (60-digit) value is cheap: Decimal.exp."""
    from decimal import Decimal, getcontext
    getcontext().prec = 60
    for x in [1.0, -1.0, 0.5, 0.3465, -0.3466, 10.0, -20.0, 100.25, -700.0, 709.0, 1e-10]:
        want = float(Decimal(x).exp())
        got = float(oracle.exp(np.array([x]))[0])
        assert abs(got - want) <= np.spacing(want), (x, got, want)


def test_exp_powers_of_two():
    """exp(n ln 2) is 2^n up to the rounding of n ln 2 itself (x has a relative
    error below 2^-53, so exp(x) is 2^n within |x| * 2^-53 relative)."""
    for n in [-1000, -500, -64, -1, 1, 2, 52, 300, 1000]:
        x = n * math.log(2.0)
        got = float(oracle.exp(np.array([x]))[0])
        assert abs(got / math.ldexp(1.0, n) - 1.0) <= abs(x) * 2.0 ** -52 + 2.0 ** -52


def test_exp_special_values():
    x = np.array([0.0, -0.0, np.nan, np.inf, -np.inf, 1000.5, -1000.5, 709.9, -745.2, -744.0])
    got = oracle.exp(x)
    assert got[0] == 1.0 and got[1] == 1.0
    assert np.isnan(got[2])
    assert got[3] == np.inf and got[4] == 0.0
    assert got[5] == np.inf and got[6] == 0.0
    assert got[7] == np.inf                        # past the largest double
    assert got[8] == 0.0                           # below half the smallest subnormal
    assert got[9] == np.exp(-744.0)                # a subnormal result, rounded once


def test_exp_subnormal_range():
    x = np.linspace(-745.0, -708.5, 20001)
    got = oracle.exp(x)
    ref = np.exp(x)
    assert np.abs(got - ref).max() <= 5e-324


@pytest.mark.parametrize("kind", ["squared", "logistic", "poisson"])
def test_objective_at_zero_margin(kind):
    """At m = 0: e^0 = 1 exactly, so p = 1/2, and every derivative is exact."""
    y = np.array([0.0, 1.0, 0.25, -3.5, 7.0], dtype=np.float32)
    m = np.zeros_like(y)
    g, h = oracle.objective(kind, m, y)
    if kind == "squared":
        want_g, want_h = -y, np.ones_like(y)
    elif kind == "logistic":
        want_g, want_h = 0.5 - y, np.full_like(y, 0.25)
    else:
        want_g, want_h = 1.0 - y, np.ones_like(y)
    assert np.array_equal(g, want_g.astype(np.float32))
    assert np.array_equal(h, want_h.astype(np.float32))


def test_squared_exact_rational():
    """g = m - y rounded once to fp32 (m - y of two fp32 values whose exponents
    are close is exact in double), h = 1."""
    m, y, _ = synth.objective_inputs(3, 20_000, "squared")
    g, h = oracle.objective("squared", m, y)
    for i in range(0, 20_000, 97):
        exact = Fraction(float(m[i])) - Fraction(float(y[i]))
        assert g[i] == np.float32(float(exact)), i
    assert (h == 1.0).all()


@pytest.mark.parametrize("kind", ["logistic", "poisson"])
def test_objective_against_numpy_exp(kind):
    """Same formulas with numpy's exp: within one fp32 ulp everywhere, and the
    same fp32 value almost always (they differ only when the two double
    results straddle an fp32 rounding boundary)."""
    m, y, _ = synth.objective_inputs(5, 200_000, kind)
    g, h = oracle.objective(kind, m, y)
    md = m.astype(np.float64)
    yd = y.astype(np.float64)
    if kind == "logistic":
        p = 1.0 / (1.0 + np.exp(-md))
        rg, rh = (p - yd).astype(np.float32), (p * (1.0 - p)).astype(np.float32)
    else:
        e = np.exp(md)
        rg, rh = (e - yd).astype(np.float32), e.astype(np.float32)
    for got, want in ((g, rg), (h, rh)):
        nz = want != 0
        assert ulp_diff(got[nz], want[nz]).max() <= 1.0
        assert (got[~nz] == 0).all() or np.abs(got[~nz]).max() < 1e-30
        assert (got == want).mean() > 0.999


def finite_difference(loss, m, y, step):
    """Central differences of the loss in exact rational arithmetic around the
    double m (only the loss's own exp/log are evaluated in floating point)."""
    return (loss(m + step, y) - loss(m - step, y)) / (2 * step)


@pytest.mark.parametrize("kind", ["squared", "logistic", "poisson"])
def test_derivatives_match_the_loss(kind):
    """g and h are the first and second derivatives of the loss in m: checked
    by central differences of the loss written independently here."""
    def loss(m, y):
        if kind == "squared":
            return 0.5 * (m - y) ** 2
        if kind == "logistic":
            return math.log1p(math.exp(m)) - y * m
        return math.exp(m) - y * m

    m, y, _ = synth.objective_inputs(9, 400, kind)
    m = np.clip(m, -15, 15).astype(np.float32)
    g, h = oracle.objective(kind, m, y)
    step = 1e-4
    for i in range(400):
        mi, yi = float(m[i]), float(y[i])
        fd_g = finite_difference(loss, mi, yi, step)
        fd_h = (loss(mi + step, yi) - 2 * loss(mi, yi) + loss(mi - step, yi)) / step ** 2
        scale = max(1.0, abs(fd_g), math.exp(mi) if kind == "poisson" else 1.0)
        assert abs(float(g[i]) - fd_g) <= 1e-6 * scale + 1e-7 * abs(loss(mi, yi)), (i, mi, yi)
        assert abs(float(h[i]) - fd_h) <= 2e-4 * max(1.0, float(h[i])), (i, mi, yi)


def test_logistic_saturation():
    """For m >= 38, e^-m < 2^-54 so 1 + e^-m rounds to 1: p = 1, h = 0 exactly.
    For very negative m, p = e^m (relatively) and h ~ p."""
    m = np.array([38.0, 50.0, 88.0, 1e30, -50.0, -80.0], dtype=np.float32)
    y = np.array([1, 0, 1, 0, 0, 1], dtype=np.float32)
    g, h = oracle.objective("logistic", m, y)
    assert np.array_equal(g[:4], np.array([0, 1, 0, 1], dtype=np.float32))
    assert (h[:4] == 0).all()
    for i, mi in ((4, -50.0), (5, -80.0)):
        assert abs(float(h[i]) / math.exp(mi) - 1) < 1e-6
    assert abs(float(g[5]) + 1.0) < 1e-30 + 1e-7


@pytest.mark.parametrize("kind", ["squared", "logistic", "poisson"])
def test_power_of_two_weights_scale_exactly(kind):
    m, y, _ = synth.objective_inputs(13, 50_000, kind)
    g1, h1 = oracle.objective(kind, m, y)
    for k in (-3, 0, 1, 5):
        w = np.full(m.shape, 2.0 ** k, dtype=np.float32)
        gw, hw = oracle.objective(kind, m, y, w)
        ok = (np.abs(g1) > 1e-30) & (np.abs(g1) < 1e30)
        assert np.array_equal(gw[ok], (g1[ok] * np.float32(2.0 ** k)))
        okh = (h1 > 1e-30) & (h1 < 1e30)
        assert np.array_equal(hw[okh], (h1[okh] * np.float32(2.0 ** k)))
    w0 = np.zeros(m.shape, dtype=np.float32)
    g0, h0 = oracle.objective(kind, m, y, w0)
    assert (g0 == 0).all() and (h0 == 0).all()


def test_general_weights_within_one_rounding():
    m, y, w = synth.objective_inputs(17, 50_000, "logistic", weighted=True)
    g1, h1 = oracle.objective("logistic", m, y)
    gw, hw = oracle.objective("logistic", m, y, w)
    ref = g1.astype(np.float64) * w
    nz = ref != 0
    # g1 carries one fp32 rounding, gw one: at most ~2 ulp apart relative to w*g
    assert (np.abs(gw[nz] - ref[nz]) / np.abs(ref[nz])).max() < 2.5 * 2.0 ** -23


def test_unknown_objective_rejected():
    m = np.zeros(4, dtype=np.float32)
    with pytest.raises(oracle.OracleError) as e:
        oracle.objective(7, m, m)
    assert e.value.status == oracle.E_INVALID


def test_c3_recipe_from_scores():
    """The c3 recipe draws scores in double; the fp32 scores it also keeps give
    logistic (g, h) within fp32 rounding of the recipe's own (g, h)."""
    w = synth.make("c3", n_rows=100_000)
    g, h = oracle.objective("logistic", w.margin, w.label)
    # a score rounded to fp32 moves p by at most 2^-24 |m| p (1-p) <= 2^-24 |m| / 4
    tol = np.abs(w.margin).astype(np.float64) * 2.0 ** -25 + 2.0 ** -23
    assert (np.abs(g.astype(np.float64) - w.grad) <= tol).all()
    assert (np.abs(h.astype(np.float64) - w.hess) <= tol).all()
