"""Pins of the oracle's fixed-point encoding (CPU only).

The pages fix int64 fixed-point cells (bonsai "9. Parallelism & determinism",
"The idea") but not the scale.  The reading pinned here: k = 30 - e with
2^(e-1) <= max|c| < 2^e, q = rint(c * 2^k) with ties to even.  These tests
check it against hand-worked values, against exact sums of the raw floats
(math.fsum) within the rounding bound, and against its range guarantee.
"""
import math

import numpy as np
import pytest

import oracle


def test_hand_pin_round_half_even():
    # M = 1 -> e = 1 -> k = 29.  2^-30 * 2^29 = 0.5 -> 0; 3 * 2^-30 * 2^29 = 1.5 -> 2.
    g = np.array([1.0, 2.0 ** -30, 3 * 2.0 ** -30], dtype=np.float32)
    q, k = oracle.quantize(g, require_nonneg=False)
    assert k == 29
    assert q.tolist() == [2 ** 29, 0, 2]


def test_ties_to_even_both_signs():
    # M = 2^29 - 2^5 ... pick M = 1.0 (k = 29) and values at exact half steps.
    step = 2.0 ** -29
    vals = [1.0, 0.5 * step, 1.5 * step, 2.5 * step, -0.5 * step, -1.5 * step, -2.5 * step,
            3.5 * step]
    q, k = oracle.quantize(np.array(vals, dtype=np.float32), require_nonneg=False)
    assert k == 29
    assert q.tolist() == [2 ** 29, 0, 2, 2, 0, -2, -2, 4]


@pytest.mark.parametrize("m,expect_k", [
    (1.0, 29), (0.5, 30), (0.75, 30), (1.5, 29), (2.0, 28), (3.0, 28),
    (2.0 ** 31, -2), (1e-30, 30 - math.frexp(np.float32(1e-30))[1]),
])
def test_scale_exponent(m, expect_k):
    q, k = oracle.quantize(np.array([m, -m / 4], dtype=np.float32), require_nonneg=False)
    assert k == expect_k
    assert abs(int(q[0])) <= 2 ** 30


def test_zero_vector_gives_k0():
    q, k = oracle.quantize(np.zeros(5, dtype=np.float32), require_nonneg=True)
    assert k == 0 and not q.any()


def test_negative_zero_is_zero_even_for_hessian():
    q, k = oracle.quantize(np.array([-0.0, 0.5], dtype=np.float32), require_nonneg=True)
    assert q.tolist() == [0, 2 ** 29]


@pytest.mark.parametrize("bad", [np.nan, np.inf, -np.inf])
def test_nonfinite_rejected(bad):
    with pytest.raises(oracle.OracleError) as e:
        oracle.quantize(np.array([0.5, bad], dtype=np.float32), require_nonneg=False)
    assert e.value.status == oracle.E_NONFINITE


def test_negative_hessian_rejected():
    with pytest.raises(oracle.OracleError):
        oracle.quantize(np.array([0.5, -1e-20], dtype=np.float32), require_nonneg=True)
    # the same vector is a valid gradient
    oracle.quantize(np.array([0.5, -1e-20], dtype=np.float32), require_nonneg=False)


@pytest.mark.parametrize("seed", range(4))
def test_range_and_sum_error_bound(seed):
    """|q| <= 2^30, max element hits [2^29, 2^30], and for any subset the
    fixed-point sum differs from the exact float sum by <= count * 2^-(k+1)."""
    rng = np.random.default_rng(seed)
    n = 5000
    scale = 10.0 ** rng.uniform(-20, 20)
    c = (rng.standard_normal(n) * scale).astype(np.float32)
    q, k = oracle.quantize(c, require_nonneg=False)
    assert np.abs(q.astype(np.int64)).max() <= 2 ** 30
    assert np.abs(q.astype(np.int64)).max() >= 2 ** 29
    for _ in range(5):
        sub = rng.random(n) < rng.uniform(0.01, 1.0)
        cnt = int(sub.sum())
        exact = math.fsum(float(x) for x in c[sub])
        fixed = math.ldexp(float(int(q[sub].astype(np.int64).sum())), -k)
        assert abs(fixed - exact) <= cnt * math.ldexp(1.0, -(k + 1)) * (1 + 1e-12) + abs(exact) * 2 ** -52


def test_wide_dynamic_range_exact_where_representable():
    # values that are multiples of 2^-k encode exactly
    c = np.array([1.0, 0.25, -0.125, 2.0 ** -29, -(2.0 ** -28)], dtype=np.float32)
    q, k = oracle.quantize(c, require_nonneg=False)
    assert k == 29
    back = [math.ldexp(int(v), -k) for v in q]
    assert back == [float(x) for x in c]


def test_precision_one_bit():
    # M = 0.75 -> e = 0 -> k = 1: 0.75 * 2 = 1.5 -> 2 (= 2^P), 0.25 * 2 = 0.5 -> 0
    q, k = oracle.quantize(np.array([0.75, 0.25, -0.5], dtype=np.float32), False, bits=1)
    assert k == 1 and q.tolist() == [2, 0, -1]


@pytest.mark.parametrize("bits", [4, 8, 19, 29])
def test_precision_bits(bits):
    """k = P - e: the largest value lands in [2^(P-1), 2^P] and half-steps round to even."""
    step = 2.0 ** -(bits - 1)          # M = 1 -> e = 1 -> k = P - 1
    vals = [1.0, 0.5 * step, 1.5 * step, -2.5 * step]
    q, k = oracle.quantize(np.array(vals, dtype=np.float32), require_nonneg=False, bits=bits)
    assert k == bits - 1
    assert q.tolist() == [2 ** (bits - 1), 0, 2, -2]


@pytest.mark.parametrize("bits", [0, 31])
def test_precision_out_of_range(bits):
    with pytest.raises(oracle.OracleError):
        oracle.quantize(np.ones(3, dtype=np.float32), require_nonneg=True, bits=bits)


@pytest.mark.parametrize("bits,expect", [(19, 2 ** 19), (23, 2 ** 23), (24, 2 ** 24 - 1), (30, 2 ** 30 - 64)])
def test_largest_code_reaches_two_to_the_p(bits, expect):
    """M = 1 - 2^-24 (the fp32 value below 1) has e = 0, so k = P and
    M * 2^P = 2^P - 2^(P - 24): below P = 24 that is within half a step of
    2^P and rounds up to it (the bound |q| <= 2^P is reached, which the
    packed sums' drain period allows for); from P = 24 on it is an integer."""
    m = np.float32(np.nextafter(np.float32(1), np.float32(0)))
    assert float(m) == 1 - 2.0 ** -24
    for sign, nonneg in ((1, False), (-1, False), (1, True)):
        q, k = oracle.quantize(np.array([sign * m, 0.25 * sign * m], dtype=np.float32), require_nonneg=nonneg,
                               bits=bits)
        assert k == bits
        assert q[0] == sign * expect
