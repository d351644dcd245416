"""Pins of the oracle's Jensen correction taken to all orders (jensen == 3).

"Quantized Keys Steal Attention: Bias Correction for KV-Cache Compression in Video
Diffusion", abstract: the correction removes, in expectation, the inflation that the
keys' rounding noise brings to their softmax weight, computed from the step sizes and
the query; the page uses its second-order Taylor form. Under the same uniform noise
model (e_c ~ U(-step_c/2, step_c/2), channels independent) the expectation has a closed
form, E[exp(tau q.e)] = prod_c sinh(a_c)/a_c with a_c = tau |q_c| step_c / 2, so the
correction to all orders is beta = sum_c log(sinh(a_c)/a_c).

Pins: values at points where sinh is known exactly (a = ln 2: sinh = 3/4; a = ln 3:
sinh = 4/3), the limits (a^2/6 - a^4/180 for small a, a - ln(2a) for large a), the
correction read back out of the oracle's log-sum-exp, and a Monte Carlo check on the
tiny workload's real INT2 and INT4 step sizes that the corrected partition-sum ratio is
1 in expectation (where the second-order form leaves a 4th-order overshoot).
"""
import math

import numpy as np
import pytest

from test_oracle_jensen_mc import _tiny_setup


@pytest.mark.parametrize("a,sinh_a", [(math.log(2.0), 0.75), (math.log(3.0), 4.0 / 3.0), (math.log(5.0), 2.4)])
def test_log_sinhc_known_points(orc, a, sinh_a):
    # sinh(ln x) = (x - 1/x) / 2: 3/4 at x = 2, 4/3 at x = 3, 12/5 at x = 5
    assert orc.log_sinhc(a) == pytest.approx(math.log(sinh_a / a), rel=1e-14)


def test_log_sinhc_limits(orc):
    assert orc.log_sinhc(0.0) == 0.0
    for a in (1e-6, 1e-3, 0.05):
        series = a ** 2 / 6 - a ** 4 / 180 + a ** 6 / 2835
        assert orc.log_sinhc(a) == pytest.approx(series, rel=1e-9, abs=1e-22)
    # the series branch near 0 and the direct branch meet: continuous at the switch
    lo, hi = orc.log_sinhc(0.01 * (1 - 1e-12)), orc.log_sinhc(0.01 * (1 + 1e-12))
    assert abs(hi - lo) <= 1e-10 * hi   # the direct branch carries ~1e-11 relative there
    for a in (25.0, 60.0, 700.0):
        # sinh(a)/a = e^a (1 - e^-2a) / (2a): the correction term is below 1e-20
        assert orc.log_sinhc(a) == pytest.approx(a - math.log(2 * a), rel=1e-15)
    # monotone and convex in a^2 near 0, below a^2/6 everywhere (the log of sinh(a)/a
    # grows like a, its second-order term like a^2)
    grid = np.linspace(0.0, 30.0, 601)
    vals = np.array([orc.log_sinhc(a) for a in grid])
    assert np.all(np.diff(vals) > 0)
    assert np.all(vals <= grid ** 2 / 6 + 1e-15)


def _beta(orc, q, k, step_row, scale, jensen):
    _, lse, _ = orc.attend_row(q, k[None], np.zeros((1, q.size)), np.zeros(1, np.int32),
                               step_row[None] ** 2, scale, jensen)
    return scale * float(q @ k) - lse


@pytest.mark.parametrize("bits", [2, 4])
def test_exact_beta_out_of_the_oracle(orc, bits):
    """A single cached key: lse is its corrected logit, so beta = scale q.k - lse; it is the
    sum over channels of the per-channel closed form, its difference from the second-order
    form is the 4th-order term to leading order, and it stays below that form."""
    K, V, step, gid, q, kc, vc = _tiny_setup(orc, bits)
    scale = 1 / np.sqrt(K.shape[1])
    for g in range(step.shape[0]):
        for i in (0, 5, 15):
            a = scale * np.abs(q[i]) * step[g] / 2
            b3 = _beta(orc, q[i], K[0], step[g], scale, 3)
            b1 = _beta(orc, q[i], K[0], step[g], scale, 1)
            want = sum(orc.log_sinhc(x) for x in a)
            np.testing.assert_allclose(b3, want, rtol=1e-10, atol=1e-13)
            assert b3 <= b1 + 1e-13
            diff4 = -(a ** 4).sum() / 180
            assert abs((b3 - b1) - diff4) <= (a ** 6).sum() / 2835 * 1.01 + 1e-13


@pytest.mark.parametrize("bits", [2, 4])
def test_monte_carlo_partition_ratio_is_one(orc, bits):
    """E over the rounding noise of Z_noisy / Z_true for the cached keys, each key's logit
    corrected by beta: the closed form says 1 exactly for the all-orders correction, and
    prod sinh(a)/a * exp(-a^2/6 summed) (below 1) for the second-order one."""
    K, V, step, gid, q, kc, vc = _tiny_setup(orc, bits)
    scale = 1 / np.sqrt(K.shape[1])
    n, d = K.shape
    R = 2000
    rng = np.random.default_rng(200 + bits)
    ssq = step ** 2
    nq = q.shape[0]
    true_lse = np.array([orc.attend_row(q[i], K, V, gid, ssq, scale, 0)[1] for i in range(nq)])
    r3 = np.zeros((R, nq))
    half = step[gid] / 2
    for r in range(R):
        Kn = K + rng.uniform(-1.0, 1.0, (n, d)) * half
        for i in range(nq):
            r3[r, i] = np.exp(orc.attend_row(q[i], Kn, V, gid, ssq, scale, 3)[1] - true_lse[i])
    for i in range(nq):
        got = r3[:, i]
        se = got.std() / np.sqrt(R)
        assert abs(got.mean() - 1.0) <= 3 * se + 1e-12, (i, got.mean(), se)
    # pooled over queries the ratio is 1 to within a fraction of a percent
    pooled = r3.mean()
    assert abs(pooled - 1.0) <= 3 * r3.mean(1).std() / np.sqrt(R) + 1e-12
