"""The chunk kernel's all-orders Jensen form sums G(a) = log2(sinh(a) / a) over channels as a
series in a^2 where a <= 1 (kExactC in csrc/attention.hip) and evaluates G directly
elsewhere. These CPU checks pin that table to the mathematics: its entries are log2(e)
times the Taylor coefficients of ln(sinh a / a) (2^2n B_2n / (2n (2n)!)), and the five
terms stay within 2.7e-7 of G on [0, 1], in float64 and with float32 coefficients.
Source: "Quantized Keys Steal Attention: Bias Correction for KV-Cache Compression in
Video Diffusion", abstract (the correction of the bias in expectation); the uniform-noise
model of the all-orders form.
"""
import math
import os
import re
from fractions import Fraction

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _table():
    src = open(os.path.join(ROOT, "bit_kv_cache_pack_amd", "csrc", "attention.hip")).read()
    m = re.search(r"kExactC\[5\]\s*=\s*\{([^}]*)\}", src)
    assert m, "kExactC not found"
    return [float(x.strip().rstrip("f")) for x in m.group(1).split(",")]


def _bernoulli(n):
    # Akiyama-Tanigawa, exact rationals
    a = [Fraction(0)] * (n + 1)
    for m in range(n + 1):
        a[m] = Fraction(1, m + 1)
        for j in range(m, 0, -1):
            a[j - 1] = j * (a[j - 1] - a[j])
    return a[0]   # B_n with B_1 = +1/2 (unused here)


def test_coefficients_are_the_taylor_series_of_log_sinhc():
    c = _table()
    for k, ck in enumerate(c):
        n = k + 1
        exact = Fraction(2 ** (2 * n)) * _bernoulli(2 * n) / (2 * n * math.factorial(2 * n))
        want = float(exact) / math.log(2.0)
        assert abs(ck - want) <= 2e-7 * abs(want), (k, ck, want)
    # the first two by hand: 1/6 and -1/180
    assert abs(c[0] * math.log(2.0) - 1 / 6) < 1e-8
    assert abs(c[1] * math.log(2.0) + 1 / 180) < 1e-9


def test_five_terms_within_bound_on_unit_interval():
    c = np.asarray(_table(), np.float64)
    a = np.linspace(1e-4, 1.0, 20001)
    u = a * a
    series = sum(ck * u ** (k + 1) for k, ck in enumerate(c))
    g = np.log(np.sinh(a) / a) / np.log(2.0)
    assert np.abs(series - g).max() < 2.7e-7
    # float32 coefficients, evaluated in float32 as the kernel's products are
    c32 = c.astype(np.float32)
    u32 = u.astype(np.float32)
    s32 = np.zeros_like(u32)
    p = u32.copy()
    for ck in c32:
        s32 = s32 + ck * p
        p = p * u32
    assert np.abs(s32.astype(np.float64) - g).max() < 4e-7
