"""Pins of the oracle's number-format conversions against library routines.

The quantizer stores step and zero as IEEE binary16 and the reader rounds dequantized
elements to bf16 (or fp16); the oracle implements both conversions itself. Here they
are checked against numpy's float16 and torch's bfloat16 casts (both round to
nearest, ties to even).
"""
import numpy as np
import pytest
import torch


def _interesting_f32(n, seed):
    rng = np.random.default_rng(seed)
    # wide exponent sweep, both signs
    e = rng.uniform(-30, 20, n)
    x = (np.sign(rng.standard_normal(n)) * np.exp2(e)).astype(np.float32)
    # exact fp16 half-way points: midpoints between adjacent binary16 values
    h = rng.integers(0, 0x7bff, n // 4).astype(np.uint16)
    lo = h.view(np.float16).astype(np.float64)
    hi = (h + 1).view(np.float16).astype(np.float64)
    mids = ((lo + hi) / 2).astype(np.float32)     # exact in float32
    # exact bf16 half-way points
    b = rng.integers(0, 0x7f7f, n // 4).astype(np.uint32)
    bmid = ((b << 16) | 0x8000).astype(np.uint32).view(np.float32)
    edges = np.array([0.0, -0.0, 65504, 65519.996, 65520, 65536, 1e-8, 2.0 ** -24, 2.0 ** -25,
                      3 * 2.0 ** -26, 2.0 ** -14, 2.0 ** -14 - 2.0 ** -25, 1.0, -1.0, np.inf,
                      -np.inf], np.float32)
    return np.concatenate([x, mids, -mids, bmid, -bmid, edges])


def test_f32_to_f16_matches_numpy(orc):
    x = _interesting_f32(200000, 1)
    ours = orc.f32_to_f16_bits(x)
    ref = x.astype(np.float16).view(np.uint16)
    bad = np.nonzero(ours != ref)[0]
    assert bad.size == 0, (x[bad[:5]], ours[bad[:5]], ref[bad[:5]])


def test_f16_to_f64_all_bit_patterns(orc):
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = orc.f16_bits_to_f64(h)
    ref = h.view(np.float16).astype(np.float64)
    finite = np.isfinite(ref)
    assert np.array_equal(ours[finite], ref[finite])
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    assert np.array_equal(np.isinf(ours), np.isinf(ref))


def test_f32_to_bf16_matches_torch(orc):
    x = _interesting_f32(200000, 2)
    x = x[np.isfinite(x)]
    ours = orc.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    bad = np.nonzero(ours != ref)[0]
    assert bad.size == 0, (x[bad[:5]], ours[bad[:5]], ref[bad[:5]])


def test_bf16_to_f32_roundtrip(orc):
    h = np.arange(0, 65536, 7, dtype=np.uint32).astype(np.uint16)
    vals = torch.from_numpy(h.view(np.int16)).view(torch.bfloat16).float().numpy()
    fin = np.isfinite(vals)
    back = orc.f32_to_bf16_bits(vals[fin])
    assert np.array_equal(back, h[fin])
