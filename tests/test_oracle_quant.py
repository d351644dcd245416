"""Pins of the oracle's quantizer (Q1), packing (Q2) and append / group table (Q3).

What pins them: hand-worked cases (tests/golden/quant_hand_examples.json), the
round-trip bound |x - dequant(x)| <= step/2, exhaustive brute force over small code
vectors, exact power-of-two scaling, permutation equivariance, packed bytes worked by
hand, and the group table of the chunk-wise cache (whole chunks appended, each chunk
split into K-groups of 128 tokens from its own first token).
"""
import json
import os

import numpy as np
import pytest
import torch

import workloads

GOLD = os.path.join(os.path.dirname(__file__), "golden", "quant_hand_examples.json")


def _f16(bits):
    return float(np.array([bits], np.uint16).view(np.float16)[0])


def test_hand_examples(orc):
    cases = json.load(open(GOLD))["cases"]
    for c in cases:
        codes, s, z = orc.quantize_group(c["x"], c["bits"])
        assert list(codes) == c["codes"], c["name"]
        assert s == int(c["step"], 16), (c["name"], hex(s))
        assert z == int(c["zero"], 16), (c["name"], hex(z))


def test_packing_bytes(orc):
    gold = json.load(open(GOLD))["packing"]
    w = orc.pack_row([1, 2, 3, 0] + [0] * 12, 2)
    assert w.view(np.uint8)[0] == int(gold["int2_codes_1_2_3_0_first_byte"], 16)
    w = orc.pack_row([0xA, 0x5] + [0] * 6, 4)
    assert w.view(np.uint8)[0] == int(gold["int4_codes_a_5_first_byte"], 16)
    # channel 17 of an INT2 row lives in word 1, bits 2..3
    codes = np.zeros(64, np.uint8)
    codes[17] = 3
    w = orc.pack_row(codes, 2)
    assert w[1] == 3 << 2 and w.sum() == w[1]
    # channel 9 of an INT4 row: word 1, bits 4..7
    codes = np.zeros(64, np.uint8)
    codes[9] = 0xC
    w = orc.pack_row(codes, 4)
    assert w[1] == 0xC << 4 and w.sum() == w[1]


@pytest.mark.parametrize("bits", [2, 4])
def test_pack_unpack_roundtrip(orc, bits):
    rng = np.random.default_rng(3)
    for d in (64, 128):
        codes = rng.integers(0, 1 << bits, d).astype(np.uint8)
        assert np.array_equal(orc.unpack_row(orc.pack_row(codes, bits), d, bits), codes)


@pytest.mark.parametrize("bits", [2, 4])
def test_brute_force_code_vectors(orc, bits):
    """Every code vector, padded with the extreme codes so step = 1 and zero = 0, comes
    back unchanged (all 4^4 INT2 vectors, all 16^2 INT4 pairs)."""
    L = (1 << bits) - 1
    n = 4 if bits == 2 else 2
    for idx in range((L + 1) ** n):
        v = [(idx // (L + 1) ** k) % (L + 1) for k in range(n)]
        x = [0.0, float(L)] + [float(c) for c in v]
        codes, s, z = orc.quantize_group(x, bits)
        assert s == 0x3C00 and z == 0
        assert list(codes) == [0, L] + v


@pytest.mark.parametrize("bits", [2, 4])
def test_roundtrip_bound_and_range(orc, bits):
    """|x - (code*step + zero)| <= step/2 (+ |min - zero| when fp16 moved the zero, + a
    few float32 ulps); codes in [0, L]; the minimum maps to 0 and the maximum to L."""
    L = (1 << bits) - 1
    rng = np.random.default_rng(10 + bits)
    worst = 0.0
    for trial in range(400):
        n = int(rng.integers(2, 130))
        scale = float(np.exp(rng.uniform(-4, 4)))
        x = (rng.standard_normal(n) * scale + rng.uniform(-3, 3) * scale).astype(np.float32)
        codes, s, z = orc.quantize_group(x, bits)
        step, zero = _f16(s), _f16(z)
        assert codes.min() >= 0 and codes.max() <= L
        if step == 0:
            assert np.all(codes == 0)
            continue
        assert codes[np.argmin(x)] == 0 and codes[np.argmax(x)] == L
        xhat = codes.astype(np.float64) * step + zero
        err = np.abs(x.astype(np.float64) - xhat)
        slack = abs(float(x.min()) - zero) + 8 * np.finfo(np.float32).eps * np.abs(x).max()
        bound = step / 2 * (1 + 2.0 ** -9) + slack
        assert np.all(err <= bound), (trial, err.max(), bound)
        worst = max(worst, float((err.max() - abs(float(x.min()) - zero)) / (step / 2)))
    assert worst > 0.9  # the bound is tight: some element sits near a half-step


@pytest.mark.parametrize("bits", [2, 4])
def test_power_of_two_scaling(orc, bits):
    """x -> 2x doubles step and zero exactly and leaves the codes unchanged (away from
    fp16 subnormals and overflow)."""
    rng = np.random.default_rng(20 + bits)
    for _ in range(200):
        x = rng.standard_normal(int(rng.integers(2, 64))).astype(np.float32)
        c1, s1, z1 = orc.quantize_group(x, bits)
        c2, s2, z2 = orc.quantize_group(2 * x, bits)
        assert np.array_equal(c1, c2)
        assert _f16(s2) == 2 * _f16(s1) and _f16(z2) == 2 * _f16(z1)


@pytest.mark.parametrize("bits", [2, 4])
def test_permutation_equivariance(orc, bits):
    rng = np.random.default_rng(30 + bits)
    for _ in range(100):
        x = rng.standard_normal(int(rng.integers(2, 128))).astype(np.float32)
        p = rng.permutation(x.size)
        c1, s1, z1 = orc.quantize_group(x, bits)
        c2, s2, z2 = orc.quantize_group(x[p], bits)
        assert (s1, z1) == (s2, z2) and np.array_equal(c1[p], c2)


def test_dequant_spec_rounding(orc):
    """A1: dequant = round_to_elem(fl32(code*step + zero)); bf16 via torch's cast,
    fp16 via numpy's cast, exact = real arithmetic."""
    rng = np.random.default_rng(7)
    for _ in range(2000):
        s = int(rng.integers(0x0400, 0x5800))
        z = int(rng.integers(0, 0x7800)) | (0x8000 if rng.random() < 0.5 else 0)
        c = int(rng.integers(0, 16))
        y = np.float32(np.float32(c) * np.float32(_f16(s))) + np.float32(_f16(z))
        want_bf = torch.tensor([float(y)], dtype=torch.float32).to(torch.bfloat16).double().item()
        want_h = float(np.float32(y).astype(np.float16))
        assert orc.dequant(c, s, z, "bf16") == want_bf
        assert orc.dequant(c, s, z, "f16") == want_h
        assert orc.dequant(c, s, z, "bf16", exact=True) == c * _f16(s) + _f16(z)


def _np_unpack(words, d, bits):
    """Layout check with numpy bit operations (channel c: word c // (32/b), shift b*(c % (32/b)))."""
    per = 32 // bits
    c = np.arange(d)
    return ((words[..., c // per] >> (bits * (c % per)).astype(np.uint32)) & ((1 << bits) - 1)).astype(np.uint8)


@pytest.mark.parametrize("bits", [2, 4])
def test_append_layout_contiguous(orc, bits):
    """Q3 contiguous: K groups of Gk tokens from the append's own first token (last one
    short), V groups per (token, 32 channels); codes and meta land in the documented
    slots; a second append continues the table."""
    rng = np.random.default_rng(40 + bits)
    B, H, d, Gk = 2, 3, 64, 32
    seg = orc.new_segment(bits, "bf16", B, H, d, capacity=200, k_group_tokens=Gk, kgroup_capacity=16)
    ks = [rng.standard_normal((B, H, n, d)).astype(np.float32) for n in (70, 45)]
    vs = [rng.standard_normal((B, H, n, d)).astype(np.float32) for n in (70, 45)]
    assert orc.append(seg, ks[0], vs[0]) == 3
    assert orc.append(seg, ks[1], vs[1]) == 2
    assert seg["n_tokens"] == 115 and seg["n_kgroups"] == 5
    assert list(seg["kgroup_start"][:6]) == [0, 32, 64, 70, 102, 115]
    kc = _np_unpack(seg["k_codes"], d, bits)
    vc = _np_unpack(seg["v_codes"], d, bits)
    starts = seg["kgroup_start"]
    src_k = np.concatenate(ks, axis=2)
    src_v = np.concatenate(vs, axis=2)
    for b in range(B):
        for h in range(H):
            for g in range(5):
                t0, t1 = starts[g], starts[g + 1]
                for ch in (0, 17, d - 1):
                    codes, s, z = orc.quantize_group(src_k[b, h, t0:t1, ch], bits)
                    assert np.array_equal(kc[b, h, t0:t1, ch], codes)
                    assert tuple(seg["k_meta"][b, h, g, ch]) == (s, z)
            for t in (0, 69, 70, 114):
                for gv in range(d // 32):
                    codes, s, z = orc.quantize_group(src_v[b, h, t, 32 * gv:32 * gv + 32], bits)
                    assert np.array_equal(vc[b, h, t, 32 * gv:32 * gv + 32], codes)
                    assert tuple(seg["v_meta"][b, h, t, gv]) == (s, z)


def test_append_gather_windows(orc):
    """Q3 gather: each listed {start, len} becomes one K-group, in list order."""
    rng = np.random.default_rng(50)
    B, H, d = 1, 2, 64
    N = 150                                  # windows of 32: 0..4, window 4 has 22 tokens
    k = rng.standard_normal((B, H, N, d)).astype(np.float32)
    v = rng.standard_normal((B, H, N, d)).astype(np.float32)
    groups = np.array([[32, 32], [128, 22], [0, 32]], np.int32)
    seg = orc.new_segment(4, "f16", B, H, d, capacity=100, k_group_tokens=32, kgroup_capacity=8)
    assert orc.append(seg, k, v, groups=groups) == 3
    assert list(seg["kgroup_start"][:4]) == [0, 32, 54, 86]
    kc = _np_unpack(seg["k_codes"], d, 4)
    for g, (s0, ln) in enumerate(groups):
        t0 = seg["kgroup_start"][g]
        for ch in range(d):
            codes, s, z = orc.quantize_group(k[0, 1, s0:s0 + ln, ch], 4)
            assert np.array_equal(kc[0, 1, t0:t0 + ln, ch], codes)
            assert tuple(seg["k_meta"][0, 1, g, ch]) == (s, z)


def test_append_rejects_overflow(orc):
    seg = orc.new_segment(2, "bf16", 1, 1, 64, capacity=40, k_group_tokens=32, kgroup_capacity=4)
    x = np.zeros((1, 1, 41, 64), np.float32)
    with pytest.raises(ValueError):
        orc.append(seg, x, x)
    assert seg["n_tokens"] == 0


def test_video_chunk_group_table(orc):
    """Chunk-wise cache of the 12-head video workload: 4 appends of 4,680 tokens with
    128-token K groups give 37 groups per append (36 x 128 + one of 72), 148 in all."""
    w = workloads.WORKLOADS["video_chunk_int2_h12_d128"]
    seg = orc.new_segment(2, "bf16", 1, 1, 64, capacity=w.n_cache, k_group_tokens=128,
                          kgroup_capacity=200)
    x = np.zeros((1, 1, w.append_tokens, 64), np.float32)
    for _ in range(w.n_appends):
        assert orc.append(seg, x, x) == 37
    st = seg["kgroup_start"][:seg["n_kgroups"] + 1]
    assert seg["n_kgroups"] == 148
    assert list(st[:3]) == [0, 128, 256] and st[36] == 4608 and st[37] == 4680 and st[-1] == 18720
    lens = np.diff(st)
    assert np.all((lens == 128) | (lens == 72)) and (lens == 72).sum() == 4
