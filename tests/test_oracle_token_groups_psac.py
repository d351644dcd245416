"""Pins of the oracle's per-token K groups and low-rank logit compensation.

Per-token K groups: "Quantized Keys Steal Attention: Bias Correction for KV-Cache
Compression in Video Diffusion", abstract, computes its correction from the cached keys'
step sizes and the query norm. The norm alone suffices when every channel of a key shares
one step, i.e. when keys are grouped per token (as values are) over all channels. Pins:
keys grouped per token in runs of 32 channels are quantized exactly as values are (the
value path is pinned in test_oracle_quant.py); with one group over all channels the
channel-weighted and the query-norm forms of the correction agree, and a single cached
key's correction is tau^2/24 |q|^2 step^2 (read back from the log-sum-exp).

Compensation: "QuantWM Preserves Attention in 2-Bit KV Cache Quantization for Video World
Models" (its PSAC item) compensates key error along the dominant query subspace; the pages
give no formula, and the one built here stores c_t = bf16(U^T (k_t - khat_t)) per token and
adds (U^T q) . c_t to the logit. Pins from that definition: for queries inside span(U)
the logits are those of the unquantized keys up to the bf16 rounding of c (checked against
float64 attention over the original keys, with a bound from that rounding), for queries
orthogonal to it the output is that of the uncompensated cache exactly, and bf16 rounding
from double is pinned by hand values.
"""
import numpy as np
import pytest
import torch


def _kv(rng, B, H, n, d, dtype=torch.bfloat16, scale=2.0):
    k = torch.from_numpy((rng.standard_normal((B, H, n, d)) * scale).astype(np.float32)).to(dtype)
    v = torch.from_numpy(rng.standard_normal((B, H, n, d)).astype(np.float32)).to(dtype)
    return k.float().numpy(), v.float().numpy()


def test_bf16_from_double_hand_values(orc):
    assert orc.f64_to_bf16_bits(1.0) == 0x3F80
    assert orc.f64_to_bf16_bits(1.0 + 2 ** -8) == 0x3F80          # half-way: to even (down)
    assert orc.f64_to_bf16_bits(1.0 + 3 * 2 ** -8) == 0x3F82       # half-way: to even (up)
    assert orc.f64_to_bf16_bits(1.0 + 2 ** -8 + 2 ** -40) == 0x3F81  # just above half: up
    assert orc.f64_to_bf16_bits(-2.5) == 0xC020
    assert orc.f64_to_bf16_bits(0.0) == 0 and orc.f64_to_bf16_bits(-0.0) == 0x8000
    assert orc.f64_to_bf16_bits(2.0 ** -130) == 0x0008               # subnormal: 8 units of 2^-133


@pytest.mark.parametrize("bits", [2, 4])
def test_token_groups_of_32_quantize_keys_as_values(orc, bits):
    rng = np.random.default_rng(4)
    B, H, n, d = 1, 2, 70, 128
    k, v = _kv(rng, B, H, n, d)
    seg = orc.new_segment(bits, "bf16", B, H, d, capacity=n, k_group_tokens=32, kgroup_capacity=4,
                          k_group_channels=32)
    assert orc.append(seg, k, k) == 0 and seg["n_kgroups"] == 0     # no K-group table
    assert np.array_equal(seg["k_codes"], seg["v_codes"])
    assert np.array_equal(seg["k_meta"], seg["v_meta"])


def test_token_groups_over_all_channels_make_the_norm_form_exact(orc):
    rng = np.random.default_rng(5)
    B, H, n, d = 1, 1, 300, 64
    k, v = _kv(rng, B, H, n, d)
    seg = orc.new_segment(2, "bf16", B, H, d, capacity=n, k_group_tokens=64, kgroup_capacity=8,
                          k_group_channels=d)
    orc.append(seg, k, v)
    q = rng.standard_normal((B, 2, 40, d)).astype(np.float32)
    o1, l1 = orc.attention(q, [seg], n_kv_heads=H, jensen=1)
    o2, l2 = orc.attention(q, [seg], n_kv_heads=H, jensen=2)
    o0, l0 = orc.attention(q, [seg], n_kv_heads=H, jensen=0)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-13)
    np.testing.assert_allclose(l1, l2, rtol=0, atol=1e-12)
    assert np.abs(o1 - o0).max() > 1e-4                               # the correction acts
    # one cached key: lse = scale q.khat - tau^2/24 |q|^2 step^2
    one = orc.new_segment(2, "bf16", 1, 1, d, capacity=1, k_group_tokens=1, kgroup_capacity=1,
                          k_group_channels=d)
    orc.append(one, k[:, :, :1], v[:, :, :1])
    step = float(one["k_meta"][0, 0, 0, 0, 0:1].view(np.float16)[0])
    tau = 1 / np.sqrt(d)
    for i in range(5):
        qi = q[:, :1, i:i + 1]
        _, l_on = orc.attention(qi, [one], n_kv_heads=1, jensen=1)
        _, l_off = orc.attention(qi, [one], n_kv_heads=1, jensen=0)
        want = tau ** 2 / 24 * float((qi.astype(np.float64) ** 2).sum()) * step ** 2
        assert float(l_off - l_on) == pytest.approx(want, rel=1e-9)


def _basis(rng, H, d, r):
    U = np.zeros((H, d, r), np.float32)
    for h in range(H):
        U[h] = np.linalg.qr(rng.standard_normal((d, r)))[0].astype(np.float32)
    return U


def _sdpa(q, K, V, scale):
    s = scale * q @ K.T
    w = np.exp(s - s.max(-1, keepdims=True))
    w /= w.sum(-1, keepdims=True)
    return w @ V


@pytest.mark.parametrize("bits", [2, 4])
def test_compensation_restores_logits_inside_the_subspace(orc, bits):
    rng = np.random.default_rng(6)
    B, H, n, d, r = 1, 2, 400, 128, 8
    k, v = _kv(rng, B, H, n, d)
    U = _basis(rng, H, d, r)
    seg = orc.new_segment(bits, "bf16", B, H, d, capacity=n, k_group_tokens=128, kgroup_capacity=4, comp_basis=U)
    plain = orc.new_segment(bits, "bf16", B, H, d, capacity=n, k_group_tokens=128, kgroup_capacity=4)
    orc.append(seg, k, v)
    orc.append(plain, k, v)
    assert np.array_equal(seg["k_codes"], plain["k_codes"]) and np.array_equal(seg["k_meta"], plain["k_meta"])
    assert np.all(seg["k_comp"][..., r:] == 0)
    tau = 1 / np.sqrt(d)
    nq = 12
    # queries inside span(U_h), of the size of ordinary queries
    a = rng.standard_normal((B, H, nq, r)) * np.sqrt(d / r)
    q = np.einsum("hdr,bhqr->bhqd", U.astype(np.float64), a).astype(np.float32)
    out_c, _ = orc.attention(q, [seg], n_kv_heads=H, jensen=0)
    out_p, _ = orc.attention(q, [plain], n_kv_heads=H, jensen=0)
    Vhat = np.zeros((H, n, d))
    for h in range(H):   # the dequantized values, from the uncompensated oracle with identity keys
        _, Vh = _dense(orc, plain, h, d)
        Vhat[h] = Vh
    cst = seg["k_comp"][0].view(np.uint16).astype(np.uint32) << 16
    cval = cst.view(np.float32)[..., :r].astype(np.float64)             # [H][n][r] stored c
    for h in range(H):
        want = _sdpa(q[0, h].astype(np.float64), k[0, h].astype(np.float64), Vhat[h], tau)
        err_c = np.abs(out_c[0, h] - want).max()
        err_p = np.abs(out_p[0, h] - want).max()
        # the stored c is within half a bf16 ulp (< 2^-8 |c|) of U^T (k - khat): every logit is
        # within delta of the unquantized one, and the output within max|v| (e^{2 delta} - 1)
        uq = np.abs(q[0, h].astype(np.float64) @ U[h].astype(np.float64))  # [nq][r]
        delta = tau * (uq @ (2.0 ** -8 * np.abs(cval[h])).T).max()
        bound = np.abs(Vhat[h]).max() * np.expm1(2 * delta)
        assert err_c <= bound and err_c * 20 < err_p, (h, err_c, bound, err_p)


def _dense(orc, seg, h, d):
    """The dequantized values of one head, from the stored codes and step/zero through the
    oracle's unpacking and dequantization (both pinned in test_oracle_quant.py)."""
    n = seg["n_tokens"]
    V = np.zeros((n, d))
    for t in range(n):
        codes = orc.unpack_row(seg["v_codes"][0, h, t], d, seg["bits"])
        for c in range(d):
            m = seg["v_meta"][0, h, t, c // 32]
            V[t, c] = orc.dequant(int(codes[c]), int(m[0]), int(m[1]), seg["elem"])
    return None, V


def test_compensation_is_invisible_to_orthogonal_queries(orc):
    rng = np.random.default_rng(7)
    B, H, n, d, r = 1, 1, 300, 64, 4
    k, v = _kv(rng, B, H, n, d)
    U = _basis(rng, H, d, r)
    seg = orc.new_segment(2, "bf16", B, H, d, capacity=n, k_group_tokens=64, kgroup_capacity=8, comp_basis=U)
    plain = orc.new_segment(2, "bf16", B, H, d, capacity=n, k_group_tokens=64, kgroup_capacity=8)
    orc.append(seg, k, v)
    orc.append(plain, k, v)
    q = rng.standard_normal((B, 1, 20, d))
    P = np.eye(d) - U[0].astype(np.float64) @ U[0].T.astype(np.float64)
    q = (q @ P.T).astype(np.float32)
    # float32 rounding of q leaves U^T q at ~1e-7: the compensation then moves logits by
    # less than 1e-7 * |c|
    o_c, l_c = orc.attention(q, [seg], n_kv_heads=H, jensen=1)
    o_p, l_p = orc.attention(q, [plain], n_kv_heads=H, jensen=1)
    np.testing.assert_allclose(o_c, o_p, rtol=0, atol=1e-6)
    np.testing.assert_allclose(l_c, l_p, rtol=0, atol=1e-6)
