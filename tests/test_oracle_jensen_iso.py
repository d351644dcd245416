"""Pins of the isotropic Jensen form (jensen == 2) against the channel-weighted one.

"Quantized Keys Steal Attention: Bias Correction for KV-Cache Compression in Video
Diffusion", abstract: the correction is computed from the step sizes of the cached keys
and the query's norm. The channel-weighted second-order term
    beta_1 = tau^2/24 * sum_c q_c^2 step_c^2
becomes a function of the norm alone when every channel's step^2 is replaced by its mean
over the group's channels:
    beta_2 = tau^2/24 * |q|^2 * mean_c step_c^2.
Neither pin below restates that formula: beta_2 is the average of beta_1 over all cyclic
shifts of the step vector, the two are equal when the steps are equal across channels
(here built through the whole quantize-and-attend path), and small hand examples fix the
constants. beta is read off the oracle as minus the log-sum-exp of a row whose only key
is a zero key of group 0.
"""
import numpy as np
import pytest
import torch


def beta_of(orc, q, step_sq, scale, jensen):
    d = q.size
    K = np.zeros((1, d)); V = np.zeros((1, d)); tg = np.zeros(1, np.int32)
    _, lse, _ = orc.attend_row(q, K, V, tg, np.asarray(step_sq, np.float64)[None, :], scale, jensen)
    return -lse


def test_hand_values(orc):
    q = np.array([1.0, 2.0])
    s2 = np.array([4.0, 16.0])
    # weighted: (1*4 + 4*16) / 24; isotropic: (1 + 4) * (4 + 16) / 2 / 24
    assert beta_of(orc, q, s2, 1.0, 1) == pytest.approx(68.0 / 24.0, rel=1e-15)
    assert beta_of(orc, q, s2, 1.0, 2) == pytest.approx(50.0 / 24.0, rel=1e-15)
    assert beta_of(orc, q, s2, 1.0, 0) == 0.0
    # the scale enters squared
    assert beta_of(orc, q, s2, 0.5, 2) == pytest.approx(50.0 / 24.0 / 4.0, rel=1e-15)


@pytest.mark.parametrize("d", [64, 128])
def test_isotropic_is_the_shift_average_of_the_weighted_form(orc, d):
    rng = np.random.default_rng(40 + d)
    q = rng.standard_normal(d)
    s2 = rng.uniform(0.0, 2.0, d) ** 2
    scale = 1.0 / np.sqrt(d)
    iso = beta_of(orc, q, s2, scale, 2)
    avg = np.mean([beta_of(orc, q, np.roll(s2, k), scale, 1) for k in range(d)])
    assert abs(iso - avg) <= 1e-12 * abs(iso)
    # and the two forms differ for unequal steps
    assert abs(beta_of(orc, q, s2, scale, 1) - iso) > 1e-3 * abs(iso)


def _latin_group_keys(rng, n_groups, G, d):
    """Keys whose channels all take the same G values inside each K-group, in shifted
    orders: every channel of a group has the same minimum and maximum, hence the same step."""
    out = np.zeros((n_groups * G, d), np.float32)
    for g in range(n_groups):
        base = torch.from_numpy(rng.standard_normal(G).astype(np.float32) * 3).bfloat16().float().numpy()
        for c in range(d):
            out[g * G:(g + 1) * G, c] = np.roll(base, c)
    return out


@pytest.mark.parametrize("bits", [2, 4])
def test_forms_agree_when_steps_are_equal_across_channels(orc, bits):
    rng = np.random.default_rng(7 + bits)
    d, G, n_groups, Hkv = 64, 32, 4, 2
    seg = orc.new_segment(bits, "bf16", 1, Hkv, d, capacity=n_groups * G, k_group_tokens=G,
                          kgroup_capacity=n_groups)
    k = np.stack([_latin_group_keys(rng, n_groups, G, d) for _ in range(Hkv)])[None]
    v = torch.from_numpy(rng.standard_normal((1, Hkv, n_groups * G, d)).astype(np.float32)).bfloat16().float().numpy()
    orc.append(seg, k, v)
    steps = seg["k_meta"][0, :, :n_groups, :, 0].copy().view(np.float16)
    assert (steps == steps[..., :1]).all() and (steps != 0).all()
    q = torch.from_numpy(rng.standard_normal((1, 4, 6, d)).astype(np.float32)).bfloat16().float().numpy()
    kc = torch.from_numpy(rng.standard_normal((1, Hkv, 5, d)).astype(np.float32)).bfloat16().float().numpy()
    vc = torch.from_numpy(rng.standard_normal((1, Hkv, 5, d)).astype(np.float32)).bfloat16().float().numpy()
    o1, l1 = orc.attention(q, [seg], kc, vc, jensen=1)
    o2, l2 = orc.attention(q, [seg], kc, vc, jensen=2)
    o0, _ = orc.attention(q, [seg], kc, vc, jensen=0)
    assert np.abs(o1 - o2).max() < 1e-13 and np.abs(l1 - l2).max() < 1e-13
    assert np.abs(o1 - o0).max() > 1e-4


def test_forms_differ_for_unequal_steps(orc):
    rng = np.random.default_rng(12)
    d, Hkv = 64, 1
    seg = orc.new_segment(2, "bf16", 1, Hkv, d, capacity=64, k_group_tokens=32, kgroup_capacity=2)
    scales = rng.lognormal(0.0, 0.5, d).astype(np.float32)
    k = torch.from_numpy(rng.standard_normal((1, Hkv, 64, d)).astype(np.float32) * scales).bfloat16().float().numpy()
    v = torch.from_numpy(rng.standard_normal((1, Hkv, 64, d)).astype(np.float32)).bfloat16().float().numpy()
    orc.append(seg, k, v)
    q = torch.from_numpy(rng.standard_normal((1, 1, 4, d)).astype(np.float32)).bfloat16().float().numpy()
    _, l1 = orc.attention(q, [seg], None, None, jensen=1)
    _, l2 = orc.attention(q, [seg], None, None, jensen=2)
    assert np.abs(l1 - l2).max() > 1e-4
