"""Pins of the oracle's Jensen-bias correction.

The pages ("Quantized Keys Steal Attention: Bias Correction for KV-Cache Compression
in Video Diffusion", abstract) state that, because exp is convex, quantization noise
on cached keys inflates their softmax weight, so they take attention mass from the
unquantized current chunk; and that a per-score correction built from the cached keys'
step sizes and the query removes this bias in expectation, in a second-order Taylor
form. Under the uniform rounding-noise model (e_c ~ U(-step_c/2, step_c/2), channels
independent):

    E[exp(tau q.e)] = prod_c sinh(a_c)/a_c,   a_c = tau |q_c| step_c / 2
    log(sinh a / a) = a^2/6 - a^4/180 + ...

so the second-order correction to subtract from the logit is sum_c a_c^2 / 6. These
tests take the oracle's correction out of its log-sum-exp and check it against that
closed form, then check by Monte Carlo on the tiny workload's real INT2 and INT4 step
sizes that (a) without the correction the cached-key mass is inflated, (b) with it
the bias shrinks at least 3x, and (c) the mean partition-sum ratios match the closed
forms within 3 standard errors.
"""
import numpy as np
import pytest

import workloads


def _lncosh_ratio(a):
    a = np.asarray(a, np.float64)
    out = np.zeros_like(a)
    nz = a > 1e-4
    out[nz] = np.log(np.sinh(a[nz]) / a[nz])
    out[~nz] = a[~nz] ** 2 / 6
    return out


def _tiny_setup(orc, bits):
    w = workloads.WORKLOADS["tiny_int2_h1_d64"]
    data = workloads.generate(w)
    d = w.head_dim
    seg = orc.new_segment(bits, "bf16", 1, 1, d, capacity=w.n_cache, k_group_tokens=w.k_group_tokens,
                          kgroup_capacity=w.n_cache // w.k_group_tokens)
    K = data["cache_k"].float().numpy()
    V = data["cache_v"].float().numpy()
    orc.append(seg, K, V)
    G = seg["n_kgroups"]
    step = seg["k_meta"][0, 0, :G, :, 0].copy().view(np.float16).astype(np.float64)   # [G][d]
    gid = np.repeat(np.arange(G), w.k_group_tokens).astype(np.int32)
    q = data["q"].float().numpy()[0, 0].astype(np.float64)
    kc = data["cur_k"].float().numpy()[0, 0].astype(np.float64)
    vc = data["cur_v"].float().numpy()[0, 0].astype(np.float64)
    return K[0, 0].astype(np.float64), V[0, 0].astype(np.float64), step, gid, q, kc, vc


def _beta_from_oracle(orc, q, k, step_row, scale):
    """The oracle's correction for one (query, key group): with a single cached key the
    log-sum-exp is the corrected logit itself, so beta = scale*q.k - lse."""
    _, lse, _ = orc.attend_row(q, k[None], np.zeros((1, q.size)), np.zeros(1, np.int32),
                               step_row[None] ** 2, scale, True)
    return scale * float(q @ k) - lse


@pytest.mark.parametrize("bits", [2, 4])
def test_beta_is_second_order_term_of_closed_form(orc, bits):
    K, V, step, gid, q, kc, vc = _tiny_setup(orc, bits)
    scale = 1 / np.sqrt(K.shape[1])
    for shrink in (1.0, 1 / 8):
        for g in range(step.shape[0]):
            for i in (0, 7, 15):
                st = step[g] * shrink
                beta = _beta_from_oracle(orc, q[i], K[0], st, scale)
                a = scale * np.abs(q[i]) * st / 2
                exact = _lncosh_ratio(a).sum()
                second = (a ** 2).sum() / 6
                # beta comes out of a difference of O(1) numbers: allow that cancellation
                np.testing.assert_allclose(beta, second, rtol=1e-10, atol=1e-14)
                # the exact log-MGF differs only by the 4th-order term
                assert abs(beta - exact) <= (a ** 4).sum() / 180 * 1.01 + 1e-15
                assert beta > 0


@pytest.mark.parametrize("bits", [2, 4])
def test_monte_carlo_mass_bias(orc, bits):
    K, V, step, gid, q, kc, vc = _tiny_setup(orc, bits)
    scale = 1 / np.sqrt(K.shape[1])
    n, d = K.shape
    R = 3000 if bits == 2 else 2000
    rng = np.random.default_rng(100 + bits)
    Kall = np.concatenate([K, kc]); Vall = np.concatenate([V, vc])
    tg = np.concatenate([gid, -np.ones(kc.shape[0], np.int32)]).astype(np.int32)
    ssq = step ** 2
    nq = q.shape[0]
    true_mass = np.array([orc.attend_row(q[i], Kall, Vall, tg, ssq, scale, False)[2] for i in range(nq)])
    true_lse_cache = np.array([orc.attend_row(q[i], K, V, gid, ssq, scale, False)[1] for i in range(nq)])
    m_off = np.zeros((R, nq)); m_on = np.zeros((R, nq))
    r_off = np.zeros((R, nq)); r_on = np.zeros((R, nq))
    half = step[gid] / 2                                             # [n][d]
    for r in range(R):
        Kn = K + rng.uniform(-1.0, 1.0, (n, d)) * half
        Knall = np.concatenate([Kn, kc])
        for i in range(nq):
            m_off[r, i] = orc.attend_row(q[i], Knall, Vall, tg, ssq, scale, False)[2]
            m_on[r, i] = orc.attend_row(q[i], Knall, Vall, tg, ssq, scale, True)[2]
            r_off[r, i] = np.exp(orc.attend_row(q[i], Kn, V, gid, ssq, scale, False)[1] - true_lse_cache[i])
            r_on[r, i] = np.exp(orc.attend_row(q[i], Kn, V, gid, ssq, scale, True)[1] - true_lse_cache[i])
    bias_off = (m_off - true_mass).mean(0)          # per query
    bias_on = (m_on - true_mass).mean(0)
    # (a) inflation without correction: the query-averaged mass bias is positive and
    # well outside its standard error. (Single queries may show a small negative bias:
    # the mass is a concave function of the cached partition sum, whose expectation
    # is what the noise inflates.)
    avg_off = (m_off - true_mass).mean(1)
    assert avg_off.mean() > 3 * avg_off.std() / np.sqrt(R)
    # (b) the correction cuts the mean absolute bias at least 3x
    assert np.abs(bias_on).mean() * 3 <= np.abs(bias_off).mean()
    # (c) partition-sum ratios against the closed forms
    for i in range(nq):
        s_true = scale * K @ q[i]
        w = np.exp(s_true - s_true.max()); w /= w.sum()
        a = scale * np.abs(q[i])[None, :] * step[gid] / 2            # [n][d]
        lmgf = _lncosh_ratio(a).sum(1)                                # [n]
        beta = (a ** 2).sum(1) / 6
        want_off = (w * np.exp(lmgf)).sum()
        want_on = (w * np.exp(lmgf - beta)).sum()
        for got, want in ((r_off[:, i], want_off), (r_on[:, i], want_on)):
            se = got.std() / np.sqrt(R)
            assert abs(got.mean() - want) <= 3 * se + 1e-12, (i, got.mean(), want, se)
