"""Pins of the oracle's chunk attention (A1-A3).

The library pin is torch's scaled_dot_product_attention in float64 on the CPU, fed
with keys/values decoded from the packed cache independently (numpy bit operations,
numpy float32 arithmetic, torch's bf16 / numpy's fp16 casts) and with the Jensen
term as an additive mask. Closed forms and invariants pin the rest: a single key, all
keys equal, zero step sizes, permutation of the history, and the log-sum-exp merge of
two halves of the history.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import workloads


def _np_unpack(words, d, bits):
    per = 32 // bits
    c = np.arange(d)
    return ((words[..., c // per] >> (bits * (c % per)).astype(np.uint32)) & ((1 << bits) - 1)).astype(np.float32)


def _round_elem(y32, elem):
    if elem == "bf16":
        return torch.from_numpy(y32).to(torch.bfloat16).double().numpy()
    return y32.astype(np.float16).astype(np.float64)


def np_decode(seg, b, h):
    """Independent decode of one (b, h) of a segment: K, V [n][d] float64, the K-group of
    each token and the fp16 step of (token, channel) for the Jensen term."""
    n, d, bits = seg["n_tokens"], seg["d"], seg["bits"]
    if bits == 16:
        to = (lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).double().numpy()) \
            if seg["elem"] == "bf16" else (lambda a: a.view(np.float16).astype(np.float64))
        return to(seg["k_raw"][b, h, :n]), to(seg["v_raw"][b, h, :n]), None, None
    starts = seg["kgroup_start"][:seg["n_kgroups"] + 1]
    gid = np.searchsorted(starts, np.arange(n), side="right") - 1
    km = seg["k_meta"][b, h][gid]                       # [n][d][2]
    ks = km[..., 0].copy().view(np.float16).astype(np.float32)
    kz = km[..., 1].copy().view(np.float16).astype(np.float32)
    vm = np.repeat(seg["v_meta"][b, h, :n], seg["Gv"], axis=1)
    vs = vm[..., 0].copy().view(np.float16).astype(np.float32)
    vz = vm[..., 1].copy().view(np.float16).astype(np.float32)
    kc = _np_unpack(seg["k_codes"][b, h, :n], d, bits)
    vc = _np_unpack(seg["v_codes"][b, h, :n], d, bits)
    K = _round_elem((kc * ks + kz).astype(np.float32), seg["elem"])
    V = _round_elem((vc * vs + vz).astype(np.float32), seg["elem"])
    return K, V, gid, ks.astype(np.float64)


def sdpa_reference(q, segs, k_cur, v_cur, Hkv, scale, jensen):
    """float64 SDPA over [decoded history; current chunk] with mask = -beta."""
    B, Hq, nq, d = q.shape
    gqa = Hq // Hkv
    out = np.zeros((B, Hq, nq, d))
    for b in range(B):
        for h in range(Hkv):
            Ks, Vs, S2 = [], [], []
            for s in segs:
                K, V, gid, st = np_decode(s, b, h)
                Ks.append(K); Vs.append(V)
                S2.append(np.zeros_like(K) if st is None else st * st)
            if k_cur is not None:
                Ks.append(k_cur[b, h].astype(np.float64)); Vs.append(v_cur[b, h].astype(np.float64))
                S2.append(np.zeros((k_cur.shape[2], d)))
            K = np.concatenate(Ks); V = np.concatenate(Vs); S2 = np.concatenate(S2)
            for r in range(gqa):
                hq = h * gqa + r
                qq = q[b, hq].astype(np.float64)                       # [nq][d]
                if jensen == 1:
                    beta = scale * scale / 24.0 * (qq * qq) @ S2.T
                elif jensen == 2:
                    beta = scale * scale / 24.0 * np.outer((qq * qq).sum(1), S2.mean(1))
                else:
                    beta = np.zeros((nq, K.shape[0]))
                o = F.scaled_dot_product_attention(
                    torch.from_numpy(qq)[None, None], torch.from_numpy(K)[None, None],
                    torch.from_numpy(V)[None, None], attn_mask=torch.from_numpy(-beta)[None, None],
                    scale=scale)
                out[b, hq] = o[0, 0].numpy()
    return out


def build_cache(orc, w, data):
    seg = orc.new_segment(w.bits, w.dtype, w.batch, w.n_kv_heads, w.head_dim,
                          capacity=w.n_cache, k_group_tokens=w.k_group_tokens,
                          kgroup_capacity=w.n_appends * (-(-w.append_tokens // w.k_group_tokens)))
    ck = data["cache_k"].float().numpy(); cv = data["cache_v"].float().numpy()
    for a in range(w.n_appends):
        sl = slice(a * w.append_tokens, (a + 1) * w.append_tokens)
        orc.append(seg, ck[:, :, sl], cv[:, :, sl])
    return seg


@pytest.mark.parametrize("jensen", [0, 1, 2])
def test_tiny_workload_vs_sdpa(orc, jensen):
    w = workloads.WORKLOADS["tiny_int2_h1_d64"]
    data = workloads.generate(w)
    seg = build_cache(orc, w, data)
    q = data["q"].float().numpy(); kc = data["cur_k"].float().numpy(); vc = data["cur_v"].float().numpy()
    scale = 1 / np.sqrt(w.head_dim)
    out, lse = orc.attention(q, [seg], kc, vc, scale=scale, jensen=jensen)
    ref = sdpa_reference(q, [seg], kc, vc, 1, scale, jensen)
    assert np.abs(out - ref).max() < 1e-12


def test_gqa_mixed_segments_vs_sdpa(orc):
    rng = np.random.default_rng(5)
    B, Hq, Hkv, d = 2, 4, 2, 64
    segs = []
    for bits, elem, n in ((4, "bf16", 90), (2, "bf16", 70), (16, "bf16", 33)):
        s = orc.new_segment(bits, elem, B, Hkv, d, capacity=100, k_group_tokens=32, kgroup_capacity=8)
        k = torch.from_numpy(rng.standard_normal((B, Hkv, n, d)).astype(np.float32) * 2).bfloat16().float().numpy()
        v = torch.from_numpy(rng.standard_normal((B, Hkv, n, d)).astype(np.float32)).bfloat16().float().numpy()
        orc.append(s, k, v)
        segs.append(s)
    q = torch.from_numpy(rng.standard_normal((B, Hq, 5, d)).astype(np.float32)).bfloat16().float().numpy()
    kc = torch.from_numpy(rng.standard_normal((B, Hkv, 10, d)).astype(np.float32)).bfloat16().float().numpy()
    vc = torch.from_numpy(rng.standard_normal((B, Hkv, 10, d)).astype(np.float32)).bfloat16().float().numpy()
    for jensen in (0, 1, 2):
        out, lse = orc.attention(q, segs, kc, vc, scale=0.125, jensen=jensen)
        ref = sdpa_reference(q, segs, kc, vc, Hkv, 0.125, jensen)
        assert np.abs(out - ref).max() < 1e-12
    # a subset of rows equals the same rows of the full computation
    out_r, lse_r = orc.attention(q, segs, kc, vc, scale=0.125, rows=[4, 0])
    out_f, lse_f = orc.attention(q, segs, kc, vc, scale=0.125)
    assert np.array_equal(out_r[:, :, 0], out_f[:, :, 4]) and np.array_equal(lse_r[:, :, 1], lse_f[:, :, 0])


def test_fp16_window_segments_vs_sdpa(orc):
    rng = np.random.default_rng(6)
    B, Hq, Hkv, d = 1, 14, 2, 64
    segs = []
    for bits, n in ((16, 40), (4, 64), (2, 96)):
        s = orc.new_segment(bits, "f16", B, Hkv, d, capacity=n, k_group_tokens=32, kgroup_capacity=4)
        k = (rng.standard_normal((B, Hkv, n, d)) * 3).astype(np.float16).astype(np.float32)
        v = rng.standard_normal((B, Hkv, n, d)).astype(np.float16).astype(np.float32)
        orc.append(s, k, v)
        segs.append(s)
    q = rng.standard_normal((B, Hq, 1, d)).astype(np.float16).astype(np.float32)
    out, _ = orc.attention(q, segs, None, None, n_kv_heads=Hkv, jensen=1)
    ref = sdpa_reference(q, segs, None, None, Hkv, 1 / 8, 1)
    assert np.abs(out - ref).max() < 1e-12


def test_single_key_closed_form(orc):
    rng = np.random.default_rng(8)
    d = 64
    q = rng.standard_normal((1, 1, 3, d)).astype(np.float32)
    kc = rng.standard_normal((1, 1, 1, d)).astype(np.float32)
    vc = rng.standard_normal((1, 1, 1, d)).astype(np.float32)
    out, lse = orc.attention(q, [], kc, vc, n_kv_heads=1, scale=0.125)
    assert np.array_equal(out[0, 0], np.repeat(vc[0, 0].astype(np.float64), 3, axis=0))
    np.testing.assert_allclose(lse[0, 0], 0.125 * (q[0, 0].astype(np.float64) @ kc[0, 0, 0]), rtol=1e-14)


def test_equal_keys_give_mean_value(orc):
    """All history keys identical (constant channels: step 0) and no current chunk: all
    logits tie, so the output is the plain mean of the decoded values, Jensen or not."""
    rng = np.random.default_rng(9)
    d, n = 64, 96
    key = rng.standard_normal(d).astype(np.float32)
    k = np.broadcast_to(key, (1, 1, n, d)).copy()
    v = rng.standard_normal((1, 1, n, d)).astype(np.float32)
    s = orc.new_segment(2, "bf16", 1, 1, d, capacity=n, k_group_tokens=32, kgroup_capacity=4)
    orc.append(s, k, v)
    assert np.all(s["k_meta"][..., 0][0, 0, :3] == 0)          # step 0 on every channel
    q = rng.standard_normal((1, 1, 4, d)).astype(np.float32)
    _, V, _, _ = np_decode(s, 0, 0)
    for jensen in (0, 1):
        out, _ = orc.attention(q, [s], None, None, n_kv_heads=1, jensen=jensen)
        np.testing.assert_allclose(out[0, 0], np.broadcast_to(V.mean(0), (4, d)), atol=1e-14)


def test_permutation_of_history_is_invisible(orc):
    """One K-group over the whole history: permuting its tokens permutes the codes and
    keeps the step/zero, so the output is unchanged up to summation order."""
    rng = np.random.default_rng(10)
    d, n = 64, 128
    k = rng.standard_normal((1, 1, n, d)).astype(np.float32)
    v = rng.standard_normal((1, 1, n, d)).astype(np.float32)
    p = rng.permutation(n)
    q = rng.standard_normal((1, 1, 6, d)).astype(np.float32)
    kc = rng.standard_normal((1, 1, 7, d)).astype(np.float32)
    outs = []
    for perm in (np.arange(n), p):
        s = orc.new_segment(2, "bf16", 1, 1, d, capacity=n, k_group_tokens=n, kgroup_capacity=1)
        orc.append(s, k[:, :, perm], v[:, :, perm])
        outs.append(orc.attention(q, [s], kc, kc, jensen=1)[0])
    np.testing.assert_allclose(outs[0], outs[1], atol=1e-14, rtol=0)


def test_lse_merge_of_history_halves(orc):
    """Attention over A and over (B + current) merged by log-sum-exp equals attention
    over A + B + current: pins multi-segment handling and the returned lse."""
    rng = np.random.default_rng(11)
    d = 64
    segs = []
    for n in (100, 60):
        s = orc.new_segment(2, "bf16", 1, 2, d, capacity=n, k_group_tokens=32, kgroup_capacity=4)
        orc.append(s, rng.standard_normal((1, 2, n, d)).astype(np.float32) * 2,
                   rng.standard_normal((1, 2, n, d)).astype(np.float32))
        segs.append(s)
    q = rng.standard_normal((1, 4, 5, d)).astype(np.float32)
    kc = rng.standard_normal((1, 2, 9, d)).astype(np.float32)
    vc = rng.standard_normal((1, 2, 9, d)).astype(np.float32)
    oa, la = orc.attention(q, segs[:1], None, None, n_kv_heads=2, jensen=1)
    ob, lb = orc.attention(q, segs[1:], kc, vc, jensen=1)
    o, l = orc.attention(q, segs, kc, vc, jensen=1)
    m = np.maximum(la, lb)
    wa, wb = np.exp(la - m), np.exp(lb - m)
    merged = (wa[..., None] * oa + wb[..., None] * ob) / (wa + wb)[..., None]
    np.testing.assert_allclose(merged, o, atol=1e-13)
    np.testing.assert_allclose(m + np.log(wa + wb), l, atol=1e-13)


def test_zero_steps_make_jensen_a_noop(orc):
    rng = np.random.default_rng(12)
    d, n = 64, 64
    # each channel constant over each 32-token group -> every K step is 0
    base = rng.standard_normal((1, 1, 2, d)).astype(np.float32)
    k = np.repeat(base, 32, axis=2)
    v = rng.standard_normal((1, 1, n, d)).astype(np.float32)
    s = orc.new_segment(4, "bf16", 1, 1, d, capacity=n, k_group_tokens=32, kgroup_capacity=2)
    orc.append(s, k, v)
    q = rng.standard_normal((1, 1, 3, d)).astype(np.float32)
    kc = rng.standard_normal((1, 1, 5, d)).astype(np.float32)
    a, _ = orc.attention(q, [s], kc, kc, jensen=0)
    b, _ = orc.attention(q, [s], kc, kc, jensen=1)
    assert np.array_equal(a, b)
