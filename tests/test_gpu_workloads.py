"""GPU parity at the full sizes of the benchmarked workloads, in the launch configuration
that bench.py times (its ``ChunkStep``: one cache built by the same appends, the same
attention call with the same workspace, then the quantize-append of the current chunk).

The oracle recomputes every packed code, step/zero and group table of the cache in full
(bit-exact), and the attention on sampled query rows of every head (all rows where a
workload has few). Bars as in test_gpu_parity: codes/meta/windows bit-exact, attention
2e-3 max-abs against the oracle in fp64 with dequantized values rounded to the element
dtype.
"""
import numpy as np
import pytest
import torch

import bit_kv_cache_pack_amd as kvq
import oracle
import workloads
from bench import ChunkStep
from parity_util import append_both, assert_segments_equal, f32, gpu_attention, make_pair, oracle_attention

pytestmark = pytest.mark.gpu
TOL = 2e-3


def _oracle_cache(w, data):
    n_groups = w.n_appends * -(-w.append_tokens // w.k_group_tokens)
    extra = -(-w.n_cur // w.k_group_tokens) if w.n_cur else 0
    oseg = oracle.new_segment(w.bits, w.dtype, w.batch, w.n_kv_heads, w.head_dim, capacity=w.n_cache + w.n_cur,
                              k_group_tokens=w.k_group_tokens, kgroup_capacity=n_groups + extra)
    ck, cv = f32(data["cache_k"]), f32(data["cache_v"])
    for a in range(w.n_appends):
        sl = slice(a * w.append_tokens, (a + 1) * w.append_tokens)
        oracle.append(oseg, ck[:, :, sl], cv[:, :, sl])
    return oseg


def _rows(n_q, stride):
    rows = list(range(0, n_q, stride))
    if rows[-1] != n_q - 1:
        rows.append(n_q - 1)
    return rows


def _check_step(name, stride):
    w = workloads.WORKLOADS[name]
    step = ChunkStep(w, n_copies=1)
    data = step.data
    oseg = _oracle_cache(w, data)
    gseg = step.segs[0]
    print("%s: cache %d tokens, %d K-groups per head" % (name, gseg.n_tokens, gseg.n_kgroups), flush=True)
    assert_segments_equal(gseg, oseg)

    step.run()
    torch.cuda.synchronize()
    got = step.out.cpu().numpy()
    rows = _rows(w.n_q, stride)
    kc = data["cur_k"] if w.n_cur else None
    vc = data["cur_v"] if w.n_cur else None
    ref, _ = oracle_attention(data["q"], [oseg], kc, vc, n_kv_heads=w.n_kv_heads, jensen=w.jensen, rows=rows)
    err = np.abs(got[:, :, rows] - ref)
    print("%s: %d rows x %d heads, max |err| %.3g" % (name, len(rows), w.n_q_heads, err.max()), flush=True)
    assert err.max() <= TOL, (name, float(err.max()), np.unravel_index(err.argmax(), err.shape))

    if w.n_cur:  # the step's quantize-append of the current chunk
        oracle.append(oseg, f32(data["cur_k"]), f32(data["cur_v"]))
        assert_segments_equal(gseg, oseg)


def test_video_chunk_int2_h12_d128():
    """Video chunk step: 18,720 cached INT2 tokens + 4,680 current, 4,680 queries x 12 heads."""
    _check_step("video_chunk_int2_h12_d128", stride=37)


@pytest.mark.parametrize("bits", [2, 4])
def test_decode_gqa32x8_32k(bits):
    """Decode, GQA 32/8, 8 sequences x 32,768 cached tokens: every query row."""
    _check_step("decode_gqa32x8_int%d_32k" % bits, stride=1)


@pytest.mark.timeout(600)
def test_rollout_chunk_int2_h40_d128():
    """Long rollout: 74,880 cached INT2 tokens + 4,680 current, 40 heads; sampled rows."""
    _check_step("rollout_chunk_int2_h40_d128", stride=390)


@pytest.mark.parametrize("jensen", [0, 1])
def test_windowquant_fp16_gqa14x2_d64(jensen):
    """WindowQuant end to end: window scores and FP16/INT4/INT2 assignment (bit-exact), the
    three grouped segments built by gathered appends (bit-exact), then one decode query of
    14 heads over the mixed-precision cache."""
    w = workloads.WORKLOADS["windowquant_fp16_gqa14x2_d64"]
    data = workloads.generate(w)
    k, v = data["cache_k"], data["cache_v"]                 # [1][2][19600][64] fp16
    N, W = w.n_cache, w.n_windows
    n16, n4 = kvq.window_budget(W, w.pct_fp16, w.pct_int4)
    assert (n16, n4, W - n16 - n4) == (61, 184, 368)
    bits, order, score = kvq.assign_windows(k[0].cuda(), data["text"].cuda(), n16, n4)
    torch.cuda.synchronize()
    osc = oracle.window_scores(f32(k[0]), data["text"].numpy(), w.window)
    ob, oo = oracle.assign_windows(osc, n16, n4)
    np.testing.assert_array_max_ulp(score.cpu().numpy(), osc, maxulp=4)
    bits_h, order_h = bits.cpu().numpy(), order.cpu().numpy()
    assert np.array_equal(bits_h, ob) and np.array_equal(order_h, oo)

    classes = kvq.window_groups(order_h.tolist(), bits_h.tolist(), N, w.window)
    gsegs, osegs = [], []
    for b in (16, 4, 2):
        groups, n_tok = classes[b]
        gseg, oseg = make_pair(b, "f16", 1, w.n_kv_heads, w.head_dim, capacity=n_tok, Gk=w.window,
                               kgroup_capacity=len(groups))
        append_both(gseg, oseg, k, v, groups=groups)
        assert_segments_equal(gseg, oseg)
        gsegs.append(gseg)
        osegs.append(oseg)
    go, gl = gpu_attention(data["q"], gsegs, n_kv_heads=w.n_kv_heads, jensen=jensen)
    oo_, ol = oracle_attention(data["q"], osegs, n_kv_heads=w.n_kv_heads, jensen=jensen)
    assert np.abs(go - oo_).max() <= TOL
    assert np.abs(gl - ol).max() <= TOL
