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


def _check_step(name, stride, jensen=None):
    w = workloads.WORKLOADS[name]
    if jensen is not None:
        w = workloads.scaled(w, jensen=jensen)
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


@pytest.mark.parametrize("jensen", [0, 1, 2, 3])
def test_video_chunk_int2_h12_d128(jensen):
    """Video chunk step: 18,720 cached INT2 tokens + 4,680 current, 4,680 queries x 12 heads
    (every Jensen form: off, channel-weighted, isotropic, all orders)."""
    _check_step("video_chunk_int2_h12_d128", stride=37, jensen=jensen)


@pytest.mark.parametrize("bits", [2, 4])
@pytest.mark.parametrize("jensen", [0, 1, 2, 3])
def test_decode_gqa32x8_32k(bits, jensen):
    """Decode, GQA 32/8, 8 sequences x 32,768 cached tokens: every query row, with the
    Jensen correction off and in each of its three forms."""
    _check_step("decode_gqa32x8_int%d_32k" % bits, stride=1, jensen=jensen)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("jensen", [0, 1, 2, 3])
def test_rollout_chunk_int2_h40_d128(jensen):
    """Long rollout: 74,880 cached INT2 tokens + 4,680 current, 40 heads; every 127th
    query row and the last one, so every 256-row block of every head holds at least two
    checked rows (every Jensen form)."""
    w = workloads.WORKLOADS["rollout_chunk_int2_h40_d128"]
    rows = _rows(w.n_q, 127)
    assert {r // 256 for r in rows} == set(range(-(-w.n_q // 256)))
    _check_step("rollout_chunk_int2_h40_d128", stride=127, jensen=jensen)


@pytest.mark.skip(reason="The WindowQuant decode query (fp16, head_dim 64, FP16 + INT4 + INT2 window segments) "
                         "faulted the GPU once in an uncommitted working copy of decode_kernel, cause not found. "
                         "decode_kernel now holds no code for raw segments, fp16, INT4 at head_dim 64 or several "
                         "segments; decode_eligible sends this call to attention_kernel, which "
                         "test_windowquant_fp16_gqa14x2_d64 checks against the oracle, and "
                         "tests/sanitize/decode_checker.cpp checks that routing on the CPU.")
def test_windowquant_decode_query_on_the_decode_kernel():
    pass


@pytest.mark.parametrize("jensen", [0, 1, 2, 3])
def test_windowquant_fp16_gqa14x2_d64(jensen):
    """WindowQuant end to end: window scores, FP16/INT4/INT2 assignment and the grouped
    layout's gather lists (bit-exact), the three grouped segments built by gathered appends
    from the device lists (bit-exact), then one decode query of 14 heads over the
    mixed-precision cache."""
    w = workloads.WORKLOADS["windowquant_fp16_gqa14x2_d64"]
    data = workloads.generate(w)
    k, v = data["cache_k"], data["cache_v"]                 # [1][2][19600][64] fp16
    N, W = w.n_cache, w.n_windows
    asg = kvq.assign_windows(k.cuda(), data["text"].cuda(), w.pct_fp16, w.pct_int4, window=w.window)
    assert (asg.n_fp16, asg.n_int4, W - asg.n_fp16 - asg.n_int4) == (61, 184, 368)
    torch.cuda.synchronize()
    osc = oracle.window_scores(f32(k[0]), data["text"].numpy(), w.window)
    ob, oo = oracle.assign_windows(osc, asg.n_fp16, asg.n_int4)
    og, oct_ = oracle.window_groups(ob, oo, N, w.window)
    np.testing.assert_array_max_ulp(asg.score[0].cpu().numpy(), osc, maxulp=4)
    assert np.array_equal(asg.bits[0].cpu().numpy(), ob) and np.array_equal(asg.order[0].cpu().numpy(), oo)
    assert np.array_equal(asg.groups[0].cpu().numpy(), og)
    class_tokens = asg.class_tokens[0].cpu().numpy()
    assert np.array_equal(class_tokens, oct_)

    rows = asg.class_rows()
    kd, vd = k.cuda(), v.cuda()
    gsegs, osegs = [], []
    for ci, b in enumerate((16, 4, 2)):
        a, e = rows[b]
        n_tok = int(class_tokens[ci])
        gseg, oseg = make_pair(b, "f16", 1, w.n_kv_heads, w.head_dim, capacity=n_tok, Gk=w.window,
                               kgroup_capacity=e - a)
        kvq.quantize_append(gseg, kd, vd, n_new=n_tok, src_groups=asg.class_list(b))
        oracle.append(oseg, f32(k), f32(v), groups=og[a:e])
        assert_segments_equal(gseg, oseg)
        gsegs.append(gseg)
        osegs.append(oseg)
    go, gl = gpu_attention(data["q"], gsegs, n_kv_heads=w.n_kv_heads, jensen=jensen)
    oo_, ol = oracle_attention(data["q"], osegs, n_kv_heads=w.n_kv_heads, jensen=jensen)
    assert np.abs(go - oo_).max() <= TOL
    assert np.abs(gl - ol).max() <= TOL
