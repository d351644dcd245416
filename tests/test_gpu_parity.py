"""GPU parity: the HIP library against the CPU oracle on the same seeded inputs.

Bars: packed codes, step/zero, group tables and window assignments bit-exact;
attention outputs within 2e-3 max-abs (fp32 output; bf16 output adds its own rounding of
half a bf16 ulp); log-sum-exp within 2e-3. Cases span several tiles, ragged K-groups
and tiles, GQA packing, token splits, mixed-precision segments and the tiny workload.
"""
import numpy as np
import pytest
import torch

import bit_kv_cache_pack_amd as kvq
import oracle
import workloads
from parity_util import check_windows as _check_windows, window_case as _window_case
from parity_util import (TORCH_DT, append_both, assert_segments_equal, bf16_half_ulp, f32, gpu_attention,
                         make_pair, oracle_attention)

pytestmark = pytest.mark.gpu
TOL = 2e-3


def _rand(shape, dtype, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=g) * scale).to(TORCH_DT[dtype])


@pytest.mark.parametrize("bits", [2, 4])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("src", ["f32", "bf16", "f16"])
def test_quantize_append_bit_exact(bits, d, src):
    elem = "f16" if src == "f16" else "bf16"
    B, H, Gk = 2, 3, 128 if d == 128 else 32
    gseg, oseg = make_pair(bits, elem, B, H, d, capacity=700, Gk=Gk, kgroup_capacity=40)
    for i, n in enumerate((300, 1, 257)):                    # ragged tails, a 1-token append
        k = _rand((B, H, n, d), src, 10 * i + 1, 3.0)
        v = _rand((B, H, n, d), src, 10 * i + 2)
        append_both(gseg, oseg, k, v)
    assert_segments_equal(gseg, oseg)


@pytest.mark.parametrize("bits", [2, 4])
@pytest.mark.parametrize("d,Gk", [(128, 512), (64, 1024)])
def test_quantize_append_long_groups_bit_exact(bits, d, Gk):
    """K-groups longer than a thread's rows held in registers (more than 8 rows per thread):
    16-bit sources take the batched reload path, with ragged tails."""
    B, H = 1, 2
    gseg, oseg = make_pair(bits, "bf16", B, H, d, capacity=2 * Gk + 300, Gk=Gk, kgroup_capacity=8)
    for i, n in enumerate((Gk + 37, Gk - 5)):
        append_both(gseg, oseg, _rand((B, H, n, d), "bf16", 40 + i, 3.0), _rand((B, H, n, d), "bf16", 50 + i))
    assert_segments_equal(gseg, oseg)


@pytest.mark.parametrize("bits", [2, 4, 16])
def test_quantize_append_gather_bit_exact(bits):
    B, H, d, N = 1, 2, 64, 200
    k = _rand((B, H, N, d), "f16", 5, 2.0)
    v = _rand((B, H, N, d), "f16", 6)
    groups = [(96, 32), (192, 8), (0, 32), (64, 32)]
    gseg, oseg = make_pair(bits, "f16", B, H, d, capacity=120, Gk=32, kgroup_capacity=8)
    append_both(gseg, oseg, k, v, groups=groups)
    assert_segments_equal(gseg, oseg)


@pytest.mark.parametrize("bits", [2, 4])
@pytest.mark.parametrize("d", [64, 128])
def test_quantize_exact_ties_bit_exact(bits, d):
    """Quotients (x - zero) / step that are exact half-integers in every K and V group:
    multiples of step / 2 between 0 and L step, so the codes depend on round-half-to-even
    (the quantizer's fast reciprocal path must hand these to the division)."""
    B, H, n = 1, 2, 200
    L = (1 << bits) - 1
    t = torch.arange(n).view(n, 1)
    c = torch.arange(d).view(1, d)
    half = (t * 3 + c * 5) % (2 * L + 1)          # 0 .. 2L, both ends in every group
    x = (half.float() * 0.25).expand(B, H, n, d).contiguous()   # step 0.5: x / step = half / 2
    gseg, oseg = make_pair(bits, "bf16", B, H, d, capacity=n, Gk=128 if d == 128 else 32, kgroup_capacity=8)
    append_both(gseg, oseg, x.to(torch.bfloat16), (x * 2.0).to(torch.bfloat16))
    assert_segments_equal(gseg, oseg)


def test_quantize_constant_and_zero_groups():
    """Degenerate groups: constant channels (step 0), signed zeros."""
    B, H, d, n = 1, 1, 64, 64
    k = torch.zeros((B, H, n, d), dtype=torch.float32)
    k[..., 1::2, :] = -0.0
    k[..., 5] = 1.25
    v = torch.full((B, H, n, d), -0.0)
    v[..., 0, :32] = 3.0
    gseg, oseg = make_pair(2, "bf16", B, H, d, capacity=n, Gk=32, kgroup_capacity=2)
    append_both(gseg, oseg, k, v)
    assert_segments_equal(gseg, oseg)


def _attention_case(bits, dtype, B, Hq, Hkv, d, appends, n_cur, n_q, jensen, seed, out_dtype=torch.float32):
    Gk = 128 if d == 128 else 32
    cap = sum(appends)
    gseg, oseg = make_pair(bits, dtype, B, Hkv, d, capacity=max(cap, 1), Gk=Gk,
                           kgroup_capacity=sum(-(-n // Gk) for n in appends) + 1)
    for i, n in enumerate(appends):
        append_both(gseg, oseg, _rand((B, Hkv, n, d), dtype, seed + 10 * i, 2.0),
                    _rand((B, Hkv, n, d), dtype, seed + 10 * i + 1))
    q = _rand((B, Hq, n_q, d), dtype, seed + 100)
    kc = _rand((B, Hkv, n_cur, d), dtype, seed + 101, 2.0) if n_cur else None
    vc = _rand((B, Hkv, n_cur, d), dtype, seed + 102) if n_cur else None
    segs_g = [gseg] if cap else []
    segs_o = [oseg] if cap else []
    go, gl = gpu_attention(q, segs_g, kc, vc, n_kv_heads=Hkv, jensen=jensen, out_dtype=out_dtype)
    oo, ol = oracle_attention(q, segs_o, kc, vc, n_kv_heads=Hkv, jensen=jensen)
    return go, gl, oo, ol


@pytest.mark.parametrize("bits", [2, 4])
@pytest.mark.parametrize("jensen", [0, 1, 2, 3])
def test_attention_chunk_small(bits, jensen):
    go, gl, oo, ol = _attention_case(bits, "bf16", 1, 2, 2, 128, appends=(200, 200), n_cur=100, n_q=150,
                                     jensen=jensen, seed=7)
    err = np.abs(go - oo).max()
    assert err <= TOL, err
    assert np.abs(gl - ol).max() <= TOL


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("jensen", [0, 1, 2, 3])
def test_attention_gqa_decode_splits(d, jensen):
    """GQA decode: one query per head, rows packed per KV head, token splits + combine."""
    go, gl, oo, ol = _attention_case(2, "bf16", 2, 8, 2, d, appends=(1500, 700), n_cur=0, n_q=1, jensen=jensen,
                                     seed=11)
    assert np.abs(go - oo).max() <= TOL
    assert np.abs(gl - ol).max() <= TOL


@pytest.mark.parametrize("bits,d", [(2, 64), (2, 128), (4, 128)])
@pytest.mark.parametrize("jensen", [0, 1, 3])
def test_attention_decode_with_current_chunk(bits, d, jensen):
    """Decode-shaped (4 query rows per KV head) over one packed segment and a 40-token
    current chunk, 340 tokens in all: one workgroup walks each (batch, KV head), so the
    decode kernel's current-chunk instances take the call."""
    go, gl, oo, ol = _attention_case(bits, "bf16", 2, 8, 2, d, appends=(300,), n_cur=40, n_q=1, jensen=jensen,
                                     seed=31 + bits + d)
    assert np.abs(go - oo).max() <= TOL
    assert np.abs(gl - ol).max() <= TOL


def test_attention_shares_span_row_blocks():
    """600 row blocks (the last one ragged) over 130 tokens: more than two rounds of
    workgroups, so every workgroup takes an equal share of about 2.3 row blocks -- a cut
    first piece, whole row blocks, a cut last piece, and pieces that hold only the padding
    past the last token -- and the cut row blocks are merged afterwards."""
    go, gl, oo, ol = _attention_case(2, "bf16", 1, 4, 1, 64, appends=(100,), n_cur=30, n_q=38390, jensen=1,
                                     seed=19)
    assert np.abs(go - oo).max() <= TOL
    assert np.abs(gl - ol).max() <= TOL


def test_attention_fp16_and_only_current_chunk():
    go, gl, oo, ol = _attention_case(4, "f16", 1, 4, 4, 64, appends=(), n_cur=77, n_q=33, jensen=1, seed=13)
    assert np.abs(go - oo).max() <= TOL


def test_attention_bf16_output():
    go, gl, oo, ol = _attention_case(2, "bf16", 1, 2, 1, 128, appends=(300,), n_cur=64, n_q=70, jensen=1,
                                     seed=17, out_dtype=torch.bfloat16)
    assert np.all(np.abs(go - oo) <= TOL + bf16_half_ulp(oo))


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float16])
def test_attention_whole_row_blocks_half_outputs(out_dtype):
    """256 row blocks over a short history: on a 256-CU part each workgroup takes one whole
    row block and writes the final 2-byte output itself (no piece merge)."""
    go, gl, oo, ol = _attention_case(2, "bf16", 1, 1, 1, 64, appends=(64,), n_cur=16, n_q=256 * 256, jensen=1,
                                     seed=23, out_dtype=out_dtype)
    if out_dtype == torch.bfloat16:
        half_ulp = bf16_half_ulp(oo)
    else:
        half_ulp = np.spacing(np.abs(oo).astype(np.float16)).astype(np.float64) / 2
    assert np.all(np.abs(go - oo) <= TOL + half_ulp)
    assert np.abs(gl - ol).max() <= TOL


def test_attention_whole_row_blocks_share_order_tail():
    """250 row blocks over a short history: on a 256-CU part each workgroup takes one whole
    row block, and the XCD-aware share order maps workgroups 0..247 to shares
    (i % 8) * 31 + i / 8 and the last two to themselves. Every row of every block must come
    out once and right (a share taken twice or never shows as a wrong or zero row)."""
    go, gl, oo, ol = _attention_case(2, "bf16", 1, 1, 1, 64, appends=(64,), n_cur=16, n_q=250 * 256, jensen=1,
                                     seed=29)
    assert np.abs(go - oo).max() <= TOL
    assert np.abs(gl - ol).max() <= TOL


@pytest.mark.parametrize("jensen", [0, 1, 2, 3])
def test_tiny_workload(jensen):
    w = workloads.WORKLOADS["tiny_int2_h1_d64"]
    data = workloads.generate(w)
    gseg, oseg = make_pair(2, "bf16", 1, 1, w.head_dim, capacity=w.n_cache, Gk=w.k_group_tokens,
                           kgroup_capacity=w.n_cache // w.k_group_tokens)
    append_both(gseg, oseg, data["cache_k"], data["cache_v"])
    assert_segments_equal(gseg, oseg)
    go, gl = gpu_attention(data["q"], [gseg], data["cur_k"], data["cur_v"], jensen=jensen)
    oo, ol = oracle_attention(data["q"], [oseg], data["cur_k"], data["cur_v"], jensen=jensen)
    assert np.abs(go - oo).max() <= TOL
    assert np.abs(gl - ol).max() <= TOL


def test_windows_scores_and_assignment():
    k, t = _window_case(1, 2, 1000, 64, 3)
    asg = kvq.assign_windows(k[0].cuda(), t[0].cuda(), 10, 30)
    torch.cuda.synchronize()
    _check_windows(asg, k, t, 1000)


def test_windows_at_the_window_limit():
    """16,384 windows in one layer, the most kvq_assign_windows takes: the ranking's widest
    grid (256 workgroups, every wave counting over 4,096 windows) and the list pass over 16
    chunks, against the oracle (its O(W^2) ranking included)."""
    N = 16384 * 32 - 5
    k, t = _window_case(1, 1, N, 64, 77)
    asg = kvq.assign_windows(k.cuda(), t.cuda(), 10, 30)
    torch.cuda.synchronize()
    _check_windows(asg, k, t, N)


def test_attention_eight_segments():
    """The most segments one attention call takes (8): INT2, INT4 and raw segments of ragged
    sizes and K-group sizes, with a current chunk, chunk-shaped (several row blocks) and
    decode-shaped (one query per head), every Jensen form, against the oracle."""
    B, Hq, Hkv, d = 1, 4, 2, 128
    specs = [(2, 128, 700), (4, 64, 333), (16, 32, 95), (2, 32, 1), (4, 128, 1200), (2, 64, 257), (16, 32, 40),
             (2, 128, 129)]
    gsegs, osegs = [], []
    for i, (bits, Gk, n) in enumerate(specs):
        gseg, oseg = make_pair(bits, "bf16", B, Hkv, d, capacity=n, Gk=Gk, kgroup_capacity=-(-n // Gk))
        append_both(gseg, oseg, _rand((B, Hkv, n, d), "bf16", 400 + i, 2.0), _rand((B, Hkv, n, d), "bf16", 420 + i))
        gsegs.append(gseg)
        osegs.append(oseg)
    kc = _rand((B, Hkv, 77, d), "bf16", 440, 2.0)
    vc = _rand((B, Hkv, 77, d), "bf16", 441)
    for n_q, jensen in ((300, 1), (1, 2), (300, 3), (1, 0)):
        q = _rand((B, Hq, n_q, d), "bf16", 442 + n_q + jensen)
        go, gl = gpu_attention(q, gsegs, kc, vc, n_kv_heads=Hkv, jensen=jensen)
        oo, ol = oracle_attention(q, osegs, kc, vc, n_kv_heads=Hkv, jensen=jensen)
        assert np.abs(go - oo).max() <= TOL, (n_q, jensen)
        assert np.abs(gl - ol).max() <= TOL, (n_q, jensen)


@pytest.mark.parametrize("n_q", [1, 260])
def test_attention_with_empty_segments(n_q):
    """Empty segments in the list, as a WindowQuant budget with an empty class leaves them
    (here the INT4 one, and an empty raw one): they hold no token and change nothing."""
    B, Hq, Hkv, d = 1, 4, 2, 64
    gsegs, osegs = [], []
    for i, (bits, n) in enumerate(((16, 0), (4, 0), (2, 333), (16, 45))):
        gseg, oseg = make_pair(bits, "f16", B, Hkv, d, capacity=max(n, 32), Gk=32, kgroup_capacity=max(-(-n // 32), 1))
        if n:
            append_both(gseg, oseg, _rand((B, Hkv, n, d), "f16", 460 + i, 2.0), _rand((B, Hkv, n, d), "f16", 470 + i))
        gsegs.append(gseg)
        osegs.append(oseg)
    q = _rand((B, Hq, n_q, d), "f16", 480 + n_q)
    go, gl = gpu_attention(q, gsegs, n_kv_heads=Hkv, jensen=1)
    oo, ol = oracle_attention(q, osegs, n_kv_heads=Hkv, jensen=1)
    assert np.abs(go - oo).max() <= TOL
    assert np.abs(gl - ol).max() <= TOL


@pytest.mark.parametrize("N", [20, 32, 64, 2080, 2081, 4129])
def test_windows_rank_boundaries(N):
    """Window counts at the ranking's edges: one window (20, 32: nothing to rank), two, 65
    (one more than a workgroup ranks), 66 and 130 windows (several workgroups, ranges not
    split evenly over the four waves); bits, order, lists and counts against the oracle,
    with tied scores (repeated windows) in the larger cases."""
    k, t = _window_case(2, 2, N, 64, 31 + N % 7)
    if N > 2000:
        k[:, :, 32 * 7:32 * 8] = k[:, :, 32 * 3:32 * 4]     # windows 3 and 7 score the same
        k[:, :, 32 * 40:32 * 41] = k[:, :, 32 * 3:32 * 4]
    asg = kvq.assign_windows(k.cuda(), t.cuda(), 10, 30)
    torch.cuda.synchronize()
    _check_windows(asg, k, t, N)


@pytest.mark.parametrize("N", [6272, 6256])
def test_windows_many_layers_one_launch(N):
    """Prefill scale: 12 independent caches (layers) scored and assigned by one pair of
    launches, each layer with its own keys and text query; a short last window (6256)
    lands in whatever class its score gives it."""
    k, t = _window_case(12, 2, N, 64, 29)
    asg = kvq.assign_windows(k.cuda(), t.cuda(), 10, 30)
    torch.cuda.synchronize()
    _check_windows(asg, k, t, N)


@pytest.mark.parametrize("dtype,d,jensen", [("f16", 64, 1), ("bf16", 128, 1), ("bf16", 128, 2), ("f16", 128, 0),
                                            ("bf16", 64, 3)])
def test_windowquant_segments_many_queries(dtype, d, jensen):
    """Chunk-shaped attention over the WindowQuant layout: 300 query rows per query head
    (GQA 4/2) over FP16 + INT4 + INT2 segments built from the device gather lists, plus an
    unquantized current chunk; every row against the oracle."""
    H, Hq, N, window = 2, 4, 3000 - 7, 32
    rng = np.random.default_rng(41 + d)
    scale = np.exp(rng.normal(0, 0.5, (H, 1, d))).astype(np.float32)
    k = torch.from_numpy((rng.standard_normal((1, H, N, d)) * scale).astype(np.float32)).to(TORCH_DT[dtype])
    v = torch.from_numpy(rng.standard_normal((1, H, N, d)).astype(np.float32)).to(TORCH_DT[dtype])
    t = torch.from_numpy(rng.standard_normal(d).astype(np.float32))
    asg = kvq.assign_windows(k.cuda(), t.cuda(), 10, 30, window=window)
    torch.cuda.synchronize()
    bits, order = asg.bits[0].cpu().numpy(), asg.order[0].cpu().numpy()
    og, oct_ = oracle.window_groups(bits, order, N, window)
    assert np.array_equal(asg.groups[0].cpu().numpy(), og)
    rows = asg.class_rows()
    gsegs, osegs = [], []
    for ci, b in enumerate((16, 4, 2)):
        a, e = rows[b]
        n_tok = int(oct_[ci])
        gseg, oseg = make_pair(b, dtype, 1, H, d, capacity=n_tok, Gk=window, kgroup_capacity=e - a)
        kvq.quantize_append(gseg, k.cuda(), v.cuda(), n_new=n_tok, src_groups=asg.class_list(b))
        oracle.append(oseg, f32(k), f32(v), groups=og[a:e])
        assert_segments_equal(gseg, oseg)
        gsegs.append(gseg)
        osegs.append(oseg)
    q = _rand((1, Hq, 300, d), dtype, 91)
    kc = _rand((1, H, 150, d), dtype, 92, 2.0)
    vc = _rand((1, H, 150, d), dtype, 93)
    go, gl = gpu_attention(q, gsegs, kc, vc, n_kv_heads=H, jensen=jensen)
    oo, ol = oracle_attention(q, osegs, kc, vc, n_kv_heads=H, jensen=jensen)
    assert np.abs(go - oo).max() <= TOL
    assert np.abs(gl - ol).max() <= TOL


@pytest.mark.parametrize("case", ["whole_row_blocks", "shares", "decode_path", "raw_segment", "int4_d64"])
def test_attention_with_fused_append(case):
    """kvq_chunk_attention with append_dst: the attention reads the cache as it was before
    the call (against the oracle), and the current chunk lands in the segment bit-exactly
    as a separate kvq_quantize_append would put it (against the oracle's append)."""
    cfg = {
        # 250 row blocks of 256 queries on a 256-CU part: one round of whole row blocks, six
        # CUs left idle for the append workgroups
        "whole_row_blocks": dict(bits=2, dtype="bf16", B=1, Hq=10, Hkv=10, d=128, n_q=6400, n_cache=700, n_cur=300),
        # 24 row blocks: equal shares on every CU, the append after them
        "shares": dict(bits=2, dtype="bf16", B=1, Hq=2, Hkv=2, d=128, n_q=3000, n_cache=900, n_cur=500),
        # few rows per KV head: the decode kernel, then the quantize-append kernel
        "decode_path": dict(bits=2, dtype="bf16", B=2, Hq=8, Hkv=2, d=128, n_q=1, n_cache=400, n_cur=40),
        "raw_segment": dict(bits=16, dtype="f16", B=1, Hq=4, Hkv=2, d=64, n_q=300, n_cache=200, n_cur=77),
        "int4_d64": dict(bits=4, dtype="f16", B=1, Hq=4, Hkv=4, d=64, n_q=600, n_cache=500, n_cur=130),
    }[case]
    bits, dtype, B, Hq, Hkv, d = (cfg[k] for k in ("bits", "dtype", "B", "Hq", "Hkv", "d"))
    n_q, n_cache, n_cur = cfg["n_q"], cfg["n_cache"], cfg["n_cur"]
    Gk = 128 if d == 128 else 32
    cap = n_cache + n_cur
    kgc = -(-n_cache // Gk) + -(-n_cur // Gk)
    gseg, oseg = make_pair(bits, dtype, B, Hkv, d, capacity=cap, Gk=Gk, kgroup_capacity=kgc)
    append_both(gseg, oseg, _rand((B, Hkv, n_cache, d), dtype, 61, 2.0), _rand((B, Hkv, n_cache, d), dtype, 62))
    q = _rand((B, Hq, n_q, d), dtype, 63)
    kc = _rand((B, Hkv, n_cur, d), dtype, 64, 2.0)
    vc = _rand((B, Hkv, n_cur, d), dtype, 65)
    oo, ol = oracle_attention(q, [oseg], kc, vc, n_kv_heads=Hkv, jensen=1)   # before the append
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
    out = kvq.chunk_attention(q.cuda(), [gseg], kc.cuda(), vc.cuda(), n_kv_heads=Hkv, jensen=1, lse=lse,
                              append_to=gseg)
    torch.cuda.synchronize()
    assert gseg.n_tokens == cap
    assert np.abs(out.cpu().numpy() - oo).max() <= TOL
    assert np.abs(lse.cpu().numpy() - ol).max() <= TOL
    oracle.append(oseg, f32(kc), f32(vc))
    assert_segments_equal(gseg, oseg)


@pytest.mark.parametrize("bits,d,kgc,dtype", [(2, 128, 32, "bf16"), (4, 128, 128, "bf16"), (2, 64, 64, "f16"),
                                              (2, 128, 64, "bf16")])
@pytest.mark.parametrize("jensen", [0, 1, 2])
def test_token_groups_attention(bits, d, kgc, dtype, jensen):
    """Per-token K groups: codes and step/zero bit-exact; chunk attention (GQA, a current
    chunk, a second plain segment) with the Jensen term carried by the extra K columns."""
    B, Hq, Hkv, n1, n2, n_cur, n_q = 1, 4, 2, 700, 300, 90, 260
    Gk = 128 if d == 128 else 32
    tseg, toseg = make_pair(bits, dtype, B, Hkv, d, capacity=n1, Gk=Gk, kgroup_capacity=1, k_group_channels=kgc)
    append_both(tseg, toseg, _rand((B, Hkv, n1, d), dtype, 71, 2.0), _rand((B, Hkv, n1, d), dtype, 72))
    assert tseg.n_kgroups == 0
    assert_segments_equal(tseg, toseg)
    pseg, poseg = make_pair(bits, dtype, B, Hkv, d, capacity=n2, Gk=Gk, kgroup_capacity=-(-n2 // Gk))
    append_both(pseg, poseg, _rand((B, Hkv, n2, d), dtype, 73, 2.0), _rand((B, Hkv, n2, d), dtype, 74))
    q = _rand((B, Hq, n_q, d), dtype, 75)
    kc = _rand((B, Hkv, n_cur, d), dtype, 76, 2.0)
    vc = _rand((B, Hkv, n_cur, d), dtype, 77)
    go, gl = gpu_attention(q, [tseg, pseg], kc, vc, n_kv_heads=Hkv, jensen=jensen)
    oo, ol = oracle_attention(q, [toseg, poseg], kc, vc, n_kv_heads=Hkv, jensen=jensen)
    assert np.abs(go - oo).max() <= TOL
    assert np.abs(gl - ol).max() <= TOL


def _basis(rng, H, d, r):
    U = np.zeros((H, d, r), np.float32)
    for h in range(H):
        U[h] = np.linalg.qr(rng.standard_normal((d, r)))[0].astype(np.float32)
    return U


@pytest.mark.parametrize("bits,d,r,dtype", [(2, 128, 8, "bf16"), (4, 64, 4, "f16"), (2, 64, 3, "bf16")])
@pytest.mark.parametrize("jensen", [0, 1])
def test_compensation_attention(bits, d, r, dtype, jensen):
    """The low-rank compensation: stored c within one bf16 step of the oracle's; attention
    (queries half inside span(U), a current chunk, a fused append into the segment) against
    the oracle."""
    B, Hq, Hkv, n, n_cur, n_q = 1, 4, 2, 900, 120, 300
    Gk = 128 if d == 128 else 32
    rng = np.random.default_rng(81 + r)
    U = _basis(rng, Hkv, d, r)
    gseg, oseg = make_pair(bits, dtype, B, Hkv, d, capacity=n + n_cur, Gk=Gk,
                           kgroup_capacity=-(-n // Gk) + -(-n_cur // Gk), comp_basis=U)
    append_both(gseg, oseg, _rand((B, Hkv, n, d), dtype, 82, 2.0), _rand((B, Hkv, n, d), dtype, 83))
    assert_segments_equal(gseg, oseg)
    q = _rand((B, Hq, n_q, d), dtype, 84).float().numpy()
    # half of every query inside the subspace of its KV head
    for hq in range(Hq):
        Uh = U[hq * Hkv // Hq].astype(np.float64)
        q[0, hq] = (0.5 * q[0, hq] + 2.0 * (q[0, hq] @ Uh) @ Uh.T).astype(np.float32)
    q = torch.from_numpy(q).to(TORCH_DT[dtype])
    kc = _rand((B, Hkv, n_cur, d), dtype, 85, 2.0)
    vc = _rand((B, Hkv, n_cur, d), dtype, 86)
    oo, ol = oracle_attention(q, [oseg], kc, vc, n_kv_heads=Hkv, jensen=jensen)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
    out = kvq.chunk_attention(q.cuda(), [gseg], kc.cuda(), vc.cuda(), n_kv_heads=Hkv, jensen=jensen, lse=lse,
                              append_to=gseg)
    torch.cuda.synchronize()
    assert np.abs(out.cpu().numpy() - oo).max() <= TOL
    assert np.abs(lse.cpu().numpy() - ol).max() <= TOL
    oracle.append(oseg, f32(kc), f32(vc))
    assert_segments_equal(gseg, oseg)
