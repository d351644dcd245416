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
@pytest.mark.parametrize("jensen", [0, 1, 2])
def test_attention_chunk_small(bits, jensen):
    go, gl, oo, ol = _attention_case(bits, "bf16", 1, 2, 2, 128, appends=(200, 200), n_cur=100, n_q=150,
                                     jensen=jensen, seed=7)
    err = np.abs(go - oo).max()
    assert err <= TOL, err
    assert np.abs(gl - ol).max() <= TOL


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("jensen", [1, 2])
def test_attention_gqa_decode_splits(d, jensen):
    """GQA decode: one query per head, rows packed per KV head, token splits + combine."""
    go, gl, oo, ol = _attention_case(2, "bf16", 2, 8, 2, d, appends=(1500, 700), n_cur=0, n_q=1, jensen=jensen,
                                     seed=11)
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


@pytest.mark.parametrize("jensen", [0, 1, 2])
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
    rng = np.random.default_rng(3)
    H, N, d = 2, 1000, 64
    k = torch.from_numpy(rng.standard_normal((H, N, d)).astype(np.float32)).half()
    t = torch.from_numpy(rng.standard_normal(d).astype(np.float32))
    W = -(-N // 32)
    n16, n4 = kvq.window_budget(W, 10, 30)
    bits, order, score = kvq.assign_windows(k.cuda(), t.cuda(), n16, n4)
    torch.cuda.synchronize()
    osc = oracle.window_scores(f32(k), t.numpy(), 32)
    ob, oo = oracle.assign_windows(osc, n16, n4)
    np.testing.assert_array_max_ulp(score.cpu().numpy(), osc, maxulp=4)
    assert np.array_equal(bits.cpu().numpy(), ob)
    assert np.array_equal(order.cpu().numpy(), oo)
