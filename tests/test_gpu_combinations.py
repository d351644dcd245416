"""GPU parity of feature combinations, against the CPU oracle: the all-orders Jensen form
with the fused append and through the no-alloc entry point; per-token K groups and the
low-rank compensation over several sequences, with the fused append; the no-alloc entry
point over per-token K groups. Same bars as test_gpu_parity.py: appended segments
bit-exact, attention within 2e-3 (fp32 output), log-sum-exp within 2e-3.
"""
import numpy as np
import pytest
import torch

import bit_kv_cache_pack_amd as kvq
import oracle
from parity_util import TORCH_DT, append_both, assert_segments_equal, f32, make_pair, oracle_attention

pytestmark = pytest.mark.gpu
TOL = 2e-3


def _rand(shape, dtype, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=g) * scale).to(TORCH_DT[dtype])


def _basis(seed, H, d, r):
    rng = np.random.default_rng(seed)
    U = np.zeros((H, d, r), np.float32)
    for h in range(H):
        U[h] = np.linalg.qr(rng.standard_normal((d, r)))[0].astype(np.float32)
    return U


def _fused_step(gseg, oseg, q, kc, vc, Hkv, jensen):
    """Attention with append_dst against the oracle on the cache as it was, then the
    appended segment against the oracle's append."""
    oo, ol = oracle_attention(q, [oseg], kc, vc, n_kv_heads=Hkv, jensen=jensen)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
    n0 = gseg.n_tokens
    out = kvq.chunk_attention(q.cuda(), [gseg], kc.cuda(), vc.cuda(), n_kv_heads=Hkv, jensen=jensen, lse=lse,
                              append_to=gseg)
    torch.cuda.synchronize()
    assert gseg.n_tokens == n0 + kc.shape[2]
    assert np.abs(out.cpu().numpy() - oo).max() <= TOL
    assert np.abs(lse.cpu().numpy() - ol).max() <= TOL
    oracle.append(oseg, f32(kc), f32(vc))
    assert_segments_equal(gseg, oseg)


@pytest.mark.parametrize("case", ["shares", "whole_row_blocks"])
def test_exact_jensen_with_fused_append(case):
    """KVQ_JENSEN_EXACT in the chunk kernel's EXACT instance, with the append workgroups in
    the same launch (equal shares, or whole row blocks with idle CUs)."""
    B, Hq, Hkv, d, n_q, n_cache, n_cur = {
        "shares": (1, 2, 2, 128, 3000, 900, 500),
        "whole_row_blocks": (1, 10, 10, 128, 6400, 700, 300),
    }[case]
    Gk = 128
    gseg, oseg = make_pair(2, "bf16", B, Hkv, d, capacity=n_cache + n_cur, Gk=Gk,
                           kgroup_capacity=-(-n_cache // Gk) + -(-n_cur // Gk))
    append_both(gseg, oseg, _rand((B, Hkv, n_cache, d), "bf16", 201, 2.0), _rand((B, Hkv, n_cache, d), "bf16", 202))
    _fused_step(gseg, oseg, _rand((B, Hq, n_q, d), "bf16", 203), _rand((B, Hkv, n_cur, d), "bf16", 204, 2.0),
                _rand((B, Hkv, n_cur, d), "bf16", 205), Hkv, jensen=3)


@pytest.mark.parametrize("kgc,jensen", [(32, 1), (128, 2), (64, 0)])
def test_token_groups_two_sequences_fused_append(kgc, jensen):
    """Per-token K groups, batch 2 with GQA 3: the attention, then the current chunk
    appended after it in the same call (the quantize-append kernel)."""
    B, Hq, Hkv, d, n_q, n_cache, n_cur = 2, 6, 2, 128, 170, 600, 140
    gseg, oseg = make_pair(4 if kgc == 128 else 2, "bf16", B, Hkv, d, capacity=n_cache + n_cur, Gk=128,
                           kgroup_capacity=1, k_group_channels=kgc)
    append_both(gseg, oseg, _rand((B, Hkv, n_cache, d), "bf16", 211, 2.0), _rand((B, Hkv, n_cache, d), "bf16", 212))
    _fused_step(gseg, oseg, _rand((B, Hq, n_q, d), "bf16", 213), _rand((B, Hkv, n_cur, d), "bf16", 214, 2.0),
                _rand((B, Hkv, n_cur, d), "bf16", 215), Hkv, jensen=jensen)


@pytest.mark.parametrize("jensen", [1, 2])
def test_compensation_two_sequences_fused_append(jensen):
    """The low-rank compensation (rank 5), batch 2 with GQA 2, fp16 elements at head_dim
    64, with the fused append."""
    B, Hq, Hkv, d, n_q, n_cache, n_cur, r = 2, 4, 2, 64, 210, 500, 96, 5
    U = _basis(221, Hkv, d, r)
    gseg, oseg = make_pair(2, "f16", B, Hkv, d, capacity=n_cache + n_cur, Gk=32,
                           kgroup_capacity=-(-n_cache // 32) + -(-n_cur // 32), comp_basis=U)
    append_both(gseg, oseg, _rand((B, Hkv, n_cache, d), "f16", 222, 2.0), _rand((B, Hkv, n_cache, d), "f16", 223))
    _fused_step(gseg, oseg, _rand((B, Hq, n_q, d), "f16", 224), _rand((B, Hkv, n_cur, d), "f16", 225, 2.0),
                _rand((B, Hkv, n_cur, d), "f16", 226), Hkv, jensen=jensen)


@pytest.mark.parametrize("case", ["exact_shares", "token_groups"])
def test_noalloc_matches_oracle(case):
    """kvq_chunk_attention_noalloc (the library's static scratch) with the all-orders form
    over equal shares, and over per-token K groups, against the oracle and bit for bit
    against kvq_chunk_attention."""
    B, Hq, Hkv, d, n_q, n_cache, n_cur = 1, 2, 2, 128, 3000, 800, 200
    kgc = 32 if case == "token_groups" else 0
    jensen = 3 if case == "exact_shares" else 1
    gseg, oseg = make_pair(2, "bf16", B, Hkv, d, capacity=n_cache, Gk=128, kgroup_capacity=-(-n_cache // 128),
                           k_group_channels=kgc)
    append_both(gseg, oseg, _rand((B, Hkv, n_cache, d), "bf16", 231, 2.0), _rand((B, Hkv, n_cache, d), "bf16", 232))
    q = _rand((B, Hq, n_q, d), "bf16", 233)
    kc = _rand((B, Hkv, n_cur, d), "bf16", 234, 2.0)
    vc = _rand((B, Hkv, n_cur, d), "bf16", 235)
    oo, ol = oracle_attention(q, [oseg], kc, vc, n_kv_heads=Hkv, jensen=jensen)
    qd, kd, vd = q.cuda(), kc.cuda(), vc.cuda()
    ref = kvq.chunk_attention(qd, [gseg], kd, vd, n_kv_heads=Hkv, jensen=jensen)
    out = torch.full(q.shape, float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
    kvq.chunk_attention_noalloc(qd, [gseg], out, kd, vd, n_kv_heads=Hkv, jensen=jensen, lse=lse)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
    assert np.abs(out.cpu().numpy() - oo).max() <= TOL
    assert np.abs(lse.cpu().numpy() - ol).max() <= TOL


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f16", 64)])
def test_exact_jensen_outlying_key_channels(dtype, d):
    """The all-orders form where some K-groups hold channels with large steps (outlier
    channels scaled up to 60x, some in every group, some in two groups only), so that the
    kernel's direct evaluation of the pairs outside its series' range runs beside the series."""
    B, Hq, Hkv, n_q, n_cache, n_cur = 1, 4, 2, 600, 1000, 100
    Gk = 128
    k = _rand((B, Hkv, n_cache, d), "bf16", 241).float()
    k[..., 5] *= 30.0
    k[:, :, 256:512, 3] *= 60.0
    k[:, 1, 640:768, d - 7] *= 45.0
    gseg, oseg = make_pair(2, dtype, B, Hkv, d, capacity=n_cache, Gk=Gk, kgroup_capacity=-(-n_cache // Gk))
    append_both(gseg, oseg, k.to(TORCH_DT[dtype]), _rand((B, Hkv, n_cache, d), dtype, 242))
    q = _rand((B, Hq, n_q, d), dtype, 243, 1.5)
    kc = _rand((B, Hkv, n_cur, d), dtype, 244)
    vc = _rand((B, Hkv, n_cur, d), dtype, 245)
    oo, ol = oracle_attention(q, [oseg], kc, vc, n_kv_heads=Hkv, jensen=3)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
    out = kvq.chunk_attention(q.cuda(), [gseg], kc.cuda(), vc.cuda(), n_kv_heads=Hkv, jensen=3, lse=lse)
    torch.cuda.synchronize()
    assert np.abs(out.cpu().numpy() - oo).max() <= TOL
    assert np.abs(lse.cpu().numpy() - ol).max() <= TOL
