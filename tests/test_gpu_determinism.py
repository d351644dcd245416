"""Repeated calls give bit-identical results: the kernels accumulate in a fixed order (no
atomics, no order that depends on scheduling), through the chunk kernel's piece merge, the
decode kernel's split merge, the fused append and the window ranking."""
import pytest
import torch

import bit_kv_cache_pack_amd as kvq

pytestmark = pytest.mark.gpu


def _rand(shape, dtype, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=g) * scale).to(dtype).cuda()


@pytest.mark.parametrize("Hq,nq,n,jensen", [(2, 3000, 700, 1), (8, 1, 20000, 3), (4, 300, 2000, 2)])
def test_attention_bitwise_repeatable(Hq, nq, n, jensen):
    Hkv, d = 2, 128
    seg = kvq.Segment(2, torch.bfloat16, 1, Hkv, d, n, k_group_tokens=128, kgroup_capacity=-(-n // 128))
    kvq.quantize_append(seg, _rand((1, Hkv, n, d), torch.bfloat16, 1, 2.0), _rand((1, Hkv, n, d), torch.bfloat16, 2))
    q = _rand((1, Hq, nq, d), torch.bfloat16, 3)
    kc = _rand((1, Hkv, 40, d), torch.bfloat16, 4, 2.0) if nq > 1 else None
    vc = _rand((1, Hkv, 40, d), torch.bfloat16, 5) if nq > 1 else None
    runs = []
    for _ in range(3):
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
        out = kvq.chunk_attention(q, [seg], kc, vc, n_kv_heads=Hkv, jensen=jensen, lse=lse)
        runs.append((out.clone(), lse.clone()))
    torch.cuda.synchronize()
    for out, lse in runs[1:]:
        assert torch.equal(out, runs[0][0]) and torch.equal(lse, runs[0][1])


def test_fused_append_and_windows_bitwise_repeatable():
    Hkv, d, n, n_cur = 2, 128, 600, 150
    outs = []
    for _ in range(2):
        seg = kvq.Segment(2, torch.bfloat16, 1, Hkv, d, n + n_cur, k_group_tokens=128, kgroup_capacity=8)
        kvq.quantize_append(seg, _rand((1, Hkv, n, d), torch.bfloat16, 6, 2.0), _rand((1, Hkv, n, d), torch.bfloat16, 7))
        q = _rand((1, 4, 500, d), torch.bfloat16, 8)
        out = kvq.chunk_attention(q, [seg], _rand((1, Hkv, n_cur, d), torch.bfloat16, 9, 2.0),
                                  _rand((1, Hkv, n_cur, d), torch.bfloat16, 10), n_kv_heads=Hkv, append_to=seg)
        outs.append((out, seg.k.clone(), seg.v.clone(), seg.k_meta.clone(), seg.v_meta.clone()))
    torch.cuda.synchronize()
    for a, b in zip(outs[0], outs[1]):
        assert torch.equal(a, b)
    k = _rand((3, 2, 5000, 64), torch.float16, 11)
    t = _rand((3, 64), torch.float32, 12)
    a1 = kvq.assign_windows(k, t, 10, 30)
    a2 = kvq.assign_windows(k, t, 10, 30)
    torch.cuda.synchronize()
    for x, y in ((a1.score, a2.score), (a1.bits, a2.bits), (a1.order, a2.order), (a1.groups, a2.groups),
                 (a1.class_tokens, a2.class_tokens)):
        assert torch.equal(x, y)
