"""kvq_chunk_attention_noalloc (the entry point for callers that cannot allocate) against
kvq_chunk_attention on the same inputs: two calls in a row, the second smaller, each
within the parity bar of the existing entry point's output (2e-3 max-abs; the same
kernels and plan normally give identical bits). The first call takes the chunk kernel's
equal-shares plan, whose partials fill most of the static scratch; the second a split
decode, whose partials overwrite the start of it."""
import numpy as np
import pytest
import torch

import bit_kv_cache_pack_amd as kvq
from parity_util import make_pair, append_both

pytestmark = pytest.mark.gpu
TOL = 2e-3


def _rand(shape, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=g) * scale).to(torch.bfloat16)


def _case(B, Hq, Hkv, d, n_cache, n_cur, n_q, seed):
    Gk = 128
    gseg, oseg = make_pair(2, "bf16", B, Hkv, d, capacity=n_cache, Gk=Gk, kgroup_capacity=-(-n_cache // Gk))
    append_both(gseg, oseg, _rand((B, Hkv, n_cache, d), seed, 2.0), _rand((B, Hkv, n_cache, d), seed + 1))
    q = _rand((B, Hq, n_q, d), seed + 2).cuda()
    kc = _rand((B, Hkv, n_cur, d), seed + 3, 2.0).cuda() if n_cur else None
    vc = _rand((B, Hkv, n_cur, d), seed + 4).cuda() if n_cur else None
    return gseg, q, kc, vc


@pytest.mark.parametrize("order", ["large_then_small"])
def test_noalloc_matches_chunk_attention(order):
    cases = [
        # 24 row blocks of 256 queries on a 256-CU part: equal shares, 35.7 MB of partials
        dict(B=1, Hq=2, Hkv=2, d=128, n_cache=2000, n_cur=500, n_q=3000, seed=5),
        # GQA decode, one query per head, split over several workgroups per KV head
        dict(B=2, Hq=8, Hkv=2, d=128, n_cache=2000, n_cur=0, n_q=1, seed=7),
    ]
    for c in cases:
        gseg, q, kc, vc = _case(**c)
        need = kvq.attention_workspace_size(q, [gseg], c["n_cur"], n_kv_heads=c["Hkv"])
        assert 0 < need <= kvq.NOALLOC_SCRATCH_BYTES, need
        lse_ref = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
        ref = kvq.chunk_attention(q, [gseg], kc, vc, n_kv_heads=c["Hkv"], lse=lse_ref)
        out = torch.full(q.shape, float("nan"), dtype=torch.float32, device="cuda")
        lse = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device="cuda")
        torch.cuda.synchronize()
        before = torch.cuda.memory_stats().get("allocation.all.allocated", 0)
        kvq.chunk_attention_noalloc(q, [gseg], out, kc, vc, n_kv_heads=c["Hkv"], lse=lse)
        torch.cuda.synchronize()
        assert torch.cuda.memory_stats().get("allocation.all.allocated", 0) == before
        a, b = out.cpu().numpy(), ref.cpu().numpy()
        err = float(np.abs(a - b).max())
        print("case %s: workspace %d bytes, max |noalloc - chunk_attention| = %.3g (identical: %s)"
              % (c, need, err, bool(np.array_equal(a, b))), flush=True)
        assert np.isfinite(a).all() and err <= TOL
        assert float(np.abs(lse.cpu().numpy() - lse_ref.cpu().numpy()).max()) <= TOL
