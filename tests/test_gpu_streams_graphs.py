"""Every launch goes to the caller's stream, and the no-allocation entry point can be
captured in a HIP graph.
- The same appends and attention calls issued on a side stream (default priority) give
  bit-identical results to those issued on the current stream: no kernel of a call (the
  piece merge, the split merge, the fused append) runs anywhere else.
- kvq_chunk_attention_noalloc, captured once in a graph (it allocates nothing and issues no
  memset), is replayed several times with new query values written in between, with the
  program's own eager work and synchronizations between the replays; every replay equals an
  eager call on the same inputs, bit for bit.
"""
import pytest
import torch

import bit_kv_cache_pack_amd as kvq

pytestmark = pytest.mark.gpu


def _rand(shape, dtype, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=g) * scale).to(dtype).cuda()


def _run(Hq, nq, n, n_cur, fused):
    Hkv, d = 2, 128
    seg = kvq.Segment(2, torch.bfloat16, 1, Hkv, d, n + (n_cur if fused else 0), k_group_tokens=128,
                      kgroup_capacity=-(-n // 128) + 2)
    kvq.quantize_append(seg, _rand((1, Hkv, n, d), torch.bfloat16, 1, 2.0), _rand((1, Hkv, n, d), torch.bfloat16, 2))
    q = _rand((1, Hq, nq, d), torch.bfloat16, 3)
    kc = _rand((1, Hkv, n_cur, d), torch.bfloat16, 4, 2.0) if n_cur else None
    vc = _rand((1, Hkv, n_cur, d), torch.bfloat16, 5) if n_cur else None
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
    out = kvq.chunk_attention(q, [seg], kc, vc, n_kv_heads=Hkv, lse=lse, append_to=seg if fused else None)
    return out, lse, seg.k, seg.v, seg.k_meta, seg.v_meta


@pytest.mark.parametrize("Hq,nq,n,n_cur,fused", [(2, 3000, 700, 200, False), (8, 1, 20000, 0, False),
                                                  (2, 600, 500, 150, True)])
def test_side_stream_matches_current_stream(Hq, nq, n, n_cur, fused):
    ref = _run(Hq, nq, n, n_cur, fused)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        got = _run(Hq, nq, n, n_cur, fused)
    side.synchronize()
    for a, b in zip(ref, got):
        assert torch.equal(a, b)


@pytest.mark.parametrize("Hq,nq,n", [(2, 3000, 800), (8, 1, 20000)])
def test_noalloc_graph_replays(Hq, nq, n):
    Hkv, d = 2, 128
    seg = kvq.Segment(2, torch.bfloat16, 1, Hkv, d, n, k_group_tokens=128, kgroup_capacity=-(-n // 128))
    kvq.quantize_append(seg, _rand((1, Hkv, n, d), torch.bfloat16, 11, 2.0), _rand((1, Hkv, n, d), torch.bfloat16, 12))
    q = _rand((1, Hq, nq, d), torch.bfloat16, 13)
    out = torch.empty(q.shape, dtype=torch.float32, device="cuda")
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
    # eager first: the library's one-time set-up (device scratch address, CU count) is done
    kvq.chunk_attention_noalloc(q, [seg], out, n_kv_heads=Hkv, lse=lse)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        with torch.cuda.graph(graph, stream=cap):
            kvq.chunk_attention_noalloc(q, [seg], out, n_kv_heads=Hkv, lse=lse)
    torch.cuda.synchronize()
    for rep in range(4):
        q.copy_(_rand(q.shape, torch.bfloat16, 100 + rep))          # new inputs, eager work
        ref_out = torch.empty_like(out)
        ref_lse = torch.empty_like(lse)
        kvq.chunk_attention(q, [seg], n_kv_heads=Hkv, out=ref_out, lse=ref_lse)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out), rep
        assert torch.equal(lse, ref_lse), rep
