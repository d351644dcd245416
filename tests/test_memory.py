"""Memory invariants of the attention path.

The pages warn that integrations of KV-cache quantization can keep the memory win only on
paper when they rebuild or keep large BF16 buffers next to the packed cache ("KV Cache
Quantization for Self-Forcing Video Generation", abstract), and the Jensen correction is
said to need no additional memory ("Quantized Keys Steal Attention", abstract). So:

* the library allocates nothing itself: no HIP allocation call appears in its sources
  (the caller brings the workspace, or the no-alloc entry point uses a fixed static array);
* the workspace the attention asks for does not grow with the cache: it is 0 for the
  long-rollout step (whole row blocks) and at most 2 x CUs x 256 rows x (2 head_dim + 16)
  bytes otherwise (35.7 MB at head_dim 128 on 256 CUs), under a third of a BF16 copy of
  the video-chunk step's cache and below the packed cache itself from 16 chunks of
  history on;
* on the GPU, a whole chunk step (attention, then quantize-append) raises the device's
  peak allocation by exactly the output, the lse and that workspace, and leaves the
  device's free memory where it was.
"""
import os
import re

import numpy as np
import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "bit_kv_cache_pack_amd", "csrc")
BM = 256
CUS = 256   # the plan's compute-unit count when no device is present (MI355X's)


def test_library_sources_allocate_nothing():
    pat = re.compile(r"\bhip(Malloc\w*|Free\w*|HostMalloc|ExtMallocWithFlags|MemPool\w*|HostRegister)\s*\(")
    for name in sorted(os.listdir(CSRC)):
        if name.endswith((".hip", ".h", ".cuh", ".cpp")):
            text = open(os.path.join(CSRC, name)).read()
            text = re.sub(r"//[^\n]*", "", text)
            assert not pat.search(text), (name, pat.search(text).group(0))


def _packed_bytes(B, Hkv, d, n, bits, Gk=128, Gv=32):
    codes = 2 * B * Hkv * n * d * bits // 8
    kmeta = B * Hkv * (-(-n // Gk)) * d * 4
    vmeta = B * Hkv * n * (d // Gv) * 4
    return codes + kmeta + vmeta


FAKE = 0x100000   # never dereferenced: the size query reads no pointer


def _ws(B, Hq, Hkv, d, n_q, n_cache, n_cur, bits=2):
    import ctypes
    import bit_kv_cache_pack_amd as kvq
    ng = -(-n_cache // 128)
    seg = kvq.KvqSegment(bits=bits, elem_dtype=kvq.BF16, batch=B, n_kv_heads=Hkv, head_dim=d,
                         capacity=n_cache + 4096, n_tokens=n_cache, k_group_tokens=128, v_group_channels=32,
                         kgroup_capacity=ng + 64, n_kgroups=ng, k=FAKE, v=FAKE, k_meta=FAKE, v_meta=FAKE,
                         kgroup_start=FAKE)
    arr = (kvq.KvqSegment * 1)(seg)
    a = kvq.KvqAttnArgs(q=FAKE, dtype=kvq.BF16, batch=B, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=d, n_q=n_q,
                        segs=arr, n_segs=1, k_cur=FAKE if n_cur else None, v_cur=FAKE if n_cur else None,
                        n_cur=n_cur, softmax_scale=0.0, jensen=1, out=FAKE, out_dtype=kvq.BF16, lse=None,
                        workspace=None, workspace_bytes=0)
    n = ctypes.c_size_t()
    assert kvq.lib().kvq_attention_workspace_size(ctypes.byref(a), ctypes.byref(n)) == kvq.OK
    return n.value


@pytest.mark.parametrize("shape", [
    # (batch, q heads, kv heads, head_dim, queries, current chunk)
    (1, 12, 12, 128, 4680, 4680),    # video chunk step
    (1, 40, 40, 128, 4680, 4680),    # long-rollout chunk step
    (1, 2, 2, 128, 3000, 500),
    (2, 8, 2, 64, 900, 0),
    (8, 32, 8, 128, 1, 0),           # GQA decode
])
def test_workspace_bounded_independent_of_cache(shape):
    B, Hq, Hkv, d, n_q, n_cur = shape
    chunk_bound = 2 * CUS * BM * (2 * d + 16)
    decode_bound = 1023 * 16 * (d + 2) * 4
    sizes = []
    for n_cache in (4680, 18720, 74880, 299520):
        w = _ws(B, Hq, Hkv, d, n_q, n_cache, n_cur)
        sizes.append(w)
        assert w <= max(chunk_bound, decode_bound), (n_cache, w)
        if n_q * Hq // Hkv > 16:
            assert w <= chunk_bound
    assert max(sizes) <= max(chunk_bound, decode_bound)


def test_long_rollout_step_needs_no_workspace():
    # 40 heads x 19 row blocks = 760 row blocks fill 3 rounds of 256 CUs to 99 %: whole row
    # blocks, no partials
    assert _ws(1, 40, 40, 128, 4680, 74880, 4680) == 0


def test_video_chunk_workspace_is_small_against_the_cache():
    w = _ws(1, 12, 12, 128, 4680, 18720, 4680)
    assert w == 2 * CUS * BM * (2 * 128 + 16)        # every CU holds two partial pieces
    assert w < 0.5 * _packed_bytes(1, 12, 128, 16 * 4680, 2)
    bf16_cache = 2 * 12 * (18720 + 4680) * 128 * 2
    assert w < bf16_cache / 3


@pytest.mark.gpu
def test_chunk_step_peak_and_free_memory():
    import bit_kv_cache_pack_amd as kvq
    torch.manual_seed(11)
    dev = "cuda"
    B, H, d, n_cache, n_cur = 1, 12, 128, 18720, 4680
    seg = kvq.Segment(2, torch.bfloat16, B, H, d, capacity=n_cache + n_cur, device=torch.device(dev))
    for i in range(4):
        k = torch.randn(B, H, 4680, d, device=dev, dtype=torch.bfloat16)
        v = torch.randn(B, H, 4680, d, device=dev, dtype=torch.bfloat16)
        kvq.quantize_append(seg, k, v)
    q = torch.randn(B, H, n_cur, d, device=dev, dtype=torch.bfloat16)
    kc = torch.randn(B, H, n_cur, d, device=dev, dtype=torch.bfloat16)
    vc = torch.randn(B, H, n_cur, d, device=dev, dtype=torch.bfloat16)
    need = kvq.attention_workspace_size(q, [seg], n_cur, n_kv_heads=H)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert need == 2 * cus * BM * (2 * d + 16), need

    def step():
        out = kvq.chunk_attention(q, [seg], kc, vc, n_kv_heads=H, out_dtype=torch.bfloat16)
        return out

    out = step()   # loads the code objects
    torch.cuda.synchronize()
    del out
    torch.cuda.empty_cache()
    free0, _ = torch.cuda.mem_get_info()
    # bytes requested from torch's allocator (its blocks are rounded up to 2 MiB)
    base = torch.cuda.memory_stats()["requested_bytes.all.current"]
    torch.cuda.reset_peak_memory_stats()
    out = step()
    torch.cuda.synchronize()
    peak = torch.cuda.memory_stats()["requested_bytes.all.peak"] - base
    out_bytes = out.numel() * out.element_size()
    # the binding allocates the output and the workspace; the library nothing more
    assert peak == out_bytes + need, (peak, out_bytes, need)
    del out
    torch.cuda.empty_cache()
    free1, _ = torch.cuda.mem_get_info()
    assert free1 == free0, (free0, free1)
