"""C ABI checks that need no GPU: libkvq.so loads, exports every function include/kvq.h
declares, and its host-side validation rejects bad arguments with the documented status
codes before anything is enqueued (no HIP call is reached on these paths)."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import bit_kv_cache_pack_amd as kvq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvq.h")


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:kvq_status|const char \*|int32_t)\s*(kvq_\w+)\s*\(", text, re.M)))


def test_header_declares_the_entry_points():
    assert _declared() == sorted(kvq.SYMBOLS)


def test_library_exports_every_declared_symbol():
    L = kvq.lib()
    for name in _declared():
        assert hasattr(L, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", kvq.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (kvq_\w+)", out))
    assert set(_declared()) <= exported
    assert L.kvq_abi_version() == 3


def test_header_compiles_as_c():
    src = '#include "kvq.h"\nint main(void){kvq_segment s; (void)s; return (int)sizeof(kvq_attn_args) > 0 ? 0 : 1;}\n'
    r = subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"), "-x", "c",
                        "-", "-o", "/dev/null"], input=src, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def test_struct_layouts_match_binding():
    """ctypes mirrors of the ABI structs have the C sizes (checked with the C compiler)."""
    src = ('#include <stdio.h>\n#include "kvq.h"\nint main(void){printf("%zu %zu %zu %zu",'
           'sizeof(kvq_segment),sizeof(kvq_append_args),sizeof(kvq_window_args),sizeof(kvq_attn_args));return 0;}\n')
    exe = "/tmp/kvq_sizes_%d" % os.getpid()
    r = subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), "-x", "c", "-", "-o", exe], input=src,
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    sizes = [int(x) for x in subprocess.run([exe], capture_output=True, text=True).stdout.split()]
    os.unlink(exe)
    assert sizes == [ctypes.sizeof(kvq.KvqSegment), ctypes.sizeof(kvq.KvqAppendArgs),
                     ctypes.sizeof(kvq.KvqWindowArgs), ctypes.sizeof(kvq.KvqAttnArgs)]


def test_status_strings():
    for code in (kvq.OK, kvq.ERR_ARG, kvq.ERR_UNSUPPORTED, kvq.ERR_CAPACITY, kvq.ERR_WORKSPACE, kvq.ERR_HIP):
        assert kvq.status_string(code)
    assert kvq.status_string(-99) == "unknown status"


FAKE = 0x100000  # a 16-byte aligned address that is never dereferenced on these paths


def _seg(**kw):
    d = dict(bits=2, elem_dtype=kvq.BF16, batch=1, n_kv_heads=2, head_dim=128, capacity=1000, n_tokens=0,
             k_group_tokens=128, v_group_channels=32, kgroup_capacity=16, n_kgroups=0,
             k=FAKE, v=FAKE, k_meta=FAKE, v_meta=FAKE, kgroup_start=FAKE)
    d.update(kw)
    return kvq.KvqSegment(**d)


def _append(seg, **kw):
    d = dict(dst=ctypes.pointer(seg), k_src=FAKE, v_src=FAKE, src_dtype=kvq.BF16, src_tokens=500, n_new=500,
             src_groups=None, n_src_groups=0)
    d.update(kw)
    a = kvq.KvqAppendArgs(**d)
    return kvq.lib().kvq_quantize_append(ctypes.byref(a), None)


@pytest.mark.parametrize("kw,status", [
    (dict(bits=3), kvq.ERR_UNSUPPORTED),
    (dict(head_dim=96), kvq.ERR_UNSUPPORTED),
    (dict(elem_dtype=kvq.F32), kvq.ERR_UNSUPPORTED),
    (dict(v_group_channels=16), kvq.ERR_UNSUPPORTED),
    (dict(k_group_tokens=0), kvq.ERR_UNSUPPORTED),
    (dict(n_tokens=900), kvq.ERR_CAPACITY),          # 900 + 500 > 1000
    (dict(n_kgroups=13), kvq.ERR_CAPACITY),          # 13 + 4 > 16
    (dict(k=None), kvq.ERR_ARG),
    (dict(k_meta=FAKE + 4), kvq.ERR_ARG),            # misaligned
    (dict(n_tokens=-1), kvq.ERR_ARG),
])
def test_append_validation(kw, status):
    seg = _seg(**kw)
    before = (seg.n_tokens, seg.n_kgroups)
    assert _append(seg) == status
    assert (seg.n_tokens, seg.n_kgroups) == before


def test_append_validation_args():
    assert _append(_seg(), n_new=-1) == kvq.ERR_ARG
    assert _append(_seg(), src_tokens=499) == kvq.ERR_ARG
    assert _append(_seg(), src_dtype=7) == kvq.ERR_UNSUPPORTED
    assert _append(_seg(), k_src=None) == kvq.ERR_ARG
    assert _append(_seg(), src_groups=FAKE, n_src_groups=0) == kvq.ERR_ARG
    assert _append(_seg(), src_groups=FAKE, n_src_groups=3) == kvq.ERR_ARG   # 3 x 128 < 500 tokens
    seg = _seg()
    assert _append(seg, n_new=0) == kvq.OK and seg.n_tokens == 0            # no-op, nothing launched
    assert kvq.lib().kvq_quantize_append(None, None) == kvq.ERR_ARG


def _attn(segs=None, **kw):
    segs = [_seg(n_tokens=300, n_kgroups=3)] if segs is None else segs
    arr = (kvq.KvqSegment * max(1, len(segs)))(*segs)
    d = dict(q=FAKE, dtype=kvq.BF16, batch=1, n_q_heads=4, n_kv_heads=2, head_dim=128, n_q=10, segs=arr,
             n_segs=len(segs), k_cur=FAKE, v_cur=FAKE, n_cur=10, softmax_scale=0.0, jensen=1, out=FAKE,
             out_dtype=kvq.F32, lse=None, workspace=None, workspace_bytes=0)
    d.update(kw)
    return kvq.KvqAttnArgs(**d), arr


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=kvq.F32), kvq.ERR_UNSUPPORTED),
    (dict(head_dim=256), kvq.ERR_UNSUPPORTED),
    (dict(n_q_heads=3), kvq.ERR_ARG),
    (dict(n_segs=9), kvq.ERR_UNSUPPORTED),
    (dict(jensen=5), kvq.ERR_UNSUPPORTED),
    (dict(jensen=4), kvq.ERR_UNSUPPORTED),
    (dict(jensen=-1), kvq.ERR_UNSUPPORTED),
    (dict(out_dtype=9), kvq.ERR_UNSUPPORTED),
    (dict(q=None), kvq.ERR_ARG),
    (dict(out=None), kvq.ERR_ARG),
    (dict(k_cur=None), kvq.ERR_ARG),
    (dict(softmax_scale=-1.0), kvq.ERR_ARG),
    (dict(n_q=0), kvq.ERR_ARG),
])
def test_attention_validation(kw, status):
    a, arr = _attn(**kw)
    assert kvq.lib().kvq_chunk_attention(ctypes.byref(a), None) == status


def test_attention_segment_checks():
    a, arr = _attn(segs=[_seg(n_tokens=300, n_kgroups=3, elem_dtype=kvq.F16)])
    assert kvq.lib().kvq_chunk_attention(ctypes.byref(a), None) == kvq.ERR_UNSUPPORTED
    a, arr = _attn(segs=[_seg(n_tokens=300, n_kgroups=3, n_kv_heads=4)])
    assert kvq.lib().kvq_chunk_attention(ctypes.byref(a), None) == kvq.ERR_ARG
    a, arr = _attn(segs=[], n_cur=0)               # no tokens at all
    assert kvq.lib().kvq_chunk_attention(ctypes.byref(a), None) == kvq.ERR_ARG
    # per-token K columns: the all-orders form is refused, and so are two segments whose
    # extra columns differ in kind; the same segments pass the checks with the default form
    tok = _seg(n_tokens=300, n_kgroups=3, k_group_channels=32)
    a, arr = _attn(segs=[tok], jensen=3)
    assert kvq.lib().kvq_chunk_attention(ctypes.byref(a), None) == kvq.ERR_UNSUPPORTED
    n = ctypes.c_size_t()
    a, arr = _attn(segs=[tok], jensen=1)
    assert kvq.lib().kvq_attention_workspace_size(ctypes.byref(a), ctypes.byref(n)) == kvq.OK
    a, arr = _attn(segs=[tok, _seg(n_tokens=300, n_kgroups=3, k_group_channels=64)], jensen=1)
    assert kvq.lib().kvq_chunk_attention(ctypes.byref(a), None) == kvq.ERR_UNSUPPORTED


def test_workspace_size_and_check():
    # decode shape over a long history: one query per head -> several workgroups per KV head
    # whose partials need a workspace
    a, arr = _attn(segs=[_seg(capacity=20000, n_tokens=20000, n_kgroups=157, kgroup_capacity=157)], n_q=1,
                   n_cur=0, k_cur=None, v_cur=None)
    n = ctypes.c_size_t()
    assert kvq.lib().kvq_attention_workspace_size(ctypes.byref(a), ctypes.byref(n)) == kvq.OK
    assert n.value > 0 and n.value % (4 * 130) == 0
    assert kvq.lib().kvq_chunk_attention(ctypes.byref(a), None) == kvq.ERR_WORKSPACE
    a.workspace, a.workspace_bytes = FAKE, n.value - 1
    assert kvq.lib().kvq_chunk_attention(ctypes.byref(a), None) == kvq.ERR_WORKSPACE
    assert kvq.lib().kvq_attention_workspace_size(ctypes.byref(a), None) == kvq.ERR_ARG
    # a short decode history fits one workgroup per KV head: no workspace
    a, arr = _attn(segs=[_seg(n_tokens=1000, n_kgroups=8)], n_q=1, n_cur=0, k_cur=None, v_cur=None)
    assert kvq.lib().kvq_attention_workspace_size(ctypes.byref(a), ctypes.byref(n)) == kvq.OK and n.value == 0
    # 512 row blocks of 256 queries fill two rounds of 256 workgroups (the CU count the
    # plan assumes without a device): one workgroup per row block, no workspace
    a, arr = _attn(n_q=8192, n_q_heads=16, n_kv_heads=16, segs=[_seg(n_kv_heads=16, n_tokens=900, n_kgroups=8)])
    assert kvq.lib().kvq_attention_workspace_size(ctypes.byref(a), ctypes.byref(n)) == kvq.OK and n.value == 0
    # 384 row blocks would leave half of the second round idle: every workgroup takes an
    # equal share and keeps two partial slots of 256 rows x (d + 4) floats
    a, arr = _attn(n_q=8192, n_q_heads=12, n_kv_heads=12, segs=[_seg(n_kv_heads=12, n_tokens=900, n_kgroups=8)])
    assert kvq.lib().kvq_attention_workspace_size(ctypes.byref(a), ctypes.byref(n)) == kvq.OK
    assert n.value > 0 and n.value % (2 * 256 * (2 * 128 + 16)) == 0 and n.value // (2 * 256 * (2 * 128 + 16)) <= 256


def test_window_validation():
    def call(**kw):
        d = dict(k=FAKE, k_dtype=kvq.F16, n_layers=1, n_kv_heads=2, head_dim=64, n_tokens=19600, window=32,
                 text_query=FAKE, pct_fp16=10, pct_int4=30, bits_out=FAKE, order_out=FAKE, score_out=FAKE,
                 groups_out=None, class_tokens_out=None)
        d.update(kw)
        a = kvq.KvqWindowArgs(**d)
        return kvq.lib().kvq_assign_windows(ctypes.byref(a), None)
    assert call(pct_fp16=70, pct_int4=40) == kvq.ERR_ARG   # shares above 100 %
    assert call(pct_int4=-1) == kvq.ERR_ARG
    assert call(score_out=None) == kvq.ERR_ARG
    assert call(bits_out=None) == kvq.ERR_ARG
    assert call(k_dtype=9) == kvq.ERR_UNSUPPORTED
    assert call(head_dim=257) == kvq.ERR_UNSUPPORTED       # the header's limits: head_dim 1..256,
    assert call(head_dim=0) == kvq.ERR_UNSUPPORTED
    assert call(n_tokens=16384 * 32 + 1) == kvq.ERR_UNSUPPORTED   # at most 16384 windows per layer,
    assert call(n_layers=65536) == kvq.ERR_UNSUPPORTED             # at most 65535 layers
    assert call(n_layers=0) == kvq.ERR_ARG
    assert call(window=0) == kvq.ERR_ARG
    assert call(n_tokens=0) == kvq.ERR_ARG
    assert kvq.lib().kvq_assign_windows(None, None) == kvq.ERR_ARG


def test_window_budget_rule():
    """kvq_window_budget: floor of the shares over all windows, window 0 inside the FP16
    share, at least one FP16 window; the 100-frame workload's 613 windows give 61 / 184 / 368."""
    assert kvq.window_budget(613, 10, 30) == (61, 184)
    assert kvq.window_budget(5, 10, 30) == (1, 2)          # floor 0 FP16 raised to window 0
    assert kvq.window_budget(1, 0, 0) == (1, 0)
    assert kvq.window_budget(10, 0, 100) == (1, 9)         # INT4 capped to what is left
    assert kvq.window_budget(100, 100, 0) == (100, 0)
    for bad in ((0, 10, 30), (10, 101, 0), (10, -1, 0), (10, 60, 50)):
        with pytest.raises(kvq.KvqError):
            kvq.window_budget(*bad)
    n = ctypes.c_int32()
    assert kvq.lib().kvq_window_budget(10, 10, 30, None, ctypes.byref(n)) == kvq.ERR_ARG


def test_binding_attention_without_segments_takes_heads_from_current_chunk():
    """No segments: the KV head count comes from the current chunk; with neither, the
    binding asks for it instead of failing inside."""
    import torch
    q = torch.zeros((1, 4, 33, 64), dtype=torch.float16)
    kc = torch.zeros((1, 4, 77, 64), dtype=torch.float16)
    a, arr = kvq._attn_args(q, [], kc, kc, None, 0.0, 1, None, kvq.F32, None, None)
    assert a.n_kv_heads == 4 and a.n_cur == 77
    assert kvq.attention_workspace_size(q, [], n_cur=77, n_kv_heads=4) >= 0
    with pytest.raises(ValueError):
        kvq.attention_workspace_size(q, [], n_cur=77)


def test_probe_validation():
    sink = FAKE
    L = kvq.lib()
    assert L.kvq_probe_hbm_read(None, 1 << 20, sink, None) == kvq.ERR_ARG
    assert L.kvq_probe_hbm_read(FAKE, 0, sink, None) == kvq.ERR_ARG
    assert L.kvq_probe_hbm_read(FAKE, 1000, sink, None) == kvq.ERR_ARG       # not a multiple of 16
    assert L.kvq_probe_hbm_read(FAKE + 8, 1 << 20, sink, None) == kvq.ERR_ARG  # misaligned
    assert L.kvq_probe_hbm_read(FAKE, 1 << 20, None, None) == kvq.ERR_ARG


def test_fused_append_validation():
    """append_dst is checked like kvq_quantize_append before anything is enqueued; on error
    neither descriptor changes."""
    dst = _seg(capacity=1000, n_tokens=995, n_kgroups=8)            # 995 + 10 current > 1000
    a, arr = _attn(append_dst=ctypes.pointer(dst))
    assert kvq.lib().kvq_chunk_attention(ctypes.byref(a), None) == kvq.ERR_CAPACITY
    assert (dst.n_tokens, dst.n_kgroups) == (995, 8)
    dst = _seg(n_tokens=100, n_kgroups=16, kgroup_capacity=16)       # no room for a new K-group
    a, arr = _attn(append_dst=ctypes.pointer(dst))
    assert kvq.lib().kvq_chunk_attention(ctypes.byref(a), None) == kvq.ERR_CAPACITY
    dst = _seg(n_kv_heads=4)                                         # not the attention's heads
    a, arr = _attn(append_dst=ctypes.pointer(dst))
    assert kvq.lib().kvq_chunk_attention(ctypes.byref(a), None) == kvq.ERR_ARG
    dst = _seg(k_meta=None)
    a, arr = _attn(append_dst=ctypes.pointer(dst))
    assert kvq.lib().kvq_chunk_attention(ctypes.byref(a), None) == kvq.ERR_ARG
    assert (dst.n_tokens, dst.n_kgroups) == (0, 0)
