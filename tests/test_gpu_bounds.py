"""No kernel writes outside what it is given. Outputs, log-sum-exp rows and workspaces are
handed over as the head of a larger buffer whose tail holds a canary pattern; after the
call the tail must be unchanged. Cache segments start zeroed: after appends, every slot
past the appended tokens (codes, V meta, compensation rows) and past the written K-groups
(K meta, the group table) must still be zero. Paths: the chunk kernel with whole row blocks
and with equal shares (piece merge), the decode kernel with splits (split merge), the
fused append, the no-allocation entry point, and contiguous, gathered, per-token-group and
compensated appends.
"""
import numpy as np
import pytest
import torch

import bit_kv_cache_pack_amd as kvq

pytestmark = pytest.mark.gpu
CANARY = 0x7FBADBAD          # a NaN payload no kernel produces
GUARD = 4096                 # guard words past every buffer


def _rand(shape, dtype, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=g) * scale).to(dtype).cuda()


def _guarded(n_words):
    """A float32 view of n_words words at the head of a canary-filled buffer, and the buffer."""
    buf = torch.full((n_words + GUARD,), CANARY, dtype=torch.int32, device="cuda")
    return buf[:n_words].view(torch.float32), buf


def _guard_intact(buf, n_words):
    tail = buf[n_words:].cpu().numpy()
    assert np.all(tail == CANARY), "%d guard words overwritten" % int((tail != CANARY).sum())


def _segment(bits, d, H, n, cap, seed, Gk=128, kgc=0, basis=None, dtype=torch.bfloat16):
    seg = kvq.Segment(bits, dtype, 1, H, d, cap, k_group_tokens=Gk, kgroup_capacity=-(-cap // Gk) + 4,
                      k_group_channels=kgc, comp_basis=basis)
    if n:
        kvq.quantize_append(seg, _rand((1, H, n, d), dtype, seed, 2.0), _rand((1, H, n, d), dtype, seed + 1))
    return seg


def _check_segment_tail(seg):
    """Every slot past the segment's tokens and K-groups is still zero."""
    torch.cuda.synchronize()
    n, G = seg.n_tokens, seg.n_kgroups
    for name in ("k", "v", "v_meta", "k_comp"):
        t = getattr(seg, name, None)
        if t is not None:
            assert not t[:, :, n:].any(), "%s written past token %d" % (name, n)
    if seg.bits != 16 and seg.k_meta is not None:
        if seg.desc.k_group_channels:
            assert not seg.k_meta[:, :, n:].any(), "per-token k_meta written past token %d" % n
        else:
            assert not seg.k_meta[:, :, G:].any(), "k_meta written past group %d" % G
            assert not seg.kgroup_start[G + 1:].any(), "group table written past entry %d" % G


def _attention_guarded(q, segs, kc, vc, Hkv, jensen=1, append_to=None):
    """chunk_attention with guarded out, lse and workspace, the guards checked afterwards;
    returns the workspace size the plan asked for."""
    B, Hq, nq, d = q.shape
    n_out, n_lse = B * Hq * nq * d, B * Hq * nq
    out, obuf = _guarded(n_out)
    lse, lbuf = _guarded(n_lse)
    need = kvq.attention_workspace_size(q, segs, 0 if kc is None else kc.shape[2], n_kv_heads=Hkv, jensen=jensen)
    nw = -(-need // 4)
    ws, wbuf = _guarded(max(nw, 1))
    kvq.chunk_attention(q, segs, kc, vc, n_kv_heads=Hkv, jensen=jensen, out=out.view(q.shape),
                        lse=lse.view(B, Hq, nq), workspace=ws.view(torch.uint8)[:need] if need else None,
                        append_to=append_to)
    torch.cuda.synchronize()
    _guard_intact(obuf, n_out)
    _guard_intact(lbuf, n_lse)
    _guard_intact(wbuf, max(nw, 1))
    assert torch.isfinite(out).all() and torch.isfinite(lse).all()
    return need


@pytest.mark.parametrize("case", ["whole_row_blocks", "equal_shares", "decode_splits", "fused_append"])
def test_attention_writes_stay_inside(case):
    d = 128
    if case == "whole_row_blocks":     # 16 heads x 16 row blocks: one round of 256 workgroups
        Hkv, Hq, nq, n, cap, n_cur = 16, 16, 4096, 300, 300, 64
    elif case == "equal_shares":
        Hkv, Hq, nq, n, cap, n_cur = 2, 2, 3000, 700, 700, 200
    elif case == "decode_splits":
        Hkv, Hq, nq, n, cap, n_cur = 2, 8, 1, 20000, 20000, 0
    else:
        Hkv, Hq, nq, n, cap, n_cur = 2, 2, 600, 500, 500 + 150, 150
    seg = _segment(2, d, Hkv, n, cap, 11)
    q = _rand((1, Hq, nq, d), torch.bfloat16, 21)
    kc = _rand((1, Hkv, n_cur, d), torch.bfloat16, 22, 2.0) if n_cur else None
    vc = _rand((1, Hkv, n_cur, d), torch.bfloat16, 23) if n_cur else None
    need = _attention_guarded(q, [seg], kc, vc, Hkv, append_to=seg if case == "fused_append" else None)
    if case in ("equal_shares", "decode_splits"):
        assert need > 0   # the merge path ran
    if case == "whole_row_blocks":
        assert need == 0  # no pieces to merge
    _check_segment_tail(seg)


def test_noalloc_writes_stay_inside():
    d, Hkv, Hq, nq = 128, 2, 2, 3000
    seg = _segment(2, d, Hkv, 800, 800, 31)
    q = _rand((1, Hq, nq, d), torch.bfloat16, 32)
    out, obuf = _guarded(Hq * nq * d)
    lse, lbuf = _guarded(Hq * nq)
    kvq.chunk_attention_noalloc(q, [seg], out.view(q.shape), n_kv_heads=Hkv, lse=lse.view(1, Hq, nq))
    torch.cuda.synchronize()
    _guard_intact(obuf, Hq * nq * d)
    _guard_intact(lbuf, Hq * nq)
    assert torch.isfinite(out).all()


@pytest.mark.parametrize("bits,d,kgc,rank,gather", [(2, 128, 0, 0, False), (4, 64, 0, 0, False),
                                                     (2, 64, 0, 0, True), (4, 128, 32, 0, False),
                                                     (2, 128, 0, 5, False), (16, 64, 0, 0, True)])
def test_appends_write_only_their_slots(bits, d, kgc, rank, gather):
    """Two appends into a segment with spare capacity and spare K-groups: nothing past the
    appended tokens and groups changes."""
    H, Gk = 2, 64
    basis = None
    if rank:
        g = torch.Generator().manual_seed(5)
        basis = torch.linalg.qr(torch.randn(H, d, rank, generator=g))[0].contiguous().cuda()
    seg = kvq.Segment(bits, torch.bfloat16, 1, H, d, 1000, k_group_tokens=Gk, kgroup_capacity=40,
                      k_group_channels=kgc, comp_basis=basis)
    for i, n in enumerate((301, 77)):
        k = _rand((1, H, n, d), torch.bfloat16, 40 + i, 2.0)
        v = _rand((1, H, n, d), torch.bfloat16, 50 + i)
        if gather:
            groups = torch.tensor([[0, 30], [40, 17], [5, 64], [n - 3, 3]], dtype=torch.int32).cuda()
            kvq.quantize_append(seg, k, v, n_new=30 + 17 + 64 + 3, src_groups=groups)
        else:
            kvq.quantize_append(seg, k, v)
        _check_segment_tail(seg)
