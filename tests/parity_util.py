"""Helpers of the GPU parity tests: build the same cache on both sides (HIP library via
the binding, CPU oracle), copy device buffers back in the oracle's layout, compare."""
import numpy as np
import torch

import bit_kv_cache_pack_amd as kvq
import oracle

TORCH_DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def f32(t: torch.Tensor) -> np.ndarray:
    """Exact float32 values of a CPU tensor of any float dtype."""
    return t.float().numpy()


def make_pair(bits, elem, B, H, d, capacity, Gk, kgroup_capacity, k_group_channels=0, comp_basis=None):
    """comp_basis: the low-rank compensation's basis [H][d][r], float32: numpy (copied to the
    device for this segment), or a CUDA tensor (the device copy itself, which segments read in
    one attention call share)."""
    if comp_basis is None:
        gb = ob = None
    elif isinstance(comp_basis, torch.Tensor):
        gb, ob = comp_basis, comp_basis.cpu().numpy()
    else:
        ob = np.ascontiguousarray(comp_basis, np.float32)
        gb = torch.from_numpy(ob).cuda()
    g = kvq.Segment(bits, TORCH_DT[elem], B, H, d, capacity, k_group_tokens=Gk, kgroup_capacity=kgroup_capacity,
                    k_group_channels=k_group_channels, comp_basis=gb)
    o = oracle.new_segment(bits, elem, B, H, d, capacity=capacity, k_group_tokens=Gk,
                           kgroup_capacity=kgroup_capacity, k_group_channels=k_group_channels,
                           comp_basis=ob)
    return g, o


def append_both(gseg, oseg, k_src: torch.Tensor, v_src: torch.Tensor, groups=None):
    """k_src/v_src CPU tensors [B][H][n][d]; groups: list of (start, len) or None."""
    kd, vd = k_src.cuda(), v_src.cuda()
    if groups is None:
        kvq.quantize_append(gseg, kd, vd)
        oracle.append(oseg, f32(k_src), f32(v_src))
    else:
        garr = np.asarray(groups, np.int32).reshape(-1, 2)
        n_new = int(garr[:, 1].sum())
        kvq.quantize_append(gseg, kd, vd, n_new=n_new, src_groups=torch.from_numpy(garr).cuda())
        oracle.append(oseg, f32(k_src), f32(v_src), groups=garr)


def host_view(gseg):
    """The GPU segment's buffers as numpy arrays in the oracle's layout."""
    out = dict(n_tokens=gseg.n_tokens, n_kgroups=gseg.n_kgroups)
    if gseg.bits == 16:
        out["k_raw"] = gseg.k.cpu().view(torch.int16).numpy().view(np.uint16)
        out["v_raw"] = gseg.v.cpu().view(torch.int16).numpy().view(np.uint16)
    else:
        out["k_codes"] = gseg.k.cpu().numpy().view(np.uint32)
        out["v_codes"] = gseg.v.cpu().numpy().view(np.uint32)
        out["k_meta"] = gseg.k_meta.cpu().numpy().view(np.uint16)
        out["v_meta"] = gseg.v_meta.cpu().numpy().view(np.uint16)
        out["kgroup_start"] = gseg.kgroup_start.cpu().numpy()
        if gseg.k_comp is not None:
            out["k_comp"] = gseg.k_comp.cpu().numpy().view(np.uint16)
    return out


def assert_segments_equal(gseg, oseg):
    h = host_view(gseg)
    assert h["n_tokens"] == oseg["n_tokens"]
    n = oseg["n_tokens"]
    if gseg.bits == 16:
        assert np.array_equal(h["k_raw"][:, :, :n], oseg["k_raw"][:, :, :n])
        assert np.array_equal(h["v_raw"][:, :, :n], oseg["v_raw"][:, :, :n])
        return
    G = oseg["n_kgroups"]
    assert h["n_kgroups"] == G
    token_groups = oseg.get("kgc", 0) > 0
    if not token_groups:
        assert np.array_equal(h["kgroup_start"][:G + 1], oseg["kgroup_start"][:G + 1])
    if "k_comp" in h:
        # the compensation is a float sum (fp32 on the device, double in the oracle) rounded
        # to bf16: within one bf16 step of the oracle's plus the fp32 sum's own error (head_dim
        # terms |U e| <= |e| <= a few units: below 2^-15 absolute), and mostly equal
        a = h["k_comp"][:, :, :n].astype(np.uint32) << 16
        b = oseg["k_comp"][:, :, :n].astype(np.uint32) << 16
        fa, fb = a.view(np.float32).astype(np.float64), b.view(np.float32).astype(np.float64)
        step = np.abs(fb) * 2.0 ** -7 + 2.0 ** -15
        assert np.all(np.abs(fa - fb) <= step), np.abs(fa - fb).max()
        assert (a == b).mean() >= 0.98, (a == b).mean()
    for name, sl in (("k_codes", np.s_[:, :, :n]), ("v_codes", np.s_[:, :, :n]),
                     ("k_meta", np.s_[:, :, :n] if token_groups else np.s_[:, :, :G]),
                     ("v_meta", np.s_[:, :, :n])):
        a, b = h[name][sl], oseg[name][sl]
        bad = np.argwhere(a != b)
        assert bad.size == 0, "%s differs at %d places, first %s: gpu %s oracle %s" % (
            name, len(bad), bad[0].tolist(), a[tuple(bad[0])], b[tuple(bad[0])])


def gpu_attention(q, gsegs, k_cur=None, v_cur=None, n_kv_heads=None, jensen=1, out_dtype=torch.float32,
                  softmax_scale=0.0):
    qd = q.cuda()
    kc = None if k_cur is None else k_cur.cuda()
    vc = None if v_cur is None else v_cur.cuda()
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
    out = kvq.chunk_attention(qd, gsegs, kc, vc, n_kv_heads=n_kv_heads, jensen=jensen, out_dtype=out_dtype,
                              lse=lse, softmax_scale=softmax_scale)
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), lse.cpu().numpy()


def oracle_attention(q, osegs, k_cur=None, v_cur=None, n_kv_heads=None, jensen=1, rows=None, scale=None):
    kc = None if k_cur is None else f32(k_cur)
    vc = None if v_cur is None else f32(v_cur)
    return oracle.attention(f32(q), osegs, kc, vc, n_kv_heads=n_kv_heads, jensen=int(jensen), rows=rows,
                            scale=scale)


def bf16_half_ulp(x: np.ndarray) -> np.ndarray:
    """Half a bf16 ulp at |x| (the rounding error of writing x as bf16)."""
    ax = np.maximum(np.abs(x), 2.0 ** -126)
    return np.exp2(np.floor(np.log2(ax)) - 8)


def window_case(nl, H, N, d, seed, dtype=torch.float16):
    """Seeded keys [nl][H][N][d] and text queries [nl][d] for window scoring."""
    rng = np.random.default_rng(seed)
    k = torch.from_numpy(rng.standard_normal((nl, H, N, d)).astype(np.float32)).to(dtype)
    t = torch.from_numpy(rng.standard_normal((nl, d)).astype(np.float32))
    return k, t


def check_windows(asg, k, t, N, window=32, pct=(10, 30)):
    """Every layer's scores (4 ulp), bits, order, gather lists and class token counts
    (bit-exact) against the oracle run on that layer alone; k [layers][H][N][d], t
    [layers][d] on the CPU."""
    W = -(-N // window)
    n16, n4 = oracle.window_budget(W, *pct)
    assert (asg.n_fp16, asg.n_int4) == (n16, n4)
    score, bits, order = asg.score.cpu().numpy(), asg.bits.cpu().numpy(), asg.order.cpu().numpy()
    groups, ct = asg.groups.cpu().numpy(), asg.class_tokens.cpu().numpy()
    for layer in range(k.shape[0]):
        osc = oracle.window_scores(f32(k[layer]), t[layer].numpy(), window)
        ob, oo = oracle.assign_windows(osc, n16, n4)
        og, oct_ = oracle.window_groups(ob, oo, N, window)
        np.testing.assert_array_max_ulp(score[layer], osc, maxulp=4)
        assert np.array_equal(bits[layer], ob), layer
        assert np.array_equal(order[layer], oo), layer
        assert np.array_equal(groups[layer], og), layer
        assert np.array_equal(ct[layer], oct_), layer
