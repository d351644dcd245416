"""A seeded sweep of small random configurations, GPU against the CPU oracle. Each case draws:
- the element dtype (bf16 or f16), head_dim (64 or 128), batch (1 or 2), the GQA ratio (1, 2,
  4 or 7) and the KV head count;
- one or two cache segments with INT2, INT4 or raw (bits 16) tokens, each filled by one to
  three appends of ragged lengths, in K-groups of 32, 64 or 128 tokens;
- a current chunk of 0 to 200 tokens;
- 1 to 4 query rows per head (decode-shaped) or up to 400 (chunk-shaped, several row blocks);
- the Jensen form (off, channel-weighted, isotropic, all orders).
Together they reach both attention kernels, their work plans (whole row blocks, equal
shares with merged pieces, decode splits) and multi-segment walks in combinations the
hand-picked cases do not. A second sweep adds, to the same draws, per-token K groups or the
low-rank compensation on the packed segments (one kind per call, as the library requires)
and the current chunk appended by the attention call itself. Appended segments are compared
bit for bit, attention within 2e-3 (fp32 output) and the log-sum-exp within 2e-3, as in
test_gpu_parity.py.
"""
import os

import numpy as np
import pytest
import torch

import bit_kv_cache_pack_amd as kvq
import oracle
from parity_util import (TORCH_DT, append_both, assert_segments_equal, f32, gpu_attention, make_pair,
                         oracle_attention)

pytestmark = pytest.mark.gpu
TOL = 2e-3
N_CASES = 160
# Wider sweeps on demand: KVQ_SWEEP_SCALE multiplies every case count and KVQ_SWEEP_OFFSET
# moves every seed (defaults 1 and 0: the committed cases).
SCALE = int(os.environ.get("KVQ_SWEEP_SCALE", "1"))
OFFSET = int(os.environ.get("KVQ_SWEEP_OFFSET", "0"))


def _cases(n):
    return range(OFFSET, OFFSET + n * SCALE)


def _rand(rng, shape, dtype, scale=1.0):
    return torch.from_numpy((rng.standard_normal(shape) * scale).astype(np.float32)).to(TORCH_DT[dtype])


def _draw(case):
    rng = np.random.default_rng(7000 + case)
    c = dict(dtype=str(rng.choice(["bf16", "f16"])), d=int(rng.choice([64, 128])), B=int(rng.choice([1, 2])),
             gqa=int(rng.choice([1, 2, 4, 7])), Hkv=int(rng.choice([1, 2, 3])))
    n_segs = int(rng.choice([1, 1, 2]))
    c["segs"] = []
    for _ in range(n_segs):
        bits = int(rng.choice([2, 2, 4, 16]))
        appends = [int(n) for n in rng.integers(1, 900, size=int(rng.integers(1, 4)))]
        c["segs"].append(dict(bits=bits, Gk=int(rng.choice([32, 64, 128])), appends=appends))
    c["n_cur"] = int(rng.choice([0, 0, int(rng.integers(1, 201))]))
    c["n_q"] = int(rng.integers(1, 5)) if rng.random() < 0.4 else int(rng.integers(50, 401))
    c["jensen"] = int(rng.choice([0, 1, 1, 2, 3]))
    return c, rng


@pytest.mark.parametrize("case", _cases(N_CASES))
def test_random_configuration(case):
    c, rng = _draw(case)
    dtype, d, B, Hkv = c["dtype"], c["d"], c["B"], c["Hkv"]
    Hq = c["gqa"] * Hkv
    gsegs, osegs = [], []
    for s in c["segs"]:
        cap = sum(s["appends"])
        kgc = sum(-(-n // s["Gk"]) for n in s["appends"])
        gseg, oseg = make_pair(s["bits"], dtype, B, Hkv, d, capacity=cap, Gk=s["Gk"], kgroup_capacity=kgc)
        for n in s["appends"]:
            append_both(gseg, oseg, _rand(rng, (B, Hkv, n, d), dtype, 2.0), _rand(rng, (B, Hkv, n, d), dtype))
        assert_segments_equal(gseg, oseg)
        gsegs.append(gseg)
        osegs.append(oseg)
    q = _rand(rng, (B, Hq, c["n_q"], d), dtype)
    kc = _rand(rng, (B, Hkv, c["n_cur"], d), dtype, 2.0) if c["n_cur"] else None
    vc = _rand(rng, (B, Hkv, c["n_cur"], d), dtype) if c["n_cur"] else None
    go, gl = gpu_attention(q, gsegs, kc, vc, n_kv_heads=Hkv, jensen=c["jensen"])
    oo, ol = oracle_attention(q, osegs, kc, vc, n_kv_heads=Hkv, jensen=c["jensen"])
    err, lerr = np.abs(go - oo).max(), np.abs(gl - ol).max()
    assert err <= TOL and lerr <= TOL, (c, err, lerr)


def _basis(rng, H, d, r):
    U = np.zeros((H, d, r), np.float32)
    for h in range(H):
        U[h] = np.linalg.qr(rng.standard_normal((d, r)))[0].astype(np.float32)
    return U


@pytest.mark.parametrize("case", _cases(64))
def test_random_configuration_extras(case):
    c, rng = _draw(100 + case)
    dtype, d, B, Hkv = c["dtype"], c["d"], c["B"], c["Hkv"]
    Hq = c["gqa"] * Hkv
    aug = str(rng.choice(["tok", "comp"]))
    kgc = int(rng.choice([32, 64] + ([128] if d == 128 else []))) if aug == "tok" else 0
    # one device copy of the basis for every segment of the call (the library requires the same)
    basis = torch.from_numpy(_basis(rng, Hkv, d, int(rng.integers(1, 9)))).cuda() if aug == "comp" else None
    jensen = 1 if c["jensen"] == 3 else c["jensen"]
    n_cur = c["n_cur"] or int(rng.integers(1, 201))
    fused = int(rng.integers(0, len(c["segs"]))) if rng.random() < 0.6 else -1
    gsegs, osegs = [], []
    for i, s in enumerate(c["segs"]):
        packed = s["bits"] != 16
        extra = n_cur if i == fused else 0
        cap = sum(s["appends"]) + extra
        groups = kgc == 0 and packed
        kcap = sum(-(-n // s["Gk"]) for n in s["appends"]) + -(-extra // s["Gk"]) if groups else 1
        gseg, oseg = make_pair(s["bits"], dtype, B, Hkv, d, capacity=cap, Gk=s["Gk"], kgroup_capacity=kcap,
                               k_group_channels=kgc if packed else 0, comp_basis=basis if packed else None)
        for n in s["appends"]:
            append_both(gseg, oseg, _rand(rng, (B, Hkv, n, d), dtype, 2.0), _rand(rng, (B, Hkv, n, d), dtype))
        assert_segments_equal(gseg, oseg)
        gsegs.append(gseg)
        osegs.append(oseg)
    q = _rand(rng, (B, Hq, c["n_q"], d), dtype)
    kc = _rand(rng, (B, Hkv, n_cur, d), dtype, 2.0)
    vc = _rand(rng, (B, Hkv, n_cur, d), dtype)
    oo, ol = oracle_attention(q, osegs, kc, vc, n_kv_heads=Hkv, jensen=jensen)
    if fused < 0:
        go, gl = gpu_attention(q, gsegs, kc, vc, n_kv_heads=Hkv, jensen=jensen)
    else:
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
        out = kvq.chunk_attention(q.cuda(), gsegs, kc.cuda(), vc.cuda(), n_kv_heads=Hkv, jensen=jensen, lse=lse,
                                  append_to=gsegs[fused])
        torch.cuda.synchronize()
        go, gl = out.float().cpu().numpy(), lse.cpu().numpy()
        oracle.append(osegs[fused], f32(kc), f32(vc))
        assert_segments_equal(gsegs[fused], osegs[fused])
    err, lerr = np.abs(go - oo).max(), np.abs(gl - ol).max()
    assert err <= TOL and lerr <= TOL, (c, aug, kgc, fused, err, lerr)


@pytest.mark.parametrize("case", _cases(96))
def test_random_appends(case):
    """Quantize-appends of random shape against the oracle, bit for bit: INT2 or INT4, head
    dim 64 or 128, fp32/bf16/fp16 sources into bf16/fp16 caches, K-groups of 32 to 256
    tokens, two or three appends of ragged lengths (1 to 700 tokens), contiguous or gathered
    from random windows (any order, ragged window lengths, a repeated window)."""
    rng = np.random.default_rng(9000 + case)
    bits, d = int(rng.choice([2, 4])), int(rng.choice([64, 128]))
    elem = str(rng.choice(["bf16", "f16"]))
    src = str(rng.choice(["f32", elem]))
    B, H, Gk = int(rng.choice([1, 2])), int(rng.choice([1, 2, 3])), int(rng.choice([32, 64, 128, 256]))
    plans = []
    for _ in range(int(rng.integers(2, 4))):
        n = int(rng.integers(1, 701))
        if rng.random() < 0.4:
            wl = int(rng.choice([16, 32, Gk]))
            starts = rng.permutation(np.arange(0, max(n - 1, 1), wl))[: int(rng.integers(1, 12))]
            groups = [(int(s0), int(min(wl, n - s0))) for s0 in starts]
            if len(groups) > 1:
                groups.append(groups[0])        # a window taken twice
            plans.append((n, [(s0, min(ln, Gk)) for s0, ln in groups]))
        else:
            plans.append((n, None))
    cap = sum(n if g is None else sum(ln for _, ln in g) for n, g in plans)
    kcap = sum(-(-n // Gk) if g is None else len(g) for n, g in plans)
    gseg, oseg = make_pair(bits, elem, B, H, d, capacity=cap, Gk=Gk, kgroup_capacity=kcap)
    for n, groups in plans:
        k = _rand(rng, (B, H, n, d), src, 3.0)
        v = _rand(rng, (B, H, n, d), src)
        append_both(gseg, oseg, k, v, groups=groups)
        assert_segments_equal(gseg, oseg)


@pytest.mark.parametrize("case", _cases(40))
def test_random_window_assignments(case):
    """Window scores, bit-widths, order, gather lists and class token counts for random
    token counts (1 to 9,000), KV heads, head dims, layers and budget percentages (the class
    boundaries move with them), against the oracle."""
    from parity_util import check_windows, window_case
    rng = np.random.default_rng(9500 + case)
    nl, H, d = int(rng.integers(1, 4)), int(rng.integers(1, 4)), int(rng.choice([64, 128]))
    N = int(rng.integers(1, 9001))
    p16 = int(rng.integers(0, 31))
    p4 = int(rng.integers(0, 101 - p16))
    k, t = window_case(nl, H, N, d, 9500 + case, dtype=TORCH_DT[str(rng.choice(["f16", "bf16"]))])
    asg = kvq.assign_windows(k.cuda(), t.cuda(), p16, p4)
    torch.cuda.synchronize()
    check_windows(asg, k, t, N, pct=(p16, p4))
