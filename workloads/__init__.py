"""Seeded synthetic inputs shaped like the pages' workloads.

This module only draws random numbers and rounds them to the storage dtype of a
workload. It holds none of the quantizer's or the attention's arithmetic, so both
the CPU oracle (``oracle/``) and the HIP path (``bit_kv_cache_pack_amd``) can take
their inputs from here without sharing any code of the method.

Shapes follow the pages' workloads:

* chunk-wise autoregressive video diffusion: 1,560 latent tokens per frame, three
  frames per chunk, a growing cache of earlier chunks ("Quantized Keys Steal
  Attention: Bias Correction for KV-Cache Compression in Video Diffusion",
  abstract; "KV Cache Quantization for Self-Forcing Video Generation", abstract);
* WindowQuant decode over 100 frames x 196 visual tokens, 32-token windows, a
  64-d text query ("WindowQuant" notes, sections on what is new and on the main
  results);
* a decode-shaped GQA cache of 32,768 tokens per sequence.

No public dataset is used; every tensor is drawn from the distributions listed
per workload below.

Recipe (one numpy ``SeedSequence(seed).spawn(9)`` child stream per tensor, in
this order): channel scales, outlier channel indices, cache K, cache V, current
K, current V, Q, per-frame drift, text vector. Values are drawn in float32 and
rounded to nearest-even into the workload dtype with torch's CPU conversion;
the rounded values are what both sides consume.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional

import numpy as np
import torch

DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    dtype: str                 # storage dtype of Q / current chunk / cache elements
    src_dtype: str             # dtype of the tensors that get quantized
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    n_appends: int             # the cache is built by this many appends ...
    append_tokens: int         # ... of this many tokens each
    n_cur: int                 # unquantized current-chunk tokens
    n_q: int                   # query rows per (batch, query head)
    bits: int                  # 2 or 4; 0 = WindowQuant mixed FP16/INT4/INT2
    k_group_tokens: int = 128
    v_group_channels: int = 32
    lognormal_sigma: float = 0.5   # key channel scale ~ LogNormal(0, sigma); 0 = no scaling
    n_outliers: int = 2
    outlier_factor: float = 8.0
    drift_sigma: float = 0.0       # per-frame key drift ~ N(0, sigma^2) per channel
    frame_tokens: int = 1560
    window: int = 32
    pct_fp16: int = 10
    pct_int4: int = 30
    jensen: int = 1
    seed: int = 1000

    @property
    def n_cache(self) -> int:
        return self.n_appends * self.append_tokens

    @property
    def n_windows(self) -> int:
        return -(-self.n_cache // self.window)


WORKLOADS: Dict[str, Workload] = {}


def _add(w: Workload) -> None:
    WORKLOADS[w.name] = w


# Tiny case: one head, d = 64, a 256-token INT2 cache (one append, 8 K-groups of
# 32 tokens), a 16-token current chunk and 16 queries. Cache source in fp32;
# queries and the current chunk are rounded to bf16.
_add(Workload("tiny_int2_h1_d64", dtype="bf16", src_dtype="f32", batch=1, n_q_heads=1,
              n_kv_heads=1, head_dim=64, n_appends=1, append_tokens=256, n_cur=16, n_q=16,
              bits=2, k_group_tokens=32, seed=1000))
# Video-diffusion chunk step: 12 heads x 128, cache of 12 latent frames (4 appends of
# one 3-frame chunk), current chunk of 3 frames = 4,680 queries and unquantized keys.
_add(Workload("video_chunk_int2_h12_d128", dtype="bf16", src_dtype="bf16", batch=1,
              n_q_heads=12, n_kv_heads=12, head_dim=128, n_appends=4, append_tokens=4680,
              n_cur=4680, n_q=4680, bits=2, seed=1001))
# Decode-shaped GQA cache, 8 sequences x 32 query heads over 8 KV heads, 32,768 tokens.
for _bits in (2, 4):
    _add(Workload(f"decode_gqa32x8_int{_bits}_32k", dtype="bf16", src_dtype="bf16", batch=8,
                  n_q_heads=32, n_kv_heads=8, head_dim=128, n_appends=1, append_tokens=32768,
                  n_cur=0, n_q=1, bits=_bits, lognormal_sigma=0.0, n_outliers=4,
                  outlier_factor=10.0, seed=1002))
# WindowQuant mixed-precision window cache: 100 frames x 196 visual tokens, fp16,
# 14 query heads over 2 KV heads, d = 64, one decode query.
_add(Workload("windowquant_fp16_gqa14x2_d64", dtype="f16", src_dtype="f16", batch=1,
              n_q_heads=14, n_kv_heads=2, head_dim=64, n_appends=1, append_tokens=19600,
              n_cur=0, n_q=1, bits=0, k_group_tokens=32, frame_tokens=196, seed=1003))
# Long-rollout chunk step: 40 heads x 128, INT2 cache of 48 latent frames (16 appends
# of one 3-frame chunk), current chunk of 4,680 tokens, keys drift per frame.
_add(Workload("rollout_chunk_int2_h40_d128", dtype="bf16", src_dtype="bf16", batch=1,
              n_q_heads=40, n_kv_heads=40, head_dim=128, n_appends=16, append_tokens=4680,
              n_cur=4680, n_q=4680, bits=2, drift_sigma=0.1, seed=1004))


def scaled(w: Workload, **changes) -> Workload:
    """A copy of ``w`` with some fields replaced (smaller parity cases)."""
    return dataclasses.replace(w, **changes)


def _round(x: np.ndarray, dtype: str) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(DTYPES[dtype])


def generate(w: Workload, seed: Optional[int] = None) -> Dict[str, torch.Tensor]:
    """Draw the inputs of workload ``w`` (CPU tensors in their storage dtypes).

    Returns ``cache_k``/``cache_v`` [B][Hkv][n_cache][d] (src dtype; the history
    before quantization), ``cur_k``/``cur_v`` [B][Hkv][n_cur][d], ``q``
    [B][Hq][n_q][d] and, for WindowQuant, ``text`` [d] (float32).
    """
    ss = np.random.SeedSequence(w.seed if seed is None else seed)
    (r_scale, r_outl, r_ck, r_cv, r_uk, r_uv, r_q, r_drift, r_text) = [
        np.random.default_rng(s) for s in ss.spawn(9)]
    B, Hkv, Hq, d = w.batch, w.n_kv_heads, w.n_q_heads, w.head_dim
    n_cache, n_cur = w.n_cache, w.n_cur

    # per (kv head, channel) key scale: log-normal, then a few distinct outlier channels
    if w.lognormal_sigma > 0:
        scale = r_scale.lognormal(0.0, w.lognormal_sigma, size=(Hkv, d)).astype(np.float32)
    else:
        scale = np.ones((Hkv, d), np.float32)
    for h in range(Hkv):
        idx = r_outl.choice(d, size=w.n_outliers, replace=False)
        scale[h, idx] *= np.float32(w.outlier_factor)

    # per (kv head, frame, channel) key drift, shared by the cached and current frames
    total_frames = -(-(n_cache + n_cur) // w.frame_tokens)
    drift = (r_drift.standard_normal((Hkv, total_frames, d), dtype=np.float32)
             * np.float32(w.drift_sigma))

    def keys(rng, n, first_token):
        k = rng.standard_normal((B, Hkv, n, d), dtype=np.float32)
        k *= scale[None, :, None, :]
        if w.drift_sigma > 0 and n > 0:
            frame_of = (first_token + np.arange(n)) // w.frame_tokens
            for h in range(Hkv):
                k[:, h] += drift[h][frame_of][None]
        return k

    out: Dict[str, torch.Tensor] = {}
    out["cache_k"] = _round(keys(r_ck, n_cache, 0), w.src_dtype)
    out["cache_v"] = _round(r_cv.standard_normal((B, Hkv, n_cache, d), dtype=np.float32), w.src_dtype)
    out["cur_k"] = _round(keys(r_uk, n_cur, n_cache), w.dtype)
    out["cur_v"] = _round(r_uv.standard_normal((B, Hkv, n_cur, d), dtype=np.float32), w.dtype)
    out["q"] = _round(r_q.standard_normal((B, Hq, w.n_q, d), dtype=np.float32), w.dtype)
    out["text"] = torch.from_numpy(r_text.standard_normal(d, dtype=np.float32))
    return out
