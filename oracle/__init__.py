"""CPU oracle for low-bit KV-cache quantize-pack and Jensen-corrected chunk attention.

TEST INFRASTRUCTURE: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package. The arithmetic lives
in ``kvq_oracle.c`` (plain scalar C, fp64 attention); this file only marshals
numpy arrays through ctypes. It shares no code with ``bit_kv_cache_pack_amd``.

Segments are plain dicts of numpy arrays in the cache layout:
  k_codes / v_codes  uint32 [B][H][cap][d*bits/32]   (bits 2, 4)
  k_meta             uint16 [B][H][kgroup_cap][d][2] {step, zero} as fp16 bits
  v_meta             uint16 [B][H][cap][d/Gv][2]
  kgroup_start       int32  [kgroup_cap + 1]
  k_raw / v_raw      uint16 [B][H][cap][d]            (bits 16, fp16/bf16 bits)
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, List, Optional, Sequence

import numpy as np

from . import build as _build

F32, F16, BF16 = 0, 1, 2
_DT = {"f32": F32, "f16": F16, "bf16": BF16}

_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB) or (
                os.path.getmtime(_build.LIB) < os.path.getmtime(_build.SRC)):
            _build.build()
        _lib = ctypes.CDLL(_build.LIB)
        _declare(_lib)
    return _lib


P = ctypes.c_void_p
I32, I64, U16, F64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint16, ctypes.c_double


class OrcSegment(ctypes.Structure):
    _fields_ = [("bits", I32), ("elem_dtype", I32), ("capacity", I32), ("n_tokens", I32),
                ("n_kgroups", I32), ("kgroup_capacity", I32), ("v_group_channels", I32),
                ("k_codes", P), ("v_codes", P), ("k_meta", P), ("v_meta", P),
                ("kgroup_start", P), ("k_raw", P), ("v_raw", P),
                ("k_group_channels", I32), ("comp_rank", I32), ("comp_basis", P), ("k_comp", P)]


def _declare(L):
    L.orc_f16_to_f64.argtypes = [U16]; L.orc_f16_to_f64.restype = F64
    L.orc_f64_to_f16.argtypes = [F64]; L.orc_f64_to_f16.restype = U16
    L.orc_f32_to_f16.argtypes = [ctypes.c_float]; L.orc_f32_to_f16.restype = U16
    L.orc_f32_to_bf16.argtypes = [ctypes.c_float]; L.orc_f32_to_bf16.restype = U16
    L.orc_bf16_to_f32.argtypes = [U16]; L.orc_bf16_to_f32.restype = ctypes.c_float
    L.orc_quantize_group.argtypes = [P, I64, I64, ctypes.c_int, P, P, P, I64]
    L.orc_quantize_group.restype = None
    L.orc_dequant.argtypes = [ctypes.c_int, U16, U16, ctypes.c_int, ctypes.c_int]
    L.orc_dequant.restype = F64
    L.orc_pack_row.argtypes = [P, ctypes.c_int, ctypes.c_int, P]; L.orc_pack_row.restype = None
    L.orc_unpack_row.argtypes = [P, ctypes.c_int, ctypes.c_int, P]; L.orc_unpack_row.restype = None
    L.orc_append.argtypes = ([ctypes.c_int] * 11 + [P] * 7 + [P, P, I64, ctypes.c_int, P, ctypes.c_int]
                             + [ctypes.c_int, ctypes.c_int, P, P])
    L.orc_f64_to_bf16.argtypes = [F64]; L.orc_f64_to_bf16.restype = U16
    L.orc_append.restype = ctypes.c_int
    L.orc_log_sinhc.argtypes = [F64]; L.orc_log_sinhc.restype = F64
    L.orc_attend_row.argtypes = [P, ctypes.c_int, P, P, P, I64, P, ctypes.c_int, F64, ctypes.c_int,
                                 P, P, P, P]
    L.orc_attend_row.restype = None
    L.orc_attention.argtypes = [P] + [ctypes.c_int] * 5 + [P, ctypes.c_int, P, P, ctypes.c_int,
                                                           F64, ctypes.c_int, ctypes.c_int, P,
                                                           ctypes.c_int, P, P, P]
    L.orc_attention.restype = ctypes.c_int
    L.orc_window_scores.argtypes = [P, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, P, P]
    L.orc_window_scores.restype = None
    L.orc_assign_windows.argtypes = [P, ctypes.c_int, ctypes.c_int, ctypes.c_int, P, P]
    L.orc_assign_windows.restype = ctypes.c_int
    L.orc_window_groups.argtypes = [P, P, ctypes.c_int, ctypes.c_int, ctypes.c_int, P, P]
    L.orc_window_groups.restype = None
    L.orc_window_budget.argtypes = [ctypes.c_int] * 3 + [P, P]
    L.orc_window_budget.restype = None
    for n in ("orc_f32_to_f16_n", "orc_f32_to_bf16_n", "orc_f16_to_f64_n"):
        getattr(L, n).argtypes = [P, I64, P]
        getattr(L, n).restype = None


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# -------------------------------------------------------------------- formats
def f32_to_f16_bits(x: np.ndarray) -> np.ndarray:
    x = _c(x, np.float32).ravel()
    out = np.zeros(x.size, np.uint16)
    lib().orc_f32_to_f16_n(_ptr(x), x.size, _ptr(out))
    return out


def f16_bits_to_f64(h: np.ndarray) -> np.ndarray:
    h = _c(h, np.uint16).ravel()
    out = np.zeros(h.size, np.float64)
    lib().orc_f16_to_f64_n(_ptr(h), h.size, _ptr(out))
    return out


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    x = _c(x, np.float32).ravel()
    out = np.zeros(x.size, np.uint16)
    lib().orc_f32_to_bf16_n(_ptr(x), x.size, _ptr(out))
    return out


# -------------------------------------------------------------------- quantizer
def quantize_group(x: Sequence[float], bits: int):
    """Q1 on one group. Returns (codes uint8[n], step fp16 bits, zero fp16 bits)."""
    x = _c(x, np.float32)
    codes = np.zeros(x.size, np.uint8)
    s, z = U16(), U16()
    lib().orc_quantize_group(_ptr(x), x.size, 1, bits, ctypes.byref(s), ctypes.byref(z),
                             _ptr(codes), 1)
    return codes, s.value, z.value


def dequant(code: int, step_h: int, zero_h: int, elem: str = "bf16", exact: bool = False) -> float:
    return lib().orc_dequant(int(code), int(step_h), int(zero_h), _DT[elem], int(exact))


def pack_row(codes: Sequence[int], bits: int) -> np.ndarray:
    codes = _c(codes, np.uint8)
    d = codes.size
    words = np.zeros(d * bits // 32, np.uint32)
    lib().orc_pack_row(_ptr(codes), d, bits, _ptr(words))
    return words


def unpack_row(words: np.ndarray, d: int, bits: int) -> np.ndarray:
    words = _c(words, np.uint32)
    codes = np.zeros(d, np.uint8)
    lib().orc_unpack_row(_ptr(words), d, bits, _ptr(codes))
    return codes


# -------------------------------------------------------------------- segments
def new_segment(bits: int, elem: str, B: int, H: int, d: int, capacity: int,
                k_group_tokens: int, kgroup_capacity: int, v_group_channels: int = 32,
                k_group_channels: int = 0, comp_basis: Optional[np.ndarray] = None) -> Dict:
    """k_group_channels > 0: per-token K groups of that many channels (k_meta [B][H][cap]
    [d/kgc][2]). comp_basis float32 [H][d][r]: the low-rank compensation, c stored as bf16
    bits in k_comp [B][H][cap][8] (the first r entries)."""
    r = 0 if comp_basis is None else comp_basis.shape[2]
    seg = dict(bits=bits, elem=elem, B=B, H=H, d=d, capacity=capacity, n_tokens=0, n_kgroups=0,
               Gk=k_group_tokens, Gv=v_group_channels, kgroup_capacity=kgroup_capacity,
               kgc=k_group_channels, comp_rank=r)
    if bits == 16:
        seg["k_raw"] = np.zeros((B, H, capacity, d), np.uint16)
        seg["v_raw"] = np.zeros((B, H, capacity, d), np.uint16)
    else:
        wpr = d * bits // 32
        seg["k_codes"] = np.zeros((B, H, capacity, wpr), np.uint32)
        seg["v_codes"] = np.zeros((B, H, capacity, wpr), np.uint32)
        if k_group_channels:
            seg["k_meta"] = np.zeros((B, H, capacity, d // k_group_channels, 2), np.uint16)
        else:
            seg["k_meta"] = np.zeros((B, H, kgroup_capacity, d, 2), np.uint16)
        seg["v_meta"] = np.zeros((B, H, capacity, d // v_group_channels, 2), np.uint16)
        seg["kgroup_start"] = np.zeros(kgroup_capacity + 1, np.int32)
        if r:
            seg["comp_basis"] = np.ascontiguousarray(comp_basis, np.float32)
            seg["k_comp"] = np.zeros((B, H, capacity, 8), np.uint16)
    return seg


def append(seg: Dict, k_src: np.ndarray, v_src: np.ndarray, n_new: Optional[int] = None,
           groups: Optional[np.ndarray] = None) -> int:
    """Q3: quantize-append; k_src/v_src float [B][H][src_tokens][d] (exact values of the
    source dtype). Returns the number of new K-groups and advances the segment."""
    k_src = _c(k_src, np.float32)
    v_src = _c(v_src, np.float32)
    src_tokens = k_src.shape[2]
    g = None if groups is None else _c(groups, np.int32).reshape(-1, 2)
    if n_new is None:
        n_new = src_tokens if g is None else int(g[:, 1].sum())
    n_groups_in = 0 if g is None else g.shape[0]
    r = lib().orc_append(seg["bits"], _DT[seg["elem"]], seg["B"], seg["H"], seg["d"],
                         seg["capacity"], seg["n_tokens"], seg["Gk"], seg["Gv"],
                         seg["kgroup_capacity"], seg["n_kgroups"],
                         _ptr(seg.get("k_codes")), _ptr(seg.get("v_codes")),
                         _ptr(seg.get("k_meta")), _ptr(seg.get("v_meta")),
                         _ptr(seg.get("kgroup_start")), _ptr(seg.get("k_raw")),
                         _ptr(seg.get("v_raw")), _ptr(k_src), _ptr(v_src), src_tokens, n_new,
                         _ptr(g), n_groups_in, seg.get("kgc", 0), seg.get("comp_rank", 0),
                         _ptr(seg.get("comp_basis")), _ptr(seg.get("k_comp")))
    if r < 0:
        raise ValueError("oracle append rejected the request")
    seg["n_tokens"] += n_new
    if seg["bits"] != 16:
        seg["n_kgroups"] += r
    return r


def _orc_seg(seg: Dict) -> OrcSegment:
    return OrcSegment(seg["bits"], _DT[seg["elem"]], seg["capacity"], seg["n_tokens"],
                      seg["n_kgroups"], seg["kgroup_capacity"], seg["Gv"],
                      _ptr(seg.get("k_codes")), _ptr(seg.get("v_codes")),
                      _ptr(seg.get("k_meta")), _ptr(seg.get("v_meta")),
                      _ptr(seg.get("kgroup_start")), _ptr(seg.get("k_raw")),
                      _ptr(seg.get("v_raw")), seg.get("kgc", 0), seg.get("comp_rank", 0),
                      _ptr(seg.get("comp_basis")), _ptr(seg.get("k_comp")))


# -------------------------------------------------------------------- attention
def attention(q: np.ndarray, segs: List[Dict], k_cur: Optional[np.ndarray] = None,
              v_cur: Optional[np.ndarray] = None, n_kv_heads: Optional[int] = None,
              scale: Optional[float] = None, jensen: int = 1, exact: bool = False,
              rows: Optional[Sequence[int]] = None, want_mass: bool = False):
    """A1-A3 in double. q float [B][Hq][nq][d]. jensen: 0 off, 1 the channel-weighted
    second-order term, 2 its isotropic (query-norm) form, 3 the same noise model to all
    orders (sum over channels of log(sinh a / a)). Returns (out [B][Hq][n_rows][d]
    float64, lse [B][Hq][n_rows]) and, with want_mass, the softmax mass on cached tokens."""
    q = _c(q, np.float32)
    B, Hq, nq, d = q.shape
    if n_kv_heads is None:
        n_kv_heads = segs[0]["H"] if segs else k_cur.shape[1]
    n_cur = 0 if k_cur is None else k_cur.shape[2]
    if k_cur is None:
        k_cur = np.zeros((B, n_kv_heads, 0, d), np.float32)
        v_cur = k_cur
    k_cur = _c(k_cur, np.float32)
    v_cur = _c(v_cur, np.float32)
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    rws = None if rows is None else _c(rows, np.int32)
    n_rows = nq if rws is None else rws.size
    out = np.zeros((B, Hq, n_rows, d), np.float64)
    lse = np.zeros((B, Hq, n_rows), np.float64)
    mass = np.zeros((B, Hq, n_rows), np.float64) if want_mass else None
    arr = (OrcSegment * max(1, len(segs)))(*[_orc_seg(s) for s in segs])
    r = lib().orc_attention(_ptr(q), B, Hq, n_kv_heads, d, nq, arr, len(segs), _ptr(k_cur),
                            _ptr(v_cur), n_cur, float(scale), int(jensen), int(exact), _ptr(rws),
                            n_rows, _ptr(out), _ptr(lse), _ptr(mass))
    if r != 0:
        raise ValueError("oracle attention rejected the request")
    return (out, lse, mass) if want_mass else (out, lse)


def attend_row(q: np.ndarray, K: np.ndarray, V: np.ndarray, tok_group: np.ndarray,
               step_sq: np.ndarray, scale: float, jensen: int, logit_add: Optional[np.ndarray] = None):
    """One query over a dense key/value list (real-valued keys, e.g. keys plus sampled
    rounding noise); jensen as in attention(). Returns (out [d], lse, mass on grouped
    tokens)."""
    q = _c(q, np.float64); K = _c(K, np.float64); V = _c(V, np.float64)
    tg = _c(tok_group, np.int32); ssq = _c(step_sq, np.float64)
    d = q.size
    out = np.zeros(d, np.float64)
    lse, mass = F64(), F64()
    la = None if logit_add is None else _c(logit_add, np.float64)
    lib().orc_attend_row(_ptr(q), d, _ptr(K), _ptr(V), _ptr(tg), K.shape[0], _ptr(ssq),
                         ssq.shape[0] if ssq.ndim == 2 else 0, float(scale), int(jensen), _ptr(la),
                         _ptr(out), ctypes.byref(lse), ctypes.byref(mass))
    return out, lse.value, mass.value


# -------------------------------------------------------------------- windows
def window_scores(k: np.ndarray, text: np.ndarray, window: int = 32) -> np.ndarray:
    k = _c(k, np.float32)
    H, N, d = k.shape
    W = -(-N // window)
    score = np.zeros(W, np.float64)
    lib().orc_window_scores(_ptr(k), H, N, d, window, _ptr(_c(text, np.float32)), _ptr(score))
    return score


def assign_windows(score: np.ndarray, n_fp16: int, n_int4: int):
    score = _c(score, np.float64)
    W = score.size
    bits = np.zeros(W, np.int8)
    order = np.zeros(W, np.int32)
    if lib().orc_assign_windows(_ptr(score), W, n_fp16, n_int4, _ptr(bits), _ptr(order)) != 0:
        raise ValueError("bad window budget")
    return bits, order


def window_budget(n_windows: int, pct_fp16: int, pct_int4: int):
    a, b = ctypes.c_int(), ctypes.c_int()
    lib().orc_window_budget(n_windows, pct_fp16, pct_int4, ctypes.byref(a), ctypes.byref(b))
    return a.value, b.value


def window_groups(bits: np.ndarray, order: np.ndarray, n_tokens: int, window: int = 32):
    """A6: gather lists in grouped order (int32 [W][2]: first token, length) and the token
    counts of the FP16, INT4 and INT2 classes."""
    bits = _c(bits, np.int8)
    order = _c(order, np.int32)
    W = bits.size
    groups = np.zeros((W, 2), np.int32)
    ct = np.zeros(3, np.int32)
    lib().orc_window_groups(_ptr(bits), _ptr(order), W, int(n_tokens), int(window), _ptr(groups), _ptr(ct))
    return groups, ct


def log_sinhc(a: float) -> float:
    """log(sinh(a) / a), a >= 0 (0 at a = 0)."""
    return lib().orc_log_sinhc(float(a))


def f64_to_bf16_bits(x: float) -> int:
    return lib().orc_f64_to_bf16(float(x))
