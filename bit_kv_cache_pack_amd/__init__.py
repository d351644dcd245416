"""Python binding of libkvq (include/kvq.h): argument marshalling only.

Every step of the computation runs in the HIP kernels of ``libkvq.so``; this module
turns torch tensors (device memory, the current HIP stream) into the C structures of
the ABI and back. There is no fallback: if the library is missing, calls raise.

Entry points (same names as the C ABI, without the ``kvq_`` prefix):
  quantize_append(segment, k_src, v_src, n_new=None, src_groups=None)
  assign_windows(k, text_query, n_fp16, n_int4, window=32, ...)
  attention_workspace_size(q, segments, n_cur, ...)
  chunk_attention(q, segments, k_cur=None, v_cur=None, ...)
  status_string(status)
``Segment`` allocates the device buffers of one cache segment (torch tensors) and keeps
the host descriptor that the C calls advance.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import List, Optional, Sequence

import numpy as np
import torch

HERE = os.path.dirname(os.path.abspath(__file__))
# KVQ_LIBRARY selects another build of the same library (e.g. a tuning variant)
LIB_PATH = os.environ.get("KVQ_LIBRARY") or os.path.join(HERE, "libkvq.so")

F32, F16, BF16 = 0, 1, 2
OK, ERR_ARG, ERR_UNSUPPORTED, ERR_CAPACITY, ERR_WORKSPACE, ERR_HIP = 0, -1, -2, -3, -4, -5
JENSEN_OFF, JENSEN_TAYLOR2, JENSEN_ISO, JENSEN_EXACT = 0, 1, 2, 3
MAX_SEGMENTS = 8

_TORCH_DT = {torch.float32: F32, torch.float16: F16, torch.bfloat16: BF16}
_DT_TORCH = {F32: torch.float32, F16: torch.float16, BF16: torch.bfloat16}

P = ctypes.c_void_p
I32 = ctypes.c_int32


class KvqSegment(ctypes.Structure):
    _fields_ = [("bits", I32), ("elem_dtype", I32), ("batch", I32), ("n_kv_heads", I32),
                ("head_dim", I32), ("capacity", I32), ("n_tokens", I32), ("k_group_tokens", I32),
                ("v_group_channels", I32), ("kgroup_capacity", I32), ("n_kgroups", I32),
                ("k", P), ("v", P), ("k_meta", P), ("v_meta", P), ("kgroup_start", P),
                ("k_group_channels", I32), ("comp_rank", I32), ("comp_basis", P), ("k_comp", P)]


class KvqAppendArgs(ctypes.Structure):
    _fields_ = [("dst", ctypes.POINTER(KvqSegment)), ("k_src", P), ("v_src", P), ("src_dtype", I32),
                ("src_tokens", ctypes.c_int64), ("n_new", I32), ("src_groups", P), ("n_src_groups", I32)]


class KvqWindowArgs(ctypes.Structure):
    _fields_ = [("k", P), ("k_dtype", I32), ("n_layers", I32), ("n_kv_heads", I32), ("head_dim", I32),
                ("n_tokens", I32), ("window", I32), ("text_query", P), ("pct_fp16", I32), ("pct_int4", I32),
                ("bits_out", P), ("order_out", P), ("score_out", P), ("groups_out", P),
                ("class_tokens_out", P)]


class KvqAttnArgs(ctypes.Structure):
    _fields_ = [("q", P), ("dtype", I32), ("batch", I32), ("n_q_heads", I32), ("n_kv_heads", I32),
                ("head_dim", I32), ("n_q", I32), ("segs", ctypes.POINTER(KvqSegment)), ("n_segs", I32),
                ("k_cur", P), ("v_cur", P), ("n_cur", I32), ("softmax_scale", ctypes.c_float),
                ("jensen", I32), ("out", P), ("out_dtype", I32), ("lse", P), ("workspace", P),
                ("workspace_bytes", ctypes.c_size_t), ("append_dst", ctypes.POINTER(KvqSegment))]


SYMBOLS = ("kvq_quantize_append", "kvq_window_budget", "kvq_assign_windows", "kvq_attention_workspace_size",
           "kvq_chunk_attention", "kvq_chunk_attention_noalloc", "kvq_probe_hbm_read", "kvq_status_string",
           "kvq_abi_version")

_lib = None


class KvqError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__("%s: %s (%d)" % (where, status_string(status), status))
        self.status = status


def lib() -> ctypes.CDLL:
    """Load libkvq.so (built by ``python -m bit_kv_cache_pack_amd.build``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libkvq.so is not built (%s); run python -m bit_kv_cache_pack_amd.build"
                               % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        L.kvq_quantize_append.argtypes = [ctypes.POINTER(KvqAppendArgs), P]
        L.kvq_quantize_append.restype = ctypes.c_int
        L.kvq_window_budget.argtypes = [I32, I32, I32, ctypes.POINTER(I32), ctypes.POINTER(I32)]
        L.kvq_window_budget.restype = ctypes.c_int
        L.kvq_assign_windows.argtypes = [ctypes.POINTER(KvqWindowArgs), P]
        L.kvq_assign_windows.restype = ctypes.c_int
        L.kvq_attention_workspace_size.argtypes = [ctypes.POINTER(KvqAttnArgs), ctypes.POINTER(ctypes.c_size_t)]
        L.kvq_attention_workspace_size.restype = ctypes.c_int
        L.kvq_chunk_attention.argtypes = [ctypes.POINTER(KvqAttnArgs), P]
        L.kvq_chunk_attention.restype = ctypes.c_int
        L.kvq_chunk_attention_noalloc.argtypes = [ctypes.POINTER(KvqAttnArgs), P]
        L.kvq_chunk_attention_noalloc.restype = ctypes.c_int
        L.kvq_probe_hbm_read.argtypes = [P, ctypes.c_size_t, P, P]
        L.kvq_probe_hbm_read.restype = ctypes.c_int
        L.kvq_status_string.argtypes = [ctypes.c_int]
        L.kvq_status_string.restype = ctypes.c_char_p
        L.kvq_abi_version.argtypes = []
        L.kvq_abi_version.restype = I32
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().kvq_status_string(int(status)).decode()


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream, t: torch.Tensor):
    """The stream to launch on: ``stream`` (a torch stream or a raw handle), or torch's
    current stream on t's device, read as the raw handle (building a torch stream object
    costs more host time than the launch itself)."""
    if stream is None:
        return ctypes.c_void_p(torch._C._cuda_getCurrentRawStream(t.device.index))
    return ctypes.c_void_p(stream.cuda_stream) if hasattr(stream, "cuda_stream") else stream


def _check(status: int, where: str) -> None:
    if status != OK:
        raise KvqError(status, where)


def _dev(t: torch.Tensor, name: str) -> torch.Tensor:
    if not t.is_cuda:
        raise ValueError("%s must be a device tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return t


class Segment:
    """Device buffers and host descriptor of one cache segment (layout: include/kvq.h)."""

    def __init__(self, bits: int, elem_dtype: torch.dtype, batch: int, n_kv_heads: int, head_dim: int,
                 capacity: int, k_group_tokens: int = 128, kgroup_capacity: Optional[int] = None,
                 v_group_channels: int = 32, device=None, k_group_channels: int = 0,
                 comp_basis: Optional[torch.Tensor] = None):
        """k_group_channels > 0: per-token K groups of that many channels. comp_basis: device
        float32 [n_kv_heads][head_dim][r] (r <= 8), the low-rank compensation's basis."""
        device = device or torch.device("cuda")
        self.bits = bits
        if kgroup_capacity is None:
            kgroup_capacity = max(1, math.ceil(capacity / k_group_tokens) + 16)
        B, H, d = batch, n_kv_heads, head_dim
        if bits == 16:
            self.k = torch.zeros((B, H, capacity, d), dtype=elem_dtype, device=device)
            self.v = torch.zeros((B, H, capacity, d), dtype=elem_dtype, device=device)
            self.k_meta = self.v_meta = self.kgroup_start = None
        else:
            wpr = d * bits // 32
            self.k = torch.zeros((B, H, capacity, wpr), dtype=torch.int32, device=device)
            self.v = torch.zeros((B, H, capacity, wpr), dtype=torch.int32, device=device)
            if k_group_channels:
                self.k_meta = torch.zeros((B, H, capacity, d // k_group_channels, 2), dtype=torch.int16,
                                          device=device)
            else:
                self.k_meta = torch.zeros((B, H, kgroup_capacity, d, 2), dtype=torch.int16, device=device)
            self.v_meta = torch.zeros((B, H, capacity, d // v_group_channels, 2), dtype=torch.int16,
                                      device=device)
            self.kgroup_start = torch.zeros(kgroup_capacity + 1, dtype=torch.int32, device=device)
        self.comp_basis = comp_basis
        r = 0 if comp_basis is None else comp_basis.shape[2]
        self.k_comp = torch.zeros((B, H, capacity, 8), dtype=torch.int16, device=device) if r else None
        self.desc = KvqSegment(bits, _TORCH_DT[elem_dtype], B, H, d, capacity, 0, k_group_tokens,
                               v_group_channels, kgroup_capacity, 0, _ptr(self.k), _ptr(self.v),
                               _ptr(self.k_meta), _ptr(self.v_meta), _ptr(self.kgroup_start),
                               k_group_channels, r, _ptr(comp_basis), _ptr(self.k_comp))

    @property
    def n_tokens(self) -> int:
        return self.desc.n_tokens

    @property
    def n_kgroups(self) -> int:
        return self.desc.n_kgroups

    def reset(self, n_tokens: int = 0, n_kgroups: int = 0) -> None:
        """Rewind the host descriptor (the device table keeps its contents)."""
        self.desc.n_tokens = n_tokens
        self.desc.n_kgroups = n_kgroups

    def nbytes(self) -> int:
        return sum(t.numel() * t.element_size() for t in (self.k, self.v, self.k_meta, self.v_meta, self.k_comp)
                   if t is not None)


def quantize_append(segment: Segment, k_src: torch.Tensor, v_src: torch.Tensor, n_new: Optional[int] = None,
                    src_groups: Optional[torch.Tensor] = None, stream=None) -> None:
    _dev(k_src, "k_src"); _dev(v_src, "v_src")
    if src_groups is not None:
        _dev(src_groups, "src_groups")
        if src_groups.dtype != torch.int32:
            raise ValueError("src_groups must be int32 [n][2]")
        n_groups = src_groups.numel() // 2
        if n_new is None:
            raise ValueError("n_new is required with src_groups (device data is not read on the host)")
    else:
        n_groups = 0
        if n_new is None:
            n_new = k_src.shape[2]
    args = KvqAppendArgs(ctypes.pointer(segment.desc), _ptr(k_src), _ptr(v_src), _TORCH_DT[k_src.dtype],
                         k_src.shape[2], int(n_new), _ptr(src_groups), n_groups)
    _check(lib().kvq_quantize_append(ctypes.byref(args), _stream(stream, k_src)), "kvq_quantize_append")


def window_budget(n_windows: int, pct_fp16: int, pct_int4: int):
    """(FP16 windows, INT4 windows) that kvq_assign_windows gives each class (the rule is
    in the library; include/kvq.h states it)."""
    a, b = I32(), I32()
    _check(lib().kvq_window_budget(int(n_windows), int(pct_fp16), int(pct_int4), ctypes.byref(a), ctypes.byref(b)),
           "kvq_window_budget")
    return a.value, b.value


class WindowAssignment:
    """Device outputs of kvq_assign_windows for n_layers caches: bits [L][W] int8, order
    [L][W] int32, score [L][W] float64, groups [L][W][2] int32 (the gather lists in
    grouped order) and class_tokens [L][3] int32 (tokens of the FP16, INT4, INT2 classes),
    plus the window counts per class."""

    def __init__(self, bits, order, score, groups, class_tokens, n_fp16, n_int4):
        self.bits, self.order, self.score = bits, order, score
        self.groups, self.class_tokens = groups, class_tokens
        self.n_fp16, self.n_int4 = n_fp16, n_int4
        self.n_windows = bits.shape[-1]

    def class_rows(self):
        """Rows of ``groups`` (per layer) holding the FP16, INT4 and INT2 gather lists."""
        a, b = self.n_fp16, self.n_fp16 + self.n_int4
        return {16: (0, a), 4: (a, b), 2: (b, self.n_windows)}

    def class_list(self, bits: int, layer: int = 0) -> torch.Tensor:
        """The device gather list of one class (a view into ``groups``)."""
        a, b = self.class_rows()[bits]
        return self.groups[layer, a:b]


def assign_windows(k: torch.Tensor, text_query: torch.Tensor, pct_fp16: int, pct_int4: int, window: int = 32,
                   out: Optional[WindowAssignment] = None, stream=None) -> WindowAssignment:
    """k: device [n_layers][Hkv][N][d] (or [Hkv][N][d] for one layer); text_query: device
    float32 [n_layers][d] (or [d])."""
    _dev(k, "k"); _dev(text_query, "text_query")
    if k.dim() == 3:
        k = k.unsqueeze(0)
    nl, H, N, d = k.shape
    if text_query.dim() == 1:
        text_query = text_query.unsqueeze(0)
    if text_query.dtype != torch.float32 or tuple(text_query.shape) != (nl, d):
        raise ValueError("text_query must be float32 [n_layers][head_dim]")
    W = -(-N // window)
    if out is None:
        n16, n4 = window_budget(W, pct_fp16, pct_int4)
        dev = k.device
        out = WindowAssignment(torch.empty((nl, W), dtype=torch.int8, device=dev),
                               torch.empty((nl, W), dtype=torch.int32, device=dev),
                               torch.empty((nl, W), dtype=torch.float64, device=dev),
                               torch.empty((nl, W, 2), dtype=torch.int32, device=dev),
                               torch.empty((nl, 3), dtype=torch.int32, device=dev), n16, n4)
    args = KvqWindowArgs(_ptr(k), _TORCH_DT[k.dtype], nl, H, d, N, window, _ptr(text_query), int(pct_fp16),
                         int(pct_int4), _ptr(out.bits), _ptr(out.order), _ptr(out.score), _ptr(out.groups),
                         _ptr(out.class_tokens))
    _check(lib().kvq_assign_windows(ctypes.byref(args), _stream(stream, k)), "kvq_assign_windows")
    return out


def _attn_args(q, segments, k_cur, v_cur, n_kv_heads, softmax_scale, jensen, out, out_dtype, lse,
               workspace, append_to=None):
    B, Hq, nq, d = q.shape
    segs = list(segments)
    if n_kv_heads is None:
        if segs:
            n_kv_heads = segs[0].desc.n_kv_heads
        elif k_cur is not None:
            n_kv_heads = k_cur.shape[1]
        else:
            raise ValueError("n_kv_heads is needed when there are neither segments nor a current chunk")
    arr = (KvqSegment * max(1, len(segs)))(*[s.desc for s in segs])
    n_cur = 0 if k_cur is None else k_cur.shape[2]
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    a = KvqAttnArgs(_ptr(q), _TORCH_DT[q.dtype], B, Hq, n_kv_heads, d, nq, arr, len(segs), _ptr(k_cur),
                    _ptr(v_cur), n_cur, float(softmax_scale), int(jensen), _ptr(out), out_dtype, _ptr(lse),
                    _ptr(workspace), ws_bytes,
                    None if append_to is None else ctypes.pointer(append_to.desc))
    return a, arr


def attention_workspace_size(q: torch.Tensor, segments: Sequence[Segment], n_cur: int = 0,
                             n_kv_heads: Optional[int] = None, jensen: int = JENSEN_TAYLOR2,
                             out_dtype: int = F32) -> int:
    a, arr = _attn_args(q, segments, None, None, n_kv_heads, 0.0, jensen, None, out_dtype, None, None)
    a.n_cur = int(n_cur)
    n = ctypes.c_size_t()
    _check(lib().kvq_attention_workspace_size(ctypes.byref(a), ctypes.byref(n)), "kvq_attention_workspace_size")
    return n.value


def chunk_attention(q: torch.Tensor, segments: Sequence[Segment], k_cur: Optional[torch.Tensor] = None,
                    v_cur: Optional[torch.Tensor] = None, n_kv_heads: Optional[int] = None,
                    softmax_scale: float = 0.0, jensen: int = JENSEN_TAYLOR2, out: Optional[torch.Tensor] = None,
                    out_dtype: torch.dtype = torch.float32, lse: Optional[torch.Tensor] = None,
                    workspace: Optional[torch.Tensor] = None, append_to: Optional[Segment] = None,
                    stream=None) -> torch.Tensor:
    """``append_to``: also quantize k_cur / v_cur into this segment in the same call (the
    attention reads the segments as they were before it)."""
    _dev(q, "q")
    if k_cur is not None:
        _dev(k_cur, "k_cur"); _dev(v_cur, "v_cur")
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype, device=q.device)
    if n_kv_heads is None and not segments and k_cur is not None:
        n_kv_heads = k_cur.shape[1]
    if workspace is None:
        need = attention_workspace_size(q, segments, 0 if k_cur is None else k_cur.shape[2], n_kv_heads,
                                        jensen, _TORCH_DT[out.dtype])
        if need:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    a, arr = _attn_args(q, segments, k_cur, v_cur, n_kv_heads, softmax_scale, jensen, out,
                        _TORCH_DT[out.dtype], lse, workspace, append_to)
    _check(lib().kvq_chunk_attention(ctypes.byref(a), _stream(stream, q)), "kvq_chunk_attention")
    return out


NOALLOC_SCRATCH_BYTES = 72 << 20   # KVQ_NOALLOC_SCRATCH_BYTES


def chunk_attention_noalloc(q: torch.Tensor, segments: Sequence[Segment], out: torch.Tensor,
                            k_cur: Optional[torch.Tensor] = None, v_cur: Optional[torch.Tensor] = None,
                            n_kv_heads: Optional[int] = None, softmax_scale: float = 0.0,
                            jensen: int = JENSEN_TAYLOR2, lse: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """kvq_chunk_attention_noalloc: chunk_attention with the partials in the library's static
    per-GPU scratch; the caller passes the output, nothing is allocated here or in the call.
    Calls that overlap on one GPU race on that scratch."""
    _dev(q, "q"); _dev(out, "out")
    if k_cur is not None:
        _dev(k_cur, "k_cur"); _dev(v_cur, "v_cur")
    if n_kv_heads is None and not segments and k_cur is not None:
        n_kv_heads = k_cur.shape[1]
    a, arr = _attn_args(q, segments, k_cur, v_cur, n_kv_heads, softmax_scale, jensen, out,
                        _TORCH_DT[out.dtype], lse, None)
    _check(lib().kvq_chunk_attention_noalloc(ctypes.byref(a), _stream(stream, q)), "kvq_chunk_attention_noalloc")
    return out


def probe_hbm_read(buf: torch.Tensor, sink: torch.Tensor, stream=None) -> None:
    """Enqueue one streaming read of ``buf`` (a measurement aid: kvq_probe_hbm_read)."""
    _dev(buf, "buf"); _dev(sink, "sink")
    nbytes = buf.numel() * buf.element_size()
    _check(lib().kvq_probe_hbm_read(_ptr(buf), nbytes, _ptr(sink), _stream(stream, buf)), "kvq_probe_hbm_read")
