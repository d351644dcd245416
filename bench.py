"""Benchmark: fused INT2-KV chunk attention (TFLOP/s, effective KV GB/s vs MI355X peaks).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

Default workload: the video-diffusion chunk step -- batch 1, 12 heads, head_dim 128, an
INT2 cache of 18,720 tokens (4 appends of one 4,680-token chunk, K groups of 128 tokens,
V groups of 32 channels) and an unquantized current chunk of 4,680 tokens that is both the
queries and the current keys/values. One step = the fused attention with the Jensen
correction, then the quantize-append of the current chunk into the cache (the descriptor
is rewound after each step, so every step does identical work). Inputs are seeded
synthetic tensors already resident in HBM when timing starts.

One JSON line on stdout. ``value`` = attention FLOPs per step (4 * B * Hq * Nq * (N_cache +
N_cur) * d, the dense QK^T and PV products) / step time. ``roofline`` is the attention
kernel against the bf16 dense MFMA peak, its duration taken with HIP events recorded on
the stream the kernels run on. ``cpu_baseline`` times the CPU oracle on a bounded sample.
"""
import argparse
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import bit_kv_cache_pack_amd as kvq  # noqa: E402
import workloads  # noqa: E402

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16/fp16 MFMA
PEAK_HBM_GBPS = 8000.0        # MI355X HBM3E
METRIC = "fused INT2-KV chunk attention: TFLOP/s + effective KV HBM GB/s vs peak"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class ChunkStep:
    """Attention of the current chunk over the packed cache + the chunk's quantize-append."""

    def __init__(self, w: workloads.Workload, n_copies: int = 1):
        self.w = w
        t0 = time.time()
        data = workloads.generate(w)
        log("generated inputs in %.1fs" % (time.time() - t0))
        self.data = data
        B, Hq, Hkv, d = w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim
        dt = workloads.DTYPES[w.dtype]
        self.bits = w.bits
        n_groups = w.n_appends * -(-w.append_tokens // w.k_group_tokens)
        extra = -(-w.n_cur // w.k_group_tokens) if w.n_cur else 0
        self.segs = []
        for c in range(n_copies):
            seg = kvq.Segment(w.bits, dt, B, Hkv, d, w.n_cache + w.n_cur, k_group_tokens=w.k_group_tokens,
                              kgroup_capacity=n_groups + extra)
            ck, cv = data["cache_k"], data["cache_v"]
            for a in range(w.n_appends):
                sl = slice(a * w.append_tokens, (a + 1) * w.append_tokens)
                kvq.quantize_append(seg, ck[:, :, sl].contiguous().cuda(), cv[:, :, sl].contiguous().cuda())
            self.segs.append(seg)
        torch.cuda.synchronize()
        self.base = (self.segs[0].n_tokens, self.segs[0].n_kgroups)
        self.q = data["q"].cuda()
        self.k_cur = data["cur_k"].cuda() if w.n_cur else None
        self.v_cur = data["cur_v"].cuda() if w.n_cur else None
        self.out = torch.empty(self.q.shape, dtype=torch.float32, device="cuda")
        need = kvq.attention_workspace_size(self.q, self.segs[:1], w.n_cur, jensen=w.jensen)
        self.ws = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")
        self.i = 0
        self.append = w.n_cur > 0

    def flops(self) -> float:
        w = self.w
        return 4.0 * w.batch * w.n_q_heads * w.n_q * (w.n_cache + w.n_cur) * w.head_dim

    def kv_bytes(self) -> float:
        """Packed codes + fp16 step/zero of the cache + raw current K/V, each read once."""
        w = self.w
        per_tok = 2 * w.head_dim * w.bits / 8 + 4 * (w.head_dim // w.v_group_channels)
        kmeta = 4 * w.head_dim * w.n_appends * -(-w.append_tokens // w.k_group_tokens)
        cache = w.batch * w.n_kv_heads * (w.n_cache * per_tok + kmeta)
        cur = 2 * w.batch * w.n_kv_heads * w.n_cur * w.head_dim * 2
        return cache + cur

    def qo_bytes(self) -> float:
        w = self.w
        return w.batch * w.n_q_heads * w.n_q * w.head_dim * (2 + 4)

    def append_bytes(self) -> float:
        """Quantize-append: read the chunk's K and V, write codes and step/zero."""
        w = self.w
        if not self.append:
            return 0.0
        n = w.n_cur
        rd = 2 * w.batch * w.n_kv_heads * n * w.head_dim * 2
        wr = w.batch * w.n_kv_heads * (2 * n * w.head_dim * w.bits / 8 + 4 * n * (w.head_dim // 32)
                                       + 4 * w.head_dim * -(-n // w.k_group_tokens))
        return rd + wr

    def run(self, events=None):
        seg = self.segs[self.i % len(self.segs)]
        self.i += 1
        seg.reset(*self.base)
        if events is not None:
            events[0].record()
        kvq.chunk_attention(self.q, [seg], self.k_cur, self.v_cur, jensen=self.w.jensen, out=self.out,
                            workspace=self.ws)
        if events is not None:
            events[1].record()
        if self.append:
            kvq.quantize_append(seg, self.k_cur, self.v_cur)
        if events is not None:
            events[2].record()


def kernel_source_digest() -> str:
    """sha256 over the HIP sources of the library (any change invalidates stored counters)."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "bit_kv_cache_pack_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        if name.endswith((".hip", ".cuh", ".h")):
            with open(os.path.join(csrc, name), "rb") as f:
                h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def stored_traffic(workload: str, kernel: str):
    """HBM bytes per launch of `kernel` on `workload` from profiles/, or None when no summary
    exists or the kernel sources changed since its counters were taken."""
    path = os.path.join(ROOT, "profiles", "%s_%s_traffic.md" % (kernel, workload))
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if line.startswith("- ") and ":" in line:
            k, v = line[2:].split(":", 1)
            vals[k.strip()] = v.strip().strip("`")
    if vals.get("source_sha256") != kernel_source_digest():
        return None
    try:
        return int(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(step: ChunkStep, target_s: float = 15.0):
    """Time the CPU oracle (as it stands) on a bounded sample of the same workload: the
    quantize-append of the current chunk in full, and the attention of every r-th query row
    of every head over the full history (r chosen so the sample costs ~target_s)."""
    import oracle
    w = step.w
    data = step.data
    threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or os.cpu_count()
    seg = oracle.new_segment(w.bits, w.dtype, w.batch, w.n_kv_heads, w.head_dim,
                             capacity=w.n_cache + w.n_cur, k_group_tokens=w.k_group_tokens,
                             kgroup_capacity=w.n_appends * -(-w.append_tokens // w.k_group_tokens)
                             + -(-max(w.n_cur, 1) // w.k_group_tokens))
    ck, cv = data["cache_k"].float().numpy(), data["cache_v"].float().numpy()
    for a in range(w.n_appends):
        sl = slice(a * w.append_tokens, (a + 1) * w.append_tokens)
        oracle.append(seg, ck[:, :, sl], cv[:, :, sl])
    q = data["q"].float().numpy()
    kc = data["cur_k"].float().numpy() if w.n_cur else None
    vc = data["cur_v"].float().numpy() if w.n_cur else None
    # calibrate: one row (the per-head dequantization of the history dominates) and 33 rows
    def timed(rows):
        t0 = time.perf_counter()
        oracle.attention(q, [seg], kc, vc, n_kv_heads=w.n_kv_heads, jensen=bool(w.jensen), rows=rows)
        return time.perf_counter() - t0
    t1 = timed([0])
    t33 = timed(list(range(0, min(w.n_q, 33))))
    per_row = max((t33 - t1) / 32.0, 1e-6)
    fixed = max(t1 - per_row, 0.0)
    n_rows = int(max(1, min(w.n_q, (target_s - fixed) / per_row)))
    stride = max(1, w.n_q // n_rows)
    rows = list(range(0, w.n_q, stride))
    t_attn = timed(rows)
    t_app = 0.0
    if w.n_cur:
        t0 = time.perf_counter()
        oracle.append(seg, kc, vc)
        t_app = time.perf_counter() - t0
    frac = len(rows) / w.n_q
    # whole-step estimate: the history dequantization once, the sampled rows scaled to all
    # rows, plus the full append
    t_rows = max(t_attn - fixed, 1e-9)
    t_step = fixed + t_rows / frac + t_app
    return {"value": round(step.flops() / t_step / 1e12, 6), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": "attention of every %d-th query row (%d of %d per head, all %d heads) over the full "
                      "%d-token history (%.1f s, of which %.1f s dequantizes the history once), rows scaled "
                      "to all %d; quantize-append of the %d-token chunk in full (%.1f s)"
                      % (stride, len(rows), w.n_q, w.n_q_heads, w.n_cache + w.n_cur, t_attn, fixed, w.n_q,
                         w.n_cur, t_app),
            "est_step_s": round(t_step, 2)}


def probe_hbm(mib=2048, reps=5):
    """Measured HBM bandwidth of this device, for context beside the published peak: a sum
    over a 2 GiB buffer (reads) and a copy of 1 GiB (reads + writes), best of a few runs,
    timed with events on the current stream. Buffers exceed the last-level cache."""
    n = (mib << 20) // 4
    x = torch.ones(n, dtype=torch.float32, device="cuda")
    y = torch.empty(n // 2, dtype=torch.float32, device="cuda")
    best_read = best_copy = float("inf")
    for _ in range(reps):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        e[0].record()
        x.sum()
        e[1].record()
        y.copy_(x[: n // 2])
        e[2].record()
        torch.cuda.synchronize()
        best_read = min(best_read, e[0].elapsed_time(e[1]))
        best_copy = min(best_copy, e[1].elapsed_time(e[2]))
    read_gbps = (n * 4) / (best_read * 1e-3) / 1e9
    copy_gbps = (n // 2 * 4 * 2) / (best_copy * 1e-3) / 1e9
    del x, y
    return {"read_gbps": round(read_gbps, 1), "copy_gbps": round(copy_gbps, 1), "buffer_mib": mib,
            "note": "torch sum (read) and copy (read + write), best of %d" % reps}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="video_chunk_int2_h12_d128", choices=sorted(workloads.WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-probe-hbm", action="store_true",
                    help="skip the HBM read/copy probe (its copies would mix into a counter run's copy calibration)")
    ap.add_argument("--copies", type=int, default=0, help="cache copies rotated per step (0: auto)")
    ap.add_argument("--probe-copy-mib", type=int, default=0,
                    help="after timing, run one plain device copy of this many MiB (the reference dispatch "
                         "for scaling FETCH_SIZE / WRITE_SIZE counters to bytes)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (--gpus %d requested)" % args.gpus,
              file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    kvq.lib()
    w = workloads.WORKLOADS[args.workload]
    if w.bits == 0:
        print("the WindowQuant workload is a parity case, not a bench line", file=sys.stderr)
        sys.exit(2)
    # decode caches can sit in the 256 MB last-level cache: rotate copies > 2x that size
    copies = args.copies
    if copies == 0:
        copies = 1 if w.n_cur else 4
    step = ChunkStep(w, n_copies=copies)
    log("cache built: %d tokens, %d K-groups per head, %d copies" % (step.base[0], step.base[1], copies))

    for _ in range(args.warmup):
        step.run()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step.run(evs[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps
    attn_ms = [e[0].elapsed_time(e[1]) for e in evs]
    app_ms = [e[1].elapsed_time(e[2]) for e in evs]
    attn_avg = float(np.mean(attn_ms))
    app_avg = float(np.mean(app_ms))

    flops = step.flops()
    kvb = step.kv_bytes()
    value = flops / (ms_step * 1e-3) / 1e12
    attn_tflops = flops / (attn_avg * 1e-3) / 1e12
    decode = w.n_cur == 0
    if decode:
        alg = kvb + step.qo_bytes()
        ach = alg / (attn_avg * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                "frac": round(ach / PEAK_HBM_GBPS, 4), "traffic": stored_traffic(w.name, "decode_kernel"),
                "kernel": "decode_kernel"}
    else:
        roof = {"bound": "mfma", "achieved": round(attn_tflops, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(attn_tflops / PEAK_BF16_TFLOPS, 4), "traffic": stored_traffic(w.name, "attention_kernel"),
                "kernel": "attention_kernel"}
    res = {
        "metric": METRIC, "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "n_q_heads": w.n_q_heads, "n_kv_heads": w.n_kv_heads,
                   "head_dim": w.head_dim, "cache_tokens": w.n_cache, "cur_tokens": w.n_cur, "queries": w.n_q,
                   "bits": w.bits, "k_group_tokens": w.k_group_tokens, "v_group_channels": w.v_group_channels,
                   "jensen": bool(w.jensen), "cache_copies": copies},
        "roofline": roof,
        "attention": {"ms": round(attn_avg, 4), "ms_p10": round(float(np.percentile(attn_ms, 10)), 4),
                      "ms_p90": round(float(np.percentile(attn_ms, 90)), 4), "tflops": round(attn_tflops, 2),
                      "kv_gbps": round(kvb / (attn_avg * 1e-3) / 1e9, 1),
                      "kv_bytes": kvb, "flops": flops},
        "append": {"ms": round(app_avg, 4), "bytes": step.append_bytes(),
                   "gbps": round(step.append_bytes() / (app_avg * 1e-3) / 1e9, 1) if step.append else None},
    }
    if not args.no_probe_hbm:
        res["probe_hbm"] = probe_hbm()
    if args.probe_copy_mib:
        n = args.probe_copy_mib << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log("copy probe: %d MiB read, %d MiB written" % (args.probe_copy_mib, args.probe_copy_mib))
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a sample ...")
        res["cpu_baseline"] = cpu_baseline(step)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
