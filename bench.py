"""Benchmark: fused INT2-KV chunk attention (TFLOP/s, effective KV GB/s vs MI355X peaks).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-extra]
                    [--no-cpu-baseline]

Default workload: the long-rollout chunk step -- batch 1, 40 heads, head_dim 128, an INT2
cache of 74,880 tokens (16 appends of one 4,680-token chunk of 3 latent frames, K groups of
128 tokens, V groups of 32 channels, keys drifting per frame) and an unquantized current
chunk of 4,680 tokens that is both the queries and the current keys/values. One step = the
fused attention with the Jensen correction, then the quantize-append of the current chunk
into the cache, back to back (the descriptor is rewound after each step, so every step does
identical work). Inputs are seeded synthetic tensors already resident in HBM when timing
starts.

One JSON line on stdout. ``value`` = attention FLOPs per step (4 * B * Hq * Nq * (N_cache +
N_cur) * d, the dense QK^T and PV products) / step time. ``roofline`` is the attention
kernel against the bf16 dense MFMA peak, its duration taken with HIP events recorded on
the stream the kernels run on. ``configs`` holds the same record for the video chunk step
and the two decode-shaped caches (INT2, INT4; rated in GB/s of algorithmic bytes against
HBM), each timed the same way. ``cpu_baseline`` times the CPU oracle on a bounded sample
of the headline workload; ``probe_hbm`` the library's streaming-read probe and a copy.
"""
import argparse
import dataclasses
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

    def __init__(self, w: workloads.Workload, n_copies: int = 1, fused: bool = True, k_group_channels: int = 0,
                 comp_rank: int = 0):
        self.w = w
        self.fused = fused   # the append in the attention's own call (append_dst) or after it
        self.kgc = k_group_channels   # per-token K groups of this many channels (0: per channel)
        self.comp_rank = comp_rank    # low-rank logit compensation of this rank (0: none)
        t0 = time.time()
        data = workloads.generate(w)
        log("generated inputs in %.1fs" % (time.time() - t0))
        self.data = data
        B, Hq, Hkv, d = w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim
        dt = workloads.DTYPES[w.dtype]
        self.bits = w.bits
        n_groups = w.n_appends * -(-w.append_tokens // w.k_group_tokens)
        extra = -(-w.n_cur // w.k_group_tokens) if w.n_cur else 0
        self.basis = None
        if comp_rank:
            # the caller's estimate of each KV head's dominant query subspace: the top right
            # singular vectors of the query rows that read it (setup, not timed)
            qh = data["q"].float().reshape(B, Hkv, Hq // Hkv, w.n_q, d).permute(1, 0, 2, 3, 4).reshape(Hkv, -1, d)
            vt = torch.linalg.svd(qh, full_matrices=False).Vh[:, :comp_rank, :]          # [Hkv][r][d]
            self.basis = vt.transpose(1, 2).contiguous().cuda()                            # [Hkv][d][r]
        self.segs = []
        for c in range(n_copies):
            seg = kvq.Segment(w.bits, dt, B, Hkv, d, w.n_cache + w.n_cur, k_group_tokens=w.k_group_tokens,
                              kgroup_capacity=n_groups + extra, k_group_channels=self.kgc, comp_basis=self.basis)
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
        if self.kgc:
            per_tok += 4 * (w.head_dim // self.kgc)   # K step/zero per (token, channel run)
            kmeta = 0
        else:
            kmeta = 4 * w.head_dim * w.n_appends * -(-w.append_tokens // w.k_group_tokens)
        if self.comp_rank:
            per_tok += 16                              # the token's compensation row
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
        kmeta = 4 * n * (w.head_dim // self.kgc) if self.kgc else 4 * w.head_dim * -(-n // w.k_group_tokens)
        wr = w.batch * w.n_kv_heads * (2 * n * w.head_dim * w.bits / 8 + 4 * n * (w.head_dim // 32) + kmeta
                                       + (16 * n if self.comp_rank else 0))
        return rd + wr

    def run(self, events=None):
        seg = self.segs[self.i % len(self.segs)]
        self.i += 1
        seg.reset(*self.base)
        if events is not None:
            events[0].record()
        fused = self.append and self.fused
        kvq.chunk_attention(self.q, [seg], self.k_cur, self.v_cur, jensen=self.w.jensen, out=self.out,
                            workspace=self.ws, append_to=seg if fused else None)
        if events is not None:
            events[1].record()
        if self.append and not fused:
            kvq.quantize_append(seg, self.k_cur, self.v_cur)
        if events is not None:
            events[2].record()


class WindowStep:
    """WindowQuant, one step: window scores, the FP16/INT4/INT2 assignment and the grouped
    layout's gather lists on the GPU; the three class token counts come back to size the
    appends (12 bytes); the three grouped segments rebuilt by gathered appends from the
    device lists; then the decode attention over them."""

    def __init__(self, w: workloads.Workload):
        self.w = w
        t0 = time.time()
        self.data = data = workloads.generate(w)
        log("generated inputs in %.1fs" % (time.time() - t0))
        self.k = data["cache_k"].cuda()            # [1][Hkv][N][d]
        self.v = data["cache_v"].cuda()
        self.text = data["text"].cuda()
        self.q = data["q"].cuda()
        self.asg = kvq.assign_windows(self.k, self.text, w.pct_fp16, w.pct_int4, window=w.window)
        self.n16, self.n4 = self.asg.n_fp16, self.asg.n_int4
        self.class_tokens = torch.empty(3, dtype=torch.int32, pin_memory=True)
        self.class_tokens.copy_(self.asg.class_tokens[0])
        dt = workloads.DTYPES[w.dtype]
        rows = self.asg.class_rows()
        self.segs = []
        self.tokens = {}
        for k, b in enumerate((16, 4, 2)):
            n_tok = int(self.class_tokens[k])
            self.tokens[b] = n_tok
            self.segs.append(kvq.Segment(b, dt, 1, w.n_kv_heads, w.head_dim, w.window * (rows[b][1] - rows[b][0]),
                                         k_group_tokens=w.window, kgroup_capacity=max(rows[b][1] - rows[b][0], 1)))
        self.out = torch.empty(self.q.shape, dtype=torch.float32, device="cuda")
        self.ws = None   # sized on the first run, once the segments hold tokens

    def attention_bytes(self) -> float:
        """The mixed cache (FP16 rows; INT4 / INT2 codes, V step/zero, K step/zero per window)
        and Q, O, each once."""
        w = self.w
        d, H = w.head_dim, w.n_kv_heads
        total = 2 * H * self.tokens[16] * d * 2
        for b in (4, 2):
            n = self.tokens[b]
            total += H * (n * (2 * d * b / 8 + 4 * (d // 32)) + 4 * d * -(-n // w.window))
        return total + w.n_q_heads * w.n_q * d * (2 + 4)

    def run(self, ev=None):
        w = self.w
        if ev is not None:
            ev[0].record()
        kvq.assign_windows(self.k, self.text, w.pct_fp16, w.pct_int4, window=w.window, out=self.asg)
        if ev is not None:
            ev[1].record()
        # the appends' token counts: the only host-side step (a 12-byte copy back)
        self.class_tokens.copy_(self.asg.class_tokens[0])
        if ev is not None:
            ev[2].record()
        for k, (seg, b) in enumerate(zip(self.segs, (16, 4, 2))):
            seg.reset()
            kvq.quantize_append(seg, self.k, self.v, n_new=int(self.class_tokens[k]),
                                src_groups=self.asg.class_list(b))
        if ev is not None:
            ev[3].record()
        if self.ws is None:
            need = kvq.attention_workspace_size(self.q, self.segs, 0, n_kv_heads=w.n_kv_heads, jensen=w.jensen)
            self.ws = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")
        kvq.chunk_attention(self.q, self.segs, n_kv_heads=w.n_kv_heads, jensen=w.jensen, out=self.out,
                            workspace=self.ws)
        if ev is not None:
            ev[4].record()


def window_cpu_baseline(step: WindowStep):
    """The oracle's whole WindowQuant step once, on the host: scores, assignment, the three
    gathered appends and the attention of every query row."""
    import oracle
    w = step.w
    threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or os.cpu_count()
    k = step.data["cache_k"].float().numpy()
    v = step.data["cache_v"].float().numpy()
    t0 = time.perf_counter()
    score = oracle.window_scores(k[0], step.data["text"].numpy(), w.window)
    n16, n4 = oracle.window_budget(w.n_windows, w.pct_fp16, w.pct_int4)
    bits, order = oracle.assign_windows(score, n16, n4)
    groups, class_tokens = oracle.window_groups(bits, order, w.n_cache, w.window)
    bounds = [0, n16, n16 + n4, w.n_windows]
    segs = []
    for k_, b in enumerate((16, 4, 2)):
        lst = groups[bounds[k_]:bounds[k_ + 1]]
        seg = oracle.new_segment(b, w.dtype, 1, w.n_kv_heads, w.head_dim, capacity=max(int(class_tokens[k_]), 1),
                                 k_group_tokens=w.window, kgroup_capacity=max(len(lst), 1))
        if len(lst):
            oracle.append(seg, k, v, groups=lst)
        segs.append(seg)
    oracle.attention(step.data["q"].float().numpy(), segs, n_kv_heads=w.n_kv_heads, jensen=int(w.jensen))
    t = time.perf_counter() - t0
    return {"value": round(t * 1e6, 1), "unit": "us", "cores": threads, "kind": "oracle", "host": host_cpu(),
            "sample": "the whole step once: window scores and assignment, the three gathered appends "
                      "(%d FP16 / %d INT4 / %d INT2 windows) and the attention of all %d query rows"
                      % (step.n16, step.n4, w.n_windows - step.n16 - step.n4, w.n_q_heads * w.n_q)}


def window_main(args, w: workloads.Workload) -> None:
    step = WindowStep(w)
    for _ in range(args.warmup):
        step.run()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        step.run(evs[i])
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / args.steps
    st = {k: [] for k in ("assign", "class_tokens_copy", "appends", "attention")}
    for e in evs:
        st["assign"].append(e[0].elapsed_time(e[1]) * 1e3)
        st["class_tokens_copy"].append(e[1].elapsed_time(e[2]) * 1e3)
        st["appends"].append(e[2].elapsed_time(e[3]) * 1e3)
        st["attention"].append(e[3].elapsed_time(e[4]) * 1e3)
    med = {k: float(np.median(v)) for k, v in st.items()}
    device_us = med["assign"] + med["appends"] + med["attention"]
    gbps = step.attention_bytes() / (med["attention"] * 1e-6) / 1e9
    res = {"metric": "WindowQuant decode step latency (window scores + FP16/INT4/INT2 assignment, grouped "
                     "appends, attention), device time",
           "value": round(device_us, 2), "unit": "us", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": round(wall * 1e3, 4), "higher_is_better": False, "scaling": "weak", "vs_baseline": None,
           "dtype": "f16", "data": "synthetic",
           "config": {"workload": w.name, "batch": w.batch, "n_q_heads": w.n_q_heads, "n_kv_heads": w.n_kv_heads,
                      "head_dim": w.head_dim, "cache_tokens": w.n_cache, "window": w.window,
                      "windows": w.n_windows, "fp16_int4_int2_windows": [step.n16, step.n4,
                                                                        w.n_windows - step.n16 - step.n4],
                      "jensen": int(w.jensen)},
           "stages_us": {k: round(v, 2) for k, v in med.items()},
           "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                        "frac": round(gbps / PEAK_HBM_GBPS, 4), "traffic": None, "kernel": "attention_kernel",
                        "note": "launch-bound: %.2f MB per attention launch is %.2f us at peak, so the "
                                "fraction says nothing about the kernel" % (
                                    step.attention_bytes() / 1e6, step.attention_bytes() / 8e6)}}
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = window_cpu_baseline(step)
    print(json.dumps(res), flush=True)


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
        oracle.attention(q, [seg], kc, vc, n_kv_heads=w.n_kv_heads, jensen=int(w.jensen), rows=rows)
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
            "host": host_cpu(),
            "sample": "attention of every %d-th query row (%d of %d per head, all %d heads) over the full "
                      "%d-token history (%.1f s, of which %.1f s dequantizes the history once), rows scaled "
                      "to all %d; quantize-append of the %d-token chunk in full (%.1f s)"
                      % (stride, len(rows), w.n_q, w.n_q_heads, w.n_cache + w.n_cur, t_attn, fixed, w.n_q,
                         w.n_cur, t_app),
            "est_step_s": round(t_step, 2)}


def probe_hbm(mib=2048, reps=5):
    """Measured HBM bandwidth of this device, for context beside the published peak: the
    library's streaming-read probe (kvq_probe_hbm_read: 16-byte loads, each byte read once)
    over a 2 GiB buffer, and a device copy of 1 GiB (reads + writes), best of a few runs,
    timed with events on the current stream. Both buffers exceed the 256 MB last-level
    cache several times over."""
    n = (mib << 20) // 4
    x = torch.ones(n, dtype=torch.float32, device="cuda")
    y = torch.empty(n // 2, dtype=torch.float32, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    best_read = best_copy = float("inf")
    for _ in range(reps):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        e[0].record()
        kvq.probe_hbm_read(x, sink)
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
            "note": "kvq_probe_hbm_read streaming read, and a torch device copy (read + write), best of %d" % reps}


def host_cpu():
    """The host CPU as /proc/cpuinfo names it (model name, and the family and model numbers
    that identify the generation where a virtual machine shows only a generic name), and the
    thread settings the oracle runs under."""
    info = {}
    try:
        for line in open("/proc/cpuinfo"):
            if ":" not in line:
                if info:
                    break   # the first processor's block is enough
                continue
            k, v = (x.strip() for x in line.split(":", 1))
            if k in ("model name", "vendor_id", "cpu family", "model") and k not in info:
                info[k] = v
    except OSError:
        pass
    return {"cpu_model": info.get("model name", "unknown"), "cpu_vendor": info.get("vendor_id"),
            "cpu_family": info.get("cpu family"), "cpu_model_number": info.get("model"),
            "nproc": os.cpu_count(), "OMP_NUM_THREADS": os.environ.get("OMP_NUM_THREADS")}


def time_steps(step: ChunkStep, steps: int, warmup: int):
    """Warm-ups, then exactly ``steps`` timed steps between device synchronizations: wall ms
    per step and, per step, the event times of the attention call and of the separate
    append (0 when the append is in the attention's call)."""
    for _ in range(warmup):
        step.run()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step.run(evs[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    return ((t1 - t0) * 1e3 / steps, [e[0].elapsed_time(e[1]) for e in evs],
            [e[1].elapsed_time(e[2]) for e in evs])


def measure_chunk(args, w: workloads.Workload, copies: int = 0):
    """The config's record: step time, value, and the roofline of the attention call as the
    step makes it; with a current chunk also the same step with the append as a launch of
    its own (``separate``: the attention alone, and the append alone)."""
    # decode caches can sit in the 256 MB last-level cache: rotate copies > 2x that size
    if copies == 0:
        copies = 1 if w.n_cur else 4
    step = ChunkStep(w, n_copies=copies, fused=args.append == "fused", k_group_channels=args.k_group_channels,
                     comp_rank=args.comp_rank)
    log("%s: cache built, %d tokens, %d K-groups per head, %d copies" % (w.name, step.base[0], step.base[1], copies))
    separate = None
    if w.n_cur:
        # the other way of running the append, first (its warm-ups also warm the fused step)
        step.fused = args.append != "fused"
        s_ms, s_attn, s_app = time_steps(step, args.steps, args.warmup)
        separate = {"mode": "fused" if step.fused else "separate", "ms_per_step": round(s_ms, 4),
                    "attention_ms": round(float(np.mean(s_attn)), 4), "append_ms": round(float(np.mean(s_app)), 4)}
        step.fused = args.append == "fused"
    ms_step, attn_ms, app_ms = time_steps(step, args.steps, args.warmup)
    attn_avg = float(np.mean(attn_ms))
    app_avg = float(np.mean(app_ms))
    # stored counters hold the workload's own mode: its Jensen form, the fused append, no extra K columns
    default_mode = (w.jensen == workloads.WORKLOADS[w.name].jensen and args.append == "fused"
                    and args.k_group_channels == 0 and args.comp_rank == 0)
    flops = step.flops()
    kvb = step.kv_bytes()
    attn_tflops = flops / (attn_avg * 1e-3) / 1e12
    decode = w.n_cur == 0
    if decode:
        alg = kvb + step.qo_bytes()
        ach = alg / (attn_avg * 1e-3) / 1e9
        kernel = "decode_kernel"
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                "frac": round(ach / PEAK_HBM_GBPS, 4),
                "traffic": stored_traffic(w.name, kernel) if default_mode else None, "kernel": kernel,
                "algorithmic_bytes": alg}
        value, unit = alg / (ms_step * 1e-3) / 1e9, "GB/s"
    else:
        kernel = "attention_kernel"
        roof = {"bound": "mfma", "achieved": round(attn_tflops, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(attn_tflops / PEAK_BF16_TFLOPS, 4),
                "traffic": stored_traffic(w.name, kernel) if default_mode else None, "kernel": kernel,
                "algorithmic_flops": flops}
        value, unit = flops / (ms_step * 1e-3) / 1e12, "TFLOP/s"
    rec = {
        "workload": w.name, "value": round(value, 3), "unit": unit, "ms_per_step": round(ms_step, 4),
        "config": {"workload": w.name, "batch": w.batch, "n_q_heads": w.n_q_heads, "n_kv_heads": w.n_kv_heads,
                   "head_dim": w.head_dim, "cache_tokens": w.n_cache, "cur_tokens": w.n_cur, "queries": w.n_q,
                   "bits": w.bits, "k_group_tokens": w.k_group_tokens, "v_group_channels": w.v_group_channels,
                   "jensen": int(w.jensen), "cache_copies": copies, "k_group_channels": args.k_group_channels,
                   "comp_rank": args.comp_rank},
        "roofline": roof,
        "attention": {"ms": round(attn_avg, 4), "ms_median": round(float(np.median(attn_ms)), 4),
                      "ms_p10": round(float(np.percentile(attn_ms, 10)), 4),
                      "ms_p90": round(float(np.percentile(attn_ms, 90)), 4), "tflops": round(attn_tflops, 2),
                      "kv_gbps": round(kvb / (attn_avg * 1e-3) / 1e9, 1), "kv_bytes": kvb, "flops": flops},
        "append": {"mode": args.append if step.append else None, "ms": round(app_avg, 4),
                   "ms_median": round(float(np.median(app_ms)), 4), "bytes": step.append_bytes()},
    }
    if separate is not None:
        rec["other_append_mode"] = separate
        app_sep = app_avg if args.append != "fused" else separate["append_ms"]
        rec["append"]["separate_launch_ms"] = round(app_sep, 4)
        rec["append"]["separate_launch_gbps"] = round(step.append_bytes() / (app_sep * 1e-3) / 1e9, 1)
        rec["append"]["separate_launch_hbm_frac"] = round(step.append_bytes() / (app_sep * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4)
    return rec, step


# the other configs reported beside the headline in the same line: the video chunk (the
# smaller chunk step) and the two decode-shaped caches (the GB/s half of the metric)
EXTRA_WORKLOADS = ("video_chunk_int2_h12_d128", "decode_gqa32x8_int2_32k", "decode_gqa32x8_int4_32k")


def trace_summary(path: str, keep: int) -> None:
    """Per-kernel durations from a rocprofv3 kernel-trace CSV (``--kernel-trace
    --output-format csv``) of a ``--no-extra --no-probe-hbm --no-cpu-baseline`` run: dispatch
    count, mean, median, min and max in microseconds over each kernel's last ``keep``
    dispatches. The selected append mode is timed last, so for the step's kernels these are
    the timed steps (warm-ups, cache building and the other mode's steps come before).
    Prints a markdown table."""
    import csv
    durs = {}
    with open(path) as f:
        for row in csv.DictReader(f):
            name = row.get("Kernel_Name", "")
            short = name.split("(")[0].split("<")[0].split("::")[-1] or name
            if "<" in name.split("(")[0]:
                short += "<" + name.split("(")[0].split("<", 1)[1]
            durs.setdefault(short, []).append((int(row["End_Timestamp"]) - int(row["Start_Timestamp"])) / 1e3)
    print("| kernel | dispatches (last %d kept) | mean us | median us | min us | max us |" % keep)
    print("|---|---|---|---|---|---|")
    for k, v in sorted(durs.items(), key=lambda kv: -sum(kv[1][-keep:])):
        v = v[-keep:]
        print("| `%s` | %d | %.1f | %.1f | %.1f | %.1f |" % (k, len(v), np.mean(v), np.median(v), min(v), max(v)))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="rollout_chunk_int2_h40_d128", choices=sorted(workloads.WORKLOADS))
    ap.add_argument("--no-extra", action="store_true",
                    help="time only --workload (a profiler run then sees one workload's dispatches)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-probe-hbm", action="store_true",
                    help="skip the HBM read/copy probe (its copies would mix into a counter run's copy calibration)")
    ap.add_argument("--copies", type=int, default=0, help="cache copies rotated per step (0: auto)")
    ap.add_argument("--append", choices=("fused", "separate"), default="fused",
                    help="the current chunk's quantize-append in the attention's own call (append_dst) or "
                         "as a launch of its own after it")
    ap.add_argument("--jensen", type=int, choices=(0, 1, 2, 3), default=None,
                    help="Jensen correction (0 off, 1 channel-weighted, 2 isotropic, 3 all orders); "
                         "default: the workload's")
    ap.add_argument("--k-group-channels", type=int, choices=(0, 32, 64, 128), default=0,
                    help="per-token K groups of this many channels (0: per-channel K groups over tokens)")
    ap.add_argument("--comp-rank", type=int, choices=range(0, 9), default=0, metavar="R",
                    help="low-rank logit compensation of rank R (0: none)")
    ap.add_argument("--probe-copy-mib", type=int, default=0,
                    help="after timing, run one plain device copy of this many MiB (the reference dispatch "
                         "for scaling FETCH_SIZE / WRITE_SIZE counters to bytes)")
    ap.add_argument("--trace-summary", metavar="CSV", default=None,
                    help="print per-kernel durations of a rocprofv3 kernel-trace CSV and exit (no GPU)")
    args = ap.parse_args()
    if args.trace_summary:
        trace_summary(args.trace_summary, args.steps)
        return
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
    if args.jensen is not None:
        w = dataclasses.replace(w, jensen=args.jensen)
    if w.bits == 0:
        window_main(args, w)
        return
    rec, step = measure_chunk(args, w, args.copies)
    res = {"metric": METRIC, "value": rec["value"], "unit": rec["unit"], "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": rec["ms_per_step"], "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic", "config": rec["config"],
           "roofline": rec["roofline"], "attention": rec["attention"], "append": rec["append"]}
    if "other_append_mode" in rec:
        res["other_append_mode"] = rec["other_append_mode"]
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a sample ...")
        res["cpu_baseline"] = cpu_baseline(step)
    del step
    torch.cuda.empty_cache()
    if not args.no_extra:
        res["configs"] = {}
        for name in EXTRA_WORKLOADS:
            if name == w.name:
                continue
            r, st = measure_chunk(args, workloads.WORKLOADS[name])
            del st
            torch.cuda.empty_cache()
            res["configs"][name] = {k: r[k] for k in ("value", "unit", "ms_per_step", "roofline", "attention",
                                                      "append", "other_append_mode") if k in r}
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
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
