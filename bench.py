"""Throughput of the layer-end KV selection path on one MI355X.

A step is one pass of the whole path over one layer of synthetic input that
is already resident in HBM, as the layer-major driver runs it: one
kvsel_layer_end call (two streaming passes over K, row statistics, max-pool,
exact top-B + window, K/V gather).  The metric is
prompt-KV tokens scored + selected + compacted per second per layer.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu]
  python bench.py --copy-calibration     # plain device copy, for counter scaling
  python bench.py --summarize-trace kernel_trace.csv --last N --title T --command C

Workloads (one JSON line each):
  qwen128k     one Qwen3-14B-shaped layer (40 q / 8 kv heads), 131072 tokens (default)
  llama8k      one Llama-3-8B-shaped layer, 8192-token prompt
  llama64k     the Llama shape at 65536 tokens, B = 4096 (first layer of the sweep)
  sweep64k     32 layers at 65536 tokens, budget 4096 -> 512, one layer resident
  qevict32k    16 x 32768-token caches, 256 decode queries, window tiers
  qevict-steps QEvict decode-time routing every 8 tokens: 16 x 32768-token caches,
               8 decode queries scored per step, INT2 backing store, 5 sinks,
               64 recent tokens, half the routed windows kept (30% full, 70% INT2)
  kara512      Kara decode-window compression: 64 sequences, Llama-3-8B shape,
               512-token window, 64-token buffer, r = 40%, gamma 8, alpha 32
  llama8k-adaptive / qwen128k-adaptive
               the same layers with a head-adaptive budget: Hkv*B picks per
               sequence over all KV heads, flattened output with head offsets
  qwen128k-stream / llama64k-stream
               the same layers through kvsel_layer_end_stream (the top-k kept
               during pass 2, no per-key score vector)

The timed region is the run's last GPU work, so the last steps x
dispatches_per_step dispatches of a kernel trace of the run are exactly it.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time
from typing import Optional

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import synth  # noqa: E402

HBM_PEAK_GBS = 8000.0           # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix cores, published
# Vector-ALU ceilings of the score passes from the chip's 1024 SIMDs at the
# 2.4 GHz peak clock and the issue cost of one wave64 instruction measured
# in a standalone probe: v_exp_f32 11 cycles, v_fma_f32 / v_add_f32 4.8.
N_SIMD, PEAK_CLOCK_HZ = 1024, 2.4e9
EXP_CYCLES, FMA_CYCLES = 11.0, 4.8
EXP_RATE = N_SIMD * 64 / EXP_CYCLES * PEAK_CLOCK_HZ          # exponentials per second
METRIC = "prompt-KV tokens scored+selected+compacted/sec per layer; % of HBM BW peak"
WORKLOADS = {
    "llama8k": (2, "llama3-8b-layer-8k"),
    "llama64k": (3, "llama3-8b-layer0-64k"),
    "qwen128k": (4, "qwen3-14b-layer-128k"),
    "sweep64k": (3, "llama3-8b-32-layer-sweep-64k"),
    "qevict32k": (5, "qevict-decode-tiers-16x32k"),
    "llama8k-adaptive": (2, "llama3-8b-layer-8k-head-adaptive"),
    "qwen128k-adaptive": (4, "qwen3-14b-layer-128k-head-adaptive"),
    "kara512": (0, "kara-decode-window-64x512"),
    "qevict-steps": (5, "qevict-routing-steps-16x32k-int2"),
    "qwen128k-stream": (4, "qwen3-14b-layer-128k-streaming-topk"),
    "llama64k-stream": (3, "llama3-8b-layer0-64k-streaming-topk"),
}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_SOURCES = ["score.hip", "select.hip", "compact.hip", "tiers.hip", "kara.hip", "qevict.hip",
                  "common.h", "select_util.h"]


def source_hash() -> str:
    """Hash of the kernel sources and the compiler flags they are built
    with; counter figures are only valid for it."""
    from attention_score_eviction_amd.build import FLAGS
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "attention_score_eviction_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    h.update(" ".join(FLAGS).encode())
    return h.hexdigest()[:16]


def algorithmic_bytes(spec: synth.LayerSpec) -> dict:
    """Bytes the path must move per layer (two K sweeps, the score vectors,
    the gather): per ABI call and the path's sum."""
    e = 2 if spec.dtype == "bf16" else 4
    H = spec.batch * spec.n_kv_heads
    S, W, D, n_keep = spec.seq_len, spec.obs_window, spec.head_dim, spec.n_keep
    k_sweep = H * S * D * e
    d = {
        # two K sweeps + raw score write + max-pool read of raw, write of pooled
        "kvsel_score": 2 * k_sweep + H * S * 4 + H * S * 4 + H * (S - W) * 4,
        # pooled read + index write; K and V rows read and written + index read
        "kvsel_select_compact": H * (S - W) * 4 + H * n_keep * 4
        + 2 * 2 * H * n_keep * D * e + H * n_keep * 4,
    }
    d["path"] = sum(d.values())
    return d


def tier_bytes(spec: synth.LayerSpec, n_full: int, n_quant: int, n_prom: int, win: int = 64) -> int:
    """Algorithmic bytes of kvsel_route_tiers: scores read; full-tier and
    int4-tier windows read; full rows, codes, metadata, promoted rows written."""
    H = spec.batch * spec.n_kv_heads
    S, D = spec.seq_len, spec.head_dim
    read = H * S * 4 + 2 * H * (n_full + n_quant) * win * D * 2 + 2 * H * n_prom * win * D // 2
    write = (2 * H * n_full * win * D * 2 + 2 * H * n_quant * win * D // 2
             + 2 * H * n_quant * D * 8 + 2 * H * n_prom * win * D * 2 + H * (S // win) * 5)
    return read + write


def cpu_baseline(spec: synth.LayerSpec, x: dict, budget_s: float = 12.0,
                 adaptive: bool = False, threads: Optional[int] = None) -> dict:
    """The oracle, as it stands, timed on this host on the same workload
    (on `threads` BLAS threads when given, else all of them).  Layers whose
    dense fp64 scoring is large run on a sample of KV heads (the oracle's work
    is the same for every head), scaled to the whole layer."""
    if threads is not None:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=threads):
            return cpu_baseline(spec, x, budget_s, adaptive)
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    S, W, G, Hkv = spec.seq_len, spec.obs_window, spec.group, spec.n_kv_heads
    heads = Hkv if adaptive or spec.n_q_heads * W * S <= 64 * 1024 * 1024 else 1
    q64 = synth.to_f64(x["q"][:, :heads * G], spec.dtype)
    k64 = synth.to_f64(x["k"][:, :heads], spec.dtype)
    ks, vs = x["k"][:, :heads], x["v"][:, :heads]
    reps, t0 = 0, time.perf_counter()
    while True:
        if adaptive:
            s = oracle.head_scores(q64, k64, causal=bool(spec.causal))
            p = oracle.max_pool(s, spec.pool_kernel, spec.n_sink, S - W)
            idx, off = oracle.select_head_adaptive(p, heads * spec.budget, spec.n_sink, W)
            oracle.compact_flat(ks, idx, off)
            oracle.compact_flat(vs, idx, off)
        else:
            oracle.layer_end_compress(q64, k64, vs, budget=spec.budget, window=W,
                                      pool_kernel=spec.pool_kernel, n_sink=spec.n_sink,
                                      causal=bool(spec.causal), k_store=ks, v_store=vs)
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s or reps >= 1000:
            break
    per_layer_s = el / reps * (Hkv / heads)
    what = (f"{reps} full layer(s)" if heads == Hkv else
            f"KV head 0 of the layer ({G} query heads x {W} queries x {S} keys: score, pool, "
            f"select, gather) {reps} time(s), scaled x{Hkv} to the layer's {Hkv} KV heads")
    return {"value": round(spec.batch * S / per_layer_s, 1), "unit": "tokens/s",
            "cores": threads, "kind": "oracle",
            "sample": f"{what} of the same workload through the fp64 oracle "
                      f"({el:.1f} s, {threads} BLAS threads)"}


def traffic_for(workload: str, kernel: str):
    """Measured HBM bytes per launch of `kernel` from the committed counter
    summary, if it was taken with the current kernel sources; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except OSError:
        return None
    if t.get("source_hash") != source_hash():
        return None
    return t.get("per_kernel_bytes", {}).get(workload, {}).get(kernel)


def event_time_us(torch, stream, fn, reps: int) -> float:
    """Average time of fn() over reps calls, HIP events on the launch stream."""
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(reps):
        fn()
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps * 1e3


def kernel_times(kvsel, torch, fn, steps: int, prefix: str = "*") -> dict:
    """Per-kernel HIP-event timing inside the library (kvsel_timing_start):
    {kernel: (average us per launch, launches per step)} over `steps` calls
    of fn()."""
    kvsel.timing_read()
    kvsel.timing_start(prefix)
    try:
        for _ in range(steps):
            fn()
        torch.cuda.synchronize()
    finally:
        kvsel.timing_start(None)
    return {name: (ms * 1e3 / n, n / steps) for name, (ms, n) in kvsel.timing_read().items()}


def kernel_work(spec: synth.LayerSpec, kernel: str, n_keep: int) -> tuple:
    """Algorithmic (bytes, flops) of one launch of a kernel of the prompt path:
    what the kernel's own step of the method must move and compute (two K
    sweeps for the two score passes; score vectors; the gather)."""
    e = 2 if spec.dtype == "bf16" else 4
    H = spec.batch * spec.n_kv_heads
    S, W, D = spec.seq_len, spec.obs_window, spec.head_dim
    GW = spec.group * W
    sweep, flops = H * S * D * e, 2 * H * GW * D * S
    if kernel == "score_keys_lds32":
        # both passes in one launch: keys and queries read once, the score
        # vector written, the products of both passes
        return sweep + H * GW * D * e + H * S * 4, 2 * flops
    if kernel.startswith("score_pass1"):
        return sweep, flops
    if kernel.startswith("score_pass2"):
        return sweep + H * S * 4, flops
    if kernel in ("maxpool_kernel", "sel_pool_hist"):
        return 2 * H * S * 4, 0
    if kernel in ("select_kernel", "sel_emit"):
        return H * (S - W) * 4 + H * n_keep * 4, 0
    if kernel.startswith("sel_hist") or kernel == "sel_cand":
        return H * (S - W) * 4, 0
    if kernel == "compact_kernel":
        return 4 * H * n_keep * D * e + H * n_keep * 4, 0
    return 0, 0


def binding_roofline(spec: synth.LayerSpec, path_bytes: int, step_us: float) -> dict:
    """The step against each ceiling: HBM (algorithmic bytes), the matrix
    cores (both passes' flops), the exponentials alone (2 per logit), and the
    vector ALU issue of the passes' per-logit arithmetic (pass 1: FMA, exp,
    add and half a max3; pass 2: FMA, exp, add); the binding one is the
    largest, and frac is it over the measured step."""
    logits = spec.batch * spec.n_q_heads * spec.obs_window * spec.seq_len
    t = {
        "hbm": path_bytes / (HBM_PEAK_GBS * 1e9),
        "mfma": 2 * 2 * logits * spec.head_dim / (MFMA_BF16_PEAK_TFLOPS * 1e12),
        "exp": 2 * logits / EXP_RATE,
        "valu": logits * (2 * (2 * FMA_CYCLES + EXP_CYCLES) + FMA_CYCLES / 2) / 64
        / N_SIMD / PEAK_CLOCK_HZ,
    }
    bound = max(t, key=t.get)
    out = {f"t_{k}_us": round(v * 1e6, 2) for k, v in t.items()}
    out.update({"bound": bound, "frac": round(t[bound] / (step_us * 1e-6), 4)})
    return out


def roofline_entry(kernel: str, us: float, nbytes: int, flops: int, traffic) -> dict:
    """Roofline of one kernel launch: the binding bound is the larger of its
    HBM time and its bf16 matrix-core time at MI355X's published peaks."""
    t_hbm = nbytes / (HBM_PEAK_GBS * 1e9)
    t_mfma = flops / (MFMA_BF16_PEAK_TFLOPS * 1e12)
    if t_mfma > t_hbm:
        ach = flops / (us * 1e-6) / 1e12
        ent = {"bound": "mfma", "achieved": round(ach, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
               "unit": "TFLOP/s", "frac": round(ach / MFMA_BF16_PEAK_TFLOPS, 4)}
    else:
        ach = nbytes / (us * 1e-6) / 1e9
        ent = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS,
               "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4)}
    ent["traffic"] = traffic
    ent.update({"kernel": kernel, "us_per_launch": round(us, 2),
                "algorithmic_bytes_per_launch": nbytes, "algorithmic_flops_per_launch": flops,
                "hbm_frac": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                "mfma_frac": round(flops / (us * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)})
    return ent


def copy_bandwidth_gbs(torch, stream, nbytes: int = 1 << 30, reps: int = 20) -> float:
    """A plain device-to-device copy on the launch stream: the achievable
    read + write bandwidth of this GPU (a STREAM-copy style reference)."""
    a = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0").fill_(1)
    b = torch.empty_like(a)
    us = event_time_us(torch, stream, lambda: b.copy_(a), reps)
    del a, b
    return 2 * nbytes / (us * 1e-6) / 1e9


class Layer:
    """One resident layer on the layer-major driver, with its preallocated
    compact cache; a step is the layer-end step as the driver runs it
    (kvsel_layer_end; kvsel_layer_end_adaptive into a flattened cache for the
    head-adaptive variant).  The per-call breakdown times the composed calls
    (kvsel_score, then kvsel_select_compact, or kvsel_select_adaptive and
    kvsel_compact_flat)."""

    def __init__(self, kvsel, torch, spec, x, adaptive=False, streaming=False):
        from attention_score_eviction_amd.driver import LayerMajorDriver
        self.kvsel, self.torch, self.spec, self.adaptive = kvsel, torch, spec, adaptive
        self.streaming = streaming
        dt = torch.bfloat16 if spec.dtype == "bf16" else torch.float32
        self.drv = LayerMajorDriver(spec.batch, spec.n_q_heads, spec.n_kv_heads, spec.head_dim,
                                    spec.seq_len, spec.obs_window, spec.pool_kernel,
                                    max_budget=spec.budget, n_sink=spec.n_sink, dtype=dt)
        self.load(x)
        self.set_budget(spec.budget)

    def load(self, x):
        """Overwrite the resident layer in place (the single active buffer)."""
        torch = self.torch
        if self.spec.dtype == "bf16":
            t = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)  # noqa: E731
        else:
            t = torch.from_numpy
        self.drv.load(t(x["q"]), t(x["k"]), t(x["v"]))

    def set_budget(self, budget):
        torch, kvsel, d = self.torch, self.kvsel, self.drv
        self.budget = budget
        self.cache = self.drv.new_cache(budget)
        # separate scratch for the composed calls (kvsel_score, then the
        # select), timed alone for the per-call breakdown
        self.score_ws = torch.empty(max(kvsel.score_workspace_bytes(d.desc), 1),
                                    dtype=torch.uint8, device=d.k.device)
        self.select_ws = torch.empty(max(kvsel.select_workspace_bytes(d.desc, budget), 1),
                                     dtype=torch.uint8, device=d.k.device)
        if self.streaming:
            nb = kvsel.layer_end_stream_workspace_bytes(d.desc, budget, d.pool_kernel)
            self.stream_ws = torch.empty(max(nb, 1), dtype=torch.uint8, device=d.k.device)
        if self.adaptive:
            Bt, Hkv = self.spec.batch, self.spec.n_kv_heads
            n_keep = Hkv * (budget + self.spec.n_sink + self.spec.obs_window)
            dev = d.k.device
            self.idx = torch.empty((Bt, n_keep), dtype=torch.int32, device=dev)
            self.head_off = torch.empty((Bt, Hkv + 1), dtype=torch.int32, device=dev)
            self.k_hat = torch.empty((Bt, n_keep, self.spec.head_dim), dtype=d.k.dtype,
                                     device=dev)
            self.v_hat = torch.empty_like(self.k_hat)
            nb = kvsel.select_adaptive_workspace_bytes(d.desc, Hkv * budget)
            self.sel_ws = torch.empty(max(nb, 1), dtype=torch.uint8, device=dev)
            self.flat = self.drv.new_flat_cache(Hkv * budget)

    def score(self, stream):
        d = self.drv
        self.kvsel.score(d.q, d.k, pool_kernel=d.pool_kernel, n_sink=d.n_sink, pooled=d.pooled,
                         raw=d.raw, workspace=self.score_ws, stream=stream)

    def select_compact(self, stream):
        d, s = self.drv, self.spec
        if self.adaptive:
            self.kvsel.select_adaptive(
                d.pooled, s.n_kv_heads * self.budget, obs_window=s.obs_window,
                n_q_heads=s.n_q_heads, head_dim=s.head_dim, n_sink=s.n_sink, idx=self.idx,
                head_off=self.head_off, dtype=d.k.dtype, workspace=self.sel_ws, stream=stream)
            self.kvsel.compact_flat(d.k, d.v, self.idx, self.head_off, k_out=self.k_hat,
                                    v_out=self.v_hat, stream=stream)
            return
        c = self.cache
        self.kvsel.select_compact(d.pooled, d.k, d.v, c.budget, obs_window=s.obs_window,
                                  n_q_heads=s.n_q_heads, n_sink=s.n_sink, idx=c.idx,
                                  k_out=c.k_hat, v_out=c.v_hat, workspace=self.select_ws,
                                  stream=stream)

    def step(self, stream):
        if self.adaptive:
            self.drv.layer_end_adaptive(self.flat, stream=stream)
        elif self.streaming:
            d, c = self.drv, self.cache
            self.kvsel.layer_end_stream(d.q, d.k, d.v, budget=c.budget, pool_kernel=d.pool_kernel,
                                        n_sink=d.n_sink, idx=c.idx, k_out=c.k_hat,
                                        v_out=c.v_hat, workspace=self.stream_ws, stream=stream)
        else:
            self.drv.layer_end(self.cache, stream=stream)


def copy_calibration(steps: int) -> int:
    """A plain device-to-device copy of a known size, so that a counter run
    over it gives the scale from FETCH_SIZE / WRITE_SIZE readings to bytes."""
    import torch
    n = 256 * 1024 * 1024
    a = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    b = torch.empty_like(a)
    for _ in range(steps):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_each_way": n, "copies": steps}), flush=True)
    return 0


def short_kernel_name(n: str) -> str:
    """A profiler's kernel name reduced to the library's base name:
    'void ns::(anonymous namespace)::score_pass1_32<128, 10, 8>(args)' ->
    'score_pass1_32'."""
    n = re.sub(r"^void ", "", n.strip())
    if n.endswith(")"):                      # drop the parameter list
        depth = 0
        for i in range(len(n) - 1, -1, -1):
            depth += {")": 1, "(": -1}.get(n[i], 0)
            if depth == 0:
                n = n[:i]
                break
    n = n.split("<")[0]                      # drop template arguments
    return n.split("::")[-1].strip()


def _counter_means(path: str, counter: str) -> dict:
    """Mean per-dispatch value of `counter` for each kernel (base name) in a
    rocprofv3 counter_collection.csv."""
    import csv
    acc = {}
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        k = short_kernel_name(r["Kernel_Name"])
        acc.setdefault(k, {})
        acc[k].setdefault(r["Dispatch_Id"], 0.0)
        acc[k][r["Dispatch_Id"]] += float(r["Counter_Value"])
    return {k: sum(v.values()) / len(v) for k, v in acc.items()}


def ingest_counters(workload: str, fetch_csv: str, write_csv: str, cal_fetch_csv: str,
                    cal_write_csv: str) -> int:
    """Turn FETCH_SIZE / WRITE_SIZE runs of this bench (and of the copy
    calibration) into measured HBM bytes per kernel launch, stored with the
    hash of the kernel sources in profiles/traffic.json."""
    cal_bytes = 256 * 1024 * 1024
    cf = max(_counter_means(cal_fetch_csv, "FETCH_SIZE").values())
    cw = max(_counter_means(cal_write_csv, "WRITE_SIZE").values())
    f_scale, w_scale = cal_bytes / cf, cal_bytes / cw
    fetch = _counter_means(fetch_csv, "FETCH_SIZE")
    write = _counter_means(write_csv, "WRITE_SIZE")
    per_kernel = {k: int(round(fetch.get(k, 0.0) * f_scale + write.get(k, 0.0) * w_scale))
                  for k in set(fetch) | set(write)}
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except OSError:
        t = {}
    if t.get("source_hash") != source_hash():
        t = {"per_kernel_bytes": {}}
    t.setdefault("per_kernel_bytes", {})
    t["source_hash"] = source_hash()
    t["scale"] = {"fetch_bytes_per_unit": f_scale, "write_bytes_per_unit": w_scale,
                  "calibration": "bench.py --copy-calibration (256 MiB device copy)"}
    t["per_kernel_bytes"][workload] = per_kernel
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(t, f, indent=1, sort_keys=True)
    print(json.dumps({"workload": workload, "per_kernel_bytes": per_kernel}))
    return 0


def _trace_rows(path: str) -> list:
    """(start, end, kernel base name) of every dispatch in a rocprofv3 kernel
    trace (kernel_trace.csv, or a results .db), in start order."""
    rows = []
    if path.endswith(".csv"):
        import csv
        for r in csv.DictReader(open(path)):
            rows.append((int(r["Start_Timestamp"]), int(r["End_Timestamp"]),
                         short_kernel_name(r["Kernel_Name"])))
    else:
        import sqlite3
        con = sqlite3.connect(path)
        cols = [c[1] for c in con.execute("pragma table_info(kernels)")]
        st = "start" if "start" in cols else "start_timestamp"
        en = "end" if "end" in cols else "end_timestamp"
        for a, b, n in con.execute(f"select {st}, {en}, name from kernels"):
            rows.append((int(a), int(b), short_kernel_name(n)))
    rows.sort()
    return rows


def summarize_trace(path: str, last: int, title: str, command: str) -> int:
    """Markdown summary of the last `last` dispatches of a kernel trace (the
    timed region of a bench run: it is the run's last GPU work), per kernel:
    launches, mean / median / min duration and share, plus the sum of the
    per-step medians."""
    import statistics
    rows = _trace_rows(path)
    if last <= 0 or last > len(rows):
        print(f"trace has {len(rows)} dispatches, asked for the last {last}", file=sys.stderr)
        return 1
    sel = rows[-last:]
    per = {}
    for a, b, n in sel:
        per.setdefault(n, []).append((b - a) / 1e3)
    tot = sum(sum(v) for v in per.values())
    span_us = (sel[-1][1] - sel[0][0]) / 1e3
    out = [f"# rocprofv3 kernel trace: {title}", "", "Command (from the repository root on "
           "the GPU host):", "", "```", command, "```", "",
           f"The last {last} dispatches of the run: the bench's timed region (its last GPU "
           f"work), {span_us:.1f} us from the first start to the last end.  Microseconds.", "",
           "| kernel | launches | mean us | median us | min us | share |",
           "|---|---|---|---|---|---|"]
    steps = None
    for n, v in sorted(per.items(), key=lambda kv: -sum(kv[1])):
        out.append(f"| {n} | {len(v)} | {statistics.mean(v):.2f} | {statistics.median(v):.2f} "
                   f"| {min(v):.2f} | {100 * sum(v) / tot:.1f}% |")
        steps = len(v) if steps is None else min(steps, len(v))
    med_sum = sum(statistics.median(v) * len(v) / steps for v in per.values()) if steps else 0
    out += ["", f"Sum of per-kernel medians per step ({steps} steps): {med_sum:.2f} us; "
                f"mean time per step from first start to last end: {span_us / steps:.2f} us."]
    print("\n".join(out))
    return 0


N_XCD, N_SIMD = 8, 1024     # MI355X: 8 XCDs, 256 CUs x 4 SIMDs


def summarize_counters(paths: list, kernels: str, title: str, command: str) -> int:
    """Markdown table of SQ/GRBM counters per kernel from rocprofv3 --pmc
    runs (one counter_collection.csv per pass), mean per dispatch, with the
    derived issue shares:

    - cycles: GRBM_GUI_ACTIVE / 8 (the counter sums the 8 XCDs);
    - MFMA busy: SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x cycles);
    - VALU busy: 4 x SQ_ACTIVE_INST_VALU / (1024 x cycles) (the counter is in
      quad-cycles, summed over waves; one wave issues VALU on a SIMD at a time);
    - co-issue: SQ_VALU_MFMA_COEXEC_CYCLES / SQ_VALU_MFMA_BUSY_CYCLES;
    - idle: the share of SIMD cycles with neither unit busy."""
    want = [k for k in kernels.split(",") if k]
    means = {}
    names = []
    for p in paths:
        import csv
        acc = {}
        for r in csv.DictReader(open(p)):
            k = short_kernel_name(r["Kernel_Name"])
            if want and k not in want:
                continue
            c = r["Counter_Name"]
            if c not in names:
                names.append(c)
            acc.setdefault((k, c), {}).setdefault(r["Dispatch_Id"], 0.0)
            acc[(k, c)][r["Dispatch_Id"]] += float(r["Counter_Value"])
        for key, v in acc.items():
            means[key] = (sum(v.values()) / len(v), len(v))
    ks = want or sorted({k for k, _ in means})
    out = [f"# rocprofv3 counters: {title}", "", "Commands (from the repository root on the "
           "GPU host; one --pmc pass each):", "", "```", command, "```", "",
           "Mean per dispatch over every dispatch of the kernel in the run.", "",
           "| counter | " + " | ".join(ks) + " |", "|---" * (len(ks) + 1) + "|"]
    for c in names:
        cells = []
        for k in ks:
            m = means.get((k, c))
            cells.append("—" if m is None else f"{m[0]:,.0f}")
        out.append(f"| {c} | " + " | ".join(cells) + " |")
    out += ["", "Derived (MI355X: 8 XCDs, 1024 SIMDs):", "",
            "| | " + " | ".join(ks) + " |", "|---" * (len(ks) + 1) + "|"]

    def val(k, c):
        m = means.get((k, c))
        return None if m is None else m[0]
    rows = {"cycles per XCD": [], "MFMA busy": [], "VALU busy": [],
            "VALU co-issued during MFMA": [], "neither busy": [],
            "VALU instructions per MFMA": [], "transcendentals per MFMA": [],
            "LDS instructions per MFMA": []}
    for k in ks:
        cyc = val(k, "GRBM_GUI_ACTIVE")
        cyc = cyc / N_XCD if cyc else None
        mf, va, co = (val(k, "SQ_VALU_MFMA_BUSY_CYCLES"), val(k, "SQ_ACTIVE_INST_VALU"),
                      val(k, "SQ_VALU_MFMA_COEXEC_CYCLES"))
        nm, nv, nt, nl = (val(k, "SQ_INSTS_MFMA"), val(k, "SQ_INSTS_VALU"),
                          val(k, "SQ_INSTS_VALU_TRANS_F32"), val(k, "SQ_INSTS_LDS"))
        f = lambda x: "—" if x is None else f"{100 * x:.0f}%"     # noqa: E731
        r = lambda a, b: "—" if a is None or not b else f"{a / b:.2f}"   # noqa: E731
        mfb = mf / (N_SIMD * cyc) if mf is not None and cyc else None
        vab = 4 * va / (N_SIMD * cyc) if va is not None and cyc else None
        cob = co / mf if co is not None and mf else None
        idle = (1 - mfb - vab + cob * mfb) if None not in (mfb, vab, cob) else None
        rows["cycles per XCD"].append("—" if cyc is None else f"{cyc:,.0f}")
        rows["MFMA busy"].append(f(mfb))
        rows["VALU busy"].append(f(vab))
        rows["VALU co-issued during MFMA"].append(f(cob))
        rows["neither busy"].append(f(idle))
        rows["VALU instructions per MFMA"].append(r(nv, nm))
        rows["transcendentals per MFMA"].append(r(nt, nm))
        rows["LDS instructions per MFMA"].append(r(nl, nm))
    for n, cells in rows.items():
        out.append(f"| {n} | " + " | ".join(cells) + " |")
    print("\n".join(out))
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="qwen128k", choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--graph", action="store_true",
                    help="also time the step captured in a HIP graph and replayed")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--ingest-counters", nargs=4,
                    metavar=("FETCH_CSV", "WRITE_CSV", "CAL_FETCH_CSV", "CAL_WRITE_CSV"),
                    help="record measured traffic for --workload from rocprofv3 csv files")
    ap.add_argument("--summarize-trace", metavar="TRACE",
                    help="markdown summary of the last --last dispatches of a kernel trace")
    ap.add_argument("--summarize-counters", nargs="+", metavar="CSV",
                    help="markdown counter table from rocprofv3 --pmc csv files")
    ap.add_argument("--kernels", default="", help="comma-separated kernel base names")
    ap.add_argument("--last", type=int, default=0)
    ap.add_argument("--title", default="")
    ap.add_argument("--command", default="")
    args = ap.parse_args()
    if args.ingest_counters:
        return ingest_counters(args.workload, *args.ingest_counters)
    if args.summarize_trace:
        return summarize_trace(args.summarize_trace, args.last, args.title, args.command)
    if args.summarize_counters:
        return summarize_counters(args.summarize_counters, args.kernels, args.title, args.command)
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(the work shards by KV head with no exchange); run with --gpus 1", file=sys.stderr)
        return 2
    if args.copy_calibration:
        return copy_calibration(max(args.steps, 1))

    import torch
    import attention_score_eviction_amd as kvsel

    cid, wname = WORKLOADS[args.workload]
    if args.workload == "kara512":
        return bench_kara(args, kvsel, torch, wname)
    spec = synth.config(cid) if cid else None
    if args.workload == "qevict-steps":
        return bench_qevict_steps(args, kvsel, torch, spec, wname)
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    if args.workload == "qevict32k":
        return bench_tiers(args, kvsel, torch, spec, wname, dev, stream)
    x = synth.make_layer(spec, cid)
    adaptive = args.workload.endswith("-adaptive")
    streaming = args.workload.endswith("-stream")
    L = Layer(kvsel, torch, spec, x, adaptive=adaptive, streaming=streaming)
    if args.workload == "sweep64k":
        return bench_sweep(args, kvsel, torch, spec, wname, L, stream)

    copy_gbs = copy_bandwidth_gbs(torch, stream)
    for _ in range(args.warmup):
        L.step(stream)
    torch.cuda.synchronize()
    # per-call breakdown (HIP events around each ABI call), then per kernel
    reps = max(args.steps // 2, 20)
    sel_name = "kvsel_select_adaptive+compact_flat" if adaptive else "kvsel_select_compact"
    us_call = {"kvsel_score": event_time_us(torch, stream, lambda: L.score(stream), reps),
               sel_name: event_time_us(torch, stream, lambda: L.select_compact(stream), reps)}
    if streaming:
        us_call["kvsel_layer_end_stream"] = event_time_us(torch, stream, lambda: L.step(stream),
                                                          reps)
        us_call["workspace_bytes"] = {"kvsel_layer_end_stream": L.stream_ws.numel(),
                                      "kvsel_layer_end": L.drv.ws.numel()}
    else:
        name = "kvsel_layer_end_adaptive" if adaptive else "kvsel_layer_end"
        us_call[name] = event_time_us(torch, stream, lambda: L.step(stream), reps)
    if args.graph:
        # the step captured once in a HIP graph and replayed (host launch cost
        # removed; the same kernels on the same buffers)
        torch.cuda.synchronize()
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            L.step(None)
        stream.wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            L.step(None)
        torch.cuda.synchronize()
        us_call["step_graph_replay"] = event_time_us(torch, stream, g.replay, reps)
    kt = kernel_times(kvsel, torch, lambda: L.step(stream), reps)
    dispatches = sum(n for _, n in kt.values())
    dom = max(kt, key=lambda k: kt[k][0] * kt[k][1])
    # timed region: the last GPU work of the run; the dominant kernel's
    # launches are bracketed by HIP events on the launch stream
    kvsel.timing_read()
    kvsel.timing_start(dom)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        L.step(stream)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kvsel.timing_start(None)
    ms_step = ev0.elapsed_time(ev1) / args.steps
    dom_ms, dom_n = kvsel.timing_read()[dom]
    dom_us = dom_ms * 1e3 / dom_n

    Bt, S = spec.batch, spec.seq_len
    n_keep = spec.n_keep
    ab = algorithmic_bytes(spec)
    value = Bt * S / (ms_step * 1e-3)
    path_gbs = ab["path"] / (ms_step * 1e-3) / 1e9
    nbytes, flops = kernel_work(spec, dom, n_keep)
    score_flops = 2 * 2 * Bt * spec.n_q_heads * spec.obs_window * spec.head_dim * S
    t_score_us = sum(us * n for k, (us, n) in kt.items()
                     if k.startswith("score_") or k == "maxpool_kernel")
    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if spec.dtype == "bf16" else "f32", "data": "synthetic",
        "config": {"workload": wname, "batch": Bt, "seq_len": S, "n_q_heads": spec.n_q_heads,
                   "n_kv_heads": spec.n_kv_heads, "head_dim": spec.head_dim,
                   "obs_window": spec.obs_window, "pool_kernel": spec.pool_kernel,
                   "budget": (f"{spec.n_kv_heads * spec.budget} per sequence over all KV heads"
                              if adaptive else spec.budget), "parallelism": "none"},
        "path_hbm_frac": round(path_gbs / HBM_PEAK_GBS, 4),
        "path_copy_frac": round(path_gbs / copy_gbs, 4),
        "copy_gbs": round(copy_gbs, 1),
        "path_algorithmic_bytes": ab["path"],
        "score_mfma_util": round(score_flops / (t_score_us * 1e-6) / 1e12
                                 / MFMA_BF16_PEAK_TFLOPS, 4),
        "binding_roofline": binding_roofline(spec, ab["path"], ms_step * 1e3),
        "us_per_call": {k: (round(v, 2) if isinstance(v, float) else v)
                        for k, v in us_call.items()},
        "us_per_kernel": {k: round(us, 2) for k, (us, n) in
                          sorted(kt.items(), key=lambda kv: -kv[1][0] * kv[1][1])},
        "dispatches_per_step": int(round(dispatches)),
        "wall_s": round(wall, 3),
        "roofline": roofline_entry(dom, dom_us, nbytes, flops, traffic_for(args.workload, dom)),
    }
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(spec, x, adaptive=adaptive)
        if S <= 8192:
            # short layers: the oracle on one host thread as well
            out["cpu_baseline_1thread"] = cpu_baseline(spec, x, adaptive=adaptive, threads=1)
    print(json.dumps(out), flush=True)
    return 0


def bench_sweep(args, kvsel, torch, spec, wname, L, stream) -> int:
    """TideKV Algorithm 1 over 32 layers with the layer-major driver: one
    resident full-prompt layer buffer refilled per layer, each layer's
    compact K/V and positions committed to the driver's per-layer store."""
    from attention_score_eviction_amd.driver import linear_budgets
    n_layers = 32
    budgets = linear_budgets(n_layers, 4096, 512)
    drv = L.drv
    per_layer_us = []
    reps = max(1, args.steps // 10)
    torch.cuda.reset_peak_memory_stats()
    for layer in range(n_layers):
        if layer > 0:
            L.load(synth.make_layer(spec, 3, layer))
        cache = drv.new_cache(budgets[layer])
        for _ in range(max(1, args.warmup // 10)):
            drv.layer_end(cache, stream=stream)
        torch.cuda.synchronize()
        per_layer_us.append(event_time_us(torch, stream,
                                          lambda: drv.layer_end(cache, stream=stream), reps))
        drv.store.append(cache)     # the layer-end commit
        print(f"layer {layer} budget {budgets[layer]}: {per_layer_us[-1]:.1f} us",
              file=sys.stderr, flush=True)
    mean_us = sum(per_layer_us) / n_layers
    S = spec.seq_len
    out = {
        "metric": METRIC, "value": round(spec.batch * S / (mean_us * 1e-6), 1),
        "unit": "tokens/s", "n_gpus": 1, "steps": reps * n_layers, "warmup": args.warmup,
        "ms_per_step": round(mean_us * 1e-3, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": wname, "layers": n_layers, "seq_len": S,
                   "n_q_heads": spec.n_q_heads, "n_kv_heads": spec.n_kv_heads,
                   "head_dim": spec.head_dim, "obs_window": spec.obs_window,
                   "budget_first": budgets[0], "budget_last": budgets[-1],
                   "parallelism": "none"},
        "per_layer_us_mean": round(mean_us, 2), "per_layer_us_max": round(max(per_layer_us), 2),
        "active_layer_bytes": drv.active_bytes,
        "compact_store_bytes": drv.store_bytes,
        "scratch_bytes": drv.scratch_bytes,
        "peak_allocated_bytes": torch.cuda.max_memory_allocated(),
    }
    print(json.dumps(out), flush=True)
    return 0


def bench_tiers(args, kvsel, torch, spec, wname, dev, stream) -> int:
    """Decode-time window tiers: score 256 decode queries against 16 caches of
    32768 tokens (no causal mask), then route 512 windows per KV head into
    128 full / 256 int4 / 128 evicted and promote 12 int4 windows."""
    x = synth.make_layer(spec, 5)
    up = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)  # noqa
    q, k, v = up(x["q"]), up(x["k"]), up(x["v"])
    Bt, Hkv, S, D = k.shape
    n_full, n_quant, n_prom = 128, 256, 12
    promote = torch.from_numpy(
        synth.promote_list(5, Bt * Hkv, n_quant, n_prom).reshape(Bt, Hkv, n_prom)).to(dev)
    desc = kvsel.make_desc(q, k, causal=False)
    ws = torch.empty(kvsel.score_workspace_bytes(desc), dtype=torch.uint8, device=dev)
    raw = torch.empty((Bt, Hkv, S), dtype=torch.float32, device=dev)
    outs = kvsel.route_tiers(raw, k, v, n_full=n_full, n_quant=n_quant, promote=promote)
    tws = torch.empty(kvsel.route_tiers_workspace_bytes(
        kvsel.TierDesc(Bt, Hkv, D, S, 64, n_full, n_quant, kvsel.BF16)), dtype=torch.uint8,
        device=dev)

    def score():
        kvsel.score(q, k, pool_kernel=1, causal=False, want_pooled=False, raw=raw, workspace=ws,
                    stream=stream)

    def tiers():
        kvsel.route_tiers(raw, k, v, n_full=n_full, n_quant=n_quant, promote=promote, out=outs,
                          workspace=tws, stream=stream)

    for _ in range(args.warmup):
        score()
        tiers()
    torch.cuda.synchronize()
    reps = max(args.steps // 4, 5)
    us = {"kvsel_score": event_time_us(torch, stream, score, reps),
          "kvsel_route_tiers": event_time_us(torch, stream, tiers, reps)}
    step_us = us["kvsel_score"] + us["kvsel_route_tiers"]
    tb = tier_bytes(spec, n_full, n_quant, n_prom)
    kt = kernel_times(kvsel, torch, lambda: (score(), tiers()), reps)
    dom = max(kt, key=lambda kk: kt[kk][0] * kt[kk][1])
    nbytes, flops = kernel_work(spec, dom, 0)
    out = {
        "metric": METRIC, "value": round(Bt * S / (step_us * 1e-6), 1), "unit": "tokens/s",
        "n_gpus": 1, "steps": reps, "warmup": args.warmup,
        "ms_per_step": round(step_us * 1e-3, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": wname, "batch": Bt, "seq_len": S, "n_q_heads": spec.n_q_heads,
                   "n_kv_heads": Hkv, "head_dim": D, "decode_queries": spec.obs_window,
                   "tiers": [n_full, n_quant, (S // 64) - n_full - n_quant], "promote": n_prom,
                   "parallelism": "none"},
        "us_per_call": {kk: round(vv, 2) for kk, vv in us.items()},
        "us_per_kernel": {kk: round(u, 2) for kk, (u, n) in kt.items()},
        "roofline": roofline_entry(dom, kt[dom][0], nbytes, flops,
                                   traffic_for(args.workload, dom)),
        "route_tiers_hbm_frac": round(tb / (us["kvsel_route_tiers"] * 1e-6) / 1e9
                                      / HBM_PEAK_GBS, 4),
    }
    print(json.dumps(out), flush=True)
    return 0


def bench_kara(args, kvsel, torch, wname) -> int:
    """Kara decode-window compression of one layer for a decode batch: the
    window's queries score its compressible keys (no mask), Token2Chunk picks
    the kept positions, the kept K/V rows are gathered.  Shapes follow the
    Kara page's settings: |W| = 512, |U| = 64, r = 40%, gamma = 8, alpha = 32,
    an 8B Llama-shaped layer (32 query / 8 KV heads, D = 128)."""
    Bt, Hq, Hkv, Wn, D, U, ratio, gamma, alpha = 64, 32, 8, 512, 128, 64, 0.4, 8, 32
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    x = synth.decode_window(7, Bt, Hq, Hkv, Wn, D)
    up = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)  # noqa
    q, k, v = up(x["q"]), up(x["k"]), up(x["v"])
    kd = kvsel.kara_desc(q, k, buffer=U, keep=kvsel.kara_keep(Wn, U, ratio), gamma=gamma,
                         alpha=alpha)
    n = Wn - U
    n_keep = min(n, kd.keep + alpha) + U
    A = torch.empty((Bt, Hkv, n), dtype=torch.float32, device=dev)
    ws = torch.empty(max(kvsel.kara_score_workspace_bytes(kd), 1), dtype=torch.uint8,
                     device=dev)
    idx = torch.empty((Bt, Hkv, n_keep), dtype=torch.int32, device=dev)
    k_hat = torch.empty((Bt, Hkv, n_keep, D), dtype=torch.bfloat16, device=dev)
    v_hat = torch.empty_like(k_hat)

    def score():
        kvsel.kara_score(q, k, kd, scores=A, workspace=ws, stream=stream)

    def select():
        kvsel.kara_select(A, kd, idx=idx, stream=stream)

    def compact():
        kvsel.compact(k, v, idx, k_out=k_hat, v_out=v_hat, stream=stream)

    def step():
        score()
        select()
        compact()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    step_us = event_time_us(torch, stream, step, args.steps)
    reps = max(args.steps, 50)
    us = {"kvsel_kara_score": event_time_us(torch, stream, score, reps),
          "kvsel_kara_select": event_time_us(torch, stream, select, reps),
          "kvsel_compact": event_time_us(torch, stream, compact, reps)}
    H = Bt * Hkv
    ab = {"kvsel_kara_score": Bt * Hq * Wn * D * 2 + 2 * H * n * D * 2 + H * n * 4,
          "kvsel_kara_select": H * n * 4 + H * n_keep * 4,
          "kvsel_compact": 2 * 2 * H * n_keep * D * 2 + H * n_keep * 4}
    path = sum(ab.values())
    # The scoring contraction has G*|W| = 2048 query rows per key: it is bound
    # by the matrix cores (and the exponentials), not by HBM.
    kt = kernel_times(kvsel, torch, step, reps)
    dom = max(kt, key=lambda kk: kt[kk][0] * kt[kk][1])
    kspec = synth.LayerSpec(Bt, Hq, Hkv, D, n, Wn, 1, 0, causal=0)
    nbytes, kflops = kernel_work(kspec, dom, n_keep)
    out = {
        "metric": METRIC, "value": round(Bt * Wn / (step_us * 1e-6), 1), "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(step_us * 1e-3, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": wname, "batch": Bt, "window": Wn, "buffer": U,
                   "n_q_heads": Hq, "n_kv_heads": Hkv, "head_dim": D, "keep": kd.keep,
                   "gamma": gamma, "alpha": alpha, "parallelism": "none"},
        "path_hbm_frac": round(path / (step_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
        "path_algorithmic_bytes": path,
        "us_per_call": {kk: round(vv, 2) for kk, vv in us.items()},
        "us_per_kernel": {kk: round(u, 2) for kk, (u, m) in kt.items()},
        "binding_roofline": binding_roofline(kspec, path, step_us),
        "roofline": roofline_entry(dom, kt[dom][0], nbytes, kflops,
                                   traffic_for(args.workload, dom)),
    }
    print(json.dumps(out), flush=True)
    return 0


def bench_qevict_steps(args, kvsel, torch, spec, wname) -> int:
    """QEvict's decode-time routing, repeated every Omega = 8 generated tokens:
    the 8 newest decode queries are scored against the whole cache (no mask),
    then kvsel_qevict_step accumulates the window scores, re-ranks the live
    windows and moves data for the transitions (first demotions into the INT2
    backing store, promotions back into the cache rows).  Query sets cycle
    so that rankings drift between steps."""
    Bt, Hq, Hkv, D, S = spec.batch, spec.n_q_heads, spec.n_kv_heads, spec.head_dim, spec.seq_len
    omega, n_sink, n_recent, bits, n_sets = 8, 5, 64, 2, 4
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    x = synth.qevict_cache(7, Bt, Hkv, S, D)
    up = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)  # noqa
    k, v = up(x["k"]), up(x["v"])
    qs = [up(synth.decode_window(40 + i, Bt, Hq, Hkv, omega, D)["q"]) for i in range(n_sets)]
    nW = max(0, (S - n_sink - n_recent) // 64)
    keep = nW // 2
    n_quant = int(round(0.7 * keep))
    n_full = keep - n_quant
    qd = kvsel.qevict_desc(k, seq_len=S, max_windows=nW, n_sink=n_sink, n_recent=n_recent,
                           n_full=n_full, n_quant=n_quant, bits=bits)
    state = kvsel.qevict_state(qd, dev)
    qws = torch.empty(kvsel.qevict_step_workspace_bytes(qd), dtype=torch.uint8, device=dev)
    desc = kvsel.make_desc(qs[0], k, causal=False)
    sws = torch.empty(kvsel.score_workspace_bytes(desc), dtype=torch.uint8, device=dev)
    raw = torch.empty((Bt, Hkv, S), dtype=torch.float32, device=dev)
    it = [0]

    def score():
        q = qs[it[0] % n_sets]
        kvsel.score(q, k, pool_kernel=1, causal=False, want_pooled=False, raw=raw, workspace=sws,
                    stream=stream)

    def route():
        kvsel.qevict_step(qd, raw, state, k, v, workspace=qws, stream=stream)

    def step():
        score()
        route()
        it[0] += 1

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    steps = max(args.steps // 4, 10)
    step_us = event_time_us(torch, stream, step, steps)
    us = {"kvsel_score": event_time_us(torch, stream, score, steps),
          "kvsel_qevict_step": event_time_us(torch, stream, route, steps)}
    t = state["tier"].cpu().numpy()
    kt = kernel_times(kvsel, torch, step, steps)
    dom = max(kt, key=lambda kk: kt[kk][0] * kt[kk][1])
    kspec = synth.LayerSpec(Bt, Hq, Hkv, D, S, omega, 1, 0, causal=0)
    nbytes, kflops = kernel_work(kspec, dom, 0)
    out = {
        "metric": METRIC, "value": round(Bt * S / (step_us * 1e-6), 1), "unit": "tokens/s",
        "n_gpus": 1, "steps": steps, "warmup": args.warmup,
        "ms_per_step": round(step_us * 1e-3, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": wname, "batch": Bt, "seq_len": S, "n_q_heads": Hq,
                   "n_kv_heads": Hkv, "head_dim": D, "queries_per_step": omega,
                   "sinks": n_sink, "recent": n_recent, "windows": nW, "full": n_full,
                   "quant": n_quant, "bits": bits, "parallelism": "none"},
        "us_per_call": {kk: round(vv, 2) for kk, vv in us.items()},
        "final_tiers": {"full": int((t == 0).sum()), "quant": int((t == 1).sum()),
                        "evicted": int((t == 2).sum())},
        "us_per_kernel": {kk: round(u, 2) for kk, (u, m) in kt.items()},
        "roofline": roofline_entry(dom, kt[dom][0], nbytes, kflops,
                                   traffic_for(args.workload, dom)),
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
