"""Throughput of the layer-end KV selection path on one MI355X.

A step is one pass of the whole path over one layer of synthetic input that
is already resident in HBM: kvsel_score (two streaming passes over K, row
statistics, max-pool) -> kvsel_select (exact top-B + window) -> kvsel_compact
(K/V gather).  The metric is prompt-KV tokens scored + selected + compacted
per second per layer.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu]
  python bench.py --copy-calibration     # plain device copy, for counter scaling

Workloads (one JSON line each):
  llama8k      one Llama-3-8B-shaped layer, 8192-token prompt (default)
  llama64k     the same shape at 65536 tokens, B = 4096
  qwen128k     one Qwen3-14B-shaped layer (40 q / 8 kv heads), 131072 tokens
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
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import synth  # noqa: E402

HBM_PEAK_GBS = 8000.0
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
}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_SOURCES = ["score.hip", "select.hip", "compact.hip", "tiers.hip", "kara.hip", "qevict.hip",
                  "common.h"]


def source_hash() -> str:
    """Hash of the kernel sources; counter figures are only valid for it."""
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "attention_score_eviction_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def algorithmic_bytes(spec: synth.LayerSpec) -> dict:
    """Bytes each ABI call must move per layer (two K sweeps, score vectors,
    gather); the sum is the path's algorithmic traffic."""
    e = 2 if spec.dtype == "bf16" else 4
    H = spec.batch * spec.n_kv_heads
    S, W, D, n_keep = spec.seq_len, spec.obs_window, spec.head_dim, spec.n_keep
    k_sweep = H * S * D * e
    d = {
        # two K sweeps + raw score write + max-pool read of raw, write of pooled
        "kvsel_score": 2 * k_sweep + H * S * 4 + H * S * 4 + H * (S - W) * 4,
        # pooled read + index write
        "kvsel_select": H * (S - W) * 4 + H * n_keep * 4,
        # K and V rows read and written + index read
        "kvsel_compact": 2 * 2 * H * n_keep * D * e + H * n_keep * 4,
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
                 adaptive: bool = False) -> dict:
    """The oracle, as it stands, timed on this host on the same layer."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    q64 = synth.to_f64(x["q"], spec.dtype)
    k64 = synth.to_f64(x["k"], spec.dtype)
    reps, t0 = 0, time.perf_counter()
    S, W = spec.seq_len, spec.obs_window
    while True:
        if adaptive:
            s = oracle.head_scores(q64, k64, causal=bool(spec.causal))
            p = oracle.max_pool(s, spec.pool_kernel, spec.n_sink, S - W)
            idx, off = oracle.select_head_adaptive(p, spec.n_kv_heads * spec.budget,
                                                   spec.n_sink, W)
            oracle.compact_flat(x["k"], idx, off)
            oracle.compact_flat(x["v"], idx, off)
        else:
            oracle.layer_end_compress(q64, k64, x["v"], budget=spec.budget,
                                      window=W, pool_kernel=spec.pool_kernel,
                                      n_sink=spec.n_sink, causal=bool(spec.causal),
                                      k_store=x["k"], v_store=x["v"])
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s or reps >= 1000:
            break
    return {"value": round(spec.batch * spec.seq_len * reps / el, 1), "unit": "tokens/s",
            "cores": threads, "kind": "oracle",
            "sample": f"{reps} full layer(s) of the same workload through the fp64 oracle "
                      f"({el:.1f} s, {threads} BLAS threads)"}


def traffic_for(workload: str, call: str):
    """Measured HBM bytes per call from the committed counter summary, if it
    was taken with the current kernel sources; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except OSError:
        return None
    if t.get("source_hash") != source_hash():
        return None
    return t.get("per_call_bytes", {}).get(workload, {}).get(call)


def event_time_us(torch, stream, fn, reps: int) -> float:
    """Average time of fn() over reps calls, HIP events on the launch stream."""
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(reps):
        fn()
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps * 1e3


class Layer:
    """Device buffers of one resident layer and its preallocated outputs."""

    def __init__(self, kvsel, torch, spec, x, dev, adaptive=False):
        self.kvsel, self.torch, self.spec = kvsel, torch, spec
        self.adaptive = adaptive
        if spec.dtype == "bf16":
            up = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)  # noqa
        else:
            up = lambda a: torch.from_numpy(a).to(dev)  # noqa
        self.q, self.k, self.v = up(x["q"]), up(x["k"]), up(x["v"])
        Bt, Hkv, S, D = self.k.shape
        self.pooled = torch.empty((Bt, Hkv, S), dtype=torch.float32, device=dev)
        self.raw = torch.empty_like(self.pooled)
        self.desc = kvsel.make_desc(self.q, self.k, n_sink=spec.n_sink, causal=bool(spec.causal))
        self.ws = torch.empty(max(kvsel.score_workspace_bytes(self.desc), 1), dtype=torch.uint8,
                              device=dev)
        self.set_budget(spec.budget)

    def set_budget(self, budget):
        torch, kvsel = self.torch, self.kvsel
        Bt, Hkv, S, D = self.k.shape
        dev = self.k.device
        self.budget = budget
        n_keep = budget + self.spec.n_sink + self.spec.obs_window
        if self.adaptive:
            # the same rows in total, chosen over all KV heads of a sequence
            self.idx = torch.empty((Bt, Hkv * n_keep), dtype=torch.int32, device=dev)
            self.head_off = torch.empty((Bt, Hkv + 1), dtype=torch.int32, device=dev)
            nb = kvsel.select_adaptive_workspace_bytes(self.desc, Hkv * budget)
            self.k_hat = torch.empty((Bt, Hkv * n_keep, D), dtype=self.k.dtype, device=dev)
        else:
            self.idx = torch.empty((Bt, Hkv, n_keep), dtype=torch.int32, device=dev)
            nb = kvsel.select_workspace_bytes(self.desc, budget)
            self.k_hat = torch.empty((Bt, Hkv, n_keep, D), dtype=self.k.dtype, device=dev)
        self.sel_ws = torch.empty(max(nb, 1), dtype=torch.uint8, device=dev)
        self.v_hat = torch.empty_like(self.k_hat)

    def load(self, x):
        """Overwrite the resident layer in place (the single active buffer)."""
        torch = self.torch
        for name, t in (("q", self.q), ("k", self.k), ("v", self.v)):
            t.copy_(torch.from_numpy(x[name].view(np.int16)).view(torch.bfloat16))

    def score(self, stream):
        s = self.spec
        self.kvsel.score(self.q, self.k, pool_kernel=s.pool_kernel, n_sink=s.n_sink,
                         causal=bool(s.causal), pooled=self.pooled, raw=self.raw,
                         workspace=self.ws, stream=stream)

    def select(self, stream):
        s = self.spec
        if self.adaptive:
            self.kvsel.select_adaptive(
                self.pooled, self.k.shape[1] * self.budget, obs_window=s.obs_window,
                n_q_heads=s.n_q_heads, head_dim=self.k.shape[3], n_sink=s.n_sink,
                causal=bool(s.causal), idx=self.idx, head_off=self.head_off, dtype=self.k.dtype,
                workspace=self.sel_ws, stream=stream)
            return
        self.kvsel.select(self.pooled, self.budget, obs_window=s.obs_window,
                          n_q_heads=s.n_q_heads, head_dim=self.k.shape[3], n_sink=s.n_sink,
                          causal=bool(s.causal), idx=self.idx, dtype=self.k.dtype,
                          workspace=self.sel_ws, stream=stream)

    def compact(self, stream):
        if self.adaptive:
            self.kvsel.compact_flat(self.k, self.v, self.idx, self.head_off, k_out=self.k_hat,
                                    v_out=self.v_hat, stream=stream)
            return
        self.kvsel.compact(self.k, self.v, self.idx, k_out=self.k_hat, v_out=self.v_hat,
                           stream=stream)

    def step(self, stream):
        self.score(stream)
        self.select(stream)
        self.compact(stream)


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


CALL_KERNELS = {
    "kvsel_score": ("score_pass1", "score_combine", "score_pass2", "maxpool_kernel",
                    "score_group_sum"),
    "kvsel_select": ("select_kernel", "sel_init", "sel_hist", "sel_cand", "sel_resolve",
                     "sel_emit"),
    "kvsel_compact": ("compact_kernel",),
    "kvsel_select_adaptive": ("sel_init", "sel_hist", "sel_cand", "sel_resolve", "sel_emit",
                              "mandatory_only_kernel"),
    "kvsel_compact_flat": ("compact_flat_kernel",),
    "kvsel_route_tiers": ("tier_rank_kernel", "tier_move_kernel", "tier_promote_kernel"),
}


def _counter_means(path: str, counter: str) -> dict:
    """Mean per-dispatch value of `counter` for each kernel in a rocprofv3
    counter_collection.csv."""
    import csv
    acc = {}
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        acc.setdefault(r["Kernel_Name"], {})
        acc[r["Kernel_Name"]].setdefault(r["Dispatch_Id"], 0.0)
        acc[r["Kernel_Name"]][r["Dispatch_Id"]] += float(r["Counter_Value"])
    return {k: sum(v.values()) / len(v) for k, v in acc.items()}


def ingest_counters(workload: str, fetch_csv: str, write_csv: str, cal_fetch_csv: str,
                    cal_write_csv: str) -> int:
    """Turn FETCH_SIZE / WRITE_SIZE runs of this bench (and of the copy
    calibration) into measured HBM bytes per ABI call, stored with the hash of
    the kernel sources in profiles/traffic.json."""
    cal_bytes = 256 * 1024 * 1024
    cf = max(_counter_means(cal_fetch_csv, "FETCH_SIZE").values())
    cw = max(_counter_means(cal_write_csv, "WRITE_SIZE").values())
    f_scale, w_scale = cal_bytes / cf, cal_bytes / cw
    fetch = _counter_means(fetch_csv, "FETCH_SIZE")
    write = _counter_means(write_csv, "WRITE_SIZE")
    per_call = {}
    adaptive = workload.endswith("-adaptive")
    for call, kernels in CALL_KERNELS.items():
        if (call in ("kvsel_select_adaptive", "kvsel_compact_flat")) != adaptive and \
                call in ("kvsel_select", "kvsel_compact", "kvsel_select_adaptive",
                         "kvsel_compact_flat"):
            continue
        tot, seen = 0.0, False
        for name in set(fetch) | set(write):
            if any(kn in name for kn in kernels):
                tot += fetch.get(name, 0.0) * f_scale + write.get(name, 0.0) * w_scale
                seen = True
        if seen:
            per_call[call] = int(round(tot))
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except OSError:
        t = {}
    if t.get("source_hash") != source_hash():
        t = {"per_call_bytes": {}}
    t["source_hash"] = source_hash()
    t["scale"] = {"fetch_bytes_per_unit": f_scale, "write_bytes_per_unit": w_scale,
                  "calibration": "bench.py --copy-calibration (256 MiB device copy)"}
    t["per_call_bytes"][workload] = per_call
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(t, f, indent=1, sort_keys=True)
    print(json.dumps({"workload": workload, "per_call_bytes": per_call}))
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="llama8k", choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--ingest-counters", nargs=4,
                    metavar=("FETCH_CSV", "WRITE_CSV", "CAL_FETCH_CSV", "CAL_WRITE_CSV"),
                    help="record measured traffic for --workload from rocprofv3 csv files")
    args = ap.parse_args()
    if args.ingest_counters:
        return ingest_counters(args.workload, *args.ingest_counters)
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
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
    L = Layer(kvsel, torch, spec, x, dev, adaptive=adaptive)
    if args.workload == "sweep64k":
        return bench_sweep(args, torch, spec, wname, L, stream)

    for _ in range(args.warmup):
        L.step(stream)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        L.step(stream)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = ev0.elapsed_time(ev1) / args.steps

    reps = max(args.steps, 50)
    sel_name = "kvsel_select_adaptive" if adaptive else "kvsel_select"
    cmp_name = "kvsel_compact_flat" if adaptive else "kvsel_compact"
    us = {"kvsel_score": event_time_us(torch, stream, lambda: L.score(stream), reps),
          sel_name: event_time_us(torch, stream, lambda: L.select(stream), reps),
          cmp_name: event_time_us(torch, stream, lambda: L.compact(stream), reps)}
    ab = algorithmic_bytes(spec)
    if adaptive:
        ab[sel_name] = ab.pop("kvsel_select") + spec.batch * (spec.n_kv_heads + 1) * 4
        ab[cmp_name] = ab.pop("kvsel_compact") + spec.batch * (spec.n_kv_heads + 1) * 4
        ab["path"] = ab["kvsel_score"] + ab[sel_name] + ab[cmp_name]
    Bt, S = spec.batch, spec.seq_len
    value = Bt * S / (ms_step * 1e-3)
    path_gbs = ab["path"] / (ms_step * 1e-3) / 1e9
    dom = max(us, key=us.get)
    dom_gbs = ab[dom] / (us[dom] * 1e-6) / 1e9
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
        "path_algorithmic_bytes": ab["path"],
        "us_per_call": {k: round(v, 2) for k, v in us.items()},
        "wall_s": round(wall, 3),
        "roofline": {"bound": "hbm", "achieved": round(dom_gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(dom_gbs / HBM_PEAK_GBS, 4),
                     "traffic": traffic_for(args.workload, dom), "kernel": dom,
                     "algorithmic_bytes_per_launch": ab[dom]},
    }
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(spec, x, adaptive=adaptive)
    print(json.dumps(out), flush=True)
    return 0


def bench_sweep(args, torch, spec, wname, L, stream) -> int:
    """32 layers, one resident full-prompt layer buffer overwritten per layer;
    each layer's compact K/V goes to a per-layer store (the only state kept)."""
    n_layers = 32
    per_layer_us, store_bytes = [], 0
    reps = max(1, args.steps // 10)
    store = []
    for layer in range(n_layers):
        b = synth.sweep_budget(layer, n_layers)
        if layer > 0:
            L.load(synth.make_layer(spec, 3, layer))
        L.set_budget(b)
        for _ in range(max(1, args.warmup // 10)):
            L.step(stream)
        torch.cuda.synchronize()
        per_layer_us.append(event_time_us(torch, stream, lambda: L.step(stream), reps))
        store.append((L.k_hat.clone(), L.v_hat.clone(), L.idx.clone()))
        store_bytes += sum(t.numel() * t.element_size() for t in store[-1])
        print(f"layer {layer} budget {b}: {per_layer_us[-1]:.1f} us", file=sys.stderr, flush=True)
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
                   "budget_first": synth.sweep_budget(0), "budget_last": synth.sweep_budget(31),
                   "parallelism": "none"},
        "per_layer_us_mean": round(mean_us, 2), "per_layer_us_max": round(max(per_layer_us), 2),
        "compact_store_bytes": store_bytes,
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
    flops = 2 * 2 * Bt * spec.n_q_heads * spec.obs_window * D * S
    tflops = flops / (us["kvsel_score"] * 1e-6) / 1e12
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
        "roofline": {"bound": "mfma", "achieved": round(tflops, 1), "peak": 2500.0,
                     "unit": "TFLOP/s", "frac": round(tflops / 2500.0, 4),
                     "traffic": traffic_for(args.workload, "kvsel_score"),
                     "kernel": "kvsel_score", "algorithmic_flops_per_launch": flops},
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
    flops = 2 * 2 * Bt * Hq * Wn * n * D
    tflops = flops / (us["kvsel_kara_score"] * 1e-6) / 1e12
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
        "roofline": {"bound": "mfma", "achieved": round(tflops, 1), "peak": 2500.0,
                     "unit": "TFLOP/s", "frac": round(tflops / 2500.0, 4),
                     "traffic": traffic_for(args.workload, "kvsel_kara_score"),
                     "kernel": "kvsel_kara_score", "algorithmic_flops_per_launch": flops},
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
    H = Bt * Hkv
    t = state["tier"].cpu().numpy()
    score_bytes = 2 * H * S * D * 2 + H * S * 4   # two K sweeps + the raw scores
    dom_gbs = score_bytes / (us["kvsel_score"] * 1e-6) / 1e9
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
        "roofline": {"bound": "hbm", "achieved": round(dom_gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(dom_gbs / HBM_PEAK_GBS, 4),
                     "traffic": traffic_for(args.workload, "kvsel_score"),
                     "kernel": "kvsel_score", "algorithmic_bytes_per_launch": score_bytes},
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
