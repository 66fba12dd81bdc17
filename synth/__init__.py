"""Seeded synthetic inputs for the KV selection path.

This module only draws and shapes input tensors; it contains none of the
method's arithmetic (no logits, softmax, pooling, selection or gather).  It is
the single source of inputs shared by the CPU oracle and the GPU path, so both
see bit-identical tensors.

Stand-in for real prompt KV: the pages evaluate on LongBench / RULER / GSM8K
prompts run through Llama-3.1-8B, Mistral-7B and Qwen3-14B (TideKV §6.1;
QEvict §5; Kara §1).  No dataset or weight is available here, so keys, values
and observation queries are seeded Gaussians with the model shapes and a few
structural features that make selection non-trivial: boosted attention-sink
keys, heavy-hitter keys aligned with the observation queries, and clustered
spans of keys sharing a direction.

Every tensor is drawn from ``numpy.random.default_rng(SeedSequence(key))`` with
``key = [config_id, layer, tensor_id]`` as fp32 N(0, 1); structure is applied in
fp64/fp32 and bf16 tensors are then rounded to nearest-even on the bit pattern.
bf16 tensors are returned as ``uint16`` bit arrays, fp32 tensors as ``float32``.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

TENSOR_Q, TENSOR_K, TENSOR_V, TENSOR_STRUCT, TENSOR_PROMOTE = 0, 1, 2, 3, 4


@dataclasses.dataclass(frozen=True)
class LayerSpec:
    """Shape and input recipe of one layer-end selection problem."""

    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    seq_len: int
    obs_window: int
    pool_kernel: int
    budget: int
    dtype: str = "bf16"          # "bf16" or "f32"
    causal: int = 1
    n_sink: int = 0              # mandatory sink count passed to the path (API)
    sink_keys: int = 4           # how many leading keys are boosted
    sink_boost: float = 4.0
    structure: str = "none"      # "none" | "heavy" | "spans"
    heavy_frac: float = 0.01
    n_spans: int = 0
    span_len: int = 32
    span_boost: float = 2.0
    name: str = "custom"

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def n_keep(self) -> int:
        return self.budget + self.n_sink + self.obs_window


def config(n: int) -> LayerSpec:
    """The five workload shapes (numbered 1..5)."""
    if n == 1:
        return LayerSpec(1, 4, 2, 64, 512, 16, 5, 64, dtype="f32", name="c1-tiny-f32")
    if n == 2:
        return LayerSpec(1, 32, 8, 128, 8192, 32, 7, 1024, structure="heavy",
                         name="c2-llama8b-8k")
    if n == 3:
        return LayerSpec(1, 32, 8, 128, 65536, 64, 7, 4096, structure="heavy",
                         name="c3-llama8b-64k-sweep")
    if n == 4:
        return LayerSpec(1, 40, 8, 128, 131072, 64, 7, 4096, structure="spans",
                         n_spans=64, name="c4-qwen3-14b-128k")
    if n == 5:
        return LayerSpec(16, 32, 8, 128, 32768, 256, 1, 0, causal=0,
                         structure="heavy", name="c5-qevict-decode")
    raise ValueError(f"unknown config {n}")


def sweep_budget(layer: int, n_layers: int = 32, b_first: int = 4096, b_last: int = 512) -> int:
    """Linear per-layer budget from b_first (layer 0) down to b_last (last layer),
    rounded down: B_l = b_first - floor((b_first - b_last) * l / (n_layers - 1))."""
    if n_layers == 1:
        return b_first
    return b_first - ((b_first - b_last) * layer) // (n_layers - 1)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest-even) and return the 16-bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def to_f64(t: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 values of a generated tensor."""
    if dtype == "bf16":
        return bf16_bits_to_f32(t).astype(np.float64)
    return np.asarray(t, dtype=np.float32).astype(np.float64)


def _rng(key) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence(list(key)))


def _normal(key, shape) -> np.ndarray:
    return _rng(key).standard_normal(size=shape, dtype=np.float32)


def _round(x: np.ndarray, dtype: str) -> np.ndarray:
    return f32_to_bf16_bits(x) if dtype == "bf16" else np.ascontiguousarray(x, np.float32)


def make_layer(spec: LayerSpec, config_id: int, layer: int = 0,
               want_v: bool = True) -> dict:
    """Draw Q_obs [Bt,Hq,W,D], K and V [Bt,Hkv,S,D] for one layer.

    Returns ``{"q": ..., "k": ..., "v": ...}`` in the spec's storage dtype
    (uint16 bf16 bits or float32).
    """
    Bt, Hq, Hkv, D, S, W = (spec.batch, spec.n_q_heads, spec.n_kv_heads,
                            spec.head_dim, spec.seq_len, spec.obs_window)
    base = (config_id, layer)
    q32 = _normal(base + (TENSOR_Q,), (Bt, Hq, W, D))
    q = _round(q32, spec.dtype)
    k32 = _normal(base + (TENSOR_K,), (Bt, Hkv, S, D))
    ns = min(spec.sink_keys, S)
    if ns:
        k32[:, :, :ns, :] *= np.float32(spec.sink_boost)
    srng = _rng(base + (TENSOR_STRUCT,))
    if spec.structure == "heavy":
        _apply_heavy(k32, to_f64(q, spec.dtype), spec, srng)
    elif spec.structure == "spans":
        _apply_spans(k32, spec, srng)
    elif spec.structure != "none":
        raise ValueError(spec.structure)
    out = {"q": q, "k": _round(k32, spec.dtype)}
    del k32
    if want_v:
        out["v"] = _round(_normal(base + (TENSOR_V,), (Bt, Hkv, S, D)), spec.dtype)
    return out


def _apply_heavy(k32: np.ndarray, q64: np.ndarray, spec: LayerSpec, rng) -> None:
    """Heavy hitters: per (batch, KV head) pick round(frac*S) keys in
    [sink_keys, S-W) and rotate each so its cosine with the head's mean
    observation query is exactly 0.5, keeping its norm."""
    Bt, Hkv, S, D = k32.shape
    G, W = spec.group, spec.obs_window
    lo, hi = min(spec.sink_keys, S), S - W
    n = int(round(spec.heavy_frac * S))
    n = min(n, max(hi - lo, 0))
    if n <= 0:
        return
    for b in range(Bt):
        for h in range(Hkv):
            qm = q64[b, h * G:(h + 1) * G].reshape(-1, D).mean(axis=0)
            u = qm / np.linalg.norm(qm)
            pos = lo + rng.choice(hi - lo, size=n, replace=False)
            kk = k32[b, h, pos].astype(np.float64)
            nk = np.linalg.norm(kk, axis=1, keepdims=True)
            perp = kk - (kk @ u)[:, None] * u[None, :]
            vhat = perp / np.linalg.norm(perp, axis=1, keepdims=True)
            k32[b, h, pos] = (nk * (0.5 * u[None, :] + (math.sqrt(3.0) / 2.0) * vhat)).astype(np.float32)


def _apply_spans(k32: np.ndarray, spec: LayerSpec, rng) -> None:
    """Clustered spans: n_spans non-overlapping spans of span_len keys on the
    grid sink_keys + span_len*j inside [sink_keys, S-W-span_len], shared by all
    KV heads; per (span, batch, KV head) a random unit direction u, and each key
    of the span becomes span_boost * |k| * u."""
    Bt, Hkv, S, D = k32.shape
    L = spec.span_len
    lo = min(spec.sink_keys, S)
    n_grid = (S - spec.obs_window - L - lo) // L + 1
    if n_grid <= 0 or spec.n_spans <= 0:
        return
    js = rng.choice(n_grid, size=min(spec.n_spans, n_grid), replace=False)
    for j in np.sort(js):
        a = lo + L * int(j)
        for b in range(Bt):
            for h in range(Hkv):
                u = rng.standard_normal(D)
                u /= np.linalg.norm(u)
                kk = k32[b, h, a:a + L].astype(np.float64)
                nk = np.linalg.norm(kk, axis=1, keepdims=True)
                k32[b, h, a:a + L] = (spec.span_boost * nk * u[None, :]).astype(np.float32)


def decode_window(seed: int, batch: int, n_q_heads: int, n_kv_heads: int, window: int,
                  head_dim: int, dtype: str = "bf16") -> dict:
    """Queries, keys and values of the most recent `window` decode tokens:
    Q [Bt,Hq,W,D], K and V [Bt,Hkv,W,D], fp32 N(0,1) rounded to the storage
    dtype.  Structure: per (sequence, KV head), round(0.05 W) seeded-uniform
    window positions get their key scaled by 2, so a few keys stand out."""
    base = (900, seed)
    q32 = _normal(base + (TENSOR_Q,), (batch, n_q_heads, window, head_dim))
    k32 = _normal(base + (TENSOR_K,), (batch, n_kv_heads, window, head_dim))
    v32 = _normal(base + (TENSOR_V,), (batch, n_kv_heads, window, head_dim))
    rng = _rng(base + (TENSOR_PROMOTE,))
    n_boost = int(round(0.05 * window))
    for b in range(batch):
        for h in range(n_kv_heads):
            k32[b, h, rng.choice(window, size=n_boost, replace=False)] *= np.float32(2.0)
    return {"q": _round(q32, dtype), "k": _round(k32, dtype), "v": _round(v32, dtype)}


def promote_list(config_id: int, n_rows: int, n_quant: int, n_promote: int,
                 layer: int = 0) -> np.ndarray:
    """Seeded-uniform choice (without replacement, ascending) of n_promote of
    the n_quant quantised-tier slots per (batch, KV head) row."""
    rng = _rng((config_id, layer, TENSOR_PROMOTE))
    out = np.empty((n_rows, n_promote), dtype=np.int32)
    for r in range(n_rows):
        out[r] = np.sort(rng.choice(n_quant, size=n_promote, replace=False))
    return out


def qevict_cache(seed: int, batch: int, n_kv_heads: int, capacity: int, head_dim: int) -> dict:
    """K and V cache rows [Bt, Hkv, capacity, D] as bf16 bit patterns, N(0,1)."""
    base = (950, seed)
    return {"k": _round(_normal(base + (TENSOR_K,), (batch, n_kv_heads, capacity, head_dim)),
                        "bf16"),
            "v": _round(_normal(base + (TENSOR_V,), (batch, n_kv_heads, capacity, head_dim)),
                        "bf16")}


def qevict_token_scores(seed: int, step: int, batch: int, n_kv_heads: int, seq_len: int,
                        integer: bool = True) -> np.ndarray:
    """Per-step attention mass per token [Bt, Hkv, seq_len] float32 with drift:
    a fixed per-token importance (heavy-tailed) plus a fresh per-step part, so
    window rankings change between steps.  integer=True gives small integers
    (sums stay exact in fp32); otherwise positive reals."""
    base = _rng((960, seed, TENSOR_STRUCT)).gamma(0.5, 2.0, size=(batch, n_kv_heads, seq_len))
    fresh = _rng((960, seed, step)).gamma(0.5, 2.0, size=(batch, n_kv_heads, seq_len))
    s = base + 1.5 * fresh
    if integer:
        return np.minimum(np.floor(s), 15).astype(np.float32)
    return (s / seq_len).astype(np.float32)
