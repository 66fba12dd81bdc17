"""Layer-major driver of the layer-end step (TideKV Algorithm 1, Section 4.1).

TideKV runs prefill layer by layer: a layer's full-prompt K/V is built over
all prompt chunks, then LayerEndCompress (Algorithm 2) keeps the retained
rows, the compact cache is committed, and the full K/V is released before
the next layer starts, so only one layer's full-prompt K/V is ever resident.

This driver holds that single active buffer (Q_obs, K, V of one layer) and
the scratch of the layer-end step, fills the buffer in place for each layer,
runs the layer-end step (kvsel_layer_end) on one stream, and commits each
layer's compact K/V and absolute positions to a per-layer store.  The model
forward that would produce the K/V is not part of it: the caller supplies
each layer's tensors.  Host orchestration only; every step of the layer-end
computation runs in the library's kernels.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import torch

import ctypes

from . import (Desc, _check, _dtype_code, _ptr, _stream, layer_end, layer_end_adaptive,
               layer_end_adaptive_workspace_bytes, layer_end_workspace_bytes, lib)


@dataclass
class LayerCache:
    """Committed compact cache of one layer."""
    budget: int
    idx: torch.Tensor        # [Bt, Hkv, budget + n_sink + W] int32, absolute positions
    k_hat: torch.Tensor      # [Bt, Hkv, budget + n_sink + W, D]
    v_hat: torch.Tensor

    @property
    def nbytes(self) -> int:
        return sum(t.numel() * t.element_size() for t in (self.idx, self.k_hat, self.v_hat))


@dataclass
class FlatLayerCache:
    """Committed compact cache of one layer under a head-adaptive budget
    (TideKV Section 4.1): every KV head's rows of a sequence in one flattened
    list, head h owning rows [head_off[b,h], head_off[b,h+1])."""
    total_budget: int
    idx: torch.Tensor        # [Bt, n_keep] int32, absolute positions
    head_off: torch.Tensor   # [Bt, Hkv + 1] int32
    k_hat: torch.Tensor      # [Bt, n_keep, D]
    v_hat: torch.Tensor

    @property
    def nbytes(self) -> int:
        return sum(t.numel() * t.element_size()
                   for t in (self.idx, self.head_off, self.k_hat, self.v_hat))


@dataclass
class LayerMajorDriver:
    """One resident layer plus the layer-end scratch; see the module docstring."""
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    seq_len: int
    obs_window: int
    pool_kernel: int
    max_budget: int
    n_sink: int = 0
    dtype: torch.dtype = torch.bfloat16
    device: str = "cuda"
    store: list = field(default_factory=list)

    def __post_init__(self):
        Bt, Hq, Hkv, D, S, W = (self.batch, self.n_q_heads, self.n_kv_heads, self.head_dim,
                                self.seq_len, self.obs_window)
        dev = torch.device(self.device)
        e = lambda *s, dt=self.dtype: torch.empty(s, dtype=dt, device=dev)  # noqa: E731
        # the active layer: the only full-prompt K/V that is resident
        self.q, self.k, self.v = e(Bt, Hq, W, D), e(Bt, Hkv, S, D), e(Bt, Hkv, S, D)
        self.pooled = e(Bt, Hkv, S, dt=torch.float32)
        self.raw = e(Bt, Hkv, S, dt=torch.float32)
        self.desc = Desc(Bt, Hq, Hkv, D, S, W, self.n_sink, 1, _dtype_code(self.k), 0.0)
        self.ws = e(max(layer_end_workspace_bytes(self.desc, self.max_budget), 1),
                    dt=torch.uint8)

    @property
    def active_bytes(self) -> int:
        """Device bytes of the active layer (Q_obs, K, V)."""
        return sum(t.numel() * t.element_size() for t in (self.q, self.k, self.v))

    @property
    def scratch_bytes(self) -> int:
        """Score vectors and workspaces of the layer-end step."""
        return sum(t.numel() * t.element_size() for t in (self.pooled, self.raw, self.ws))

    @property
    def store_bytes(self) -> int:
        return sum(c.nbytes for c in self.store)

    def load(self, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor) -> None:
        """Fill the active buffer with a layer's Q_obs, K, V (host or device
        tensors of the active shapes), overwriting the previous layer."""
        for dst, src in ((self.q, q), (self.k, k), (self.v, v)):
            if tuple(src.shape) != tuple(dst.shape) or src.dtype != dst.dtype:
                raise ValueError(f"layer tensor {tuple(src.shape)} {src.dtype} does not match "
                                 f"the active buffer {tuple(dst.shape)} {dst.dtype}")
            dst.copy_(src)

    def new_cache(self, budget: int) -> LayerCache:
        """Output buffers of a layer's compact cache at `budget`."""
        if not 0 <= budget <= self.max_budget:
            raise ValueError(f"budget {budget} outside [0, {self.max_budget}]")
        n_keep = budget + self.n_sink + self.obs_window
        shape = (self.batch, self.n_kv_heads, n_keep)
        dev = self.k.device
        return LayerCache(budget, torch.empty(shape, dtype=torch.int32, device=dev),
                          torch.empty(shape + (self.head_dim,), dtype=self.dtype, device=dev),
                          torch.empty(shape + (self.head_dim,), dtype=self.dtype, device=dev))

    def layer_end(self, cache: LayerCache, stream=None) -> LayerCache:
        """LayerEndCompress of the active layer into `cache` (score ->
        max-pool -> top-budget + window -> gather), enqueued on `stream`.
        The call's arguments are marshalled once per cache and reused (every
        buffer is the driver's or the cache's), so a call costs one ctypes
        call on the host."""
        call = getattr(cache, "_call", None)
        if call is None:
            # checks of the generic binding, once: shapes and dtypes
            layer_end(self.q, self.k, self.v, budget=cache.budget, pool_kernel=self.pool_kernel,
                      n_sink=self.n_sink, raw=self.raw, pooled=self.pooled, idx=cache.idx,
                      k_out=cache.k_hat, v_out=cache.v_hat, workspace=self.ws, stream=stream)
            args = (ctypes.byref(self.desc), _ptr(self.q), _ptr(self.k), _ptr(self.v),
                    int(cache.budget), int(self.pool_kernel), _ptr(self.raw), _ptr(self.pooled),
                    _ptr(cache.idx), _ptr(cache.k_hat), _ptr(cache.v_hat), _ptr(self.ws),
                    self.ws.numel())
            fn = lib().kvsel_layer_end
            cache._call = lambda s: _check(fn(*args, s), "kvsel_layer_end")
            return cache
        call(_stream(stream))
        return cache

    def new_flat_cache(self, total_budget: int) -> FlatLayerCache:
        """Output buffers of a layer's flattened cache at a head-adaptive
        budget of `total_budget` picks per sequence (at most Hkv times the
        per-head maximum the scratch was sized for)."""
        if not 0 <= total_budget <= self.n_kv_heads * self.max_budget:
            raise ValueError(f"total budget {total_budget} outside "
                             f"[0, {self.n_kv_heads * self.max_budget}]")
        n_keep = self.n_kv_heads * (self.n_sink + self.obs_window) + total_budget
        dev = self.k.device
        Bt, D = self.batch, self.head_dim
        return FlatLayerCache(total_budget,
                              torch.empty((Bt, n_keep), dtype=torch.int32, device=dev),
                              torch.empty((Bt, self.n_kv_heads + 1), dtype=torch.int32,
                                          device=dev),
                              torch.empty((Bt, n_keep, D), dtype=self.dtype, device=dev),
                              torch.empty((Bt, n_keep, D), dtype=self.dtype, device=dev))

    def layer_end_adaptive(self, cache: FlatLayerCache, stream=None) -> FlatLayerCache:
        """LayerEndCompress of the active layer with one head-adaptive budget
        per sequence (kvsel_layer_end_adaptive) into `cache`, enqueued on
        `stream`; marshalled once per cache like layer_end."""
        call = getattr(cache, "_call", None)
        if call is None:
            ws = getattr(self, "_ws_adaptive", None)
            need = max(layer_end_adaptive_workspace_bytes(self.desc, cache.total_budget), 1)
            if ws is None or ws.numel() < need:
                ws = torch.empty(need, dtype=torch.uint8, device=self.k.device)
                self._ws_adaptive = ws
            cache._ws = ws      # the prepared call below holds its address
            layer_end_adaptive(self.q, self.k, self.v, total_budget=cache.total_budget,
                               pool_kernel=self.pool_kernel, n_sink=self.n_sink, raw=self.raw,
                               pooled=self.pooled, idx=cache.idx, head_off=cache.head_off,
                               k_out=cache.k_hat, v_out=cache.v_hat, workspace=ws, stream=stream)
            args = (ctypes.byref(self.desc), _ptr(self.q), _ptr(self.k), _ptr(self.v),
                    int(cache.total_budget), int(self.pool_kernel), _ptr(self.raw),
                    _ptr(self.pooled), _ptr(cache.idx), _ptr(cache.head_off), _ptr(cache.k_hat),
                    _ptr(cache.v_hat), _ptr(ws), ws.numel())
            fn = lib().kvsel_layer_end_adaptive
            cache._call = lambda s: _check(fn(*args, s), "kvsel_layer_end_adaptive")
            return cache
        call(_stream(stream))
        return cache

    def commit(self, budget: int, stream=None) -> LayerCache:
        """Compress the active layer at `budget` and append its compact cache
        to the store (the layer-end commit; the active buffer may then be
        refilled with the next layer)."""
        cache = self.layer_end(self.new_cache(budget), stream=stream)
        self.store.append(cache)
        return cache

    def run(self, layers, budgets, stream=None) -> list:
        """Algorithm 1's outer loop over an iterable of (q, k, v) per layer
        with its budget schedule; returns the store."""
        for (q, k, v), b in zip(layers, budgets):
            self.load(q, k, v)
            self.commit(b, stream=stream)
        return self.store


def linear_budgets(n_layers: int, first: int, last: int) -> list:
    """A PyramidKV-style per-layer budget schedule falling linearly from
    `first` (layer 0) to `last` (layer n_layers-1), rounded down:
    B_l = first - floor((first - last) * l / (n_layers - 1))."""
    if n_layers == 1:
        return [first]
    return [first - ((first - last) * l) // (n_layers - 1) for l in range(n_layers)]
