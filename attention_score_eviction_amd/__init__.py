"""Python binding of libkvsel (attention-score KV selection and compaction).

Argument marshalling only: every step of the path runs in the HIP kernels of
``libkvsel.so``; PyTorch supplies device memory and the current stream.  The
function names follow the C ABI in ``include/kvsel.h``:

    score(q_obs, k, ...)         -> (pooled, raw)     kvsel_score
    select(pooled, budget, ...)  -> idx               kvsel_select
    compact(k, v, idx, ...)      -> (k_hat, v_hat)    kvsel_compact
    route_tiers(scores, k, v, ...) -> dict            kvsel_route_tiers

There is no CPU fallback: without the built library every call raises.
"""
from __future__ import annotations

import ctypes
import os
from contextlib import nullcontext
from dataclasses import dataclass
from fractions import Fraction
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkvsel.so")

OK, ERR_ARG, ERR_BUDGET, ERR_WORKSPACE, ERR_UNSUPPORTED, ERR_DEVICE = range(6)
BF16, F32 = 0, 1


class KvselError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_str(status)} (status {status})")


class Desc(ctypes.Structure):
    """kvsel_desc."""
    _fields_ = [
        ("batch", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("seq_len", ctypes.c_int32), ("obs_window", ctypes.c_int32),
        ("n_sink", ctypes.c_int32), ("causal", ctypes.c_int32),
        ("dtype", ctypes.c_int32), ("scale", ctypes.c_float),
    ]


class TierDesc(ctypes.Structure):
    """kvsel_tier_desc."""
    _fields_ = [
        ("batch", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("seq_len", ctypes.c_int32),
        ("win", ctypes.c_int32), ("n_full", ctypes.c_int32),
        ("n_quant", ctypes.c_int32), ("dtype", ctypes.c_int32),
    ]


class QevictDesc(ctypes.Structure):
    """kvsel_qevict_desc."""
    _fields_ = [
        ("batch", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("seq_len", ctypes.c_int32),
        ("capacity", ctypes.c_int32), ("max_windows", ctypes.c_int32),
        ("win", ctypes.c_int32), ("n_sink", ctypes.c_int32),
        ("n_recent", ctypes.c_int32), ("n_full", ctypes.c_int32),
        ("n_quant", ctypes.c_int32), ("bits", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
    ]


class KaraDesc(ctypes.Structure):
    """kvsel_kara_desc."""
    _fields_ = [
        ("batch", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("window", ctypes.c_int32), ("buffer", ctypes.c_int32),
        ("keep", ctypes.c_int32), ("gamma", ctypes.c_int32),
        ("alpha", ctypes.c_int32), ("dtype", ctypes.c_int32),
        ("scale", ctypes.c_float),
    ]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libkvsel.so; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m attention_score_eviction_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    P, I32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    DP, TP = ctypes.POINTER(Desc), ctypes.POINTER(TierDesc)
    L.kvsel_status_str.argtypes = [ctypes.c_int]
    L.kvsel_status_str.restype = ctypes.c_char_p
    L.kvsel_score_workspace.argtypes = [DP]
    L.kvsel_score_workspace.restype = SZ
    L.kvsel_score.argtypes = [DP, P, P, P, P, I32, P, SZ, P]
    L.kvsel_score.restype = ctypes.c_int
    L.kvsel_select_workspace.argtypes = [DP, I32]
    L.kvsel_select_workspace.restype = SZ
    L.kvsel_select.argtypes = [DP, P, I32, P, P, SZ, P]
    L.kvsel_select.restype = ctypes.c_int
    L.kvsel_compact.argtypes = [DP, P, P, P, I32, P, P, P]
    L.kvsel_compact.restype = ctypes.c_int
    L.kvsel_select_compact.argtypes = [DP, P, I32, P, P, P, P, P, P, SZ, P]
    L.kvsel_select_compact.restype = ctypes.c_int
    L.kvsel_select_adaptive_workspace.argtypes = [DP, I32]
    L.kvsel_select_adaptive_workspace.restype = SZ
    L.kvsel_select_adaptive.argtypes = [DP, P, I32, P, P, P, SZ, P]
    L.kvsel_select_adaptive.restype = ctypes.c_int
    L.kvsel_compact_flat.argtypes = [DP, P, P, P, P, I32, P, P, P]
    L.kvsel_compact_flat.restype = ctypes.c_int
    KP = ctypes.POINTER(KaraDesc)
    L.kvsel_kara_score_workspace.argtypes = [KP]
    L.kvsel_kara_score_workspace.restype = SZ
    L.kvsel_kara_score.argtypes = [KP, P, P, P, P, SZ, P]
    L.kvsel_kara_score.restype = ctypes.c_int
    L.kvsel_kara_select.argtypes = [KP, P, P, P]
    L.kvsel_kara_select.restype = ctypes.c_int
    L.kvsel_route_tiers_workspace.argtypes = [TP]
    L.kvsel_route_tiers_workspace.restype = SZ
    L.kvsel_route_tiers.argtypes = [TP, P, P, P, P, P, P, P, P, P, P, P, P, I32, P, P, P, SZ, P]
    L.kvsel_route_tiers.restype = ctypes.c_int
    QP = ctypes.POINTER(QevictDesc)
    L.kvsel_qevict_step_workspace.argtypes = [QP]
    L.kvsel_qevict_step_workspace.restype = SZ
    L.kvsel_qevict_step.argtypes = [QP, P, P, P, P, P, P, P, P, P, P, P, SZ, P]
    L.kvsel_qevict_step.restype = ctypes.c_int
    L.kvsel_kara_keep.argtypes = [I32, I32, I32, I32]
    L.kvsel_kara_keep.restype = I32
    L.kvsel_timing_start.argtypes = [ctypes.c_char_p]
    L.kvsel_timing_start.restype = ctypes.c_int
    L.kvsel_timing_read.argtypes = [P, I32, P, P, I32]
    L.kvsel_timing_read.restype = I32
    L.kvsel_layer_end_workspace.argtypes = [DP, I32]
    L.kvsel_layer_end_workspace.restype = SZ
    L.kvsel_layer_end.argtypes = [DP, P, P, P, I32, I32, P, P, P, P, P, P, SZ, P]
    L.kvsel_layer_end.restype = ctypes.c_int
    L.kvsel_layer_end_adaptive_workspace.argtypes = [DP, I32]
    L.kvsel_layer_end_adaptive_workspace.restype = SZ
    L.kvsel_layer_end_adaptive.argtypes = [DP, P, P, P, I32, I32, P, P, P, P, P, P, P, SZ, P]
    L.kvsel_layer_end_adaptive.restype = ctypes.c_int
    L.kvsel_layer_end_stream_workspace.argtypes = [DP, I32, I32]
    L.kvsel_layer_end_stream_workspace.restype = SZ
    L.kvsel_layer_end_stream.argtypes = [DP, P, P, P, I32, I32, P, P, P, P, SZ, P]
    L.kvsel_layer_end_stream.restype = ctypes.c_int
    L.kvsel_score_static.argtypes = [DP, P, P, P, P, I32, P]
    L.kvsel_score_static.restype = ctypes.c_int
    _lib = L
    return L


def status_str(status: int) -> str:
    return lib().kvsel_status_str(status).decode()


def _check(status: int, where: str) -> None:
    if status != OK:
        raise KvselError(status, where)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("kvsel operates on device tensors only")
    if not t.is_contiguous():
        raise ValueError("kvsel needs contiguous tensors")
    return t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _on(stream):
    """Context in which the binding allocates outputs and workspaces: the
    launch stream, so that torch's caching allocator orders any reuse of
    those blocks after the kernels enqueued there."""
    if stream is None:
        return nullcontext()
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    if handle == torch.cuda.current_stream().cuda_stream:
        return nullcontext()          # already the current stream
    if not isinstance(stream, torch.cuda.Stream):
        stream = torch.cuda.ExternalStream(int(stream))
    return torch.cuda.stream(stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise ValueError(f"unsupported dtype {t.dtype}")


def make_desc(q_obs: torch.Tensor, k: torch.Tensor, *, n_sink: int = 0, causal: bool = True,
              scale: float = 0.0) -> Desc:
    """kvsel_desc from Q_obs [Bt,Hq,W,D] and K [Bt,Hkv,S,D]."""
    Bt, Hq, W, D = q_obs.shape
    Bk, Hkv, S, Dk = k.shape
    if Bk != Bt or Dk != D or q_obs.dtype != k.dtype:
        raise ValueError("q_obs / k shape or dtype mismatch")
    return Desc(Bt, Hq, Hkv, D, S, W, n_sink, int(bool(causal)), _dtype_code(k), float(scale))


def desc_of(batch, n_q_heads, n_kv_heads, head_dim, seq_len, obs_window, *, n_sink=0,
            causal=True, dtype=torch.bfloat16, scale=0.0) -> Desc:
    return Desc(batch, n_q_heads, n_kv_heads, head_dim, seq_len, obs_window, n_sink,
                int(bool(causal)), BF16 if dtype == torch.bfloat16 else F32, float(scale))


def score_workspace_bytes(desc: Desc) -> int:
    return int(lib().kvsel_score_workspace(ctypes.byref(desc)))


def select_workspace_bytes(desc: Desc, budget: int) -> int:
    return int(lib().kvsel_select_workspace(ctypes.byref(desc), int(budget)))


def score(q_obs: torch.Tensor, k: torch.Tensor, *, pool_kernel: int, n_sink: int = 0,
          causal: bool = True, scale: float = 0.0, pooled: Optional[torch.Tensor] = None,
          raw: Optional[torch.Tensor] = None, want_raw: bool = True,
          want_pooled: bool = True, workspace: Optional[torch.Tensor] = None, stream=None):
    """kvsel_score: returns (pooled [Bt,Hkv,S] fp32 or None, raw [Bt,Hkv,S] fp32 or
    None).  want_pooled=False skips the max filter (raw scores only)."""
    with _on(stream):
        d = make_desc(q_obs, k, n_sink=n_sink, causal=causal, scale=scale)
        shape = (d.batch, d.n_kv_heads, d.seq_len)
        if not want_pooled:
            pooled = None
            want_raw = True
        elif pooled is None:
            pooled = torch.empty(shape, dtype=torch.float32, device=k.device)
        if raw is None and want_raw:
            raw = torch.empty(shape, dtype=torch.float32, device=k.device)
        nbytes = score_workspace_bytes(d)
        if workspace is None:
            workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=k.device)
        st = lib().kvsel_score(ctypes.byref(d), _ptr(q_obs), _ptr(k), _ptr(raw), _ptr(pooled),
                               int(pool_kernel), _ptr(workspace), workspace.numel(),
                               _stream(stream))
        _check(st, "kvsel_score")
        return pooled, raw


def select(pooled: torch.Tensor, budget: int, *, obs_window: int, n_q_heads: int,
           head_dim: int, n_sink: int = 0, causal: bool = True,
           idx: Optional[torch.Tensor] = None, dtype=torch.bfloat16,
           workspace: Optional[torch.Tensor] = None, stream=None):
    """kvsel_select: returns idx [Bt,Hkv,budget+n_sink+W] int32 (ascending)."""
    with _on(stream):
        Bt, Hkv, S = pooled.shape
        d = desc_of(Bt, n_q_heads, Hkv, head_dim, S, obs_window, n_sink=n_sink, causal=causal,
                    dtype=dtype)
        n_keep = budget + n_sink + obs_window
        if idx is None:
            idx = torch.empty((Bt, Hkv, max(n_keep, 0)), dtype=torch.int32, device=pooled.device)
        nbytes = select_workspace_bytes(d, budget)
        if workspace is None and nbytes > 0:
            workspace = torch.empty(nbytes, dtype=torch.uint8, device=pooled.device)
        ws_ptr = _ptr(workspace) if workspace is not None else None
        ws_n = workspace.numel() if workspace is not None else 0
        st = lib().kvsel_select(ctypes.byref(d), _ptr(pooled), int(budget), _ptr(idx), ws_ptr, ws_n,
                                _stream(stream))
        _check(st, "kvsel_select")
        return idx


def compact(k: torch.Tensor, v: Optional[torch.Tensor], idx: torch.Tensor, *,
            k_out: Optional[torch.Tensor] = None, v_out: Optional[torch.Tensor] = None,
            stream=None):
    """kvsel_compact: returns (k_hat, v_hat) [Bt,Hkv,n_keep,D]."""
    with _on(stream):
        Bt, Hkv, S, D = k.shape
        n_keep = idx.shape[-1]
        d = Desc(Bt, Hkv, Hkv, D, S, 1, 0, 1, _dtype_code(k), 0.0)
        if k_out is None:
            k_out = torch.empty((Bt, Hkv, n_keep, D), dtype=k.dtype, device=k.device)
        if v is not None and v_out is None:
            v_out = torch.empty((Bt, Hkv, n_keep, D), dtype=v.dtype, device=v.device)
        st = lib().kvsel_compact(ctypes.byref(d), _ptr(k), _ptr(v), _ptr(idx), int(n_keep),
                                 _ptr(k_out), _ptr(v_out), _stream(stream))
        _check(st, "kvsel_compact")
        return k_out, v_out


def select_compact(pooled: torch.Tensor, k: torch.Tensor, v: Optional[torch.Tensor],
                   budget: int, *, obs_window: int, n_q_heads: int, n_sink: int = 0,
                   causal: bool = True, idx: Optional[torch.Tensor] = None,
                   k_out: Optional[torch.Tensor] = None, v_out: Optional[torch.Tensor] = None,
                   workspace: Optional[torch.Tensor] = None, stream=None):
    """kvsel_select_compact: returns (idx, k_hat, v_hat), the outputs of
    select() followed by compact()."""
    with _on(stream):
        Bt, Hkv, S, D = k.shape
        d = Desc(Bt, n_q_heads, Hkv, D, S, obs_window, n_sink, int(causal), _dtype_code(k), 0.0)
        n_keep = budget + n_sink + obs_window
        if idx is None:
            idx = torch.empty((Bt, Hkv, n_keep), dtype=torch.int32, device=k.device)
        if k_out is None:
            k_out = torch.empty((Bt, Hkv, n_keep, D), dtype=k.dtype, device=k.device)
        if v is not None and v_out is None:
            v_out = torch.empty((Bt, Hkv, n_keep, D), dtype=v.dtype, device=v.device)
        if workspace is None:
            workspace = torch.empty(max(select_workspace_bytes(d, budget), 1), dtype=torch.uint8,
                                    device=k.device)
        st = lib().kvsel_select_compact(ctypes.byref(d), _ptr(pooled), int(budget), _ptr(idx),
                                        _ptr(k), _ptr(v), _ptr(k_out), _ptr(v_out),
                                        _ptr(workspace), workspace.numel(), _stream(stream))
        _check(st, "kvsel_select_compact")
        return idx, k_out, v_out


def select_adaptive_workspace_bytes(desc: Desc, total_budget: int) -> int:
    return int(lib().kvsel_select_adaptive_workspace(ctypes.byref(desc), int(total_budget)))


def select_adaptive(pooled: torch.Tensor, total_budget: int, *, obs_window: int,
                    n_q_heads: int, head_dim: int, n_sink: int = 0, causal: bool = True,
                    idx: Optional[torch.Tensor] = None, head_off: Optional[torch.Tensor] = None,
                    dtype=torch.bfloat16, workspace: Optional[torch.Tensor] = None, stream=None):
    """kvsel_select_adaptive: returns (idx [Bt, Hkv*(n_sink+W)+total_budget] int32,
    head_off [Bt, Hkv+1] int32)."""
    with _on(stream):
        Bt, Hkv, S = pooled.shape
        d = desc_of(Bt, n_q_heads, Hkv, head_dim, S, obs_window, n_sink=n_sink, causal=causal,
                    dtype=dtype)
        n_keep = Hkv * (n_sink + obs_window) + total_budget
        if idx is None:
            idx = torch.empty((Bt, max(n_keep, 0)), dtype=torch.int32, device=pooled.device)
        if head_off is None:
            head_off = torch.empty((Bt, Hkv + 1), dtype=torch.int32, device=pooled.device)
        nbytes = select_adaptive_workspace_bytes(d, total_budget)
        if workspace is None and nbytes > 0:
            workspace = torch.empty(nbytes, dtype=torch.uint8, device=pooled.device)
        ws_ptr = _ptr(workspace) if workspace is not None else None
        ws_n = workspace.numel() if workspace is not None else 0
        st = lib().kvsel_select_adaptive(ctypes.byref(d), _ptr(pooled), int(total_budget),
                                         _ptr(idx), _ptr(head_off), ws_ptr, ws_n,
                                         _stream(stream))
        _check(st, "kvsel_select_adaptive")
        return idx, head_off


def compact_flat(k: torch.Tensor, v: Optional[torch.Tensor], idx: torch.Tensor,
                 head_off: torch.Tensor, *, k_out: Optional[torch.Tensor] = None,
                 v_out: Optional[torch.Tensor] = None, stream=None):
    """kvsel_compact_flat: returns (k_hat, v_hat) [Bt, n_keep, D]."""
    with _on(stream):
        Bt, Hkv, S, D = k.shape
        n_keep = idx.shape[-1]
        d = Desc(Bt, Hkv, Hkv, D, S, 1, 0, 1, _dtype_code(k), 0.0)
        if k_out is None:
            k_out = torch.empty((Bt, n_keep, D), dtype=k.dtype, device=k.device)
        if v is not None and v_out is None:
            v_out = torch.empty((Bt, n_keep, D), dtype=v.dtype, device=v.device)
        st = lib().kvsel_compact_flat(ctypes.byref(d), _ptr(k), _ptr(v), _ptr(idx), _ptr(head_off),
                                      int(n_keep), _ptr(k_out), _ptr(v_out), _stream(stream))
        _check(st, "kvsel_compact_flat")
        return k_out, v_out


def layer_end_workspace_bytes(desc: Desc, budget: int) -> int:
    return int(lib().kvsel_layer_end_workspace(ctypes.byref(desc), int(budget)))


def layer_end(q_obs: torch.Tensor, k: torch.Tensor, v: Optional[torch.Tensor], *, budget: int,
              pool_kernel: int, n_sink: int = 0, causal: bool = True, scale: float = 0.0,
              raw: Optional[torch.Tensor] = None, pooled: Optional[torch.Tensor] = None,
              idx: Optional[torch.Tensor] = None, k_out: Optional[torch.Tensor] = None,
              v_out: Optional[torch.Tensor] = None, want_scores: bool = True,
              workspace: Optional[torch.Tensor] = None, stream=None):
    """kvsel_layer_end: TideKV's LayerEndCompress in one call.  Returns
    (idx, k_hat, v_hat, raw, pooled); raw and pooled are None when
    want_scores is False and none were given (then kept in the workspace)."""
    # the stream context only when something is allocated here (a caller
    # that passes every buffer, like the layer-major driver, pays nothing)
    alloc = (want_scores and (raw is None or pooled is None)) or idx is None or k_out is None \
        or (v is not None and v_out is None) or workspace is None
    with (_on(stream) if alloc else nullcontext()):
        d = make_desc(q_obs, k, n_sink=n_sink, causal=causal, scale=scale)
        Bt, Hkv, S, D = k.shape
        n_keep = budget + n_sink + q_obs.shape[2]
        dev = k.device
        if want_scores:
            raw = torch.empty((Bt, Hkv, S), dtype=torch.float32, device=dev) if raw is None \
                else raw
            pooled = torch.empty_like(raw) if pooled is None else pooled
        if idx is None:
            idx = torch.empty((Bt, Hkv, n_keep), dtype=torch.int32, device=dev)
        if k_out is None:
            k_out = torch.empty((Bt, Hkv, n_keep, D), dtype=k.dtype, device=dev)
        if v is not None and v_out is None:
            v_out = torch.empty((Bt, Hkv, n_keep, D), dtype=v.dtype, device=dev)
        if workspace is None:
            workspace = torch.empty(max(layer_end_workspace_bytes(d, budget), 1),
                                    dtype=torch.uint8, device=dev)
        st = lib().kvsel_layer_end(ctypes.byref(d), _ptr(q_obs), _ptr(k), _ptr(v), int(budget),
                                   int(pool_kernel), _ptr(raw), _ptr(pooled), _ptr(idx),
                                   _ptr(k_out), _ptr(v_out), _ptr(workspace), workspace.numel(),
                                   _stream(stream))
        _check(st, "kvsel_layer_end")
        return idx, k_out, v_out, raw, pooled


def layer_end_stream_workspace_bytes(desc: Desc, budget: int, pool_kernel: int) -> int:
    return int(lib().kvsel_layer_end_stream_workspace(ctypes.byref(desc), int(budget),
                                                      int(pool_kernel)))


def layer_end_stream(q_obs: torch.Tensor, k: torch.Tensor, v: Optional[torch.Tensor], *,
                     budget: int, pool_kernel: int, n_sink: int = 0, causal: bool = True,
                     scale: float = 0.0, idx: Optional[torch.Tensor] = None,
                     k_out: Optional[torch.Tensor] = None, v_out: Optional[torch.Tensor] = None,
                     workspace: Optional[torch.Tensor] = None, stream=None):
    """kvsel_layer_end_stream: the layer-end step with the streaming top-k of
    pass 2 (no per-key score vector).  Returns (idx, k_hat, v_hat)."""
    alloc = idx is None or k_out is None or (v is not None and v_out is None) or workspace is None
    with (_on(stream) if alloc else nullcontext()):
        d = make_desc(q_obs, k, n_sink=n_sink, causal=causal, scale=scale)
        Bt, Hkv, S, D = k.shape
        n_keep = budget + n_sink + q_obs.shape[2]
        dev = k.device
        if idx is None:
            idx = torch.empty((Bt, Hkv, n_keep), dtype=torch.int32, device=dev)
        if k_out is None:
            k_out = torch.empty((Bt, Hkv, n_keep, D), dtype=k.dtype, device=dev)
        if v is not None and v_out is None:
            v_out = torch.empty((Bt, Hkv, n_keep, D), dtype=v.dtype, device=dev)
        if workspace is None:
            nbytes = layer_end_stream_workspace_bytes(d, budget, pool_kernel)
            workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
        st = lib().kvsel_layer_end_stream(ctypes.byref(d), _ptr(q_obs), _ptr(k), _ptr(v),
                                          int(budget), int(pool_kernel), _ptr(idx), _ptr(k_out),
                                          _ptr(v_out), _ptr(workspace), workspace.numel(),
                                          _stream(stream))
        _check(st, "kvsel_layer_end_stream")
        return idx, k_out, v_out


def layer_end_adaptive_workspace_bytes(desc: Desc, total_budget: int) -> int:
    return int(lib().kvsel_layer_end_adaptive_workspace(ctypes.byref(desc), int(total_budget)))


def layer_end_adaptive(q_obs: torch.Tensor, k: torch.Tensor, v: Optional[torch.Tensor], *,
                       total_budget: int, pool_kernel: int, n_sink: int = 0, causal: bool = True,
                       scale: float = 0.0, raw: Optional[torch.Tensor] = None,
                       pooled: Optional[torch.Tensor] = None, idx: Optional[torch.Tensor] = None,
                       head_off: Optional[torch.Tensor] = None,
                       k_out: Optional[torch.Tensor] = None, v_out: Optional[torch.Tensor] = None,
                       want_scores: bool = True, workspace: Optional[torch.Tensor] = None,
                       stream=None):
    """kvsel_layer_end_adaptive: the layer-end step with one head-adaptive
    budget per sequence, into the flattened cache.  Returns (idx [Bt, n_keep],
    head_off [Bt, Hkv+1], k_hat, v_hat [Bt, n_keep, D], raw, pooled) with
    n_keep = Hkv*(n_sink+W) + total_budget; raw and pooled are None when
    want_scores is False and none were given."""
    alloc = (want_scores and (raw is None or pooled is None)) or idx is None or \
        head_off is None or k_out is None or (v is not None and v_out is None) or \
        workspace is None
    with (_on(stream) if alloc else nullcontext()):
        d = make_desc(q_obs, k, n_sink=n_sink, causal=causal, scale=scale)
        Bt, Hkv, S, D = k.shape
        n_keep = Hkv * (n_sink + q_obs.shape[2]) + total_budget
        dev = k.device
        if want_scores:
            raw = torch.empty((Bt, Hkv, S), dtype=torch.float32, device=dev) if raw is None \
                else raw
            pooled = torch.empty_like(raw) if pooled is None else pooled
        if idx is None:
            idx = torch.empty((Bt, max(n_keep, 0)), dtype=torch.int32, device=dev)
        if head_off is None:
            head_off = torch.empty((Bt, Hkv + 1), dtype=torch.int32, device=dev)
        if k_out is None:
            k_out = torch.empty((Bt, max(n_keep, 0), D), dtype=k.dtype, device=dev)
        if v is not None and v_out is None:
            v_out = torch.empty((Bt, max(n_keep, 0), D), dtype=v.dtype, device=dev)
        if workspace is None:
            workspace = torch.empty(max(layer_end_adaptive_workspace_bytes(d, total_budget), 1),
                                    dtype=torch.uint8, device=dev)
        st = lib().kvsel_layer_end_adaptive(ctypes.byref(d), _ptr(q_obs), _ptr(k), _ptr(v),
                                            int(total_budget), int(pool_kernel), _ptr(raw),
                                            _ptr(pooled), _ptr(idx), _ptr(head_off), _ptr(k_out),
                                            _ptr(v_out), _ptr(workspace), workspace.numel(),
                                            _stream(stream))
        _check(st, "kvsel_layer_end_adaptive")
        return idx, head_off, k_out, v_out, raw, pooled


def layer_end_compress(q_obs: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, budget: int,
                       pool_kernel: int, n_sink: int = 0, causal: bool = True,
                       scale: float = 0.0, stream=None) -> dict:
    """TideKV's layer-end step (kvsel_layer_end) on one stream, as a dict."""
    idx, k_hat, v_hat, raw, pooled = layer_end(q_obs, k, v, budget=budget,
                                               pool_kernel=pool_kernel, n_sink=n_sink,
                                               causal=causal, scale=scale, stream=stream)
    return {"s": raw, "p": pooled, "idx": idx, "k_hat": k_hat, "v_hat": v_hat}


def layer_end_compress_adaptive(q_obs: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *,
                                total_budget: int, pool_kernel: int, n_sink: int = 0,
                                causal: bool = True, scale: float = 0.0, stream=None) -> dict:
    """The head-adaptive layer-end step (kvsel_layer_end_adaptive) on one
    stream, as a dict."""
    idx, off, k_hat, v_hat, raw, pooled = layer_end_adaptive(
        q_obs, k, v, total_budget=total_budget, pool_kernel=pool_kernel, n_sink=n_sink,
        causal=causal, scale=scale, stream=stream)
    return {"s": raw, "p": pooled, "idx": idx, "head_off": off, "k_hat": k_hat, "v_hat": v_hat}


def kara_desc(q_win: torch.Tensor, k_win: torch.Tensor, *, buffer: int, keep: int, gamma: int,
              alpha: int, scale: float = 0.0) -> KaraDesc:
    Bt, Hq, Wn, D = q_win.shape
    return KaraDesc(Bt, Hq, k_win.shape[1], D, Wn, int(buffer), int(keep), int(gamma),
                    int(alpha), _dtype_code(k_win), float(scale))


def kara_keep(window: int, buffer: int, ratio) -> int:
    """kvsel_kara_keep: |I| = ceil(r * (|W| - |U|)) of Kara Eq. (5), computed
    exactly by the library.  `ratio` is a fraction (num, den), a
    fractions.Fraction, or a number, which is read as the nearest fraction
    with a denominator of at most 10**6 (0.4 -> 2/5)."""
    if isinstance(ratio, tuple):
        num, den = ratio
    else:
        f = Fraction(ratio).limit_denominator(10 ** 6)
        num, den = f.numerator, f.denominator
    n = lib().kvsel_kara_keep(int(window), int(buffer), int(num), int(den))
    if n < 0:
        raise ValueError(f"kvsel_kara_keep: invalid window {window}, buffer {buffer} or "
                         f"ratio {num}/{den}")
    return int(n)


def kara_score_workspace_bytes(kd: KaraDesc) -> int:
    return int(lib().kvsel_kara_score_workspace(ctypes.byref(kd)))


def kara_score(q_win: torch.Tensor, k_win: torch.Tensor, kd: KaraDesc, *,
               scores: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
               stream=None) -> torch.Tensor:
    """kvsel_kara_score: importance [Bt,Hkv,window-buffer] float32."""
    with _on(stream):
        n = kd.window - kd.buffer
        if scores is None:
            scores = torch.empty((kd.batch, kd.n_kv_heads, n), dtype=torch.float32,
                                 device=k_win.device)
        nbytes = kara_score_workspace_bytes(kd)
        if workspace is None:
            workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=k_win.device)
        st = lib().kvsel_kara_score(ctypes.byref(kd), _ptr(q_win), _ptr(k_win), _ptr(scores),
                                    _ptr(workspace), workspace.numel(), _stream(stream))
        _check(st, "kvsel_kara_score")
        return scores


def kara_select(scores: torch.Tensor, kd: KaraDesc, *, idx: Optional[torch.Tensor] = None,
                stream=None) -> torch.Tensor:
    """kvsel_kara_select: window-relative kept positions [Bt,Hkv,n_out+buffer]."""
    with _on(stream):
        n = kd.window - kd.buffer
        n_out = min(n, kd.keep + kd.alpha)
        if idx is None:
            idx = torch.empty((kd.batch, kd.n_kv_heads, n_out + kd.buffer), dtype=torch.int32,
                              device=scores.device)
        st = lib().kvsel_kara_select(ctypes.byref(kd), _ptr(scores), _ptr(idx), _stream(stream))
        _check(st, "kvsel_kara_select")
        return idx


def kara_compress(q_win: torch.Tensor, k_win: torch.Tensor, v_win: torch.Tensor, *,
                  buffer: int, ratio: float, gamma: int, alpha: int, stream=None) -> dict:
    """One Kara window compression: score -> Token2Chunk select -> gather."""
    kd = kara_desc(q_win, k_win, buffer=buffer, keep=kara_keep(q_win.shape[2], buffer, ratio),
                   gamma=gamma, alpha=alpha)
    A = kara_score(q_win, k_win, kd, stream=stream)
    idx = kara_select(A, kd, stream=stream)
    k_hat, v_hat = compact(k_win, v_win, idx, stream=stream)
    return {"A": A, "idx": idx, "k_hat": k_hat, "v_hat": v_hat, "desc": kd}


@dataclass
class TierOutputs:
    tier: torch.Tensor
    rank: torch.Tensor
    k_full: torch.Tensor
    v_full: torch.Tensor
    k_codes: torch.Tensor
    v_codes: torch.Tensor
    k_meta: torch.Tensor
    v_meta: torch.Tensor
    k_prom: torch.Tensor
    v_prom: torch.Tensor


def route_tiers_workspace_bytes(td: TierDesc) -> int:
    return int(lib().kvsel_route_tiers_workspace(ctypes.byref(td)))


def route_tiers(scores: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, n_full: int,
                n_quant: int, win: int = 64, promote: Optional[torch.Tensor] = None,
                out: Optional[TierOutputs] = None, workspace: Optional[torch.Tensor] = None,
                stream=None) -> TierOutputs:
    """kvsel_route_tiers (QEvict window tiers with int4 and promotion)."""
    with _on(stream):
        Bt, Hkv, S, D = k.shape
        td = TierDesc(Bt, Hkv, D, S, win, n_full, n_quant, _dtype_code(k))
        nW = S // win
        n_prom = 0 if promote is None else promote.shape[-1]
        dev = k.device
        if out is None:
            e = lambda *s, dt: torch.empty(s, dtype=dt, device=dev)  # noqa: E731
            out = TierOutputs(
                e(Bt, Hkv, nW, dt=torch.int8), e(Bt, Hkv, nW, dt=torch.int32),
                e(Bt, Hkv, n_full * win, D, dt=k.dtype), e(Bt, Hkv, n_full * win, D, dt=k.dtype),
                e(Bt, Hkv, n_quant, win, D // 2, dt=torch.uint8),
                e(Bt, Hkv, n_quant, win, D // 2, dt=torch.uint8),
                e(Bt, Hkv, n_quant, D, 2, dt=torch.float32),
                e(Bt, Hkv, n_quant, D, 2, dt=torch.float32),
                e(Bt, Hkv, n_prom * win, D, dt=k.dtype), e(Bt, Hkv, n_prom * win, D, dt=k.dtype))
        nbytes = route_tiers_workspace_bytes(td)
        if workspace is None:
            workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
        nz = lambda t: _ptr(t) if t is not None and t.numel() > 0 else None  # noqa: E731
        st = lib().kvsel_route_tiers(
            ctypes.byref(td), _ptr(scores), _ptr(k), _ptr(v), _ptr(out.tier), _ptr(out.rank),
            nz(out.k_full), nz(out.v_full), nz(out.k_codes), nz(out.v_codes), nz(out.k_meta),
            nz(out.v_meta), nz(promote), int(n_prom), nz(out.k_prom), nz(out.v_prom),
            _ptr(workspace), workspace.numel(), _stream(stream))
        _check(st, "kvsel_route_tiers")
        return out
EXPORTS = ("kvsel_status_str", "kvsel_score_workspace", "kvsel_score", "kvsel_select_workspace",
           "kvsel_select", "kvsel_compact", "kvsel_route_tiers_workspace", "kvsel_route_tiers",
           "kvsel_select_adaptive_workspace", "kvsel_select_adaptive", "kvsel_compact_flat",
           "kvsel_kara_score_workspace", "kvsel_kara_score", "kvsel_kara_select",
           "kvsel_qevict_step_workspace", "kvsel_qevict_step", "kvsel_select_compact",
           "kvsel_kara_keep", "kvsel_timing_start", "kvsel_timing_read", "kvsel_score_static",
           "kvsel_layer_end_workspace", "kvsel_layer_end", "kvsel_layer_end_stream_workspace",
           "kvsel_layer_end_stream", "kvsel_layer_end_adaptive_workspace",
           "kvsel_layer_end_adaptive")

STATIC_SCRATCH_BYTES = 32 << 20   # KVSEL_STATIC_SCRATCH_BYTES


def score_static(q_obs: torch.Tensor, k: torch.Tensor, *, pooled: torch.Tensor,
                 raw: Optional[torch.Tensor] = None, pool_kernel: int, n_sink: int = 0,
                 causal: bool = True, scale: float = 0.0, stream=None):
    """kvsel_score_static: kvsel_score into caller-provided outputs with the
    library's static scratch; allocates nothing (usable under graph capture).
    Calls that overlap on one GPU race on the shared scratch."""
    d = make_desc(q_obs, k, n_sink=n_sink, causal=causal, scale=scale)
    st = lib().kvsel_score_static(ctypes.byref(d), _ptr(q_obs), _ptr(k), _ptr(raw),
                                  _ptr(pooled), int(pool_kernel), _stream(stream))
    _check(st, "kvsel_score_static")
    return pooled, raw


def timing_start(prefix: Optional[str] = "*") -> None:
    """kvsel_timing_start: bracket every later launch of a kernel whose name
    starts with `prefix` ("*" = all, None = stop) with HIP events."""
    _check(lib().kvsel_timing_start(prefix.encode() if prefix else None), "kvsel_timing_start")


def timing_read(max_kernels: int = 64) -> dict:
    """kvsel_timing_read: {kernel name: (total ms, launches)} since the last
    read; waits for the recorded events."""
    nb = 96
    names = ctypes.create_string_buffer(nb * max_kernels)
    ms = (ctypes.c_double * max_kernels)()
    cnt = (ctypes.c_int32 * max_kernels)()
    n = lib().kvsel_timing_read(names, nb, ms, cnt, max_kernels)
    if n < 0:
        raise RuntimeError(f"kvsel_timing_read failed ({n})")
    out = {}
    for i in range(min(n, max_kernels)):
        nm = names.raw[i * nb:(i + 1) * nb].split(b"\0", 1)[0].decode()
        out[nm] = (float(ms[i]), int(cnt[i]))
    return out


# ---------------------------------------------------------------------------
# Repeated recoverable routing (kvsel_qevict_step)
# ---------------------------------------------------------------------------


def qevict_desc(k: torch.Tensor, *, seq_len: int, max_windows: int, n_sink: int,
                n_recent: int, n_full: int, n_quant: int, bits: int = 2,
                win: int = 64) -> QevictDesc:
    """Descriptor for a cache k [Bt, Hkv, capacity, D] (bf16).  `win` is
    passed through as given; the library decides which window lengths it
    supports (KVSEL_ERR_UNSUPPORTED otherwise)."""
    Bt, Hkv, cap, D = k.shape
    return QevictDesc(Bt, Hkv, D, int(seq_len), cap, int(max_windows), int(win), int(n_sink),
                      int(n_recent), int(n_full), int(n_quant), int(bits), _dtype_code(k))


def qevict_state(qd: QevictDesc, device) -> dict:
    """Zeroed routing state: every window full precision, no backing-store
    entry, accumulated score 0."""
    Bt, H, M, D = qd.batch, qd.n_kv_heads, qd.max_windows, qd.head_dim
    z = lambda shape, dt: torch.zeros(shape, dtype=dt, device=device)  # noqa: E731
    return {
        "w_acc": z((Bt, H, M), torch.float32),
        "tier": z((Bt, H, M), torch.int8),
        "has_codes": z((Bt, H, M), torch.uint8),
        "k_codes": z((Bt, H, M, qd.win, D * qd.bits // 8), torch.uint8),
        "v_codes": z((Bt, H, M, qd.win, D * qd.bits // 8), torch.uint8),
        "k_meta": z((Bt, H, M, D, 2), torch.float32),
        "v_meta": z((Bt, H, M, D, 2), torch.float32),
    }


def qevict_step_workspace_bytes(qd: QevictDesc) -> int:
    return int(lib().kvsel_qevict_step_workspace(ctypes.byref(qd)))


def qevict_step(qd: QevictDesc, token_scores: torch.Tensor, state: dict, k: torch.Tensor,
                v: torch.Tensor, *, workspace: Optional[torch.Tensor] = None,
                stream=None) -> dict:
    """kvsel_qevict_step: updates state (and promoted rows of k, v) in place."""
    with _on(stream):
        if workspace is None:
            workspace = torch.empty(max(qevict_step_workspace_bytes(qd), 1), dtype=torch.uint8,
                                    device=k.device)
        st = lib().kvsel_qevict_step(
            ctypes.byref(qd), _ptr(token_scores), _ptr(state["w_acc"]), _ptr(state["tier"]),
            _ptr(state["has_codes"]), _ptr(k), _ptr(v), _ptr(state["k_codes"]),
            _ptr(state["v_codes"]), _ptr(state["k_meta"]), _ptr(state["v_meta"]), _ptr(workspace),
            workspace.numel(), _stream(stream))
        _check(st, "kvsel_qevict_step")
        return state
