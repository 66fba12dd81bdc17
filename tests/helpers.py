"""Shared test helpers: moving seeded numpy inputs onto the device and the
comparison rules used by the parity tests.  No method arithmetic lives here."""
from __future__ import annotations

import numpy as np

import synth


def dev_tensor(arr: np.ndarray, dtype: str, device="cuda"):
    """numpy bf16 bits (uint16) or float32 -> torch tensor on the device."""
    import torch
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32))
    return t.to(device)


def host_bits(t) -> np.ndarray:
    """Device tensor -> numpy array of its raw bits (uint16 for bf16)."""
    import torch
    c = t.detach().cpu().contiguous()
    if c.dtype == torch.bfloat16:
        return c.view(torch.int16).numpy().view(np.uint16)
    return c.numpy()


def assert_scores_close(gpu: np.ndarray, ref: np.ndarray, rtol: float = 1e-3, what: str = ""):
    """Element-wise relative tolerance |g - r| <= rtol * |r| (exact zeros must match)."""
    gpu = np.asarray(gpu, dtype=np.float64)
    err = np.abs(gpu - ref)
    bad = err > rtol * np.abs(ref)
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(
            f"{what}: {int(bad.sum())} elements off; first at {tuple(i)}: gpu={gpu[tuple(i)]!r} "
            f"oracle={ref[tuple(i)]!r}; max rel err {np.max(err / np.maximum(np.abs(ref), 1e-300)):.3e}")


def check_selection(idx_gpu: np.ndarray, p_ref: np.ndarray, budget: int, n_sink: int, W: int,
                    band: float = 1e-4):
    """The GPU's retained set equals the oracle's except at candidates whose
    oracle score lies within `band` (relative) of the budget-th score; it is
    ascending, holds the mandatory set and has exactly budget+n_sink+W entries."""
    S = p_ref.shape[-1]
    lo, hi = n_sink, S - W
    rows_g = idx_gpu.reshape(-1, idx_gpu.shape[-1])
    rows_p = p_ref.reshape(-1, S)
    for r in range(rows_g.shape[0]):
        g = rows_g[r].astype(np.int64)
        assert g.shape[0] == budget + n_sink + W
        assert (np.diff(g) > 0).all(), f"row {r}: not strictly ascending"
        assert g[:n_sink].tolist() == list(range(n_sink)), f"row {r}: sinks missing"
        assert g[n_sink + budget:].tolist() == list(range(hi, S)), f"row {r}: window missing"
        picks = g[n_sink:n_sink + budget]
        assert ((picks >= lo) & (picks < hi)).all()
        if budget == 0:
            continue
        cand = rows_p[r, lo:hi]
        kth = np.sort(cand)[::-1][budget - 1]
        sure_in = np.flatnonzero(cand > kth * (1 + band)) + lo
        sure_out = np.flatnonzero(cand < kth * (1 - band)) + lo
        ps = set(picks.tolist())
        missing = [i for i in sure_in.tolist() if i not in ps]
        extra = [i for i in sure_out.tolist() if i in ps]
        assert not missing, f"row {r}: clearly-kept positions missing: {missing[:10]}"
        assert not extra, f"row {r}: clearly-dropped positions kept: {extra[:10]}"


def layer_inputs(spec: synth.LayerSpec, config_id: int, layer: int = 0, want_v: bool = True):
    x = synth.make_layer(spec, config_id, layer, want_v=want_v)
    return x
