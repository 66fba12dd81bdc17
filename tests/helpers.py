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


def check_adaptive_selection(idx_g: np.ndarray, off_g: np.ndarray, p_ref: np.ndarray,
                             total: int, n_sink: int, W: int, band: float = 1e-4):
    """Head-adaptive selection in the flattened layout: per-head segments are
    ascending, hold their head's mandatory set, and the picks over all heads
    of a sequence equal the oracle's except at candidates whose oracle score
    lies within `band` (relative) of the sequence's total-th score."""
    Bt, H, S = p_ref.shape
    lo, hi = n_sink, S - W
    n_keep = H * (n_sink + W) + total
    assert idx_g.shape == (Bt, n_keep) and off_g.shape == (Bt, H + 1)
    for b in range(Bt):
        off = off_g[b].astype(np.int64)
        assert off[0] == 0 and off[H] == n_keep and (np.diff(off) >= n_sink + W).all()
        picked = np.zeros((H, S), bool)
        for h in range(H):
            g = idx_g[b, off[h]:off[h + 1]].astype(np.int64)
            assert (np.diff(g) > 0).all(), f"seq {b} head {h}: not ascending"
            assert g[:n_sink].tolist() == list(range(n_sink))
            assert g[g.size - W:].tolist() == list(range(hi, S))
            picks = g[n_sink:g.size - W]
            assert ((picks >= lo) & (picks < hi)).all()
            picked[h, picks] = True
        assert picked.sum() == total
        if total == 0:
            continue
        cand = p_ref[b, :, lo:hi]
        kth = np.sort(cand.reshape(-1))[::-1][total - 1]
        sure_in = cand > kth * (1 + band)
        sure_out = cand < kth * (1 - band)
        got = picked[:, lo:hi]
        assert not (sure_in & ~got).any(), f"seq {b}: clearly-kept candidates missing"
        assert not (sure_out & got).any(), f"seq {b}: clearly-dropped candidates kept"


def rows_gathered(out_bits: np.ndarray, src_bits: np.ndarray, idx: np.ndarray,
                  head_off: np.ndarray = None) -> bool:
    """Every output row is the source row its index names, byte for byte
    (per-head layout [Bt,Hkv,n,D], or flattened [Bt,n,D] with head offsets)."""
    if head_off is None:
        want = np.take_along_axis(src_bits, idx.astype(np.int64)[..., None], axis=2)
        return out_bits.tobytes() == want.tobytes()
    H = src_bits.shape[1]
    for b in range(idx.shape[0]):
        for h in range(H):
            r0, r1 = int(head_off[b, h]), int(head_off[b, h + 1])
            if out_bits[b, r0:r1].tobytes() != src_bits[b, h, idx[b, r0:r1]].tobytes():
                return False
    return True


def layer_inputs(spec: synth.LayerSpec, config_id: int, layer: int = 0, want_v: bool = True):
    x = synth.make_layer(spec, config_id, layer, want_v=want_v)
    return x
