"""Dense float64 definitions of the layer-end selection path.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources (the pages' titles; section / equation / algorithm of each):

* TideKV -- "Delayed KV Eviction via Layer-Wise Chunked Prefill for
  Memory-Efficient Long-Context LLM Inference": §4.2 Eqs. (4)-(8),
  Algorithm 2 (LayerEndCompress), §4.3 memory model, §6.1 setup.
* QEvict -- "Recoverable Quantized KV Eviction for Attention-Drift-Robust
  Long-Context Decoding": §4.1 protected regions and windows, §4.2
  cumulative window scoring repeated every Omega tokens, §4.3 recoverable
  hierarchy, Appendix A routing, §1 persistent backing store, §B.5 defaults
  (INT2 tier, five sinks).
* Kara -- "Kara: Efficient Reasoning LLM Serving via Sliding-Window KV Cache
  Compression": §3.1 Eq. (4) bidirectional window scoring, §3.2 Eqs. (5)-(8)
  Token2Chunk and its fill-up rule.

Readings where the pages are silent:
pooling weights w_q = 1; GQA aggregation is a sum over the group with query
head h mapped to KV head floor(h / G); the 1-D max-pool over key positions runs
over the candidate range only, stride 1, window clipped at its edges; ties in
the pooled score are broken by lowest position; the retained set is emitted in
ascending position order; ``budget`` counts non-mandatory picks.  Head-adaptive
selection picks over all KV heads of a sequence with no per-head floor beyond
the mandatory set, ties broken by (head, position) ascending.
"""
from __future__ import annotations

import math

import numpy as np


def default_scale(head_dim: int) -> float:
    """1/sqrt(D), the logit scale of TideKV Eq. (4)."""
    return 1.0 / math.sqrt(head_dim)


def logits(q: np.ndarray, k: np.ndarray, *, causal: bool, scale: float) -> np.ndarray:
    """Observation logits l[q, i] = (Q_q . K_i) * scale   (TideKV Eq. (4)).

    q: [W, D] float64 observation queries, k: [S, D] float64 keys.  With
    ``causal`` the W queries sit at absolute positions S-W .. S-1 and a key past
    the query's own position gets -inf ("logits for keys beyond its causal
    position are set to -inf", §4.2).  Without it (decode queries that follow
    the cache) every key is visible.
    """
    W = q.shape[0]
    S = k.shape[0]
    l = (q @ k.T) * scale
    if causal:
        qpos = (S - W) + np.arange(W)
        future = np.arange(S)[None, :] > qpos[:, None]
        l = np.where(future, -np.inf, l)
    return l


def softmax_rows(l: np.ndarray) -> np.ndarray:
    """a[q, i] = exp(l[q, i] - M_q) / Z_q with M_q = max_i l, Z_q = sum_i exp(l - M_q).

    This is the fixed point of TideKV's two-pass recurrence (Eqs. (5)-(6) give
    M_q and Z_q after the last key block; Eq. (7), left, forms a): computed
    here densely, whole rows at once.
    """
    M = l.max(axis=1, keepdims=True)
    e = np.exp(l - M)
    Z = e.sum(axis=1, keepdims=True)
    return e / Z


def head_scores(q_obs: np.ndarray, k: np.ndarray, *, causal: bool = True,
                scale: float | None = None) -> np.ndarray:
    """Per-KV-head key importance s[b, h_kv, i]   (TideKV Eq. (7), right; §4.2 GQA).

    s = sum over the G query heads of the KV group and over the W window
    queries of a[q, i] (pooling weights w_q = 1).  Query head h belongs to KV
    head floor(h / G).  q_obs: [Bt, Hq, W, D], k: [Bt, Hkv, S, D] (float64).
    Returns float64 [Bt, Hkv, S].  Loops per query head so that only one
    [W, S] logit matrix is alive at a time.
    """
    Bt, Hq, W, D = q_obs.shape
    _, Hkv, S, _ = k.shape
    assert Hq % Hkv == 0 and k.shape[3] == D
    G = Hq // Hkv
    if scale is None:
        scale = default_scale(D)
    s = np.zeros((Bt, Hkv, S), dtype=np.float64)
    for b in range(Bt):
        for h in range(Hq):
            hk = h // G
            a = softmax_rows(logits(q_obs[b, h], k[b, hk], causal=causal, scale=scale))
            s[b, hk] += a.sum(axis=0)
    return s


def max_pool(s: np.ndarray, kernel: int, lo: int, hi: int) -> np.ndarray:
    """1-D max-pool of the key scores along positions over the candidate range.

    p[i] = max{ s[j] : j in [i-h, i+h] and lo <= j < hi },  h = (kernel-1)/2,
    for lo <= i < hi; entries outside [lo, hi) are 0.  This is the smoothing
    step "pool to p_i" of TideKV Algorithm 2 read as a stride-1, same-length
    max filter that does not reach into the mandatory ranges (the pages give
    no kernel; its size comes from the workload).
    """
    assert kernel >= 1 and kernel % 2 == 1
    h = (kernel - 1) // 2
    S = s.shape[-1]
    p = np.zeros_like(s)
    if hi <= lo:
        return p
    ext = np.full(s.shape[:-1] + (S + 2 * h,), -np.inf)
    ext[..., lo + h:hi + h] = s[..., lo:hi]
    best = np.full(s.shape[:-1] + (hi - lo,), -np.inf)
    for off in range(-h, h + 1):
        best = np.maximum(best, ext[..., lo + h + off:hi + h + off])
    p[..., lo:hi] = best
    return p


def select(p: np.ndarray, budget: int, n_sink: int, window: int) -> np.ndarray:
    """Retained positions per (b, h_kv)   (TideKV Eq. (8); Algorithm 2 selection).

    R = Top_budget{ p_i : n_sink <= i < S-W }  U  [0, n_sink)  U  [S-W, S),
    where the mandatory set (sinks and the observation window) is always kept
    and ``budget`` counts the non-mandatory picks, so |R| = budget + n_sink + W.
    Candidates are ordered by (p descending, position ascending); R is returned
    in ascending position order as int32 [Bt, Hkv, budget + n_sink + W].
    """
    S = p.shape[-1]
    lo, hi = n_sink, S - window
    if not (0 <= n_sink and 1 <= window <= S and lo <= hi and 0 <= budget <= hi - lo):
        raise ValueError("infeasible budget / window")
    lead = p.shape[:-1]
    flat = p.reshape(-1, S)
    out = np.empty((flat.shape[0], budget + n_sink + window), dtype=np.int32)
    cand = np.arange(lo, hi)
    for r in range(flat.shape[0]):
        order = np.lexsort((cand, -flat[r, lo:hi]))   # last key is primary
        top = cand[order[:budget]]
        keep = np.concatenate([np.arange(0, lo), top, np.arange(hi, S)])
        keep.sort()
        assert keep.size == budget + n_sink + window
        out[r] = keep
    return out.reshape(lead + (out.shape[1],))


def compact_rows(x: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """Gather retained rows x[b, h, idx[b, h, r], :]   (TideKV Algorithm 2, GATHER).

    x: [Bt, Hkv, S, D] of any dtype (bit patterns are copied unchanged),
    idx: [Bt, Hkv, n]. Returns [Bt, Hkv, n, D].
    """
    return np.take_along_axis(x, idx.astype(np.int64)[..., None], axis=2)


def select_head_adaptive(p: np.ndarray, total_budget: int, n_sink: int, window: int):
    """Head-adaptive retained positions per sequence, in a flattened layout with
    per-head offsets   (TideKV Section 4.1, head-adaptive budget; Eq. (8)
    applied to the union of a sequence's KV heads).

    The sequence's candidates are the pairs (h, i) with n_sink <= i < S-W over
    all of its KV heads; the ``total_budget`` largest pooled scores among them
    are picked, ordered by (p descending, head ascending, position ascending),
    so a head receives as many rows as it has scores above the sequence-wide
    threshold.  Every head still keeps its own mandatory set (sinks and the
    observation window).  Head h's retained positions, ascending, occupy rows
    [off[b, h], off[b, h+1]) of the sequence's flattened index row.

    p: [Bt, Hkv, S].  Returns (idx int32 [Bt, Hkv*(n_sink+W) + total_budget],
    off int32 [Bt, Hkv+1]).
    """
    Bt, H, S = p.shape
    lo, hi = n_sink, S - window
    ncand = hi - lo
    if not (0 <= n_sink and 1 <= window <= S and lo <= hi and 0 <= total_budget <= H * ncand):
        raise ValueError("infeasible budget / window")
    n_keep = H * (n_sink + window) + total_budget
    idx = np.empty((Bt, n_keep), dtype=np.int32)
    off = np.empty((Bt, H + 1), dtype=np.int32)
    heads = np.repeat(np.arange(H), ncand)
    pos = np.tile(np.arange(lo, hi), H)
    for b in range(Bt):
        score = p[b, :, lo:hi].reshape(-1)
        order = np.lexsort((pos, heads, -score))      # last key is primary
        chosen = order[:total_budget]
        at = 0
        for h in range(H):
            mine = pos[chosen[heads[chosen] == h]]
            keep = np.concatenate([np.arange(0, lo), mine, np.arange(hi, S)])
            keep.sort()
            off[b, h] = at
            idx[b, at:at + keep.size] = keep
            at += keep.size
        off[b, H] = at
        assert at == n_keep
    return idx, off


def compact_flat(x: np.ndarray, idx: np.ndarray, off: np.ndarray) -> np.ndarray:
    """Gather a flattened head-adaptive cache: row r of sequence b, with
    off[b, h] <= r < off[b, h+1], is x[b, h, idx[b, r], :]   (TideKV
    Algorithm 2 GATHER into the flattened per-head-offset layout of Section
    4.1).

    x: [Bt, Hkv, S, D] (bit patterns copied unchanged).  Returns [Bt, n, D].
    """
    Bt, H = x.shape[:2]
    n = idx.shape[1]
    out = np.empty((Bt, n, x.shape[3]), dtype=x.dtype)
    for b in range(Bt):
        for h in range(H):
            r0, r1 = int(off[b, h]), int(off[b, h + 1])
            out[b, r0:r1] = x[b, h, idx[b, r0:r1].astype(np.int64)]
    return out


def layer_end_compress(q_obs, k, v, *, budget, window, pool_kernel, n_sink=0,
                       causal=True, scale=None, k_store=None, v_store=None):
    """LayerEndCompress end to end: scores -> pool -> select -> gather.

    q_obs/k are float64 values; k_store/v_store are the stored tensors (bits)
    to gather from (default: k and v themselves).  Returns a dict with s, p,
    idx, k_hat, v_hat.
    """
    S = k.shape[2]
    s = head_scores(q_obs, k, causal=causal, scale=scale)
    p = max_pool(s, pool_kernel, n_sink, S - window)
    idx = select(p, budget, n_sink, window)
    ks = k if k_store is None else k_store
    vs = v if v_store is None else v_store
    return {"s": s, "p": p, "idx": idx,
            "k_hat": compact_rows(ks, idx), "v_hat": compact_rows(vs, idx)}


# ---------------------------------------------------------------------------
# Kara: sliding-window bidirectional scoring and Token2Chunk
# ---------------------------------------------------------------------------

def kara_scores(q_win: np.ndarray, k_comp: np.ndarray, scale: float | None = None) -> np.ndarray:
    """Importance A_j of each compressible key of a decode window   (Kara,
    Section 3.1, Eq. 4): every query of the window (bidirectional: no causal
    mask) takes a softmax over the compressible keys (W minus U) only, and A_j sums
    the weights key j receives over the window's queries and, per KV head,
    over the GQA group (the same group reading as head_scores).

    q_win: [Bt, Hq, |W|, D]; k_comp: [Bt, Hkv, |W|-|U|, D].  Returns
    [Bt, Hkv, |W|-|U|] float64.
    """
    return head_scores(q_win, k_comp, causal=False, scale=scale)


def kara_select(A: np.ndarray, keep: int, gamma: int, alpha: int, buffer: int) -> np.ndarray:
    """Retained window positions per (b, h_kv)   (Kara Section 3.2, Eqs. 5-8,
    and the fill-up rule that follows them).

    A: [Bt, Hkv, n] importance of the compressible positions 0..n-1 (the
    buffer U occupies n..n+buffer-1 and is always kept).
      I  = the `keep` largest A (Eq. 5; ties -> lower position), ascending;
      R_k = (A[I[k]] + A[I[k+1]]) * (I[k+1] - I[k] - 1)  for consecutive
            picks with I[k+1] - I[k] <= gamma (Eq. 6), evaluated in float32
            because the kernel decides in float32;
      P  = the floor(alpha / gamma) largest R_k (Eq. 7; ties -> lower k);
      I^ = I plus the interior positions of the chunks in P (Eq. 8);
      fill-up: while fewer than alpha positions were added, add the highest-A
            positions not yet kept (ties -> lower position).
    Returns int32 [Bt, Hkv, min(n, keep + alpha) + buffer], ascending.
    """
    Bt, H, n = A.shape
    if not (0 <= keep <= n and gamma >= 1 and alpha >= 0 and buffer >= 0):
        raise ValueError("invalid Kara parameters")
    n_out = min(n, keep + alpha)
    out = np.empty((Bt, H, n_out + buffer), dtype=np.int32)
    pos = np.arange(n)
    for b in range(Bt):
        for h in range(H):
            a = A[b, h]
            order = np.lexsort((pos, -a))
            chosen = np.zeros(n, bool)
            chosen[order[:keep]] = True
            I = np.flatnonzero(chosen)
            a32 = a.astype(np.float32)
            chunks = []
            for k in range(len(I) - 1):
                gap = int(I[k + 1] - I[k])
                if gap <= gamma:
                    r = np.float32(np.float32(a32[I[k]] + a32[I[k + 1]]) * np.float32(gap - 1))
                    chunks.append((-float(r), k))
            chunks.sort()
            added = np.zeros(n, bool)
            for _, k in chunks[:alpha // gamma]:
                added[I[k] + 1:I[k + 1]] = True
            n_add = int(added.sum())
            rest = [j for j in order if not chosen[j] and not added[j]]
            for j in rest[:max(0, alpha - n_add)]:
                added[j] = True
            keep_pos = np.flatnonzero(chosen | added)
            assert keep_pos.size == n_out
            out[b, h] = np.concatenate([keep_pos, np.arange(n, n + buffer)])
    return out


# ---------------------------------------------------------------------------
# QEvict-style window tiers
# ---------------------------------------------------------------------------

def window_sums(s: np.ndarray, win: int) -> np.ndarray:
    """Cumulative window score w_j = sum_{i in window j} s_i over contiguous
    windows of ``win`` tokens (QEvict §4.2: windows are ranked by accumulated
    attention).  s: [..., S] with S a multiple of win -> [..., S/win]."""
    S = s.shape[-1]
    assert S % win == 0
    return s.reshape(s.shape[:-1] + (S // win, win)).sum(axis=-1)


def route_tiers(w: np.ndarray, n_full: int, n_quant: int):
    """Rank windows by (w descending, index ascending); the first n_full go to
    the full-precision tier (0), the next n_quant to the low-bit tier (1) and
    the rest are evicted (2)   (QEvict §4.3 and Appendix A: routing by rank
    under the tier capacities).

    Returns (tier int8 [..., nW], rank int32 [..., nW]) where rank[j] is the
    0-based position of window j in that order.
    """
    nW = w.shape[-1]
    flat = w.reshape(-1, nW)
    tier = np.empty(flat.shape, dtype=np.int8)
    rank = np.empty(flat.shape, dtype=np.int32)
    j = np.arange(nW)
    for r in range(flat.shape[0]):
        order = np.lexsort((j, -flat[r]))
        rank[r, order] = j
    tier[:] = np.where(rank < n_full, 0, np.where(rank < n_full + n_quant, 1, 2))
    return tier.reshape(w.shape), rank.reshape(w.shape)


def quant_int4(x: np.ndarray):
    """Asymmetric 4-bit codes of one group of values along axis 0.

    QEvict quantises the recoverable tier with an asymmetric low-bit code
    (§4.3; the summary names no formula).  Reading used: per group, lo = min,
    hi = max, scale = (hi - lo) / 15, code = clip(rint((x - lo) / scale), 0, 15)
    with round-half-to-even, codes 0 when scale == 0.  Evaluated in float32
    with exactly this operation order so the codes are decided in the same
    precision as on the device.

    x: float32 [n, ...] -> (codes uint8 [n, ...], lo float32 [...], scale float32 [...]).
    """
    x = np.asarray(x, dtype=np.float32)
    lo = x.min(axis=0)
    hi = x.max(axis=0)
    scale = np.float32(hi - lo) / np.float32(15.0)
    scale = np.asarray(scale, dtype=np.float32)
    safe = np.where(scale == 0, np.float32(1.0), scale).astype(np.float32)
    q = np.rint((x - lo).astype(np.float32) / safe).astype(np.float32)
    q = np.clip(q, 0, 15)
    q = np.where(scale == 0, np.float32(0.0), q)
    return q.astype(np.uint8), lo.astype(np.float32), scale


def dequant_int4(codes: np.ndarray, lo: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """x_hat = lo + code * scale in float32 with two roundings (multiply, then
    add; no fused multiply-add).  Returns float32; the caller rounds to bf16."""
    prod = (codes.astype(np.float32) * scale.astype(np.float32)).astype(np.float32)
    return (lo.astype(np.float32) + prod).astype(np.float32)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest, ties to
    even: keep the high 16 bits after adding half an ulp of bf16 plus the
    parity of the kept least-significant bit.  Finite inputs only."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    keep_lsb = (u >> np.uint64(16)) & np.uint64(1)
    return ((u + np.uint64(0x7FFF) + keep_lsb) >> np.uint64(16)).astype(np.uint16)


def pack_nibbles(codes: np.ndarray) -> np.ndarray:
    """Pack 4-bit codes along the last axis two per byte, the even channel in
    the low nibble: [..., D] -> [..., D/2] uint8."""
    c = np.asarray(codes, dtype=np.uint8)
    assert c.shape[-1] % 2 == 0 and int(c.max(initial=0)) <= 15
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def tier_outputs(k_bits: np.ndarray, v_bits: np.ndarray, tier: np.ndarray, win: int,
                 promote: np.ndarray | None = None) -> dict:
    """Tier payloads for a given window routing (QEvict Section 4.3).

    k_bits/v_bits: bf16 bit patterns [Bt, Hkv, S, D]; tier: [Bt, Hkv, S/win]
    with 0 = full precision, 1 = int4, 2 = evicted.  Within a tier the
    windows keep ascending index order.  Returns k_full/v_full (copied bits),
    k_codes/v_codes (packed int4 per window, [n_quant, win, D/2]),
    k_meta/v_meta ([n_quant, D, 2] fp32 lo and scale) and, for the int4-tier
    slots listed in `promote` ([Bt, Hkv, n_promote]), k_prom/v_prom: the
    dequantised windows rounded to bf16 bit patterns.  Groups are one
    channel of one window (win values); see quant_int4.
    """
    Bt, Hkv, S, D = k_bits.shape
    out = {key: [] for key in ("k_full", "v_full", "k_codes", "v_codes", "k_meta", "v_meta",
                               "k_prom", "v_prom")}
    for b in range(Bt):
        for h in range(Hkv):
            full = [j for j in range(S // win) if tier[b, h, j] == 0]
            quant = [j for j in range(S // win) if tier[b, h, j] == 1]
            for name, x in (("k", k_bits), ("v", v_bits)):
                rows = x[b, h].reshape(S // win, win, D)
                out[name + "_full"].append(rows[full].reshape(-1, D))
                codes, metas, deq = [], [], []
                for j in quant:
                    vals = (rows[j].astype(np.uint32) << np.uint32(16)).view(np.float32)
                    c, lo, sc = quant_int4(vals)
                    codes.append(pack_nibbles(c))
                    metas.append(np.stack([lo, sc], axis=-1))
                    deq.append(round_bf16(dequant_int4(c, lo, sc)))
                out[name + "_codes"].append(np.array(codes, dtype=np.uint8).reshape(-1, win, D // 2))
                out[name + "_meta"].append(np.array(metas, dtype=np.float32).reshape(-1, D, 2))
                if promote is not None:
                    out[name + "_prom"].append(
                        np.concatenate([deq[int(p)] for p in promote[b, h]], axis=0)
                        if promote.shape[-1] else np.zeros((0, D), np.uint16))
    res = {}
    for key, lst in out.items():
        if lst:
            res[key] = np.stack(lst).reshape((Bt, Hkv) + lst[0].shape)
    return res


# ---------------------------------------------------------------------------
# Memory model
# ---------------------------------------------------------------------------

def cache_bytes(n_layers: int, batch: int, n_kv_heads: int, tokens: int,
                head_dim: int, elem_bytes: int) -> int:
    """Bytes of a K+V cache: 2 * N * B * H_kv * tokens * D * b
    (TideKV §3, prompt KV size; §4.3 active-layer KV with N = 1)."""
    return 2 * n_layers * batch * n_kv_heads * tokens * head_dim * elem_bytes


# ---------------------------------------------------------------------------
# QEvict: recoverable routing repeated over decode steps
# ---------------------------------------------------------------------------

TIER_FULL, TIER_QUANT, TIER_EVICT = 0, 1, 2


def quant_lowbit(x: np.ndarray, bits: int):
    """Asymmetric codes of `bits` bits (2 or 4) of one group along axis 0:
    the int4 rule of quant_int4 with 2^bits - 1 steps between the group's
    minimum and maximum (QEvict's recoverable tier is INT2 by default, §B.5;
    §G.3 compares INT4).  float32, fixed operation order, round half to even.
    """
    levels = np.float32((1 << bits) - 1)
    x = np.asarray(x, dtype=np.float32)
    lo = x.min(axis=0)
    hi = x.max(axis=0)
    scale = np.asarray(np.float32(hi - lo) / levels, dtype=np.float32)
    safe = np.where(scale == 0, np.float32(1.0), scale).astype(np.float32)
    q = np.rint((x - lo).astype(np.float32) / safe).astype(np.float32)
    q = np.clip(q, 0, levels)
    q = np.where(scale == 0, np.float32(0.0), q)
    return q.astype(np.uint8), lo.astype(np.float32), scale


def pack_codes(codes: np.ndarray, bits: int) -> np.ndarray:
    """Pack `bits`-bit codes along the last axis, 8/bits per byte, channel c
    at bit offset bits*(c mod (8/bits)) of byte c // (8/bits) (the lowest
    channel in the lowest bits): [..., D] -> [..., D*bits/8] uint8."""
    per = 8 // bits
    c = np.asarray(codes, dtype=np.uint8)
    assert c.shape[-1] % per == 0 and int(c.max(initial=0)) < (1 << bits)
    out = np.zeros(c.shape[:-1] + (c.shape[-1] // per,), dtype=np.uint8)
    for u in range(per):
        out |= (c[..., u::per] << np.uint8(bits * u)).astype(np.uint8)
    return out


def unpack_codes(packed: np.ndarray, bits: int) -> np.ndarray:
    """Inverse of pack_codes."""
    per = 8 // bits
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * per,), dtype=np.uint8)
    for u in range(per):
        out[..., u::per] = (p >> np.uint8(bits * u)) & np.uint8((1 << bits) - 1)
    return out


def qevict_windows(seq_len: int, n_sink: int, n_recent: int, win: int) -> int:
    """Routed windows of a cache of seq_len tokens: the historical region
    between the protected sinks and the protected recent tokens (§4.1) cut
    into whole windows from its start; a partial window at its end stays
    with the protected recent tokens."""
    return max(0, (seq_len - n_sink - n_recent) // win)


def qevict_init(batch: int, heads: int, max_windows: int, head_dim: int, win: int,
                bits: int) -> dict:
    """Routing state before the first step: every window full precision,
    no backing-store entry, zero accumulated score."""
    bpt = head_dim * bits // 8
    return {
        "w_acc": np.zeros((batch, heads, max_windows), dtype=np.float64),
        "tier": np.zeros((batch, heads, max_windows), dtype=np.int8),
        "has_codes": np.zeros((batch, heads, max_windows), dtype=np.uint8),
        "k_codes": np.zeros((batch, heads, max_windows, win, bpt), dtype=np.uint8),
        "v_codes": np.zeros((batch, heads, max_windows, win, bpt), dtype=np.uint8),
        "k_meta": np.zeros((batch, heads, max_windows, head_dim, 2), dtype=np.float32),
        "v_meta": np.zeros((batch, heads, max_windows, head_dim, 2), dtype=np.float32),
    }


def qevict_step(state: dict, token_scores: np.ndarray, k_bits: np.ndarray, v_bits: np.ndarray,
                *, seq_len: int, n_sink: int, n_recent: int, win: int, n_full: int,
                n_quant: int, bits: int) -> dict:
    """One routing step of QEvict's recoverable hierarchy (§4.1-4.3,
    Appendix A), run every Omega decode tokens (§4.2), with the persistent
    backing store of §1.  Returns a new state; k_bits / v_bits (bf16 bit
    patterns [Bt, Hkv, capacity, D]) are updated in place by promotions.

    Per (sequence, KV head), for the nW = qevict_windows(...) routed windows
    (window j = tokens n_sink + win*j .. n_sink + win*(j+1) - 1):
      1. accumulate: w_acc[j] += sum of this step's token scores over window j
         (the prompt's attention initialises the scores at the first step);
      2. rank the windows that are not evicted by (w_acc desc, j asc): the
         first n_full are full precision, the next n_quant quantised, the rest
         evicted; eviction is permanent (an evicted window never ranks again);
      3. a window entering the quantised tier from full precision is
         quantised from its cache rows only at its first demotion; later
         demotions reuse that backing-store entry unchanged, so repeated
         transitions do not accumulate error;
      4. a window promoted from the quantised tier back to full precision has
         its cache rows rewritten with the dequantised values (bf16 RNE of
         lo + code*scale, two roundings): promotion restores residency, not
         the original values (Appendix K).
    Groups are one channel of one window, K and V separately (quant_lowbit).
    """
    st = {key: val.copy() for key, val in state.items()}
    Bt, H, _ = st["tier"].shape
    nW = qevict_windows(seq_len, n_sink, n_recent, win)
    for b in range(Bt):
        for h in range(H):
            for j in range(nW):
                a = n_sink + win * j
                st["w_acc"][b, h, j] += float(np.sum(token_scores[b, h, a:a + win],
                                                     dtype=np.float64))
            live = [j for j in range(nW) if st["tier"][b, h, j] != TIER_EVICT]
            order = sorted(live, key=lambda j: (-st["w_acc"][b, h, j], j))
            new = {}
            for r, j in enumerate(order):
                new[j] = TIER_FULL if r < n_full else (
                    TIER_QUANT if r < n_full + n_quant else TIER_EVICT)
            for j in live:
                old, nt = int(st["tier"][b, h, j]), new[j]
                a = n_sink + win * j
                if old == TIER_FULL and nt == TIER_QUANT and not st["has_codes"][b, h, j]:
                    for name, x in (("k", k_bits), ("v", v_bits)):
                        vals = (x[b, h, a:a + win].astype(np.uint32) << np.uint32(16)).view(
                            np.float32)
                        c, lo, sc = quant_lowbit(vals, bits)
                        st[name + "_codes"][b, h, j] = pack_codes(c, bits)
                        st[name + "_meta"][b, h, j] = np.stack([lo, sc], axis=-1)
                    st["has_codes"][b, h, j] = 1
                elif old == TIER_QUANT and nt == TIER_FULL:
                    for name, x in (("k", k_bits), ("v", v_bits)):
                        c = unpack_codes(st[name + "_codes"][b, h, j], bits)
                        meta = st[name + "_meta"][b, h, j]
                        x[b, h, a:a + win] = round_bf16(
                            dequant_int4(c, meta[:, 0][None, :], meta[:, 1][None, :]))
                st["tier"][b, h, j] = nt
    return st
