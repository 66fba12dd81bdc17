"""Parity of kvsel_route_tiers (window scores, three-tier routing, int4
quantisation, promotion by dequantisation) with the CPU oracle.

Routing: exact when window sums are exact in fp32 (integer-valued scores);
otherwise identical except for windows whose oracle sum lies within 1e-4
relative of a tier-boundary sum.  Payloads (full-tier rows, int4 codes,
(lo, scale) metadata, promoted bf16 rows) are bit-exact against the oracle's
payloads for its own routing, window by window, for every window both sides
put in the same tier (all of them when the routings agree).
"""
import numpy as np
import pytest

import oracle
import synth
from helpers import dev_tensor, host_bits

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

WIN = 64


def _kvsel():
    import attention_score_eviction_amd as kvsel
    kvsel.lib()
    return kvsel


def _rand_bf16(rng, shape, scale=1.0):
    return synth.f32_to_bf16_bits((rng.standard_normal(shape) * scale).astype(np.float32))


def _payload_check(got, want, tier_g, tier_ref, promote, min_agree=0.9):
    """got / want: payload dicts (GPU outputs as numpy, oracle outputs for the
    oracle's routing tier_ref) for the same [Bt, Hkv] rows.  Each window that
    both routings put in the full or int4 tier must carry identical bytes in
    its slot on each side; promoted slots are compared where both sides'
    promoted window is the same."""
    Bt, Hkv, nW = tier_ref.shape
    D = got["k_full"].shape[-1] if got["k_full"].size else got["k_meta"].shape[-2]
    per_win = {"k_full": (WIN, D), "v_full": (WIN, D), "k_codes": (WIN, D // 2),
               "v_codes": (WIN, D // 2), "k_meta": (D, 2), "v_meta": (D, 2),
               "k_prom": (WIN, D), "v_prom": (WIN, D)}
    view = lambda a, name: a.reshape((Bt, Hkv, -1) + per_win[name])  # noqa
    agree = 0
    for b in range(Bt):
        for h in range(Hkv):
            agree += int((tier_g[b, h] == tier_ref[b, h]).sum())
            for t, names in ((0, ("k_full", "v_full")),
                             (1, ("k_codes", "v_codes", "k_meta", "v_meta"))):
                wg = np.flatnonzero(tier_g[b, h] == t)
                wr = np.flatnonzero(tier_ref[b, h] == t)
                common = np.intersect1d(wg, wr)
                sg, sr = np.searchsorted(wg, common), np.searchsorted(wr, common)
                for name in names:
                    g = view(got[name], name)[b, h][sg]
                    w = view(want[name], name)[b, h][sr]
                    assert g.tobytes() == w.tobytes(), f"{name} row ({b},{h})"
            qg = np.flatnonzero(tier_g[b, h] == 1)
            qr = np.flatnonzero(tier_ref[b, h] == 1)
            for i, slot in enumerate(promote[b, h]):
                if qg[slot] != qr[slot]:
                    continue
                for name in ("k_prom", "v_prom"):
                    g = view(got[name], name)[b, h][i]
                    w = view(want[name], name)[b, h][i]
                    assert g.tobytes() == w.tobytes(), f"{name} row ({b},{h}) slot {i}"
    assert agree >= min_agree * Bt * Hkv * nW


def _gpu_payloads(out, rows=None):
    res = {}
    for name in ("k_full", "v_full", "k_codes", "v_codes", "k_prom", "v_prom", "k_meta",
                 "v_meta"):
        t = getattr(out, name)
        if rows is not None:
            t = t[rows]
        res[name] = t.cpu().numpy() if name.endswith("meta") else host_bits(t)
    return res


def _check_routing_band(tier_g, rank_g, w_ref, n_full, n_quant, band=1e-4):
    """GPU tiers equal the oracle's except for windows within `band` of a
    tier-boundary sum; the GPU's ranks are a permutation consistent with its
    tiers."""
    rows_t = tier_g.reshape(-1, tier_g.shape[-1])
    rows_r = rank_g.reshape(-1, rank_g.shape[-1])
    rows_w = w_ref.reshape(-1, w_ref.shape[-1])
    nW = rows_t.shape[1]
    for r in range(rows_t.shape[0]):
        assert sorted(rows_r[r].tolist()) == list(range(nW))
        want_t = np.where(rows_r[r] < n_full, 0, np.where(rows_r[r] < n_full + n_quant, 1, 2))
        assert (rows_t[r] == want_t).all()
        order = np.sort(rows_w[r])[::-1]
        bounds = [order[n_full - 1], order[n_full]] if 0 < n_full < nW else []
        if n_full + n_quant < nW:
            bounds += [order[n_full + n_quant - 1], order[n_full + n_quant]]
        ref_t, _ = oracle.route_tiers(rows_w[r][None], n_full, n_quant)
        diff = np.flatnonzero(ref_t[0] != rows_t[r])
        for j in diff:
            assert any(abs(rows_w[r][j] - bnd) <= band * abs(bnd) for bnd in bounds), \
                f"row {r} window {j} routed differently away from a boundary"


@pytest.mark.parametrize("D", [128, 64])
def test_route_tiers_exact_on_integer_scores(D):
    kvsel = _kvsel()
    rng = np.random.default_rng(30 + D)
    Bt, Hkv, nW = 2, 3, 40
    S = nW * WIN
    n_full, n_quant, n_prom = 8, 16, 4
    scores = rng.integers(0, 8, size=(Bt, Hkv, S)).astype(np.float32)
    kb = _rand_bf16(rng, (Bt, Hkv, S, D), 2.0)
    vb = _rand_bf16(rng, (Bt, Hkv, S, D))
    kb[0, 1, 5 * WIN:6 * WIN, 3] = kb[0, 1, 5 * WIN, 3]       # a constant channel
    vb[1, 2, :, 7] = synth.f32_to_bf16_bits(np.full(S, 0.5, np.float32))
    promote = synth.promote_list(77, Bt * Hkv, n_quant, n_prom).reshape(Bt, Hkv, n_prom)
    out = kvsel.route_tiers(torch.from_numpy(scores).cuda(), dev_tensor(kb, "bf16"),
                            dev_tensor(vb, "bf16"), n_full=n_full, n_quant=n_quant,
                            promote=torch.from_numpy(promote).cuda())
    torch.cuda.synchronize()
    w = oracle.window_sums(scores.astype(np.float64), WIN)
    tier, rank = oracle.route_tiers(w, n_full, n_quant)
    np.testing.assert_array_equal(out.tier.cpu().numpy(), tier)
    np.testing.assert_array_equal(out.rank.cpu().numpy(), rank)
    want = oracle.tier_outputs(kb, vb, tier, WIN, promote)
    _payload_check(_gpu_payloads(out), want, tier, tier, promote, min_agree=1.0)


def test_route_tiers_float_scores_and_edges():
    kvsel = _kvsel()
    rng = np.random.default_rng(31)
    Bt, Hkv, nW, D = 1, 4, 64, 128
    S = nW * WIN
    scores = rng.random((Bt, Hkv, S)).astype(np.float32)
    kb = _rand_bf16(rng, (Bt, Hkv, S, D), 3.0)
    vb = _rand_bf16(rng, (Bt, Hkv, S, D), 0.1)
    for n_full, n_quant, n_prom in [(16, 32, 5), (0, 64, 0), (64, 0, 0), (10, 0, 0), (1, 1, 1)]:
        promote = (synth.promote_list(78, Bt * Hkv, n_quant, n_prom).reshape(Bt, Hkv, n_prom)
                   if n_prom else None)
        out = kvsel.route_tiers(torch.from_numpy(scores).cuda(), dev_tensor(kb, "bf16"),
                                dev_tensor(vb, "bf16"), n_full=n_full, n_quant=n_quant,
                                promote=None if promote is None else torch.from_numpy(promote).cuda())
        torch.cuda.synchronize()
        tier_g = out.tier.cpu().numpy()
        w = oracle.window_sums(scores.astype(np.float64), WIN)
        _check_routing_band(tier_g, out.rank.cpu().numpy(), w, n_full, n_quant)
        prom = promote if promote is not None else np.zeros((Bt, Hkv, 0), np.int32)
        tier_ref, _ = oracle.route_tiers(w, n_full, n_quant)
        want = oracle.tier_outputs(kb, vb, tier_ref, WIN, prom)
        _payload_check(_gpu_payloads(out), want, tier_g, tier_ref, prom)


def test_full_c5_decode_tiers_sampled_rows():
    """16 sequences x 32768 cached tokens, 256 decode queries (no causal mask),
    512 windows per KV head -> 128 full / 256 int4 / 128 evicted, 12 promoted:
    score + route on the GPU; two (sequence, KV head) rows checked against the
    oracle (scores within 1e-3, routing within the band, payloads exact)."""
    kvsel = _kvsel()
    spec = synth.config(5)
    x = synth.make_layer(spec, 5)
    print("case c5 full size", flush=True)
    q, k, v = (dev_tensor(x[n], "bf16") for n in ("q", "k", "v"))
    pooled, raw = kvsel.score(q, k, pool_kernel=1, causal=False)
    n_full, n_quant, n_prom = 128, 256, 12
    Bt, Hkv = spec.batch, spec.n_kv_heads
    promote = synth.promote_list(5, Bt * Hkv, n_quant, n_prom).reshape(Bt, Hkv, n_prom)
    out = kvsel.route_tiers(raw, k, v, n_full=n_full, n_quant=n_quant,
                            promote=torch.from_numpy(promote).cuda())
    torch.cuda.synchronize()
    s_g = raw.cpu().numpy()
    G = spec.group
    for b, h in [(0, 0), (11, 5)]:
        s_ref = oracle.head_scores(synth.to_f64(x["q"][b:b + 1, h * G:(h + 1) * G], "bf16"),
                                   synth.to_f64(x["k"][b:b + 1, h:h + 1], "bf16"), causal=False)
        err = np.abs(s_g[b, h] - s_ref[0, 0]) / s_ref[0, 0]
        assert err.max() <= 1e-3
        w_ref = oracle.window_sums(s_ref, WIN)
        tier_g = out.tier[b:b + 1, h:h + 1].cpu().numpy()
        _check_routing_band(tier_g, out.rank[b:b + 1, h:h + 1].cpu().numpy(), w_ref, n_full,
                            n_quant)
        tier_ref, _ = oracle.route_tiers(w_ref, n_full, n_quant)
        want = oracle.tier_outputs(x["k"][b:b + 1, h:h + 1], x["v"][b:b + 1, h:h + 1], tier_ref,
                                   WIN, promote[b:b + 1, h:h + 1])
        got = _gpu_payloads(out, (slice(b, b + 1), slice(h, h + 1)))
        _payload_check(got, want, tier_g, tier_ref, promote[b:b + 1, h:h + 1])
