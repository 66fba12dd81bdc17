"""Parity of kvsel_qevict_step (repeated recoverable routing) with the oracle.

Both sides evolve their own state over several steps from the same seeded
cache and per-step token scores; after every step the tiers, backing-store
flags, accumulated scores, codes, metadata and cache rows are compared.
Integer-valued scores keep every window sum exact in fp32, so everything is
compared bit for bit; with real-valued scores the tiers may differ only for
windows whose accumulated score is within 1e-5 (relative) of a tier
boundary's."""
import numpy as np
import pytest
import torch

import attention_score_eviction_amd as kvsel
import oracle
import synth

pytestmark = pytest.mark.gpu


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _bf16_dev(bits):
    return torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).cuda()


def _bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


CASES = [
    # Bt, Hkv, D, nW, extra tail, n_sink, n_recent, n_full, n_quant, bits, steps
    (2, 3, 128, 20, 17, 5, 64, 5, 9, 2, 6),
    (1, 2, 64, 33, 0, 0, 64, 7, 14, 4, 5),
    (2, 1, 128, 9, 63, 5, 0, 3, 3, 2, 7),
    (1, 2, 128, 6, 1, 5, 64, 4, 4, 2, 3),       # capacity above the window count: nothing evicted
]


@pytest.mark.parametrize("case", CASES)
def test_qevict_steps_exact(case):
    Bt, H, D, nW, tail, n_sink, n_recent, n_full, n_quant, bits, steps = case
    S = n_sink + 64 * nW + n_recent + tail
    cap = S + 40
    M = nW + 3
    assert oracle.qevict_windows(S, n_sink, n_recent, 64) == nW
    cache = synth.qevict_cache(1, Bt, H, cap, D)
    k_o, v_o = cache["k"].copy(), cache["v"].copy()
    k_g, v_g = _bf16_dev(cache["k"]), _bf16_dev(cache["v"])
    st_o = oracle.qevict_init(Bt, H, M, D, 64, bits)
    qd = kvsel.qevict_desc(k_g, seq_len=S, max_windows=M, n_sink=n_sink, n_recent=n_recent,
                           n_full=n_full, n_quant=n_quant, bits=bits)
    st_g = kvsel.qevict_state(qd, k_g.device)
    print(f"qevict case {case}", flush=True)
    for step in range(steps):
        sc = synth.qevict_token_scores(3, step, Bt, H, S)
        st_o = oracle.qevict_step(st_o, sc, k_o, v_o, seq_len=S, n_sink=n_sink,
                                  n_recent=n_recent, win=64, n_full=n_full, n_quant=n_quant,
                                  bits=bits)
        kvsel.qevict_step(qd, _dev(sc), st_g, k_g, v_g)
        torch.cuda.synchronize()
        tier = st_g["tier"].cpu().numpy()
        assert np.array_equal(tier, st_o["tier"]), f"step {step}: tiers differ"
        assert np.array_equal(st_g["has_codes"].cpu().numpy(), st_o["has_codes"]), step
        assert np.array_equal(st_g["w_acc"].cpu().numpy().astype(np.float64), st_o["w_acc"]), step
        for name in ("k_codes", "v_codes"):
            assert np.array_equal(st_g[name].cpu().numpy(), st_o[name]), (step, name)
        for name in ("k_meta", "v_meta"):
            assert np.array_equal(st_g[name].cpu().numpy().view(np.uint32),
                                  st_o[name].view(np.uint32)), (step, name)
        assert np.array_equal(_bits(k_g), k_o) and np.array_equal(_bits(v_g), v_o), step
    # every transition kind happened in the longer cases
    if n_full + n_quant < nW:
        assert np.any(st_o["tier"][..., :nW] == 2) and np.any(st_o["has_codes"])


def test_qevict_growing_cache_exact():
    """Routing every Omega = 8 decode tokens on a growing cache (QEvict §4.2):
    seq_len grows by 8 per step at a fixed capacity, so the routed region
    gains a window each time 64 more tokens have left the protected recent
    region; the new window joins the ranking with the score of its own
    tokens.  Tiers, flags, accumulated scores, codes, metadata and cache rows
    stay bit-exact with the oracle at every step."""
    Bt, H, D, n_sink, n_recent, bits, omega = 2, 3, 128, 5, 64, 2, 8
    nW0, tail0, steps = 12, 40, 20
    S0 = n_sink + 64 * nW0 + n_recent + tail0
    S_end = S0 + omega * (steps - 1)
    cap = S_end + 16
    M = oracle.qevict_windows(S_end, n_sink, n_recent, 64) + 1
    n_full, n_quant = 3, 5
    cache = synth.qevict_cache(11, Bt, H, cap, D)
    k_o, v_o = cache["k"].copy(), cache["v"].copy()
    k_g, v_g = _bf16_dev(cache["k"]), _bf16_dev(cache["v"])
    st_o = oracle.qevict_init(Bt, H, M, D, 64, bits)
    st_g = None
    grew = 0
    print(f"qevict growing cache S {S0} -> {S_end}, capacity {cap}", flush=True)
    for step in range(steps):
        S = S0 + omega * step
        nW = oracle.qevict_windows(S, n_sink, n_recent, 64)
        if step and nW > oracle.qevict_windows(S - omega, n_sink, n_recent, 64):
            grew += 1
        qd = kvsel.qevict_desc(k_g, seq_len=S, max_windows=M, n_sink=n_sink, n_recent=n_recent,
                               n_full=n_full, n_quant=n_quant, bits=bits)
        if st_g is None:
            st_g = kvsel.qevict_state(qd, k_g.device)
        sc = synth.qevict_token_scores(12, step, Bt, H, S)
        st_o = oracle.qevict_step(st_o, sc, k_o, v_o, seq_len=S, n_sink=n_sink,
                                  n_recent=n_recent, win=64, n_full=n_full, n_quant=n_quant,
                                  bits=bits)
        kvsel.qevict_step(qd, _dev(sc), st_g, k_g, v_g)
        torch.cuda.synchronize()
        assert np.array_equal(st_g["tier"].cpu().numpy(), st_o["tier"]), f"step {step}: tiers"
        assert np.array_equal(st_g["has_codes"].cpu().numpy(), st_o["has_codes"]), step
        assert np.array_equal(st_g["w_acc"].cpu().numpy().astype(np.float64), st_o["w_acc"]), step
        for name in ("k_codes", "v_codes"):
            assert np.array_equal(st_g[name].cpu().numpy(), st_o[name]), (step, name)
        for name in ("k_meta", "v_meta"):
            assert np.array_equal(st_g[name].cpu().numpy().view(np.uint32),
                                  st_o[name].view(np.uint32)), (step, name)
        assert np.array_equal(_bits(k_g), k_o) and np.array_equal(_bits(v_g), v_o), step
        # slots past the routed windows are untouched (zero state)
        assert not st_o["w_acc"][..., nW:].any() and not st_o["tier"][..., nW:].any()
    assert grew == 3
    assert np.any(st_o["tier"] == 2) and np.any(st_o["has_codes"])


def test_qevict_real_scores_band():
    """One step with real-valued scores: tiers equal except for windows whose
    oracle score lies within 1e-5 (relative) of a boundary window's score;
    the quantised windows that match carry bit-exact codes."""
    Bt, H, D, nW, n_sink, n_recent, n_full, n_quant, bits = 2, 4, 128, 40, 5, 64, 10, 20, 2
    S = n_sink + 64 * nW + n_recent
    cache = synth.qevict_cache(2, Bt, H, S, D)
    k_o, v_o = cache["k"].copy(), cache["v"].copy()
    k_g, v_g = _bf16_dev(cache["k"]), _bf16_dev(cache["v"])
    st_o = oracle.qevict_init(Bt, H, nW, D, 64, bits)
    qd = kvsel.qevict_desc(k_g, seq_len=S, max_windows=nW, n_sink=n_sink, n_recent=n_recent,
                           n_full=n_full, n_quant=n_quant, bits=bits)
    st_g = kvsel.qevict_state(qd, k_g.device)
    sc = synth.qevict_token_scores(4, 0, Bt, H, S, integer=False)
    st_o = oracle.qevict_step(st_o, sc, k_o, v_o, seq_len=S, n_sink=n_sink, n_recent=n_recent,
                              win=64, n_full=n_full, n_quant=n_quant, bits=bits)
    kvsel.qevict_step(qd, _dev(sc), st_g, k_g, v_g)
    torch.cuda.synchronize()
    w = st_o["w_acc"]
    np.testing.assert_allclose(st_g["w_acc"].cpu().numpy(), w, rtol=1e-5)
    tier = st_g["tier"].cpu().numpy()
    kc = st_g["k_codes"].cpu().numpy()
    for b in range(Bt):
        for h in range(H):
            order = np.argsort(-w[b, h], kind="stable")
            bounds = [w[b, h, order[n_full - 1]], w[b, h, order[n_full]],
                      w[b, h, order[n_full + n_quant - 1]], w[b, h, order[n_full + n_quant]]]
            for j in np.flatnonzero(tier[b, h] != st_o["tier"][b, h]):
                assert min(abs(w[b, h, j] - x) for x in bounds) <= 1e-5 * w[b, h, j], (b, h, j)
            same_q = (tier[b, h] == 1) & (st_o["tier"][b, h] == 1)
            assert np.array_equal(kc[b, h][same_q], st_o["k_codes"][b, h][same_q])


def test_qevict_decode_tiers_full_size_sampled():
    """16 sequences x 8 KV heads, 32768-token caches, 5 sinks, 64 recent
    tokens, INT2, 30% of the routed budget full precision (QEvict's
    defaults); four steps on the GPU; three (sequence, head) rows replayed
    through the oracle and compared bit for bit."""
    Bt, H, D, S = 16, 8, 128, 32768
    n_sink, n_recent, bits = 5, 64, 2
    nW = oracle.qevict_windows(S, n_sink, n_recent, 64)
    keep = nW // 2
    n_quant = int(round(0.7 * keep))
    n_full = keep - n_quant
    cache = synth.qevict_cache(5, Bt, H, S, D)
    k_g, v_g = _bf16_dev(cache["k"]), _bf16_dev(cache["v"])
    qd = kvsel.qevict_desc(k_g, seq_len=S, max_windows=nW, n_sink=n_sink, n_recent=n_recent,
                           n_full=n_full, n_quant=n_quant, bits=bits)
    st_g = kvsel.qevict_state(qd, k_g.device)
    rows = [(0, 0), (7, 3), (15, 7)]
    st_o = {r: oracle.qevict_init(1, 1, nW, D, 64, bits) for r in rows}
    ko = {r: cache["k"][r[0]:r[0] + 1, r[1]:r[1] + 1].copy() for r in rows}
    vo = {r: cache["v"][r[0]:r[0] + 1, r[1]:r[1] + 1].copy() for r in rows}
    for step in range(4):
        sc = synth.qevict_token_scores(6, step, Bt, H, S)
        kvsel.qevict_step(qd, _dev(sc), st_g, k_g, v_g)
        for (b, h) in rows:
            st_o[(b, h)] = oracle.qevict_step(
                st_o[(b, h)], sc[b:b + 1, h:h + 1], ko[(b, h)], vo[(b, h)], seq_len=S,
                n_sink=n_sink, n_recent=n_recent, win=64, n_full=n_full, n_quant=n_quant,
                bits=bits)
    torch.cuda.synchronize()
    for (b, h) in rows:
        o = st_o[(b, h)]
        assert np.array_equal(st_g["tier"][b, h].cpu().numpy(), o["tier"][0, 0])
        assert np.array_equal(st_g["k_codes"][b, h].cpu().numpy(), o["k_codes"][0, 0])
        assert np.array_equal(st_g["v_meta"][b, h].cpu().numpy().view(np.uint32),
                              o["v_meta"][0, 0].view(np.uint32))
        assert np.array_equal(_bits(k_g[b, h]), ko[(b, h)][0, 0])
        assert np.array_equal(_bits(v_g[b, h]), vo[(b, h)][0, 0])
    t = st_g["tier"].cpu().numpy()
    assert np.all((t == 0).sum(-1) == n_full) and np.all((t == 1).sum(-1) == n_quant)
