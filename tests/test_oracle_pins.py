"""Pins of the CPU oracle against facts that do not come from the oracle:
brute force in plain Python, closed forms, invariants the pages state, and
the memory figures the pages print (tests/golden/memory_pins.json)."""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


# ---------------------------------------------------------------- scores ----

def _brute_scores(q, k, causal, scale):
    """Triple loops with math.exp: every logit, row max, normaliser and sum
    written out element by element (independent of numpy matmul/broadcast)."""
    Bt, Hq, W, D = q.shape
    _, Hkv, S, _ = k.shape
    G = Hq // Hkv
    s = [[[0.0] * S for _ in range(Hkv)] for _ in range(Bt)]
    for b in range(Bt):
        for h in range(Hq):
            hk = h // G
            for qi in range(W):
                pos = S - W + qi
                row = []
                for i in range(S):
                    if causal and i > pos:
                        row.append(None)
                        continue
                    acc = 0.0
                    for d in range(D):
                        acc += float(q[b, h, qi, d]) * float(k[b, hk, i, d])
                    row.append(acc * scale)
                m = max(x for x in row if x is not None)
                z = sum(math.exp(x - m) for x in row if x is not None)
                for i, x in enumerate(row):
                    if x is not None:
                        s[b][hk][i] += math.exp(x - m) / z
    return np.array(s)


@pytest.mark.parametrize("causal", [True, False])
def test_scores_match_brute_force(causal):
    q = _rand((2, 4, 3, 5), 1)
    k = _rand((2, 2, 11, 5), 2, 1.5)
    sc = 0.37
    got = oracle.head_scores(q, k, causal=causal, scale=sc)
    ref = _brute_scores(q, k, causal, sc)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-15)


def test_default_scale_is_inverse_sqrt_d():
    q = _rand((1, 2, 2, 16), 3)
    k = _rand((1, 1, 9, 16), 4)
    np.testing.assert_allclose(oracle.head_scores(q, k),
                               _brute_scores(q, k, True, 0.25), rtol=1e-12)


@pytest.mark.parametrize("causal", [True, False])
def test_row_sums_give_w_times_group(causal):
    spec = synth.config(1)
    x = synth.make_layer(spec, 1)
    q = synth.to_f64(x["q"], spec.dtype)
    k = synth.to_f64(x["k"], spec.dtype)
    s = oracle.head_scores(q, k, causal=causal)
    np.testing.assert_allclose(s.sum(-1), spec.obs_window * spec.group, rtol=1e-12)


def _harmonic(n):
    return sum(Fraction(1, j) for j in range(1, n + 1))


@pytest.mark.parametrize("how", ["equal_keys", "zero_queries"])
def test_closed_form_uniform_attention(how):
    """All logits of a row equal -> a[q,i] = 1/(S-W+q+1) on visible keys, so a
    prefix key gets G*(H_S - H_{S-W}) and window key S-W+r gets
    G*(H_S - H_{S-W+r})."""
    Bt, Hq, Hkv, D, S, W = 1, 4, 2, 64, 512, 16
    G = Hq // Hkv
    q = _rand((Bt, Hq, W, D), 5)
    k = _rand((Bt, Hkv, S, D), 6)
    if how == "equal_keys":
        k[:] = k[:, :, :1, :]
    else:
        q[:] = 0.0
    s = oracle.head_scores(q, k)
    HS = _harmonic(S)
    prefix = float(G * (HS - _harmonic(S - W)))
    assert abs(prefix - 0.0634344342767) < 1e-12
    np.testing.assert_allclose(s[..., :S - W], prefix, rtol=1e-12)
    for r in range(W):
        np.testing.assert_allclose(s[..., S - W + r], float(G * (HS - _harmonic(S - W + r))),
                                   rtol=1e-12)
    # every candidate ties: the selection is the lowest positions
    p = oracle.max_pool(s, 5, 0, S - W)
    idx = oracle.select(p, 64, 0, W)
    want = np.concatenate([np.arange(64), np.arange(S - W, S)])
    assert (idx == want).all()
    idx = oracle.select(p, 10, 3, W)
    want = np.concatenate([np.arange(3), np.arange(3, 13), np.arange(S - W, S)])
    assert (idx == want).all()


def test_spike_key_takes_almost_all_mass():
    """One prefix key aligned with every query at logit +60 takes all of the
    normalised weight: s[i*] ~= W*G and the max-pool plateau is
    [i*-h, i*+h] clipped to the candidates."""
    Bt, Hq, Hkv, D, S, W = 1, 2, 1, 8, 64, 4
    q = np.zeros((Bt, Hq, W, D)); q[..., 0] = 1.0
    k = _rand((Bt, Hkv, S, D), 7, 0.01)
    k[..., 0] = 0.0
    i_star = 20
    k[0, 0, i_star, 0] = 60.0 * math.sqrt(D)
    s = oracle.head_scores(q, k)
    assert abs(s[0, 0, i_star] - W * Hq) < W * Hq * S * math.exp(-59)
    p = oracle.max_pool(s, 7, 0, S - W)
    plateau = np.flatnonzero(p[0, 0] == s[0, 0, i_star])
    assert plateau.tolist() == list(range(i_star - 3, i_star + 4))
    # a spike at the candidate edge is clipped
    p2 = oracle.max_pool(s, 7, 18, S - W)
    assert np.flatnonzero(p2[0, 0] == s[0, 0, i_star]).tolist() == list(range(18, 24))


def test_causal_mask_hides_future_window_key():
    """A window key S-W+r with a huge logit for every query is seen only by
    the W-r queries at or after its position: its score is G*(W-r) up to
    exp(-huge) terms, and a non-causal run gives it G*W."""
    Bt, Hq, Hkv, D, S, W, r = 1, 3, 1, 4, 40, 8, 5
    q = np.zeros((Bt, Hq, W, D)); q[..., 1] = 1.0
    k = _rand((Bt, Hkv, S, D), 8, 0.01); k[..., 1] = 0.0
    j = S - W + r
    k[0, 0, j, 1] = 80.0 * 2.0          # logit 80 at scale 1/2
    s = oracle.head_scores(q, k)
    assert abs(s[0, 0, j] - Hq * (W - r)) < Hq * W * S * math.exp(-70)
    s_nc = oracle.head_scores(q, k, causal=False)
    assert abs(s_nc[0, 0, j] - Hq * W) < Hq * W * S * math.exp(-70)


def test_gqa_group_is_contiguous():
    """Query heads [h_kv*G, (h_kv+1)*G) read KV head h_kv."""
    Bt, Hq, Hkv, D, S, W = 1, 4, 2, 4, 24, 2
    q = np.zeros((Bt, Hq, W, D)); q[0, 0:2, :, 2] = 1.0     # heads 0,1 -> KV head 0
    k = _rand((Bt, Hkv, S, D), 9, 0.01); k[..., 2] = 0.0
    k[0, 0, 5, 2] = 100.0 * 2.0
    s = oracle.head_scores(q, k)
    assert abs(s[0, 0, 5] - 2 * W) < 1e-12          # both heads of group 0
    assert s[0, 1].max() < 0.2                        # group 1 stays near uniform


# ------------------------------------------------------------------ pool ----

@pytest.mark.parametrize("kernel", [1, 3, 5, 7, 9])
@pytest.mark.parametrize("lo,hi", [(0, 50), (3, 41), (10, 12), (7, 7)])
def test_max_pool_matches_sliding_window(kernel, lo, hi):
    S = 50
    s = _rand((2, 3, S), kernel * 100 + lo)
    got = oracle.max_pool(s, kernel, lo, hi)
    h = (kernel - 1) // 2
    pad = np.full((2, 3, S + 2 * h), -np.inf)
    pad[..., h + lo:h + hi] = s[..., lo:hi]
    win = np.lib.stride_tricks.sliding_window_view(pad, kernel, axis=-1)
    want = np.zeros_like(s)
    if hi > lo:
        want[..., lo:hi] = win.max(-1)[..., lo:hi]
    np.testing.assert_array_equal(got, want)


# ---------------------------------------------------------------- select ----

def test_select_matches_brute_force_sort():
    spec = synth.config(1)
    x = synth.make_layer(spec, 1)
    s = oracle.head_scores(synth.to_f64(x["q"], "f32"), synth.to_f64(x["k"], "f32"))
    S, W = spec.seq_len, spec.obs_window
    for n_sink, B, kern in [(0, 64, 5), (4, 64, 5), (0, 0, 3), (2, S - W - 2, 1), (0, 200, 9)]:
        p = oracle.max_pool(s, kern, n_sink, S - W)
        idx = oracle.select(p, B, n_sink, W)
        assert idx.shape == (1, 2, B + n_sink + W)
        for h in range(2):
            cand = sorted(range(n_sink, S - W), key=lambda i: (-p[0, h, i], i))
            want = sorted(list(range(n_sink)) + cand[:B] + list(range(S - W, S)))
            assert idx[0, h].tolist() == want
            assert (np.diff(idx[0, h]) > 0).all()


def test_select_ties_take_lowest_positions():
    p = np.array([[0.0, 3.0, 1.0, 3.0, 3.0, 2.0, 3.0, 0.5, 9.0, 9.0]])
    # candidates [1, 8), window W = 2 -> positions 8, 9 mandatory; sinks 1
    idx = oracle.select(p, 3, 1, 2)
    assert idx.tolist() == [[0, 1, 3, 4, 8, 9]]


@pytest.mark.parametrize("B,n_sink,W", [(5, 0, 8), (-1, 0, 2), (0, 0, 0), (0, 0, 11), (2, 9, 1)])
def test_select_rejects_infeasible(B, n_sink, W):
    with pytest.raises(ValueError):
        oracle.select(np.zeros((1, 10)), B, n_sink, W)


# ------------------------------------------------- head-adaptive select ----

def _flat_heads(idx, off, b, H):
    return [idx[b, off[b, h]:off[b, h + 1]].tolist() for h in range(H)]


def test_head_adaptive_matches_subset_brute_force():
    """With distinct scores the picked set is the unique T-subset of a
    sequence's candidates (over all heads) with the largest score sum."""
    import itertools
    rng = np.random.default_rng(41)
    H, S, n_sink, W = 3, 9, 1, 2
    for T in [0, 1, 4, 7, 18]:
        p = rng.permutation(2 * H * S).reshape(2, H, S)[:, :, :].astype(np.float64) + 0.5
        idx, off = oracle.select_head_adaptive(p, T, n_sink, W)
        assert idx.shape == (2, H * (n_sink + W) + T) and off.shape == (2, H + 1)
        for b in range(2):
            cand = [(h, i) for h in range(H) for i in range(n_sink, S - W)]
            best = max(itertools.combinations(cand, T),
                       key=lambda c: sum(p[b, h, i] for h, i in c)) if T else ()
            for h in range(H):
                want = sorted(list(range(n_sink)) + [i for g, i in best if g == h]
                              + list(range(S - W, S)))
                assert _flat_heads(idx, off, b, H)[h] == want
            assert off[b, 0] == 0 and off[b, H] == idx.shape[1]


def test_head_adaptive_ties_go_to_lower_head_then_position():
    p = np.zeros((1, 2, 8))
    p[0, 0] = [0, 5, 2, 5, 1, 0, 9, 9]
    p[0, 1] = [0, 5, 5, 3, 5, 0, 9, 9]
    # sinks 1, window 2 -> candidates 1..5; T = 4: the five 5s tie for four
    # places -> head 0 positions 1, 3, then head 1 positions 1, 2.
    idx, off = oracle.select_head_adaptive(p, 4, 1, 2)
    assert off.tolist() == [[0, 5, 10]]
    assert idx.tolist() == [[0, 1, 3, 6, 7, 0, 1, 2, 6, 7]]


def test_head_adaptive_separable_scores_reduce_to_uniform_budget():
    """When every head's top-B scores exceed all other candidates of the
    sequence, the head-adaptive picks equal the per-head selection."""
    rng = np.random.default_rng(42)
    Bt, H, S, n_sink, W, B = 2, 4, 64, 2, 6, 5
    p = rng.random((Bt, H, S))
    for b in range(Bt):
        for h in range(H):
            top = rng.choice(np.arange(n_sink, S - W), B, replace=False)
            p[b, h, top] += 10.0
    idx, off = oracle.select_head_adaptive(p, H * B, n_sink, W)
    uni = oracle.select(p, B, n_sink, W)
    assert (off == np.arange(H + 1)[None] * (B + n_sink + W)).all()
    assert (idx == uni.reshape(Bt, -1)).all()


def test_head_adaptive_dominant_head_takes_every_pick():
    p = np.full((1, 3, 20), 0.25)
    p[0, 1, 2:17] = np.linspace(1.0, 2.0, 15)
    idx, off = oracle.select_head_adaptive(p, 10, 0, 3)
    segs = _flat_heads(idx, off, 0, 3)
    assert segs[0] == [17, 18, 19] and segs[2] == [17, 18, 19]
    assert segs[1] == list(range(7, 20))


def test_head_adaptive_single_head_equals_select():
    spec = synth.config(1)
    x = synth.make_layer(spec, 1)
    s = oracle.head_scores(synth.to_f64(x["q"], "f32"), synth.to_f64(x["k"], "f32"))
    S, W = spec.seq_len, spec.obs_window
    p = oracle.max_pool(s, 5, 4, S - W)
    for h in range(2):
        idx, off = oracle.select_head_adaptive(p[:, h:h + 1], 64, 4, W)
        assert off.tolist() == [[0, 64 + 4 + W]]
        assert (idx == oracle.select(p[:, h:h + 1], 64, 4, W)[:, 0]).all()


@pytest.mark.parametrize("T,n_sink,W", [(-1, 0, 2), (2 * 8 + 1, 0, 2), (0, 0, 0), (0, 9, 2)])
def test_head_adaptive_rejects_infeasible(T, n_sink, W):
    with pytest.raises(ValueError):
        oracle.select_head_adaptive(np.zeros((1, 2, 10)), T, n_sink, W)


def test_compact_flat_rows_follow_their_head():
    rng = np.random.default_rng(43)
    kb = rng.integers(0, 65536, size=(2, 3, 30, 4), dtype=np.uint16)
    p = rng.random((2, 3, 30))
    idx, off = oracle.select_head_adaptive(p, 11, 1, 3)
    out = oracle.compact_flat(kb, idx, off)
    for b in range(2):
        h = 0
        for r in range(idx.shape[1]):
            while r >= off[b, h + 1]:
                h += 1
            assert out[b, r].tobytes() == kb[b, h, idx[b, r]].tobytes()


# --------------------------------------------------------------- Kara ----

def test_kara_scores_brute_force_more_queries_than_keys():
    """Kara Eq. 4 written out with math.exp: |W| = 7 window queries (two
    query heads per KV head) against the n = 5 compressible keys, no mask."""
    rng = np.random.default_rng(51)
    q = rng.standard_normal((1, 4, 7, 8))
    k = rng.standard_normal((1, 2, 5, 8))
    A = oracle.kara_scores(q, k)
    for hk in range(2):
        for j in range(5):
            tot = 0.0
            for h in (2 * hk, 2 * hk + 1):
                for i in range(7):
                    num = math.exp(sum(q[0, h, i, d] * k[0, hk, j, d] for d in range(8)) / math.sqrt(8))
                    den = sum(math.exp(sum(q[0, h, i, d] * k[0, hk, jj, d] for d in range(8))
                                       / math.sqrt(8)) for jj in range(5))
                    tot += num / den
            assert abs(A[0, hk, j] - tot) <= 1e-12 * tot
        # every window query's weights over the compressible keys sum to one
        assert abs(A[0, hk].sum() - 2 * 7) <= 1e-12


def test_kara_scores_identical_keys_are_uniform():
    q = np.random.default_rng(52).standard_normal((1, 3, 9, 4))
    k = np.tile(np.array([0.3, -1.0, 2.0, 0.5]), (1, 1, 6, 1))
    assert np.allclose(oracle.kara_scores(q, k), 3 * 9 / 6, rtol=1e-13)


def test_kara_select_worked_example():
    """TopK 4 -> I = {0, 3, 5, 9}; chunk (0,3) scores (0.9+0.8)*2, chunk (3,5)
    (0.8+0.7)*1, chunk (5,9) is wider than gamma = 3; floor(4/3) = 1 chunk
    adds {1, 2}; fill-up adds the two best remaining, 10 and 6; the buffer
    (12, 13) is kept."""
    A = np.array([[[0.9, 0.1, 0.2, 0.8, 0.05, 0.7, 0.3, 0.01, 0.02, 0.6, 0.4, 0.03]]])
    out = oracle.kara_select(A, keep=4, gamma=3, alpha=4, buffer=2)
    assert out.tolist() == [[[0, 1, 2, 3, 5, 6, 9, 10, 12, 13]]]


def test_kara_select_gamma_one_reduces_to_top_k():
    """gamma = 1 leaves no chunk interior, so the fill-up makes the result the
    plain top-(keep + alpha) set."""
    rng = np.random.default_rng(53)
    A = rng.random((2, 3, 40))
    out = oracle.kara_select(A, keep=10, gamma=1, alpha=6, buffer=0)
    for b in range(2):
        for h in range(3):
            want = sorted(sorted(range(40), key=lambda j: (-A[b, h, j], j))[:16])
            assert out[b, h].tolist() == want


def test_kara_select_ties_and_edges():
    flat = np.full((1, 1, 10), 0.5)
    # all equal: I = first positions, chunks add nothing, fill-up by position
    assert oracle.kara_select(flat, 3, 4, 2, 1).tolist() == [[[0, 1, 2, 3, 4, 10]]]
    rng = np.random.default_rng(54)
    A = rng.random((1, 2, 30))
    # alpha = 0: exactly the top-k set, ascending
    out = oracle.kara_select(A, 7, 8, 0, 3)
    for h in range(2):
        assert out[0, h, :7].tolist() == sorted(np.argsort(-A[0, h], kind="stable")[:7].tolist())
        assert out[0, h, 7:].tolist() == [30, 31, 32]
    # keep everything
    assert oracle.kara_select(A, 30, 8, 16, 0)[0, 0].tolist() == list(range(30))
    # near the end: fewer unselected positions than alpha
    assert oracle.kara_select(A, 25, 8, 16, 0).shape == (1, 2, 30)


def test_kara_select_chunks_are_contiguous_and_bounded():
    rng = np.random.default_rng(55)
    A = rng.random((3, 4, 448)) ** 4
    keep, gamma, alpha = 179, 8, 32
    out = oracle.kara_select(A, keep, gamma, alpha, 64)
    for b in range(3):
        for h in range(4):
            row = out[b, h]
            assert row.size == keep + alpha + 64 and (np.diff(row) > 0).all()
            top = set(sorted(range(448), key=lambda j: (-A[b, h, j], j))[:keep])
            assert top <= set(row.tolist())


# ---------------------------------------------------------------- gather ----

def test_compact_rows_are_byte_identical():
    rng = np.random.default_rng(11)
    kb = rng.integers(0, 65536, size=(2, 3, 40, 8), dtype=np.uint16)
    idx = np.sort(rng.choice(40, size=(2, 3, 12)), axis=-1).astype(np.int32)
    out = oracle.compact_rows(kb, idx)
    for b in range(2):
        for h in range(3):
            for r in range(12):
                assert out[b, h, r].tobytes() == kb[b, h, idx[b, h, r]].tobytes()


def test_layer_end_compress_keeps_budget_plus_window():
    spec = synth.config(1)
    x = synth.make_layer(spec, 1)
    q, k = synth.to_f64(x["q"], "f32"), synth.to_f64(x["k"], "f32")
    out = oracle.layer_end_compress(q, k, x["v"], budget=spec.budget,
                                    window=spec.obs_window, pool_kernel=spec.pool_kernel,
                                    k_store=x["k"], v_store=x["v"])
    n = spec.budget + spec.obs_window
    assert out["idx"].shape == (1, 2, n)
    S, W = spec.seq_len, spec.obs_window
    for h in range(2):
        assert out["idx"][0, h, -W:].tolist() == list(range(S - W, S))
        assert (np.diff(out["idx"][0, h]) > 0).all()
    assert out["k_hat"].tobytes() == np.stack(
        [x["k"][0, h, out["idx"][0, h]] for h in range(2)])[None].tobytes()
    # sinks are boosted x4 in the generator and win on score
    assert set(range(4)) <= set(out["idx"][0, 0].tolist())


# ----------------------------------------------------------------- tiers ----

def test_window_sums_and_ranks():
    s = np.arange(24, dtype=np.float64).reshape(1, 24)
    w = oracle.window_sums(s, 4)
    assert w.tolist() == [[6, 22, 38, 54, 70, 86]]
    tier, rank = oracle.route_tiers(w, 1, 3)
    assert rank.tolist() == [[5, 4, 3, 2, 1, 0]]
    assert tier.tolist() == [[2, 2, 1, 1, 1, 0]]
    # equal sums rank by index
    tier, rank = oracle.route_tiers(np.ones((2, 5)), 2, 2)
    assert rank.tolist() == [[0, 1, 2, 3, 4]] * 2
    assert tier.tolist() == [[0, 0, 1, 1, 2]] * 2


def test_route_tiers_brute_force():
    w = np.random.default_rng(12).integers(0, 5, size=(3, 16)).astype(np.float64)
    tier, rank = oracle.route_tiers(w, 4, 8)
    for r in range(3):
        order = sorted(range(16), key=lambda j: (-w[r, j], j))
        for pos, j in enumerate(order):
            assert rank[r, j] == pos
            assert tier[r, j] == (0 if pos < 4 else 1 if pos < 12 else 2)


# ------------------------------------------------------------------ int4 ----

def test_int4_range_and_extremes():
    x = np.random.default_rng(13).standard_normal((64, 128)).astype(np.float32)
    codes, lo, scale = oracle.quant_int4(x)
    assert codes.dtype == np.uint8 and codes.max() <= 15
    assert (codes[x.argmin(0), np.arange(128)] == 0).all()
    assert (codes[x.argmax(0), np.arange(128)] == 15).all()
    xh = oracle.dequant_int4(codes, lo, scale)
    assert (np.abs(x - xh) <= scale / 2 * (1 + 1e-5) + 4 * np.spacing(np.abs(x) + np.abs(lo))).all()


def test_int4_constant_group_is_exact():
    x = np.full((64, 3), 1.375, dtype=np.float32)
    codes, lo, scale = oracle.quant_int4(x)
    assert (codes == 0).all() and (scale == 0).all()
    assert (oracle.dequant_int4(codes, lo, scale) == x).all()


def test_int4_identity_codes_and_half_even():
    lo_v, sc = np.float32(-2.0), np.float32(0.25)       # hi = -2 + 15*0.25 = 1.75
    c = np.array([0, 15] + list(range(16)) + [3, 7], dtype=np.float32)
    x = (lo_v + c * sc).astype(np.float32)[:, None]
    codes, lo, scale = oracle.quant_int4(x)
    assert lo[0] == lo_v and scale[0] == sc
    assert codes[:, 0].tolist() == c.astype(int).tolist()
    # half-way points lo + (c + 0.5) * scale round to the even code
    half = (lo_v + (np.arange(15) + 0.5) * sc).astype(np.float32)
    xx = np.concatenate([[lo_v, lo_v + 15 * sc], half]).astype(np.float32)[:, None]
    codes, _, _ = oracle.quant_int4(xx)
    want = [0, 15] + [int(2 * round((c + 0.5) / 2)) for c in range(15)]
    assert codes[:, 0].tolist() == want


# ---------------------------------------------------------------- memory ----

def test_memory_figures_printed_by_the_pages():
    with open(os.path.join(GOLDEN, "memory_pins.json")) as f:
        pins = json.load(f)["pins"]
    unit = {"GiB": 2**30, "MiB": 2**20, "GB": 10**9}
    for p in pins:
        got = oracle.cache_bytes(p["layers"], p["batch"], p["kv_heads"], p["tokens"],
                                 p["head_dim"], p["elem_bytes"])
        want = p["printed_value"] * unit[p["printed_unit"]]
        assert abs(got - want) <= p["rel_tol"] * want, p["what"]
        if "reading_gib" in p:          # an exact check resting on a reading of the page
            assert p["reading"] and got == p["reading_gib"] * 2**30, p["what"]


def test_linear_budget_schedule():
    b = [synth.sweep_budget(l) for l in range(32)]
    assert b[0] == 4096 and b[31] == 512
    assert all(x >= y for x, y in zip(b, b[1:]))
    assert sum(b) == 73743


# ------------------------------------------------------------- tier output ---

def test_round_bf16_matches_torch_conversion():
    """Round-to-nearest-even to bfloat16, pinned to torch's own conversion,
    including exact halfway cases in both parities."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(21)
    x = np.concatenate([rng.standard_normal(20000).astype(np.float32) * 50,
                        np.array([1.0, -2.5, 3.0e-30, 65504.0, 0.0, -0.0], np.float32)])
    # halfway: low 16 bits exactly 0x8000 with even and odd kept parts
    half = (np.arange(64, dtype=np.uint32) << 16 | 0x3F800000 | 0x8000).view(np.float32)
    x = np.concatenate([x, half, -half])
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(oracle.round_bf16(x), want)


def test_pack_nibbles_layout():
    codes = np.array([[1, 2, 15, 0, 7, 8]], dtype=np.uint8)
    assert oracle.pack_nibbles(codes).tolist() == [[0x21, 0x0F, 0x87]]


def test_tier_outputs_small_brute_force():
    """Full-tier rows are the routed windows' bits in window order; int4 slots
    follow window order; metadata is the per-channel min and range/15."""
    rng = np.random.default_rng(22)
    Bt, Hkv, win, nW, D = 1, 2, 4, 5, 6
    kb = synth.f32_to_bf16_bits(rng.standard_normal((Bt, Hkv, nW * win, D)).astype(np.float32))
    vb = synth.f32_to_bf16_bits(rng.standard_normal((Bt, Hkv, nW * win, D)).astype(np.float32))
    tier = np.array([[[1, 0, 2, 1, 0], [2, 0, 0, 1, 1]]], dtype=np.int8)
    prom = np.array([[[1], [0]]], dtype=np.int32)
    out = oracle.tier_outputs(kb, vb, tier, win, prom)
    assert out["k_full"][0, 0].tobytes() == np.concatenate([kb[0, 0, 4:8], kb[0, 0, 16:20]]).tobytes()
    assert out["v_full"][0, 1].tobytes() == vb[0, 1, 4:12].tobytes()
    assert out["k_codes"].shape == (1, 2, 2, win, D // 2)
    f = synth.bf16_bits_to_f32(kb[0, 0, 12:16])            # window 3 = int4 slot 1 of head 0
    lo, hi = f.min(0), f.max(0)
    np.testing.assert_array_equal(out["k_meta"][0, 0, 1, :, 0], lo)
    np.testing.assert_array_equal(out["k_meta"][0, 0, 1, :, 1],
                                  ((hi - lo).astype(np.float32) / np.float32(15)).astype(np.float32))
    # promoted slot 1 of head 0 is window 3 dequantised; every value within
    # half a quantisation step (plus bf16 rounding) of the source
    deq = synth.bf16_bits_to_f32(out["k_prom"][0, 0])
    step = out["k_meta"][0, 0, 1, :, 1]
    assert (np.abs(deq - f) <= step / 2 + np.abs(f) * 2 ** -8 + 1e-30).all()


# ------------------------------------------------- QEvict routing steps ----

def _bf16_bits(vals):
    """Exactly representable float32 values -> bf16 bit patterns."""
    u = np.asarray(vals, dtype=np.float32).view(np.uint32)
    assert np.all((u & 0xFFFF) == 0)
    return (u >> 16).astype(np.uint16)


def test_int2_extremes_constant_identity_and_half_even():
    """INT2 rule written out: min -> 0, max -> 3, a constant group gives
    zeros, lo + c*scale with an exact scale gives c, and half-way values
    round to even (lo + 0.5 s -> 0, lo + 1.5 s -> 2, lo + 2.5 s -> 2)."""
    x = _rand((64, 8), 31).astype(np.float32)
    c, lo, sc = oracle.quant_lowbit(x, 2)
    assert c.max() <= 3
    assert np.all(c[np.argmin(x, axis=0), np.arange(8)] == 0)
    assert np.all(c[np.argmax(x, axis=0), np.arange(8)] == 3)
    c0, lo0, sc0 = oracle.quant_lowbit(np.full((64, 1), 1.25, np.float32), 2)
    assert np.all(c0 == 0) and sc0[0] == 0 and lo0[0] == np.float32(1.25)
    # lo = 1, hi = 2.5 -> scale = 0.5 exactly
    g = np.array([1.0, 1.5, 2.0, 2.5, 1.25, 1.75, 2.25, 2.5], np.float32)[:, None]
    c1, lo1, sc1 = oracle.quant_lowbit(g, 2)
    assert sc1[0] == np.float32(0.5) and lo1[0] == np.float32(1.0)
    assert c1[:, 0].tolist() == [0, 1, 2, 3, 0, 2, 2, 3]


def test_lowbit_four_bits_is_the_int4_rule():
    x = _rand((64, 16), 32).astype(np.float32)
    a = oracle.quant_lowbit(x, 4)
    b = oracle.quant_int4(x)
    for u, w in zip(a, b):
        assert np.array_equal(u, w)


def test_pack_codes_layout():
    """Lowest channel in the lowest bits: [1, 2, 3, 0] -> 1 | 2<<2 | 3<<4 = 57;
    4-bit packing equals the nibble layout."""
    assert oracle.pack_codes(np.array([[1, 2, 3, 0]], np.uint8), 2).tolist() == [[57]]
    c = np.random.default_rng(3).integers(0, 16, (5, 32)).astype(np.uint8)
    assert np.array_equal(oracle.pack_codes(c, 4), oracle.pack_nibbles(c))
    c2 = np.random.default_rng(4).integers(0, 4, (5, 32)).astype(np.uint8)
    assert np.array_equal(oracle.unpack_codes(oracle.pack_codes(c2, 2), 2), c2)


def _qe_setup(nW=6, win=4, D=8, n_sink=2, n_recent=3, seed=5, bits=2):
    S = n_sink + nW * win + n_recent + 1          # one leftover token joins the recent region
    rng = np.random.default_rng(seed)
    vals = (rng.integers(-64, 64, (1, 1, S, D)) / 16.0).astype(np.float32)
    k = _bf16_bits(vals)
    v = _bf16_bits(-vals)
    st = oracle.qevict_init(1, 1, nW + 2, D, win, bits)
    return S, k, v, st


def _window_scores(S, n_sink, win, per_window):
    s = np.zeros((1, 1, S), np.float32)
    for j, w in enumerate(per_window):
        s[0, 0, n_sink + win * j] = w          # the whole window's mass on its first token
    return s


def test_qevict_routing_steps_by_hand():
    """Six windows, capacities 2 full / 2 quantised.  Step 1 ranks 5,4 | 3,2 |
    1,0; step 2 makes windows 0 and 1 the strongest, but eviction is
    permanent, so the live windows 2..5 are re-ranked among themselves."""
    S, k, v, st = _qe_setup()
    kw = dict(seq_len=S, n_sink=2, n_recent=3, win=4, n_full=2, n_quant=2, bits=2)
    st = oracle.qevict_step(st, _window_scores(S, 2, 4, [1, 2, 3, 4, 5, 6]), k, v, **kw)
    assert st["tier"][0, 0, :6].tolist() == [2, 2, 1, 1, 0, 0]
    assert st["has_codes"][0, 0, :6].tolist() == [0, 0, 1, 1, 0, 0]
    # step 2: accumulated 0+100, 2+100, 3+10, 4, 5, 6+1 -> live order 2 (13), 5 (7), 4, 3
    st = oracle.qevict_step(st, _window_scores(S, 2, 4, [100, 100, 10, 0, 0, 1]), k, v, **kw)
    assert st["w_acc"][0, 0, :6].tolist() == [101, 102, 13, 4, 5, 7]
    assert st["tier"][0, 0, :6].tolist() == [2, 2, 0, 1, 1, 0]
    # windows beyond nW are never touched
    assert st["tier"][0, 0, 6:].tolist() == [0, 0] and st["w_acc"][0, 0, 6:].tolist() == [0, 0]


def test_qevict_backing_store_is_reused_and_promotion_writes_dequantised_rows():
    """F -> Q quantises the window once; Q -> F writes the dequantised values
    (brute force per value) into the cache rows; a second demotion keeps the
    first codes although the rows changed; protected rows never change."""
    S, k, v, st = _qe_setup()
    k0, v0 = k.copy(), v.copy()
    kw = dict(seq_len=S, n_sink=2, n_recent=3, win=4, n_full=5, n_quant=1, bits=2)
    # step 1: window 0 weakest -> quantised
    st = oracle.qevict_step(st, _window_scores(S, 2, 4, [1, 9, 9, 9, 9, 9]), k, v, **kw)
    assert st["tier"][0, 0, :6].tolist() == [1, 0, 0, 0, 0, 0]
    codes1 = st["k_codes"][0, 0, 0].copy()
    meta1 = st["k_meta"][0, 0, 0].copy()
    rows = (k0[0, 0, 2:6].astype(np.uint32) << 16).view(np.float32)
    lo = rows.min(axis=0)
    sc = (rows.max(axis=0) - lo) / np.float32(3)
    assert np.array_equal(meta1[:, 0], lo) and np.array_equal(meta1[:, 1], sc.astype(np.float32))
    # step 2: window 0 strongest, window 1 weakest -> 0 promoted, 1 quantised
    st = oracle.qevict_step(st, _window_scores(S, 2, 4, [100, 0, 1, 1, 1, 1]), k, v, **kw)
    assert st["tier"][0, 0, :6].tolist() == [0, 1, 0, 0, 0, 0]
    cu = oracle.unpack_codes(codes1, 2)
    for t in range(4):
        for ch in range(8):
            x = float(np.float32(meta1[ch, 0]) + np.float32(np.float32(cu[t, ch]) * meta1[ch, 1]))
            want = oracle.round_bf16(np.array([x], np.float32))[0]
            assert k[0, 0, 2 + t, ch] == want
    promoted = k[0, 0, 2:6].copy()
    # Re-quantising the dequantised rows would give the same codes here, so
    # make reuse observable: overwrite the window's cache rows; a re-demotion
    # must still hold the first codes, and the next promotion restores the
    # rows from them.
    k[0, 0, 2:6] = 0
    v[0, 0, 2:6] = 0
    # step 3: accumulated 101, 1009, 210 x 4 -> window 0 is the weakest and is
    # demoted again: the first codes, not a re-quantisation of its new rows
    st = oracle.qevict_step(st, _window_scores(S, 2, 4, [0, 1000, 200, 200, 200, 200]), k, v, **kw)
    assert st["tier"][0, 0, 0] == 1
    assert np.array_equal(st["k_codes"][0, 0, 0], codes1)
    assert np.array_equal(st["k_meta"][0, 0, 0], meta1)
    # step 4: promoted again -> the same rows as after the first promotion
    st = oracle.qevict_step(st, _window_scores(S, 2, 4, [10000, 0, 0, 0, 0, 0]), k, v, **kw)
    assert st["tier"][0, 0, 0] == 0 and np.array_equal(k[0, 0, 2:6], promoted)
    # protected sinks and recent rows (incl. the partial window) untouched
    assert np.array_equal(k[0, 0, :2], k0[0, 0, :2]) and np.array_equal(k[0, 0, 26:], k0[0, 0, 26:])
    assert np.array_equal(v[0, 0, :2], v0[0, 0, :2])


def test_qevict_capacities_and_permanent_eviction_random():
    """Over random steps: at most n_full full and n_quant quantised windows,
    the full tier holds the best live windows, evicted windows stay evicted,
    and with enough capacity nothing is ever evicted."""
    rng = np.random.default_rng(9)
    S, k, v, st = _qe_setup(nW=12, seed=11, bits=4)
    kw = dict(seq_len=S, n_sink=2, n_recent=3, win=4, n_full=3, n_quant=4, bits=4)
    evicted = np.zeros(12, bool)
    for _ in range(6):
        sc = rng.integers(0, 5, (1, 1, S)).astype(np.float32)
        st = oracle.qevict_step(st, sc, k, v, **kw)
        t = st["tier"][0, 0, :12]
        assert np.sum(t == 0) <= 3 and np.sum(t == 1) <= 4
        assert np.all(t[evicted] == 2)
        evicted = t == 2
        live = np.flatnonzero(t != 2)
        w = st["w_acc"][0, 0]
        best = sorted(live, key=lambda j: (-w[j], j))[:3]
        assert sorted(best) == sorted(np.flatnonzero(t == 0).tolist())
    S, k, v, st = _qe_setup(nW=5, seed=12)
    st = oracle.qevict_step(st, rng.random((1, 1, S)).astype(np.float32), k, v, seq_len=S,
                            n_sink=2, n_recent=3, win=4, n_full=2, n_quant=3, bits=2)
    assert not np.any(st["tier"][0, 0, :5] == 2)


def test_qevict_window_count():
    assert oracle.qevict_windows(32768, 5, 64, 64) == 510      # 32699 // 64
    assert oracle.qevict_windows(100, 5, 64, 64) == 0
    assert oracle.qevict_windows(5 + 64 + 64, 5, 64, 64) == 1
