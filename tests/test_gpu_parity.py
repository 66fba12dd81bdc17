"""Parity of the HIP path (through the C ABI) with the fp64 CPU oracle.

Tolerances: per-key raw and pooled scores within 1e-3 relative of the
oracle; retained sets identical except at candidates whose oracle score lies
within 1e-4 relative of the budget-th score; gathered rows byte-identical to
the source rows; selection from identical fp32 inputs bit-exact.
"""
import dataclasses

import numpy as np
import pytest

import oracle
import synth
from helpers import (assert_scores_close, check_adaptive_selection, check_selection, dev_tensor,
                     host_bits, rows_gathered)

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

L = synth.LayerSpec


def _kvsel():
    import attention_score_eviction_amd as kvsel
    kvsel.lib()
    return kvsel


# Small cases the oracle finishes in seconds.  Each spans several key chunks
# and query tiles and most have a ragged key tail.
SMALL = [
    ("c1-tiny-f32", synth.config(1), 1),
    ("bf16-ragged-sinks", L(2, 8, 2, 128, 1000, 20, 5, 100, n_sink=3, structure="heavy"), 101),
    ("bf16-noncausal", L(1, 4, 1, 128, 777, 8, 3, 50, causal=0, structure="heavy"), 102),
    ("bf16-d64", L(1, 6, 3, 64, 1500, 16, 7, 200, structure="heavy"), 103),
    ("bf16-gw320", L(1, 10, 2, 128, 2085, 64, 7, 256, structure="heavy"), 104),
    ("bf16-gw384-groups", L(1, 8, 1, 128, 1200, 48, 5, 128, n_sink=2), 105),
    ("f32-d128-groups", L(1, 2, 1, 128, 600, 80, 3, 64, dtype="f32"), 106),
    ("f32-d64-gqa1", L(1, 3, 3, 64, 333, 5, 1, 40, dtype="f32"), 107),
    ("bf16-budget-all", L(1, 2, 1, 128, 300, 12, 5, 288), 108),
    ("bf16-budget-zero", L(1, 2, 1, 128, 300, 12, 5, 0), 109),
    ("bf16-window-is-all", L(1, 2, 1, 128, 64, 64, 5, 0), 110),
    ("bf16-single-key", L(1, 2, 2, 64, 1, 1, 1, 0), 111),
    ("bf16-spans", L(1, 5, 1, 128, 4096, 64, 7, 512, structure="spans", n_spans=8), 112),
    # unmasked, at most 512 keys in whole tiles, >= 256 query rows per KV
    # head: one scoring launch per KV head with its keys in LDS
    ("bf16-noncausal-keys-on-chip", L(1, 32, 8, 128, 512, 64, 7, 200, n_sink=2, causal=0,
                                      structure="heavy"), 113),
    ("bf16-noncausal-keys-on-chip-d64", L(2, 16, 2, 64, 320, 40, 5, 100, causal=0), 114),
    # prompts of 4096 keys or more run the 32x32 tiling: D = 64, a ragged
    # tail, sinks, no mask, and two query groups (640 rows: 512 + 128)
    ("bf16-long-d64-ragged", L(1, 4, 2, 64, 4500, 24, 5, 300, n_sink=2, structure="heavy"), 113),
    ("bf16-long-gw640-groups", L(1, 20, 2, 128, 4160, 64, 7, 256), 114),
    ("bf16-long-noncausal", L(1, 8, 2, 128, 5000, 40, 3, 100, causal=0, structure="heavy"), 115),
    ("bf16-long-gw320", L(1, 10, 2, 128, 4100, 64, 7, 128, n_sink=4), 116),
    ("bf16-long-d64-gw384", L(1, 12, 2, 64, 4200, 64, 5, 100, structure="heavy"), 117),
    ("bf16-long-batch2-gw320", L(2, 10, 2, 128, 4300, 64, 7, 200, n_sink=2, structure="heavy"),
     118),
    # fp32 prompts past 4096 keys (16-row tiles), and the widest max filter
    ("f32-long-d128", L(1, 4, 2, 128, 9000, 32, 5, 500, n_sink=1, dtype="f32"), 119),
    ("bf16-long-pool129", L(1, 8, 2, 128, 5000, 32, 129, 300, structure="heavy"), 120),
]


def _run_and_check(spec, cid, heads=None):
    kvsel = _kvsel()
    x = synth.make_layer(spec, cid)
    q = dev_tensor(x["q"], spec.dtype)
    k = dev_tensor(x["k"], spec.dtype)
    v = dev_tensor(x["v"], spec.dtype)
    S, W = spec.seq_len, spec.obs_window
    print(f"case {spec.name} seed {cid} shape Bt={spec.batch} Hq={spec.n_q_heads} "
          f"Hkv={spec.n_kv_heads} D={spec.head_dim} S={S} W={W}", flush=True)
    out = kvsel.layer_end_compress(q, k, v, budget=spec.budget, pool_kernel=spec.pool_kernel,
                                   n_sink=spec.n_sink, causal=bool(spec.causal))
    torch.cuda.synchronize()
    s_g = out["s"].cpu().numpy()
    p_g = out["p"].cpu().numpy()
    idx_g = out["idx"].cpu().numpy()
    G = spec.group
    hs = list(range(spec.n_kv_heads)) if heads is None else heads
    q64 = synth.to_f64(x["q"], spec.dtype)
    k64 = synth.to_f64(x["k"], spec.dtype)
    for hk in hs:
        s_ref = oracle.head_scores(q64[:, hk * G:(hk + 1) * G], k64[:, hk:hk + 1],
                                   causal=bool(spec.causal))
        p_ref = oracle.max_pool(s_ref, spec.pool_kernel, spec.n_sink, S - W)
        assert_scores_close(s_g[:, hk:hk + 1], s_ref, what=f"raw scores head {hk}")
        assert_scores_close(p_g[:, hk:hk + 1], p_ref, what=f"pooled scores head {hk}")
        np.testing.assert_allclose(s_g[:, hk].astype(np.float64).sum(-1), G * W, rtol=1e-5)
        check_selection(idx_g[:, hk:hk + 1], p_ref, spec.budget, spec.n_sink, W)
    # every gathered row is, byte for byte, the source row its index names
    assert rows_gathered(host_bits(out["k_hat"]), x["k"], idx_g)
    assert rows_gathered(host_bits(out["v_hat"]), x["v"], idx_g)
    return out


@pytest.mark.parametrize("name,spec,cid", SMALL, ids=[c[0] for c in SMALL])
def test_small_parity(name, spec, cid):
    _run_and_check(dataclasses.replace(spec, name=name), cid)


@pytest.mark.parametrize("seed,Bt,Hq,Hkv,D,S,W,n_sink,budget,dtype,with_v", [
    (0, 1, 32, 8, 128, 8192, 32, 0, 1024, "bf16", True),     # the 8K layer
    (1, 2, 8, 2, 128, 3001, 20, 3, 200, "bf16", True),       # ragged, sinks
    (2, 1, 4, 2, 64, 900, 16, 0, 0, "f32", True),            # budget 0
    (3, 1, 4, 4, 128, 5000, 40, 2, 4000, "bf16", False),     # n_keep 4042, K only
    (4, 1, 8, 2, 128, 20000, 64, 0, 4096, "bf16", True),     # long rows: two launches
])
def test_select_compact_equals_select_then_compact(seed, Bt, Hq, Hkv, D, S, W, n_sink, budget,
                                                   dtype, with_v):
    """kvsel_select_compact gives exactly the outputs of kvsel_select followed
    by kvsel_compact."""
    kvsel = _kvsel()
    g = torch.Generator(device="cuda").manual_seed(seed)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    # pooled-like scores: non-negative with repeated values (plateaus)
    pooled = torch.rand((Bt, Hkv, S), generator=g, device="cuda")
    pooled = torch.floor(pooled * 4096) / 4096
    k = torch.randn((Bt, Hkv, S, D), generator=g, device="cuda").to(tdt)
    v = torch.randn((Bt, Hkv, S, D), generator=g, device="cuda").to(tdt) if with_v else None
    print(f"case select_compact seed {seed} S={S} budget={budget}", flush=True)
    idx1 = kvsel.select(pooled, budget, obs_window=W, n_q_heads=Hq, head_dim=D, n_sink=n_sink,
                        dtype=tdt)
    k1, v1 = kvsel.compact(k, v, idx1)
    idx2, k2, v2 = kvsel.select_compact(pooled, k, v, budget, obs_window=W, n_q_heads=Hq,
                                        n_sink=n_sink)
    torch.cuda.synchronize()
    bits = torch.int16 if tdt == torch.bfloat16 else torch.int32
    assert torch.equal(idx1, idx2)
    assert torch.equal(k1.view(bits), k2.view(bits))
    if with_v:
        assert torch.equal(v1.view(bits), v2.view(bits))
    else:
        assert v2 is None


def test_raw_only_scores_equal_pooled_call():
    """kvsel_score with pooled = NULL (raw scores only, no max filter) gives
    the same raw scores, bit for bit, as the full call."""
    kvsel = _kvsel()
    spec = dataclasses.replace(synth.config(2), seq_len=5000, obs_window=32)
    x = synth.make_layer(spec, 2)
    q, k = dev_tensor(x["q"], "bf16"), dev_tensor(x["k"], "bf16")
    _, raw_full = kvsel.score(q, k, pool_kernel=7)
    pooled, raw_only = kvsel.score(q, k, pool_kernel=7, want_pooled=False)
    torch.cuda.synchronize()
    assert pooled is None
    assert torch.equal(raw_full, raw_only)


def test_score_is_deterministic():
    kvsel = _kvsel()
    spec = synth.config(2)
    spec = dataclasses.replace(spec, seq_len=3000, obs_window=32)
    x = synth.make_layer(spec, 2, want_v=False)
    q, k = dev_tensor(x["q"], "bf16"), dev_tensor(x["k"], "bf16")
    p1, s1 = kvsel.score(q, k, pool_kernel=7)
    p2, s2 = kvsel.score(q, k, pool_kernel=7)
    torch.cuda.synchronize()
    assert torch.equal(s1, s2) and torch.equal(p1, p2)


@pytest.mark.parametrize("seed,S", [(0, 9000), (1, 9777), (2, 10554), (3, 70001), (4, 131072),
                                    (5, 50000), (6, 8000), (7, 4000), (8, 2000)])
def test_select_exact_on_identical_inputs(seed, S):
    """Given the same fp32 scores, the GPU selection is bit-exact with the
    oracle's (ties -> lowest positions), including heavy tie plateaus."""
    kvsel = _kvsel()
    rng = np.random.default_rng(seed)
    Bt, Hkv, W, n_sink = 2, 3, 40, seed % 3
    if seed in (0, 4):
        p = rng.random((Bt, Hkv, S)).astype(np.float32)
    elif seed == 5:
        # a dense band of near-equal values around the threshold
        p = (np.float32(1.0) + rng.integers(0, 3000, size=(Bt, Hkv, S)).astype(np.float32)
             * np.float32(2.0 ** -20)).astype(np.float32)
    elif seed in (1, 3, 6, 8):
        p = rng.integers(0, 5, size=(Bt, Hkv, S)).astype(np.float32) * np.float32(0.25)
    else:
        p = np.full((Bt, Hkv, S), 0.125, np.float32)
        p[..., ::97] = 3.0
        p[..., 5::11] = 0.0
    p[..., :n_sink] = 0
    p[..., S - W:] = 0
    pt = torch.from_numpy(p).cuda()
    for budget in [b for b in (1, 7, 1000, 4096, S - W - n_sink) if b <= S - W - n_sink]:
        got = kvsel.select(pt, budget, obs_window=W, n_q_heads=Hkv, head_dim=128,
                           n_sink=n_sink).cpu().numpy()
        want = oracle.select(p.astype(np.float64), budget, n_sink, W)
        np.testing.assert_array_equal(got, want)


@pytest.mark.parametrize("S,kind,budget", [(8192, "quarters", 1024), (8192, "plateau", 1024),
                                           (8192, "quarters", 3), (4000, "band", 700),
                                           (2000, "quarters", 1500)])
def test_select_compact_short_rows_with_ties(S, kind, budget):
    """The one-launch select + gather of short rows against the oracle when
    many scores tie at the cut: the ties before a thread that are not kept
    must not shift that thread's picks."""
    kvsel = _kvsel()
    rng = np.random.default_rng(S + budget)
    Bt, Hkv, Hq, D, W, n_sink = 1, 4, 16, 128, 32, 2
    p = _tie_heavy_scores(rng, kind, (Bt, Hkv, S))
    p[..., :n_sink] = 0
    p[..., S - W:] = 0
    k = torch.from_numpy(rng.standard_normal((Bt, Hkv, S, D)).astype(np.float32)).to(torch.bfloat16)
    v = torch.from_numpy(rng.standard_normal((Bt, Hkv, S, D)).astype(np.float32)).to(torch.bfloat16)
    print(f"case select_compact ties S={S} kind={kind} budget={budget}", flush=True)
    idx, k_out, v_out = kvsel.select_compact(torch.from_numpy(p).cuda(), k.cuda(), v.cuda(),
                                             budget, obs_window=W, n_q_heads=Hq, n_sink=n_sink)
    torch.cuda.synchronize()
    want = oracle.select(p.astype(np.float64), budget, n_sink, W)
    np.testing.assert_array_equal(idx.cpu().numpy(), want)
    kb = k.view(torch.int16).numpy()
    vb = v.view(torch.int16).numpy()
    np.testing.assert_array_equal(k_out.view(torch.int16).cpu().numpy(),
                                  np.take_along_axis(kb, want[..., None], axis=2))
    np.testing.assert_array_equal(v_out.view(torch.int16).cpu().numpy(),
                                  np.take_along_axis(vb, want[..., None], axis=2))


@pytest.mark.parametrize("S,kind", [(4194365, "band"), (4194366, "plateau")])
def test_select_exact_at_slice_limits(S, kind):
    """One row of 1024 slices of 4096 candidates (S = 4194365 with W = 64),
    the most the layer-end select chain takes, and one slice more (the
    generic sliced select): bit-exact with the oracle from one pick to all."""
    kvsel = _kvsel()
    rng = np.random.default_rng(S)
    W = 64
    p = _tie_heavy_scores(rng, kind, (1, 1, S))
    p[..., S - W:] = 0
    ncand = S - W
    print(f"case select slice limit S={S} kind={kind}", flush=True)
    pt = torch.from_numpy(p).cuda()
    p64 = p.astype(np.float64)
    for budget in [1, 4096, 123457, ncand]:
        got = kvsel.select(pt, budget, obs_window=W, n_q_heads=1, head_dim=128).cpu().numpy()
        np.testing.assert_array_equal(got, oracle.select(p64, budget, 0, W))


def test_compact_exact_with_oracle_indices():
    kvsel = _kvsel()
    rng = np.random.default_rng(5)
    Bt, Hkv, S, D = 2, 3, 700, 128
    kb = rng.integers(0, 65536, size=(Bt, Hkv, S, D), dtype=np.uint16)
    vb = rng.integers(0, 65536, size=(Bt, Hkv, S, D), dtype=np.uint16)
    idx = np.sort(rng.choice(S, size=(Bt, Hkv, 130)), axis=-1).astype(np.int32)
    idx[0, 0, 3] = -1          # out of range -> zero row
    idx[1, 2, 5] = S
    kh, vh = kvsel.compact(dev_tensor(kb, "bf16"), dev_tensor(vb, "bf16"),
                           torch.from_numpy(idx).cuda())
    torch.cuda.synchronize()
    safe = np.clip(idx, 0, S - 1)
    want_k = oracle.compact_rows(kb, safe)
    want_v = oracle.compact_rows(vb, safe)
    bad = (idx < 0) | (idx >= S)
    want_k[bad] = 0
    want_v[bad] = 0
    assert host_bits(kh).tobytes() == want_k.tobytes()
    assert host_bits(vh).tobytes() == want_v.tobytes()


def test_full_c2_llama_8k():
    """The bench workload (Llama-3-8B layer, S = 8192): every head checked."""
    _run_and_check(synth.config(2), 2)


def test_full_c3_layer0_64k_all_heads():
    """S = 65536, B = 4096 (first layer of the sweep): every KV head's scores
    and selection against the oracle, every row gathered byte for byte."""
    _run_and_check(synth.config(3), 3)


def test_full_c4_qwen_128k_all_heads():
    """S = 131072, 40 query heads (G = 5, G*W = 320), B = 4096: every KV
    head's scores and selection against the oracle."""
    _run_and_check(synth.config(4), 4)


def test_side_stream_equals_default_stream():
    """layer_end_compress enqueued on a side stream (its outputs and
    workspaces allocated on that stream) gives exactly the default-stream
    result."""
    kvsel = _kvsel()
    spec = dataclasses.replace(synth.config(2), seq_len=20000, obs_window=32, budget=2048)
    x = synth.make_layer(spec, 2)
    q, k, v = (dev_tensor(x[n], "bf16") for n in ("q", "k", "v"))
    ref = kvsel.layer_end_compress(q, k, v, budget=spec.budget, pool_kernel=spec.pool_kernel)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    outs = []
    for _ in range(3):      # repeated calls reuse freed blocks on the side stream
        outs.append(kvsel.layer_end_compress(q, k, v, budget=spec.budget,
                                             pool_kernel=spec.pool_kernel, stream=side))
    side.synchronize()
    for out in outs:
        for name in ("s", "p", "idx"):
            assert torch.equal(out[name], ref[name]), name
        for name in ("k_hat", "v_hat"):
            assert torch.equal(out[name].view(torch.int16), ref[name].view(torch.int16)), name


def test_scores_do_not_depend_on_key_blocking():
    """TideKV Section 4.2: the block size only trades work for memory; the
    result is the same.  One KV head scored alone (few, short key chunks) and
    the same head inside a batch of 8 heads (different chunking and grid)
    give scores within 1e-6 relative, and identical selections."""
    kvsel = _kvsel()
    spec = synth.config(2)
    x = synth.make_layer(spec, 2, want_v=False)
    q, k = dev_tensor(x["q"], "bf16"), dev_tensor(x["k"], "bf16")
    p_all, s_all = kvsel.score(q, k, pool_kernel=7)
    G = spec.group
    for hk in (0, 5):
        q1 = q[:, hk * G:(hk + 1) * G].contiguous()
        k1 = k[:, hk:hk + 1].contiguous()
        p1, s1 = kvsel.score(q1, k1, pool_kernel=7)
        torch.cuda.synchronize()
        rel = ((s1[:, 0] - s_all[:, hk]).abs() / s_all[:, hk].abs()).max().item()
        assert rel <= 1e-6, rel
        i1 = kvsel.select(p1, spec.budget, obs_window=spec.obs_window, n_q_heads=G, head_dim=128)
        ia = kvsel.select(p_all, spec.budget, obs_window=spec.obs_window, n_q_heads=spec.n_q_heads,
                          head_dim=128)
        s_ref = p_all[:, hk:hk + 1].double().cpu().numpy()
        check_selection(i1.cpu().numpy(), s_ref, spec.budget, 0, spec.obs_window)
        check_selection(ia[:, hk:hk + 1].cpu().numpy(), s_ref, spec.budget, 0, spec.obs_window)


# ----------------------------------------------- head-adaptive selection ----

def _tie_heavy_scores(rng, kind, shape):
    if kind == "uniform":
        return rng.random(shape).astype(np.float32)
    if kind == "quarters":
        return rng.integers(0, 5, size=shape).astype(np.float32) * np.float32(0.25)
    if kind == "band":
        return (np.float32(1.0) + rng.integers(0, 3000, size=shape).astype(np.float32)
                * np.float32(2.0 ** -20)).astype(np.float32)
    p = np.full(shape, 0.125, np.float32)       # plateau with sparse spikes
    p[..., ::97] = 3.0
    p[..., 5::11] = 0.0
    return p


@pytest.mark.parametrize("seed,Bt,Hkv,S,W,n_sink,kind", [
    (0, 2, 8, 1000, 40, 0, "uniform"),
    (1, 1, 8, 8192, 32, 4, "quarters"),
    (2, 2, 3, 9777, 64, 1, "plateau"),
    (3, 1, 8, 20000, 64, 0, "band"),
    (4, 3, 2, 5, 2, 1, "uniform"),
    (5, 1, 8, 131072, 64, 4, "uniform"),
    # more than 1024 slices in the group: the generic sliced select
    (6, 1, 8, 540000, 64, 0, "band"),
])
def test_select_adaptive_exact_on_identical_inputs(seed, Bt, Hkv, S, W, n_sink, kind):
    """Given the same fp32 scores, the head-adaptive picks and per-head
    offsets are bit-exact with the oracle's (ties -> lower head, then lower
    position), from one pick to every candidate of the sequence."""
    kvsel = _kvsel()
    rng = np.random.default_rng(200 + seed)
    p = _tie_heavy_scores(rng, kind, (Bt, Hkv, S))
    if kind == "uniform" and Hkv > 1:
        p[:, 1] *= np.float32(3.0)          # one head dominates the budget
    p[..., :n_sink] = 0
    p[..., S - W:] = 0
    ncand = S - W - n_sink
    print(f"case adaptive seed {seed} Bt={Bt} Hkv={Hkv} S={S} kind={kind}", flush=True)
    pt = torch.from_numpy(p).cuda()
    for T in sorted({min(t, Hkv * ncand) for t in (0, 1, 7, 1000, Hkv * 1024, Hkv * ncand)}):
        idx, off = kvsel.select_adaptive(pt, T, obs_window=W, n_q_heads=Hkv, head_dim=128,
                                         n_sink=n_sink)
        torch.cuda.synchronize()
        want_idx, want_off = oracle.select_head_adaptive(p.astype(np.float64), T, n_sink, W)
        np.testing.assert_array_equal(off.cpu().numpy(), want_off)
        np.testing.assert_array_equal(idx.cpu().numpy(), want_idx)


def test_compact_flat_exact_with_oracle_selection():
    kvsel = _kvsel()
    rng = np.random.default_rng(7)
    Bt, Hkv, S, D, W = 2, 4, 900, 64, 16
    kb = rng.integers(0, 65536, size=(Bt, Hkv, S, D), dtype=np.uint16)
    vb = rng.integers(0, 65536, size=(Bt, Hkv, S, D), dtype=np.uint16)
    p = rng.random((Bt, Hkv, S))
    p[:, 2] *= 4.0
    idx, off = oracle.select_head_adaptive(p, 777, 2, W)
    kh, vh = kvsel.compact_flat(dev_tensor(kb, "bf16"), dev_tensor(vb, "bf16"),
                                torch.from_numpy(idx).cuda(), torch.from_numpy(off).cuda())
    torch.cuda.synchronize()
    assert host_bits(kh).tobytes() == oracle.compact_flat(kb, idx, off).tobytes()
    assert host_bits(vh).tobytes() == oracle.compact_flat(vb, idx, off).tobytes()
    # an index outside [0, S) gives a zero row
    bad = idx.copy()
    bad[0, 5] = -3
    bad[1, 40] = S
    kh2, _ = kvsel.compact_flat(dev_tensor(kb, "bf16"), None, torch.from_numpy(bad).cuda(),
                                torch.from_numpy(off).cuda())
    torch.cuda.synchronize()
    got = host_bits(kh2)
    assert not got[0, 5].any() and not got[1, 40].any()
    want = oracle.compact_flat(kb, idx, off)
    want[0, 5] = 0
    want[1, 40] = 0
    assert got.tobytes() == want.tobytes()


@pytest.mark.parametrize("cid,heads_for_scores", [(2, None), (1, None)])
def test_adaptive_layer_end_against_oracle(cid, heads_for_scores):
    """Score -> head-adaptive select (sequence budget Hkv*B) -> flattened
    compact, against the oracle's scores and head-adaptive selection."""
    kvsel = _kvsel()
    spec = synth.config(cid)
    x = synth.make_layer(spec, cid)
    q, k, v = (dev_tensor(x[n], spec.dtype) for n in ("q", "k", "v"))
    T = spec.n_kv_heads * spec.budget
    print(f"case adaptive layer-end config {cid} T={T}", flush=True)
    out = kvsel.layer_end_compress_adaptive(q, k, v, total_budget=T,
                                            pool_kernel=spec.pool_kernel, n_sink=spec.n_sink)
    torch.cuda.synchronize()
    S, W = spec.seq_len, spec.obs_window
    s_ref = oracle.head_scores(synth.to_f64(x["q"], spec.dtype), synth.to_f64(x["k"], spec.dtype))
    p_ref = oracle.max_pool(s_ref, spec.pool_kernel, spec.n_sink, S - W)
    assert_scores_close(out["p"].cpu().numpy(), p_ref, what="pooled scores")
    idx_g, off_g = out["idx"].cpu().numpy(), out["head_off"].cpu().numpy()
    check_adaptive_selection(idx_g, off_g, p_ref, T, spec.n_sink, W)
    assert rows_gathered(host_bits(out["k_hat"]), x["k"], idx_g, off_g)
    assert rows_gathered(host_bits(out["v_hat"]), x["v"], idx_g, off_g)
