"""kvsel_layer_end (TideKV Algorithm 2 in one call; for long rows the max
filter, selection and gather run fused behind the score passes) gives
exactly the outputs of kvsel_score followed by kvsel_select_compact: raw and
pooled scores, indices and gathered rows, bit for bit."""
import dataclasses

import numpy as np
import pytest

import oracle
import synth
from helpers import dev_tensor

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

L = synth.LayerSpec

CASES = [
    # long rows: the fused path
    ("qwen-like-40k", L(1, 40, 8, 128, 40000, 64, 7, 4096, structure="spans", n_spans=16), 41),
    ("sinks-ragged", L(2, 8, 2, 128, 30001, 32, 5, 2000, n_sink=3, structure="heavy"), 42),
    ("budget-1", L(1, 8, 2, 128, 20000, 16, 3, 1, structure="heavy"), 43),
    ("budget-all", L(1, 4, 1, 64, 18000, 16, 7, 18000 - 16 - 2, n_sink=2), 44),
    ("pool-1", L(1, 8, 4, 128, 25000, 32, 1, 3000, structure="heavy"), 45),
    ("pool-129", L(1, 8, 2, 128, 20000, 32, 129, 3000, structure="heavy"), 46),
    ("f32-long", L(1, 4, 2, 64, 20000, 16, 5, 1000, dtype="f32"), 47),
    ("noncausal", L(1, 8, 2, 128, 24000, 40, 7, 2500, causal=0, structure="heavy"), 48),
    # two sequences on the 10-tile (G*W = 320) 8-wave passes, with sinks
    ("batch2-gw320", L(2, 10, 2, 128, 20000, 64, 7, 1500, n_sink=4, structure="spans",
                       n_spans=8), 50),
    # short rows (one workgroup per row): the gather fused into the select
    # while the kept rows fit its LDS list, else a separate gather
    ("short-8k", synth.config(2), 2),
    ("short-pool-129", L(1, 8, 2, 128, 9000, 32, 129, 1000, structure="heavy"), 63),
    ("short-sinks-ragged", L(2, 8, 2, 64, 7001, 16, 5, 700, n_sink=3), 64),
    ("short-no-fused-gather", L(1, 8, 2, 128, 16000, 32, 7, 4500, structure="heavy"), 65),
    ("short-no-candidates", L(1, 4, 2, 64, 64, 60, 3, 0, n_sink=4), 66),
    ("short-f32", L(1, 4, 2, 64, 3000, 16, 7, 200, dtype="f32"), 67),
    ("short-budget-all", L(1, 8, 2, 128, 4000, 32, 3, 4000 - 32 - 1, n_sink=1), 68),
    # unmasked, 512 keys, 256 query rows per KV head: keys-in-LDS scoring
    ("short-noncausal-keys-on-chip", L(1, 32, 8, 128, 512, 64, 7, 300, causal=0), 69),
    # more candidates than one workgroup's register batches, budget 0: the
    # composed path
    ("budget-0", L(1, 8, 2, 128, 20000, 32, 7, 0), 49),
]


@pytest.mark.parametrize("name,spec,seed", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("with_v", [True, False])
def test_layer_end_equals_composed_calls(name, spec, seed, with_v):
    import attention_score_eviction_amd as kvsel
    x = synth.make_layer(spec, seed, want_v=with_v)
    q, k = dev_tensor(x["q"], spec.dtype), dev_tensor(x["k"], spec.dtype)
    v = dev_tensor(x["v"], spec.dtype) if with_v else None
    kw = dict(n_sink=spec.n_sink, causal=bool(spec.causal))
    print(f"case layer_end {name} S={spec.seq_len} B={spec.budget} v={with_v}", flush=True)
    pooled, raw = kvsel.score(q, k, pool_kernel=spec.pool_kernel, **kw)
    idx, kh, vh = kvsel.select_compact(pooled, k, v, spec.budget, obs_window=spec.obs_window,
                                       n_q_heads=spec.n_q_heads, **kw)
    idx2, kh2, vh2, raw2, pooled2 = kvsel.layer_end(q, k, v, budget=spec.budget,
                                                    pool_kernel=spec.pool_kernel, **kw)
    torch.cuda.synchronize()
    bits = torch.int16 if spec.dtype == "bf16" else torch.int32
    assert torch.equal(raw2, raw)
    assert torch.equal(pooled2, pooled)
    assert torch.equal(idx2, idx)
    assert torch.equal(kh2.view(bits), kh.view(bits))
    if with_v:
        assert torch.equal(vh2.view(bits), vh.view(bits))
    else:
        assert vh2 is None


def test_layer_end_without_score_outputs():
    """raw and pooled kept in the workspace: the same selection and rows."""
    import attention_score_eviction_amd as kvsel
    spec = dataclasses.replace(synth.config(3), seq_len=30000)
    x = synth.make_layer(spec, 3)
    q, k, v = (dev_tensor(x[n], "bf16") for n in ("q", "k", "v"))
    a = kvsel.layer_end(q, k, v, budget=spec.budget, pool_kernel=spec.pool_kernel)
    b = kvsel.layer_end(q, k, v, budget=spec.budget, pool_kernel=spec.pool_kernel,
                        want_scores=False)
    torch.cuda.synchronize()
    assert b[3] is None and b[4] is None
    assert torch.equal(a[0], b[0])
    assert torch.equal(a[1].view(torch.int16), b[1].view(torch.int16))
    assert torch.equal(a[2].view(torch.int16), b[2].view(torch.int16))


DEGENERATE = [
    # every key zero: uniform attention, every candidate has the same score,
    # so the whole row sits in one bin and the cut is a pure position tie
    ("zero-keys", L(1, 8, 2, 128, 40000, 32, 7, 3000), 0.0, 51),
    # keys scaled down: a few distinct values crowded into a handful of bins
    ("crowded", L(1, 8, 2, 128, 40000, 32, 3, 5000), 1e-3, 52),
    ("crowded-b1", L(1, 8, 2, 128, 30000, 32, 1, 1), 1e-3, 53),
    # more slices per row than the 128K workload, ragged tail
    ("long-ragged", L(1, 8, 2, 64, 200003, 64, 7, 4096, structure="heavy"), 1.0, 54),
]


@pytest.mark.parametrize("name,spec,kscale,seed", DEGENERATE, ids=[c[0] for c in DEGENERATE])
def test_layer_end_degenerate_scores(name, spec, kscale, seed):
    """Rows whose scores crowd into few bins (the compacted boundary bin larger
    than the fused selection keeps in LDS) and all-equal rows: the fused path
    still equals the composed calls bit for bit."""
    import attention_score_eviction_amd as kvsel
    x = synth.make_layer(spec, seed)
    if kscale != 1.0:
        k32 = synth.bf16_bits_to_f32(x["k"]) * np.float32(kscale)
        x["k"] = synth.f32_to_bf16_bits(k32)
    q, k, v = (dev_tensor(x[n], spec.dtype) for n in ("q", "k", "v"))
    print(f"case layer_end degenerate {name} S={spec.seq_len} B={spec.budget}", flush=True)
    pooled, raw = kvsel.score(q, k, pool_kernel=spec.pool_kernel)
    idx, kh, vh = kvsel.select_compact(pooled, k, v, spec.budget, obs_window=spec.obs_window,
                                       n_q_heads=spec.n_q_heads)
    idx2, kh2, vh2, raw2, pooled2 = kvsel.layer_end(q, k, v, budget=spec.budget,
                                                    pool_kernel=spec.pool_kernel)
    torch.cuda.synchronize()
    assert torch.equal(raw2, raw)
    assert torch.equal(pooled2, pooled)
    assert torch.equal(idx2, idx)
    assert torch.equal(kh2.view(torch.int16), kh.view(torch.int16))
    assert torch.equal(vh2.view(torch.int16), vh.view(torch.int16))
    # the exact (score desc, position asc) selection on these fp32 scores
    S, W = spec.seq_len, spec.obs_window
    ref = oracle.select(pooled2.cpu().numpy().astype(np.float64), spec.budget, 0, W)
    assert (idx2.cpu().numpy() == ref).all()
    # a head whose candidates all tie keeps the first `budget` positions
    pc = pooled2.cpu().numpy()[0, :, :S - W]
    got = idx2.cpu().numpy()[0, :, :spec.budget]
    ties = [h for h in range(spec.n_kv_heads) if (pc[h] == pc[h, 0]).all()]
    for h in ties:
        assert (got[h] == np.arange(spec.budget)).all()
    print(f"heads with all candidates tied: {ties}", flush=True)


@pytest.mark.parametrize("ndup,budget", [(300, 150), (40, 20), (40, 40)])
def test_layer_end_duplicate_keys_tie_across_slices(ndup, budget):
    """Every key zero except ndup identical keys at scattered positions, which
    take the top scores, all exactly equal (no pooling): the budget cuts
    inside that tie, so the picks are its first `budget` positions.  More than
    64 tied candidates settle the last digit and the cut by scan, up to 64 by
    direct ranking, and a budget equal to the tie keeps its bin whole."""
    import attention_score_eviction_amd as kvsel
    spec = L(1, 8, 2, 128, 40000, 32, 1, budget)
    x = synth.make_layer(spec, 61)
    rng = np.random.default_rng(62)
    S, W, G = spec.seq_len, spec.obs_window, spec.group
    pos = np.sort(rng.choice(S - W, size=ndup, replace=False))
    q32 = synth.bf16_bits_to_f32(x["q"])
    k32 = np.zeros_like(synth.bf16_bits_to_f32(x["k"]))
    for hk in range(spec.n_kv_heads):
        d = q32[0, hk * G:(hk + 1) * G].reshape(-1, spec.head_dim).mean(axis=0)
        k32[0, hk, pos] = (d / np.linalg.norm(d) * 40.0).astype(np.float32)
    x["k"] = synth.f32_to_bf16_bits(k32)
    q, k, v = (dev_tensor(x[n], spec.dtype) for n in ("q", "k", "v"))
    print(f"case layer_end duplicate keys ndup={ndup} B={budget}", flush=True)
    pooled, raw = kvsel.score(q, k, pool_kernel=1)
    idx, kh, vh = kvsel.select_compact(pooled, k, v, budget, obs_window=W,
                                       n_q_heads=spec.n_q_heads)
    idx2, kh2, vh2, raw2, pooled2 = kvsel.layer_end(q, k, v, budget=budget, pool_kernel=1)
    torch.cuda.synchronize()
    assert torch.equal(pooled2, pooled)
    assert torch.equal(idx2, idx)
    assert torch.equal(kh2.view(torch.int16), kh.view(torch.int16))
    assert torch.equal(vh2.view(torch.int16), vh.view(torch.int16))
    ref = oracle.select(pooled2.cpu().numpy().astype(np.float64), budget, 0, W)
    assert (idx2.cpu().numpy() == ref).all()
    p = pooled2.cpu().numpy()[0]
    got = idx2.cpu().numpy()[0, :, :budget]
    for hk in range(spec.n_kv_heads):
        vals = p[hk, pos]
        assert (vals == vals[0]).all() and vals[0] > np.delete(p[hk, :S - W], pos).max()
        assert (got[hk] == pos[:budget]).all()


@pytest.mark.parametrize("S", [4194317, 4194318])
def test_layer_end_at_slice_limit(S):
    """The longest rows of the fused path: 1024 slices of 4096 candidates
    (S = 4194317 with W = 16), and one slice more, where the composed calls
    run instead.  Both equal the composed calls bit for bit and the oracle's
    selection on the same pooled scores; the raw scores sum to G*W."""
    import attention_score_eviction_amd as kvsel
    Hq, Hkv, D, W, B = 2, 1, 64, 16, 100000
    g = torch.Generator(device="cuda").manual_seed(S)
    q = torch.randn((1, Hq, W, D), generator=g, device="cuda").to(torch.bfloat16)
    k = torch.randn((1, Hkv, S, D), generator=g, device="cuda").to(torch.bfloat16)
    v = torch.randn((1, Hkv, S, D), generator=g, device="cuda").to(torch.bfloat16)
    print(f"case layer_end slice limit S={S}", flush=True)
    pooled, raw = kvsel.score(q, k, pool_kernel=7)
    idx, kh, vh = kvsel.select_compact(pooled, k, v, B, obs_window=W, n_q_heads=Hq)
    idx2, kh2, vh2, raw2, pooled2 = kvsel.layer_end(q, k, v, budget=B, pool_kernel=7)
    torch.cuda.synchronize()
    assert torch.equal(raw2, raw)
    assert torch.equal(pooled2, pooled)
    assert torch.equal(idx2, idx)
    assert torch.equal(kh2.view(torch.int16), kh.view(torch.int16))
    assert torch.equal(vh2.view(torch.int16), vh.view(torch.int16))
    p = pooled2.cpu().numpy().astype(np.float64)
    ref = oracle.select(p, B, 0, W)
    assert (idx2.cpu().numpy() == ref).all()
    total = raw2.cpu().numpy().astype(np.float64).sum()
    assert abs(total - (Hq // Hkv) * W) <= 1e-4 * (Hq // Hkv) * W
    rows = idx2[0, 0].long()
    assert torch.equal(kh2[0, 0].view(torch.int16), k[0, 0, rows].view(torch.int16))
