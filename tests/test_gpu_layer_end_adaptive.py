"""kvsel_layer_end_adaptive (TideKV Algorithm 2 with the head-adaptive
budget of Section 4.1, in one call; on long rows the max filter runs fused
with the first histogram of the head-group select) gives exactly the outputs
of kvsel_score, then kvsel_select_adaptive, then kvsel_compact_flat: raw and
pooled scores, indices, head offsets and gathered rows, bit for bit.  The
oracle check of the same call is in test_gpu_parity."""
import dataclasses

import numpy as np
import pytest

import synth
from helpers import dev_tensor

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

L = synth.LayerSpec


def _all(spec):
    return spec.n_kv_heads * (spec.seq_len - spec.obs_window - spec.n_sink)


CASES = [
    # long rows: the fused path
    ("qwen-like-40k", L(1, 40, 8, 128, 40000, 64, 7, 4096, structure="spans", n_spans=16), 51,
     None),
    ("sinks-ragged-batch2", L(2, 8, 2, 128, 30001, 32, 5, 2000, n_sink=3, structure="heavy"),
     52, None),
    ("budget-1", L(1, 8, 2, 128, 20000, 16, 3, 1, structure="heavy"), 53, 1),
    ("budget-all", L(1, 4, 2, 64, 18000, 16, 7, 100, n_sink=2), 54, "all"),
    ("pool-1", L(1, 8, 4, 128, 25000, 32, 1, 3000, structure="heavy"), 55, None),
    ("f32-long", L(1, 4, 2, 64, 20000, 16, 5, 1000, dtype="f32"), 56, None),
    ("noncausal", L(1, 8, 2, 128, 24000, 40, 7, 2500, causal=0, structure="heavy"), 57, None),
    ("llama-8k", synth.config(2), 2, None),
    ("qwen-128k", synth.config(4), 4, None),
    # one workgroup per sequence, and budget 0: the composed path
    ("tiny-f32", synth.config(1), 1, None),
    ("budget-0", L(1, 8, 2, 128, 20000, 32, 7, 100), 58, 0),
]


def _inputs(spec, seed, with_v, twin=False):
    x = synth.make_layer(spec, seed, want_v=with_v)
    if twin:
        # KV heads 0 and 1 get identical keys and query groups: every score
        # of head 1 ties with head 0's at the same position
        G = spec.n_q_heads // spec.n_kv_heads
        x["k"][:, 1] = x["k"][:, 0]
        x["q"][:, G:2 * G] = x["q"][:, 0:G]
    q, k = dev_tensor(x["q"], spec.dtype), dev_tensor(x["k"], spec.dtype)
    v = dev_tensor(x["v"], spec.dtype) if with_v else None
    return q, k, v


def _composed(kvsel, spec, q, k, v, T):
    kw = dict(n_sink=spec.n_sink, causal=bool(spec.causal))
    pooled, raw = kvsel.score(q, k, pool_kernel=spec.pool_kernel, **kw)
    idx, off = kvsel.select_adaptive(pooled, T, obs_window=spec.obs_window,
                                     n_q_heads=spec.n_q_heads, head_dim=spec.head_dim,
                                     dtype=k.dtype, **kw)
    kh, vh = kvsel.compact_flat(k, v, idx, off)
    return idx, off, kh, vh, raw, pooled


def _assert_equal(spec, got, want, with_v):
    bits = torch.int16 if spec.dtype == "bf16" else torch.int32
    idx, off, kh, vh, raw, pooled = got
    idx0, off0, kh0, vh0, raw0, pooled0 = want
    assert torch.equal(raw, raw0)
    assert torch.equal(pooled, pooled0)
    assert torch.equal(off, off0)
    assert torch.equal(idx, idx0)
    assert torch.equal(kh.view(bits), kh0.view(bits))
    if with_v:
        assert torch.equal(vh.view(bits), vh0.view(bits))
    else:
        assert vh is None


@pytest.mark.parametrize("name,spec,seed,total", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("with_v", [True, False])
def test_layer_end_adaptive_equals_composed_calls(name, spec, seed, total, with_v):
    import attention_score_eviction_amd as kvsel
    T = spec.n_kv_heads * spec.budget if total is None else (
        _all(spec) if total == "all" else total)
    print(f"case layer_end_adaptive {name} S={spec.seq_len} T={T} v={with_v}", flush=True)
    q, k, v = _inputs(spec, seed, with_v)
    want = _composed(kvsel, spec, q, k, v, T)
    got = kvsel.layer_end_adaptive(q, k, v, total_budget=T, pool_kernel=spec.pool_kernel,
                                   n_sink=spec.n_sink, causal=bool(spec.causal))
    torch.cuda.synchronize()
    _assert_equal(spec, got, want, with_v)
    idx, off = got[0].cpu().numpy(), got[1].cpu().numpy()
    S, W, ns = spec.seq_len, spec.obs_window, spec.n_sink
    for b in range(spec.batch):
        assert off[b, 0] == 0 and off[b, -1] == idx.shape[1]
        for h in range(spec.n_kv_heads):
            row = idx[b, off[b, h]:off[b, h + 1]]
            assert np.all(np.diff(row) > 0)
            assert row[:ns].tolist() == list(range(ns))
            assert row[-W:].tolist() == list(range(S - W, S))


@pytest.mark.parametrize("T", [1, 999, 2 * 2048, "all"])
def test_layer_end_adaptive_ties_across_heads(T):
    """Two KV heads with identical scores: every pick at a tied score goes to
    the lower head first, in both paths."""
    import attention_score_eviction_amd as kvsel
    spec = L(1, 8, 4, 128, 24000, 32, 5, 2048, structure="heavy")
    T = _all(spec) if T == "all" else T
    print(f"case layer_end_adaptive twin heads T={T}", flush=True)
    q, k, v = _inputs(spec, 59, True, twin=True)
    want = _composed(kvsel, spec, q, k, v, T)
    got = kvsel.layer_end_adaptive(q, k, v, total_budget=T, pool_kernel=spec.pool_kernel)
    torch.cuda.synchronize()
    _assert_equal(spec, got, want, True)
    p = got[5].cpu().numpy()
    assert np.array_equal(p[0, 0], p[0, 1])          # the twin rows really tie
    off = got[1].cpu().numpy()[0]
    n0, n1 = off[1] - off[0], off[2] - off[1]
    assert n0 >= n1                                  # ties go to the lower head


def test_driver_adaptive_prepared_call():
    """The layer-major driver's head-adaptive layer end: the first call goes
    through the checked binding, later ones through the prepared call; both
    equal the composed calls, for two layers through one resident buffer."""
    import attention_score_eviction_amd as kvsel
    from attention_score_eviction_amd.driver import LayerMajorDriver
    spec = dataclasses.replace(synth.config(2), seq_len=20000)
    drv = LayerMajorDriver(spec.batch, spec.n_q_heads, spec.n_kv_heads, spec.head_dim,
                           spec.seq_len, spec.obs_window, spec.pool_kernel,
                           max_budget=spec.budget, n_sink=spec.n_sink)
    T = spec.n_kv_heads * spec.budget
    cache = drv.new_flat_cache(T)
    for layer, seed in enumerate((61, 62)):
        print(f"case driver adaptive layer {layer}", flush=True)
        x = synth.make_layer(spec, seed)
        t = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)  # noqa: E731
        drv.load(t(x["q"]), t(x["k"]), t(x["v"]))
        for _ in range(2):
            drv.layer_end_adaptive(cache)
            torch.cuda.synchronize()
            want = _composed(kvsel, spec, drv.q, drv.k, drv.v, T)
            torch.cuda.synchronize()
            got = (cache.idx, cache.head_off, cache.k_hat, cache.v_hat, drv.raw, drv.pooled)
            _assert_equal(spec, got, want, True)
    with pytest.raises(ValueError):
        drv.new_flat_cache(T + 1)
