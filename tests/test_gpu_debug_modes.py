"""The library's debug switches on the GPU: KVSEL_SYNC=1 waits for the stream
after every call (and would report a device error as KVSEL_ERR_DEVICE) with
the same results as the asynchronous calls; KVSEL_VALIDATE_ONLY=1 enqueues
nothing, so the outputs keep what they held."""
import pytest

import synth
from helpers import dev_tensor

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _layer():
    spec = synth.config(2)
    x = synth.make_layer(spec, 2)
    return spec, (dev_tensor(x[n], spec.dtype) for n in ("q", "k", "v"))


def test_sync_mode_gives_the_same_results(monkeypatch):
    import attention_score_eviction_amd as kvsel
    spec, (q, k, v) = _layer()
    kw = dict(budget=spec.budget, pool_kernel=spec.pool_kernel)
    a = kvsel.layer_end(q, k, v, **kw)
    torch.cuda.synchronize()
    monkeypatch.setenv("KVSEL_SYNC", "1")
    b = kvsel.layer_end(q, k, v, **kw)
    c_idx, c_off, c_k, c_v, _, _ = kvsel.layer_end_adaptive(
        q, k, v, total_budget=spec.n_kv_heads * spec.budget, pool_kernel=spec.pool_kernel)
    monkeypatch.setenv("KVSEL_SYNC", "0")
    d_idx, d_off, d_k, d_v, _, _ = kvsel.layer_end_adaptive(
        q, k, v, total_budget=spec.n_kv_heads * spec.budget, pool_kernel=spec.pool_kernel)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int16) if x.dtype == torch.bfloat16 else x,
                           y.view(torch.int16) if y.dtype == torch.bfloat16 else y)
    assert torch.equal(c_idx, d_idx) and torch.equal(c_off, d_off)
    assert torch.equal(c_k.view(torch.int16), d_k.view(torch.int16))
    assert torch.equal(c_v.view(torch.int16), d_v.view(torch.int16))


def test_validate_only_mode_enqueues_nothing(monkeypatch):
    import attention_score_eviction_amd as kvsel
    spec, (q, k, v) = _layer()
    S, Hkv = spec.seq_len, spec.n_kv_heads
    n_keep = spec.budget + spec.n_sink + spec.obs_window
    idx = torch.full((1, Hkv, n_keep), -7, dtype=torch.int32, device="cuda")
    k_out = torch.zeros((1, Hkv, n_keep, spec.head_dim), dtype=k.dtype, device="cuda")
    v_out = torch.zeros_like(k_out)
    raw = torch.full((1, Hkv, S), 5.0, device="cuda")
    pooled = torch.full_like(raw, 6.0)
    monkeypatch.setenv("KVSEL_VALIDATE_ONLY", "1")
    kvsel.layer_end(q, k, v, budget=spec.budget, pool_kernel=spec.pool_kernel, raw=raw,
                    pooled=pooled, idx=idx, k_out=k_out, v_out=v_out)
    with pytest.raises(kvsel.KvselError):     # the checks still run
        kvsel.layer_end(q, k, v, budget=S, pool_kernel=spec.pool_kernel)
    monkeypatch.setenv("KVSEL_VALIDATE_ONLY", "0")
    torch.cuda.synchronize()
    assert (idx == -7).all() and (raw == 5.0).all() and (pooled == 6.0).all()
    assert not k_out.view(torch.int16).any() and not v_out.view(torch.int16).any()


def _kernels_of(call):
    """Names of the kernels one call launches (the library's launch timing)."""
    import attention_score_eviction_amd as kvsel
    torch.cuda.synchronize()
    kvsel.timing_read()
    kvsel.timing_start("*")
    try:
        out = call()
        torch.cuda.synchronize()
    finally:
        kvsel.timing_start(None)
    return out, set(kvsel.timing_read())


def test_score_combine_mode_gives_the_same_bits(monkeypatch):
    """Small score problems (the 8K layer, the decode-time routing step) merge
    the per-chunk row statistics inside the second pass, in the combine
    kernel's order; KVSEL_SCORE_COMBINE=1 runs the separate combine launch
    instead.  Raw scores, selection and compacted cache are the same bits."""
    import attention_score_eviction_amd as kvsel
    spec, (q, k, v) = _layer()
    kw = dict(budget=spec.budget, pool_kernel=spec.pool_kernel)
    a, names_a = _kernels_of(lambda: kvsel.layer_end(q, k, v, **kw))
    monkeypatch.setenv("KVSEL_SCORE_COMBINE", "1")
    b, names_b = _kernels_of(lambda: kvsel.layer_end(q, k, v, **kw))
    monkeypatch.setenv("KVSEL_SCORE_COMBINE", "0")
    assert "score_combine" not in names_a and "score_combine" in names_b
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int16) if x.dtype == torch.bfloat16 else x,
                           y.view(torch.int16) if y.dtype == torch.bfloat16 else y)
    # eight decode queries per KV head over 32K keys, two sequences
    g = torch.Generator(device="cuda").manual_seed(5)
    qd = torch.randn((2, 32, 8, 128), generator=g, device="cuda").to(torch.bfloat16)
    kd = torch.randn((2, 8, 32768, 128), generator=g, device="cuda").to(torch.bfloat16)
    (p1, s1), names_1 = _kernels_of(lambda: kvsel.score(qd, kd, pool_kernel=1, causal=False))
    monkeypatch.setenv("KVSEL_SCORE_COMBINE", "1")
    (p2, s2), names_2 = _kernels_of(lambda: kvsel.score(qd, kd, pool_kernel=1, causal=False))
    monkeypatch.setenv("KVSEL_SCORE_COMBINE", "0")
    assert "score_combine" not in names_1 and "score_combine" in names_2
    assert torch.equal(s1, s2) and torch.equal(p1, p2)


def test_score_combine_mode_ragged_query_group(monkeypatch):
    """A query group that does not fill its 32-row tiles (G·W = 5 x 8 = 40
    rows in two tiles) over 8K keys: the rows past the group's end take no
    part in the merged statistics, with or without the combine launch."""
    import attention_score_eviction_amd as kvsel
    g = torch.Generator(device="cuda").manual_seed(6)
    q = torch.randn((1, 40, 8, 128), generator=g, device="cuda").to(torch.bfloat16)
    k = torch.randn((1, 8, 8192, 128), generator=g, device="cuda").to(torch.bfloat16)
    (p1, s1), names_1 = _kernels_of(lambda: kvsel.score(q, k, pool_kernel=5))
    monkeypatch.setenv("KVSEL_SCORE_COMBINE", "1")
    (p2, s2), names_2 = _kernels_of(lambda: kvsel.score(q, k, pool_kernel=5))
    monkeypatch.setenv("KVSEL_SCORE_COMBINE", "0")
    assert "score_combine" not in names_1 and "score_combine" in names_2
    assert torch.equal(s1, s2) and torch.equal(p1, p2)
    # every query row's weights sum to one: each key column sums to the
    # group's 40 rows in total
    assert abs(float(s1.double().sum()) - 8 * 40) < 1e-2
