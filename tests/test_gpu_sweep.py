"""The layer-major sweep (TideKV Algorithm 1, Section 4.1) at 65536 tokens on
the GPU, through the same driver the benchmark times: one active full-prompt
K/V buffer filled in place per layer, each layer's compact cache committed to
a per-layer store, budgets from the linear 4096 -> 512 schedule.

Layers 0, 15 and 31 (budgets 4096, 2362, 512) are driven in order through
the one resident buffer.  For every layer and every KV head: raw and pooled
scores within 1e-3 of the oracle, the retained set equal to the oracle's
except at candidates within 1e-4 of the budget-th score, rows gathered byte
for byte.  The device memory high-water mark stays within one active layer
plus the committed store and the step's scratch.
"""
import numpy as np
import pytest

import oracle
import synth
from helpers import assert_scores_close, check_selection, dev_tensor, host_bits, rows_gathered

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def test_sweep_layers_through_one_resident_buffer():
    from attention_score_eviction_amd.driver import LayerMajorDriver, linear_budgets
    spec = synth.config(3)
    S, W, G = spec.seq_len, spec.obs_window, spec.group
    budgets = linear_budgets(32, 4096, 512)
    layers = [0, 15, 31]
    assert [budgets[l] for l in layers] == [4096, 2362, 512]
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    base = torch.cuda.memory_allocated()
    drv = LayerMajorDriver(spec.batch, spec.n_q_heads, spec.n_kv_heads, spec.head_dim, S, W,
                           spec.pool_kernel, max_budget=max(budgets))
    for layer in layers:
        print(f"case sweep layer {layer} budget {budgets[layer]} S={S}", flush=True)
        x = synth.make_layer(spec, 3, layer)
        # host tensors, copied into the resident buffer (nothing else is kept)
        drv.load(*(dev_tensor(x[n], "bf16", device="cpu") for n in ("q", "k", "v")))
        cache = drv.commit(budgets[layer])
        torch.cuda.synchronize()
        s_g, p_g = drv.raw.cpu().numpy(), drv.pooled.cpu().numpy()
        idx = cache.idx.cpu().numpy()
        assert idx.shape == (1, spec.n_kv_heads, budgets[layer] + W)
        q64, k64 = synth.to_f64(x["q"], "bf16"), synth.to_f64(x["k"], "bf16")
        for hk in range(spec.n_kv_heads):
            s_ref = oracle.head_scores(q64[:, hk * G:(hk + 1) * G], k64[:, hk:hk + 1])
            p_ref = oracle.max_pool(s_ref, spec.pool_kernel, 0, S - W)
            assert_scores_close(s_g[:, hk:hk + 1], s_ref, what=f"layer {layer} head {hk} raw")
            assert_scores_close(p_g[:, hk:hk + 1], p_ref, what=f"layer {layer} head {hk} pooled")
            check_selection(idx[:, hk:hk + 1], p_ref, budgets[layer], 0, W)
        assert rows_gathered(host_bits(cache.k_hat), x["k"], idx)
        assert rows_gathered(host_bits(cache.v_hat), x["v"], idx)
    # earlier layers' committed caches are untouched by later layers
    assert [c.budget for c in drv.store] == [budgets[l] for l in layers]
    x0 = synth.make_layer(spec, 3, 0)
    idx0 = drv.store[0].idx.cpu().numpy()
    assert rows_gathered(host_bits(drv.store[0].k_hat), x0["k"], idx0)
    # residency: one full-prompt layer, never two
    peak = torch.cuda.max_memory_allocated() - base
    layer_kv = 2 * spec.n_kv_heads * S * spec.head_dim * 2
    assert drv.active_bytes < layer_kv + (1 << 20)
    bound = drv.active_bytes + drv.store_bytes + drv.scratch_bytes + (8 << 20)
    print(f"peak {peak / 2**20:.1f} MiB, bound {bound / 2**20:.1f} MiB "
          f"(active {drv.active_bytes / 2**20:.1f}, store {drv.store_bytes / 2**20:.1f}, "
          f"scratch {drv.scratch_bytes / 2**20:.1f})", flush=True)
    assert peak <= bound
    assert peak < 2 * layer_kv
