"""The layer-end step captured in a HIP graph (for callers that replay it in
a serving loop): nothing in it allocates or clears memory with a memset, so
every replay of the graph, with other work on the stream between replays,
gives exactly what an eager call gives on the same inputs."""
import numpy as np
import pytest

import synth
from helpers import dev_tensor

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

L = synth.LayerSpec

CASES = [
    ("short-8k", synth.config(2), 2),                                      # one-launch select
    ("long-40k", L(1, 32, 8, 128, 40000, 64, 7, 4096, structure="heavy"), 71),  # fused long rows
]


@pytest.mark.parametrize("name,spec,seed", CASES, ids=[c[0] for c in CASES])
def test_graph_replays_equal_eager(name, spec, seed):
    from attention_score_eviction_amd.driver import LayerMajorDriver
    drv = LayerMajorDriver(spec.batch, spec.n_q_heads, spec.n_kv_heads, spec.head_dim,
                           spec.seq_len, spec.obs_window, spec.pool_kernel,
                           max_budget=spec.budget)
    layers = [synth.make_layer(spec, seed, layer) for layer in range(4)]

    def put(x):
        drv.load(*(dev_tensor(x[n], "bf16", device="cpu") for n in ("q", "k", "v")))

    print(f"case graph {name} S={spec.seq_len} B={spec.budget}", flush=True)
    put(layers[0])
    cache_g = drv.new_cache(spec.budget)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):           # warm-up outside the capture
        drv.layer_end(cache_g)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        drv.layer_end(cache_g)
    torch.cuda.synchronize()
    for rep, x in enumerate(layers[1:] + layers[:1]):
        put(x)                                        # eager work between replays
        g.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in (cache_g.idx, cache_g.k_hat, cache_g.v_hat, drv.raw, drv.pooled)]
        cache_e = drv.new_cache(spec.budget)
        drv.layer_end(cache_e)                        # eager, same inputs
        torch.cuda.synchronize()
        want = [cache_e.idx, cache_e.k_hat, cache_e.v_hat, drv.raw, drv.pooled]
        for a, b in zip(got, want):
            assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                               b.view(torch.int16) if b.dtype == torch.bfloat16 else b), \
                f"replay {rep}"
        assert not np.array_equal(got[0].cpu().numpy(), np.zeros_like(got[0].cpu().numpy()))


@pytest.mark.parametrize("name,spec,seed", CASES, ids=[c[0] for c in CASES])
def test_graph_replays_equal_eager_head_adaptive(name, spec, seed):
    """The head-adaptive layer end (kvsel_layer_end_adaptive) under capture:
    its histograms are cleared by kernels, so replays equal eager calls."""
    from attention_score_eviction_amd.driver import LayerMajorDriver
    drv = LayerMajorDriver(spec.batch, spec.n_q_heads, spec.n_kv_heads, spec.head_dim,
                           spec.seq_len, spec.obs_window, spec.pool_kernel,
                           max_budget=spec.budget)
    layers = [synth.make_layer(spec, seed + 100, layer) for layer in range(3)]
    T = spec.n_kv_heads * spec.budget

    def put(x):
        drv.load(*(dev_tensor(x[n], "bf16", device="cpu") for n in ("q", "k", "v")))

    print(f"case graph head-adaptive {name} S={spec.seq_len} T={T}", flush=True)
    put(layers[0])
    cache_g = drv.new_flat_cache(T)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        drv.layer_end_adaptive(cache_g)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        drv.layer_end_adaptive(cache_g)
    torch.cuda.synchronize()
    for rep, x in enumerate(layers[1:] + layers[:1]):
        put(x)
        g.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in (cache_g.idx, cache_g.head_off, cache_g.k_hat, cache_g.v_hat,
                                   drv.pooled)]
        cache_e = drv.new_flat_cache(T)
        drv.layer_end_adaptive(cache_e)
        torch.cuda.synchronize()
        want = [cache_e.idx, cache_e.head_off, cache_e.k_hat, cache_e.v_hat, drv.pooled]
        for a, b in zip(got, want):
            assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                               b.view(torch.int16) if b.dtype == torch.bfloat16 else b), \
                f"replay {rep}"
