"""The streaming top-k path (kvsel_layer_end_stream: TideKV Algorithm 2's
top-k kept during pass 2, no per-key score vector) selects exactly what the
oracle selects from the same scores, and returns the same indices and rows
as kvsel_layer_end."""
import numpy as np
import pytest

import oracle
import synth
from helpers import check_selection, dev_tensor

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

L = synth.LayerSpec

CASES = [
    # chunks smaller than the budget (every candidate kept by its chunk)
    ("qwen-like-40k-b4096", L(1, 40, 8, 128, 40000, 64, 7, 4096, structure="spans", n_spans=16), 61),
    # chunks larger than the budget: the per-chunk top-k decides
    ("llama-like-64k-b300", L(1, 32, 8, 128, 65536, 64, 7, 300, structure="heavy"), 62),
    ("sinks-ragged-b50", L(2, 8, 2, 128, 30001, 32, 5, 50, n_sink=3, structure="heavy"), 63),
    ("d64-b1", L(1, 8, 4, 64, 20000, 16, 3, 1, structure="heavy"), 64),
    ("noncausal-b700", L(1, 8, 2, 128, 24000, 40, 7, 700, causal=0, structure="heavy"), 65),
    ("pool1-b2000", L(1, 16, 4, 128, 50000, 32, 1, 2000), 66),
    ("budget-0", L(1, 8, 2, 128, 20000, 32, 7, 0), 67),
]


@pytest.mark.parametrize("name,spec,seed", CASES, ids=[c[0] for c in CASES])
def test_stream_matches_oracle_and_layer_end(name, spec, seed):
    import attention_score_eviction_amd as kvsel
    x = synth.make_layer(spec, seed)
    q, k, v = (dev_tensor(x[n], "bf16") for n in ("q", "k", "v"))
    kw = dict(n_sink=spec.n_sink, causal=bool(spec.causal))
    print(f"case stream {name} S={spec.seq_len} B={spec.budget}", flush=True)
    idx_s, kh_s, vh_s = kvsel.layer_end_stream(q, k, v, budget=spec.budget,
                                               pool_kernel=spec.pool_kernel, **kw)
    idx, kh, vh, raw, pooled = kvsel.layer_end(q, k, v, budget=spec.budget,
                                               pool_kernel=spec.pool_kernel, **kw)
    torch.cuda.synchronize()
    # the same scores, so the same selection, bit for bit
    want = oracle.select(pooled.double().cpu().numpy(), spec.budget, spec.n_sink,
                         spec.obs_window)
    np.testing.assert_array_equal(idx_s.cpu().numpy(), want)
    assert torch.equal(idx_s, idx)
    assert torch.equal(kh_s.view(torch.int16), kh.view(torch.int16))
    assert torch.equal(vh_s.view(torch.int16), vh.view(torch.int16))
    # and against the oracle's own scores, within the near-tie band
    if spec.budget > 0 and spec.n_kv_heads <= 4:
        G, S, W = spec.group, spec.seq_len, spec.obs_window
        q64, k64 = synth.to_f64(x["q"], "bf16"), synth.to_f64(x["k"], "bf16")
        for hk in range(spec.n_kv_heads):
            s_ref = oracle.head_scores(q64[:, hk * G:(hk + 1) * G], k64[:, hk:hk + 1],
                                       causal=bool(spec.causal))
            p_ref = oracle.max_pool(s_ref, spec.pool_kernel, spec.n_sink, S - W)
            check_selection(idx_s[:, hk:hk + 1].cpu().numpy(), p_ref, spec.budget,
                            spec.n_sink, W)


def test_stream_workspace_stops_growing_with_the_prompt():
    """With the chunk count fixed by the GPU, the scratch of the streaming
    path is the per-chunk candidate lists, so once every chunk holds more
    candidates than the budget it no longer grows with S; the score-vector
    path's scratch keeps growing."""
    import attention_score_eviction_amd as kvsel
    d = lambda S: kvsel.desc_of(1, 40, 8, 128, S, 64)  # noqa: E731
    ws_s = [kvsel.layer_end_stream_workspace_bytes(d(S), 4096, 7) for S in (262144, 524288)]
    ws_r = [kvsel.layer_end_workspace_bytes(d(S), 4096) for S in (262144, 524288)]
    assert ws_s[0] > 0 and ws_s[0] == ws_s[1]
    assert ws_r[1] > ws_r[0] > ws_s[0]
