"""kvsel_layer_end (TideKV Algorithm 2 in one call; for long rows the max
filter, selection and gather run fused behind the score passes) gives
exactly the outputs of kvsel_score followed by kvsel_select_compact: raw and
pooled scores, indices and gathered rows, bit for bit."""
import dataclasses

import pytest

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
    # short rows and budget 0: the composed path
    ("short-8k", synth.config(2), 2),
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
