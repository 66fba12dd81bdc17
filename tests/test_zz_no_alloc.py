"""kvsel_score_static (scratch in a static device array, no allocation) gives
exactly kvsel_score's outputs, through the C ABI, on two calls in a row
(the second smaller), and refuses a problem larger than its array."""
import ctypes

import numpy as np
import pytest

import synth
from helpers import dev_tensor

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _lib():
    import attention_score_eviction_amd as kvsel
    L = kvsel.lib()
    P, I32 = ctypes.c_void_p, ctypes.c_int32
    L.kvsel_score_static.argtypes = [ctypes.POINTER(kvsel.Desc), P, P, P, P, I32, P]
    L.kvsel_score_static.restype = ctypes.c_int
    return kvsel, L


def _case(kvsel, L, spec, seed, with_raw):
    x = synth.make_layer(spec, seed, want_v=False)
    q, k = dev_tensor(x["q"], spec.dtype), dev_tensor(x["k"], spec.dtype)
    d = kvsel.make_desc(q, k, n_sink=spec.n_sink, causal=bool(spec.causal))
    shape = (spec.batch, spec.n_kv_heads, spec.seq_len)
    ref_p, ref_s = kvsel.score(q, k, pool_kernel=spec.pool_kernel, n_sink=spec.n_sink,
                               causal=bool(spec.causal))
    pooled = torch.full(shape, -1.0, device="cuda")
    raw = torch.full(shape, -1.0, device="cuda") if with_raw else None
    stream = torch.cuda.current_stream().cuda_stream
    st = L.kvsel_score_static(ctypes.byref(d), q.data_ptr(), k.data_ptr(),
                              raw.data_ptr() if with_raw else None, pooled.data_ptr(),
                              spec.pool_kernel, stream)
    assert st == kvsel.OK, kvsel.status_str(st)
    torch.cuda.synchronize()
    assert torch.equal(pooled, ref_p)
    if with_raw:
        assert torch.equal(raw, ref_s)


def test_static_scratch_matches_workspace_call():
    kvsel, L = _lib()
    big = synth.LayerSpec(1, 40, 8, 128, 40000, 64, 7, 0, structure="spans", n_spans=16)
    small = synth.LayerSpec(2, 8, 2, 128, 3000, 32, 5, 0, n_sink=2, structure="heavy")
    print("case static scratch: 40000 keys x 8 heads, then 2 x 3000 keys x 2 heads", flush=True)
    _case(kvsel, L, big, 31, with_raw=True)
    _case(kvsel, L, small, 32, with_raw=False)   # raw scores kept in the static scratch
    _case(kvsel, L, synth.config(1), 1, with_raw=True)


def test_static_scratch_refuses_oversized_problem():
    kvsel, L = _lib()
    d = kvsel.desc_of(16, 32, 8, 128, 1 << 20, 64)       # ~0.5 GiB of raw scores in scratch
    assert kvsel.score_workspace_bytes(d) > (32 << 20)
    st = L.kvsel_score_static(ctypes.byref(d), 0x10000, 0x10000, None, 0x10000, 7, None)
    assert st == kvsel.ERR_WORKSPACE
