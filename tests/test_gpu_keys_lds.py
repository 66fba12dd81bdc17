"""Scoring with a KV head's keys held in LDS (no causal mask, at most 512
keys in whole 32-key tiles, at least 256 query rows per KV head: a decode
window scoring its own keys, as Kara's does): raw scores against the fp64
oracle's dense definition (TideKV Eq. (7) with no mask; Kara Eq. (4)), over
the kernel's instantiations (one to sixteen key tiles, D = 64 and 128),
ragged query groups and batches, and the launch really is the one-kernel
path."""
import numpy as np
import pytest

import oracle
from helpers import assert_scores_close

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

CASES = [
    # Bt, Hq, Hkv, W, D, S
    (1, 8, 2, 64, 128, 64),      # two key tiles, G·W = 256
    (2, 16, 4, 100, 64, 512),    # sixteen tiles, D = 64, 400 rows (a partial last tile)
    (1, 40, 8, 64, 128, 448),    # fourteen tiles, G = 5
    (1, 8, 1, 32, 128, 32),      # one tile, G = 8 (the window is the whole sequence)
]


@pytest.mark.parametrize("Bt,Hq,Hkv,W,D,S", CASES)
def test_keys_in_lds_scores_match_the_oracle(Bt, Hq, Hkv, W, D, S):
    import attention_score_eviction_amd as kvsel
    rng = np.random.default_rng(S + W + D)
    q = torch.from_numpy(rng.standard_normal((Bt, Hq, W, D)).astype(np.float32)).to(torch.bfloat16)
    k = torch.from_numpy(rng.standard_normal((Bt, Hkv, S, D)).astype(np.float32)).to(torch.bfloat16)
    k[:, :, ::7] *= 2      # a few keys that draw more attention
    print(f"case keys-in-LDS Bt={Bt} Hq={Hq} Hkv={Hkv} W={W} D={D} S={S}", flush=True)
    torch.cuda.synchronize()
    kvsel.timing_read()
    kvsel.timing_start("*")
    try:
        _, raw = kvsel.score(q.cuda(), k.cuda(), pool_kernel=1, causal=False)
        torch.cuda.synchronize()
    finally:
        kvsel.timing_start(None)
    names = set(kvsel.timing_read())
    assert "score_keys_lds32" in names, names
    assert not any(n.startswith(("score_pass", "score_combine", "score_group")) for n in names), names
    want = oracle.head_scores(q.double().numpy(), k.double().numpy(), causal=False)
    got = raw.cpu().numpy()
    assert_scores_close(got, want, rtol=1e-3, what="raw scores")
    # every query row's weights sum to one
    np.testing.assert_allclose(got.astype(np.float64).sum(-1), (Hq // Hkv) * W, rtol=1e-4)
