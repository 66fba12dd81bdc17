"""Parity of the Kara decode-window path (kvsel_kara_score, kvsel_kara_select,
then kvsel_compact on the window) with the CPU oracle.

Scores: within 1e-3 relative of the oracle's float64 definition.
Selection: bit-exact with the oracle on identical float32 scores.  End to
end (GPU scores vs oracle scores), a row must match the oracle exactly
unless one of the oracle's own decisions (the keep-th score, the chunk cut,
the fill-up cut) is a near tie, within 1e-5 relative; every row is checked
for size, order, the buffer and the clearly-kept positions.  Gathered rows
are byte copies of the window rows their indices name.
"""
import numpy as np
import pytest

import oracle
import synth
from helpers import assert_scores_close, dev_tensor, host_bits, rows_gathered

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _kvsel():
    import attention_score_eviction_amd as kvsel
    kvsel.lib()
    return kvsel


def _ties_kind(rng, kind, shape):
    if kind == "uniform":
        return rng.random(shape).astype(np.float32)
    if kind == "quarters":
        return (rng.integers(0, 6, size=shape) * 0.25).astype(np.float32)
    if kind == "peaks":
        p = (rng.random(shape) * 0.01).astype(np.float32)
        p[..., ::9] += np.float32(1.0)
        return p
    return np.full(shape, 0.5, np.float32)


@pytest.mark.parametrize("seed,n,buffer,keep,gamma,alpha,kind", [
    (0, 448, 64, 180, 8, 32, "uniform"),
    (1, 448, 64, 90, 8, 16, "quarters"),
    (2, 320, 64, 64, 8, 32, "peaks"),
    (3, 200, 0, 40, 4, 12, "flat"),
    (4, 17, 3, 5, 3, 4, "uniform"),
    (5, 448, 32, 0, 8, 32, "uniform"),
    (6, 448, 32, 448, 8, 32, "uniform"),
    (7, 300, 10, 100, 1, 20, "uniform"),
    (8, 2048, 16, 700, 8, 32, "uniform"),
    (9, 1, 1, 1, 8, 32, "uniform"),
])
def test_kara_select_exact_on_identical_scores(seed, n, buffer, keep, gamma, alpha, kind):
    kvsel = _kvsel()
    rng = np.random.default_rng(300 + seed)
    Bt, Hkv = 3, 4
    A = _ties_kind(rng, kind, (Bt, Hkv, n))
    print(f"case kara select seed {seed} n={n} keep={keep} gamma={gamma} alpha={alpha}",
          flush=True)
    kd = kvsel.KaraDesc(Bt, Hkv, Hkv, 128, n + buffer, buffer, keep, gamma, alpha, kvsel.BF16,
                        0.0)
    got = kvsel.kara_select(torch.from_numpy(A).cuda(), kd).cpu().numpy()
    want = oracle.kara_select(A.astype(np.float64), keep, gamma, alpha, buffer)
    np.testing.assert_array_equal(got, want)


def _margins_ok(a, keep, gamma, alpha, rel=1e-5):
    """True when none of the oracle's three cuts on score row `a` is a near
    tie: the keep-th score (Eq. 5), the chunk cut (Eq. 7) and the fill-up
    cut.  Orders inside a kept set do not matter, only the cuts."""
    n = a.size
    order = np.lexsort((np.arange(n), -a))

    def gap_ok(vals, k):
        if k <= 0 or k >= len(vals):
            return True
        return abs(vals[k - 1] - vals[k]) > rel * max(abs(vals[k - 1]), 1e-30)
    if not gap_ok(a[order], keep):
        return False
    I = np.sort(order[:keep])
    a32 = a.astype(np.float32)
    chunks = sorted(((float(np.float32(a32[I[k]] + a32[I[k + 1]])
                             * np.float32(I[k + 1] - I[k] - 1)), k)
                     for k in range(len(I) - 1) if I[k + 1] - I[k] <= gamma),
                    key=lambda t: (-t[0], t[1]))
    if not gap_ok([c[0] for c in chunks], alpha // gamma):
        return False
    taken = set(I.tolist())
    for _, k in chunks[:alpha // gamma]:
        taken.update(range(I[k] + 1, I[k + 1]))
    need = alpha - (len(taken) - len(I))
    rest = [a[j] for j in order if j not in taken]
    return gap_ok(rest, need)


def test_kara_select_alpha_int32_max():
    """A chunk budget of INT32_MAX (every free position is added by the
    fill-up): exact with the oracle, n_out = n."""
    kvsel = _kvsel()
    rng = np.random.default_rng(310)
    Bt, Hkv, n, U, keep, gamma, alpha = 2, 3, 200, 16, 50, 8, 2 ** 31 - 1
    A = rng.random((Bt, Hkv, n)).astype(np.float32)
    kd = kvsel.KaraDesc(Bt, Hkv, Hkv, 128, n + U, U, keep, gamma, alpha, kvsel.BF16, 0.0)
    got = kvsel.kara_select(torch.from_numpy(A).cuda(), kd).cpu().numpy()
    want = oracle.kara_select(A.astype(np.float64), keep, gamma, alpha, U)
    assert got.shape == (Bt, Hkv, n + U)
    np.testing.assert_array_equal(got, want)


def _token2chunk_structure(row, A32, n, keep, gamma, alpha):
    """Validity of a Token2Chunk output against the scores it was computed
    from: the keep best positions are present, every other kept position is
    either inside a qualifying chunk (strictly between consecutive members
    of I, at most gamma apart) or a fill-up pick, and exactly min(alpha,
    n - keep) positions were added."""
    comp = row[row < n]
    order = np.lexsort((np.arange(n), -A32.astype(np.float64)))
    I = np.sort(order[:keep])
    assert set(I.tolist()) <= set(comp.tolist())
    added = sorted(set(comp.tolist()) - set(I.tolist()))
    assert len(added) == min(alpha, n - keep)
    in_chunk = set()
    for k in range(len(I) - 1):
        if I[k + 1] - I[k] <= gamma:
            in_chunk.update(range(I[k] + 1, I[k + 1]))
    fill = [j for j in added if j not in in_chunk]
    # fill-up picks are the best of what remained: none of them is beaten by a
    # position left out that is not inside a chunk interior
    left = [j for j in range(n) if j not in set(comp.tolist()) and j not in in_chunk]
    if fill and left:
        key = lambda j: (-float(A32[j]), j)  # noqa: E731
        assert max(key(j) for j in fill) < min(key(j) for j in left)


# Kara Eq. (5) for r = 0.4, worked by hand: ceil(0.4 * (|W| - |U|)).
KARA_KEEP_04 = {(512, 64): 180, (384, 32): 141, (256, 32): 90, (97, 13): 34}


@pytest.mark.parametrize("shape,dtype,seed", [
    # (Bt, Hq, Hkv, window, buffer, D), as Qwen3-14B and R1-Llama-8B decode windows
    ((4, 40, 8, 512, 64, 128), "bf16", 1),
    ((2, 32, 8, 384, 32, 128), "bf16", 2),
    ((2, 8, 2, 256, 32, 64), "bf16", 3),
    ((1, 4, 2, 97, 13, 64), "f32", 4),
])
def test_kara_window_end_to_end(shape, dtype, seed):
    """Scores within 1e-3 of the oracle.  Every row is exactly Token2Chunk
    of the GPU's own scores (the oracle replayed on them) and structurally
    valid; rows whose oracle cuts are not near ties equal the oracle's
    selection from its own scores."""
    kvsel = _kvsel()
    Bt, Hq, Hkv, Wn, U, D = shape
    x = synth.decode_window(seed, Bt, Hq, Hkv, Wn, D, dtype)
    q, k, v = (dev_tensor(x[t], dtype) for t in ("q", "k", "v"))
    ratio, gamma, alpha = 0.4, 8, 32
    print(f"case kara window seed {seed} shape {shape} {dtype}", flush=True)
    out = kvsel.kara_compress(q, k, v, buffer=U, ratio=ratio, gamma=gamma, alpha=alpha)
    torch.cuda.synchronize()
    n = Wn - U
    A_ref = oracle.kara_scores(synth.to_f64(x["q"], dtype), synth.to_f64(x["k"], dtype)[:, :, :n])
    assert_scores_close(out["A"].cpu().numpy(), A_ref, what="Kara importance")
    keep = out["desc"].keep
    assert keep == KARA_KEEP_04[(Wn, U)]
    want = oracle.kara_select(A_ref, keep, gamma, alpha, U)
    got = out["idx"].cpu().numpy()
    A_gpu = out["A"].cpu().numpy()
    assert got.shape == want.shape
    np.testing.assert_array_equal(got, oracle.kara_select(A_gpu.astype(np.float64), keep, gamma,
                                                          alpha, U))
    exact_rows = 0
    for b in range(Bt):
        for h in range(Hkv):
            row = got[b, h]
            _token2chunk_structure(row, A_gpu[b, h], n, keep, gamma, alpha)
            assert (np.diff(row) > 0).all() and row[-U:].tolist() == list(range(n, Wn)) if U \
                else (np.diff(row) > 0).all()
            top = np.sort(A_ref[b, h])[::-1]
            assert set(np.flatnonzero(A_ref[b, h] > top[keep - 1] * (1 + 1e-4)).tolist()) \
                <= set(row.tolist())
            if _margins_ok(A_ref[b, h], keep, gamma, alpha):
                assert row.tolist() == want[b, h].tolist(), (b, h)
                exact_rows += 1
    assert exact_rows >= max(1, Bt * Hkv // 4)
    assert rows_gathered(host_bits(out["k_hat"]), x["k"], got)
    assert rows_gathered(host_bits(out["v_hat"]), x["v"], got)


def test_kara_bench_config_sampled_rows():
    """The benchmarked configuration in full (64 sequences of a 32/8-head,
    D = 128 layer, 512-token windows, 64-token buffer, r = 40%, gamma 8,
    alpha 32); three sequences replayed through the oracle."""
    kvsel = _kvsel()
    Bt, Hq, Hkv, Wn, U, D = 64, 32, 8, 512, 64, 128
    x = synth.decode_window(7, Bt, Hq, Hkv, Wn, D)
    q, k, v = (dev_tensor(x[t], "bf16") for t in ("q", "k", "v"))
    ratio, gamma, alpha = 0.4, 8, 32
    print("case kara bench config 64 x 512", flush=True)
    out = kvsel.kara_compress(q, k, v, buffer=U, ratio=ratio, gamma=gamma, alpha=alpha)
    torch.cuda.synchronize()
    n = Wn - U
    keep = out["desc"].keep
    assert keep == KARA_KEEP_04[(Wn, U)]
    A = out["A"].cpu().numpy()
    got = out["idx"].cpu().numpy()
    # every row is exactly Token2Chunk of the GPU's own scores
    np.testing.assert_array_equal(got, oracle.kara_select(A.astype(np.float64), keep, gamma,
                                                          alpha, U))
    exact = 0
    for b in (0, 31, 63):
        A_ref = oracle.kara_scores(synth.to_f64(x["q"][b:b + 1], "bf16"),
                                   synth.to_f64(x["k"][b:b + 1], "bf16")[:, :, :n])
        assert_scores_close(A[b:b + 1], A_ref, what=f"Kara importance, sequence {b}")
        want = oracle.kara_select(A_ref, keep, gamma, alpha, U)
        for h in range(Hkv):
            if _margins_ok(A_ref[0, h], keep, gamma, alpha):
                assert got[b, h].tolist() == want[0, h].tolist(), (b, h)
                exact += 1
        assert rows_gathered(host_bits(out["k_hat"][b:b + 1]), x["k"][b:b + 1], got[b:b + 1])
    assert exact >= 6
