"""Host logic of bench.py (no GPU): the algorithmic byte and flop counts the
roofline lines are built on, written out here from their definitions for the
128K Qwen3-14B layer; the binding-roofline composition; kernel-name
reduction; the trace summary and the traffic ingestion on small synthetic
rocprofv3 files."""
import csv
import json
import os

import pytest

import bench
import synth


def test_algorithmic_bytes_of_the_128k_layer():
    """Two K sweeps, the raw and pooled score vectors written and read, the
    gather (K and V rows read and written) and the indices, for Hkv = 8,
    S = 131072, D = 128, bf16, W = 64, B = 4096."""
    spec = synth.config(4)
    Hkv, S, D, e, W, B = 8, 131072, 128, 2, 64, 4096
    want = (2 * Hkv * S * D * e
            + 2 * Hkv * S * 4 + 2 * Hkv * (S - W) * 4
            + 2 * 2 * Hkv * (B + W) * D * e
            + 2 * Hkv * (B + W) * 4)
    assert want == 587988992
    assert bench.algorithmic_bytes(spec)["path"] == want


def test_kernel_work_of_the_score_passes():
    spec = synth.config(4)
    sweep = 8 * 131072 * 128 * 2                      # one K sweep, bf16
    flops = 2 * 8 * (5 * 64) * 128 * 131072          # 2 * Hkv * G*W * D * S
    assert bench.kernel_work(spec, "score_pass1_32", 4160) == (sweep, flops)
    b2, f2 = bench.kernel_work(spec, "score_pass2_32", 4160)
    assert (b2, f2) == (sweep + 8 * 131072 * 4, flops)  # plus the raw score write
    assert bench.kernel_work(spec, "compact_kernel", 4160)[0] == \
        4 * 8 * 4160 * 128 * 2 + 8 * 4160 * 4


def test_kernel_work_of_the_keys_in_lds_scoring():
    """Kara's 64 x 512 window batch (32 query / 8 KV heads, D = 128, 448
    compressible keys): the one-launch scoring reads every key and every
    query once, writes the score vector and does both passes' products."""
    spec = synth.LayerSpec(64, 32, 8, 128, 448, 512, 1, 0, causal=0)
    H, GW = 64 * 8, 4 * 512
    keys, queries, scores = H * 448 * 128 * 2, H * GW * 128 * 2, H * 448 * 4
    assert queries == 64 * 32 * 512 * 128 * 2
    b, f = bench.kernel_work(spec, "score_keys_lds32", 0)
    assert b == keys + queries + scores
    assert f == 2 * (2 * H * GW * 128 * 448)


def test_binding_roofline_of_the_128k_layer():
    spec = synth.config(4)
    r = bench.binding_roofline(spec, 587988992, 210.0)
    logits = 40 * 64 * 131072
    assert r["t_hbm_us"] == pytest.approx(587988992 / 8e12 * 1e6, abs=0.01)
    assert r["t_mfma_us"] == pytest.approx(4 * logits * 128 / 2.5e15 * 1e6, abs=0.01)
    # two exponentials per logit at 1024 SIMDs x 64 lanes / 11 cycles x 2.4 GHz
    assert r["t_exp_us"] == pytest.approx(2 * logits / (1024 * 64 / 11 * 2.4e9) * 1e6, abs=0.01)
    # pass 1: FMA, exp, add, half a max3; pass 2: FMA, exp, add
    per_logit = ((4.8 + 11 + 4.8 + 2.4) + (4.8 + 11 + 4.8)) / 64
    assert r["t_valu_us"] == pytest.approx(logits * per_logit / 1024 / 2.4e9 * 1e6, abs=0.01)
    assert r["bound"] == "valu"
    assert r["frac"] == pytest.approx(r["t_valu_us"] / 210.0, abs=1e-4)


def test_short_kernel_name():
    n = "void kvsel::(anonymous namespace)::score_pass1_32<128, 10, 8>(kvsel::ScoreArgs)"
    assert bench.short_kernel_name(n) == "score_pass1_32"
    assert bench.short_kernel_name("compact_kernel") == "compact_kernel"
    assert bench.short_kernel_name(
        "void kvsel::(anonymous namespace)::le_emit(kvsel::(anonymous namespace)::SelArgs, int)"
    ) == "le_emit"


def _write_trace(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        for name, a, b in rows:
            w.writerow([name, a, b])


def test_summarize_trace_takes_the_last_dispatches(tmp_path, capsys):
    # a warm-up dispatch, then two steps of two kernels (times in ns)
    rows = [("void warm(int)", 0, 9000),
            ("void a<1>(int)", 10000, 12000), ("void b(int)", 12500, 13500),
            ("void a<1>(int)", 20000, 23000), ("void b(int)", 23500, 24500)]
    p = tmp_path / "t.csv"
    _write_trace(p, rows)
    assert bench.summarize_trace(str(p), 4, "t", "cmd") == 0
    out = capsys.readouterr().out
    assert "| a | 2 | 2.50 | 2.50 | 2.00 |" in out
    assert "| b | 2 | 1.00 | 1.00 | 1.00 |" in out
    assert "warm" not in out
    # per step: median 2.5 + 1.0; span 10.0 .. 24.5 us over 2 steps
    assert "(2 steps): 3.50 us" in out and "7.25 us" in out
    assert bench.summarize_trace(str(p), 9, "t", "cmd") == 1


def _write_counters(path, counter, per_dispatch):
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for d, (name, values) in enumerate(per_dispatch):
            for v in values:                       # one row per XCD / instance
                w.writerow([d, name, counter, v])


def test_ingest_counters_scales_by_the_copy(tmp_path, monkeypatch):
    """A 256 MiB copy reading 131072 units and writing 262144 fixes 2 KiB and
    1 KiB per unit; a kernel's bytes are its mean per-dispatch units times
    those, fetch plus write, stored under the current source hash."""
    cal = 256 * 1024 * 1024
    _write_counters(tmp_path / "cf.csv", "FETCH_SIZE", [("void copy(int)", [65536, 65536])])
    _write_counters(tmp_path / "cw.csv", "WRITE_SIZE", [("void copy(int)", [131072, 131072])])
    _write_counters(tmp_path / "f.csv", "FETCH_SIZE",
                    [("void k<2>(int)", [100, 50]), ("void k<2>(int)", [300, 150])])
    _write_counters(tmp_path / "w.csv", "WRITE_SIZE", [("void k<2>(int)", [10, 10])])
    out = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(out))
    assert bench.ingest_counters("wl", str(tmp_path / "f.csv"), str(tmp_path / "w.csv"),
                                 str(tmp_path / "cf.csv"), str(tmp_path / "cw.csv")) == 0
    t = json.load(open(out))
    assert t["scale"]["fetch_bytes_per_unit"] == cal / 131072
    assert t["scale"]["write_bytes_per_unit"] == cal / 262144
    # fetch: mean of 150 and 450 units = 300 units x 2 KiB; write 20 units x 1 KiB
    assert t["per_kernel_bytes"]["wl"]["k"] == 300 * 2048 + 20 * 1024
    assert t["source_hash"] == bench.source_hash()
    assert bench.traffic_for("wl", "k") == 300 * 2048 + 20 * 1024
    os.remove(out)
    assert bench.traffic_for("wl", "k") is None
