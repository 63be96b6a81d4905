"""Host-side checks of bench.py (no GPU): the algorithmic work it credits
matches the figures worked out independently for each workload (FLOP and
byte counts of the measurement table), the launch statistics, the input-copy
rule, the single-GPU guard, and the traffic record's source guard."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402
from causal_attention_amd import inputs  # noqa: E402


@pytest.mark.parametrize("name,flops,nbytes", [
    ("c1_f32_s128", 2_113_536, 131_584),
    ("c2_mha12_s512", 403_439_616, 3_170_304),
    ("c3_gqa_b4_s2048", 34_376_515_584, 42_205_184),
    ("c5_gqa_s32768", 2_199_090_364_416, 168_820_736),
])
def test_prefill_work_matches_the_table(name, flops, nbytes):
    w = inputs.WORKLOADS[name]
    elt = 4 if w.dtype == "f32" else 2
    assert bench.prefill_flops(w.B, w.Hq, w.S, w.D, w.causal) == flops
    assert bench.prefill_bytes(w.B, w.Hq, w.Hkv, w.S, w.D, elt) == nbytes


def test_full_attention_counts_every_pair():
    assert bench.prefill_flops(1, 1, 10, 64, causal=False) == 4 * 64 * 100
    assert bench.prefill_flops(1, 1, 10, 64, causal=True) == 4 * 64 * 55


def test_decode_bytes_match_the_table():
    w = inputs.WORKLOADS["c4_decode_b32"]
    sl = inputs.decode_seqlens(w.B, w.lmin, w.lmax, w.seed)
    assert int(sl.sum()) == 72_951
    # K and V once per KV head (74,701,824 B) plus q and o (131,072 B)
    assert bench.decode_bytes(sl, w.Hq, w.Hkv, w.D) == 74_701_824 + 131_072


def test_launch_stats():
    st = bench.launch_stats([0.003, 0.001, 0.002, 0.010])
    assert st == {"mean_us": 4.0, "median_us": 2.5, "min_us": 1.0,
                  "launches": 4}
    assert bench.launch_stats([0.002])["median_us"] == 2.0


def test_copies_outlast_the_last_level_cache():
    for nbytes in (131_584, 3_170_304, 42_205_184, 74_832_896, 168_820_736):
        r = bench.copies_for(nbytes)
        assert 2 <= r <= 64
        if r < 64:
            # a copy is reused only after more than the cache's worth of
            # the other copies has been read
            assert (r - 1) * nbytes > bench.LLC_BYTES


def test_peaks():
    assert bench.peak_tflops("bf16") == 2500.0
    assert bench.peak_tflops("f16") == 2500.0
    assert bench.peak_tflops("f32") == 157.3
    assert bench.PEAK_HBM_GBS == 8000.0


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"),
                          "--gpus", "2"], capture_output=True, text=True,
                         timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr


def test_traffic_record_needs_the_current_sources(tmp_path, monkeypatch):
    rec = tmp_path / "traffic.txt"
    rec.write_text("# comment\nkernel_sources_sha256: 0000\n"
                   "c3_gqa_b4_s2048_hbm_bytes_per_launch: 123\n")
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(rec))
    assert bench.measured_traffic() == {}
    rec.write_text(f"kernel_sources_sha256: {bench.kernel_source_hash()}\n"
                   "c3_gqa_b4_s2048_hbm_bytes_per_launch: 123\n")
    tr = bench.measured_traffic()
    assert bench.traffic_for(tr, "c3_gqa_b4_s2048") == 123
    assert bench.traffic_for(tr, "c5_gqa_s32768") is None


def test_source_hash_ignores_comments_and_whitespace(tmp_path, monkeypatch):
    a = tmp_path / "a.hpp"
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "KERNEL_SOURCES", ("a.hpp",))
    a.write_text("int f() { return 1; }  // one\n/* block */\n")
    h = bench.kernel_source_hash()
    assert len(h) == 16
    a.write_text("int  f()\n{ return 1; }  // another comment\n")
    assert bench.kernel_source_hash() == h
    a.write_text("int f() { return 2; }\n")
    assert bench.kernel_source_hash() != h
