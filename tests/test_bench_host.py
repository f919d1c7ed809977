"""Host-side logic of bench.py: no GPU needed."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_flop_convention_matches_the_documented_work():
    # 131072 tokens, cp = 8, 32 query heads, d = 128: 1 073 750 016 allowed
    # pairs per head on every rank; 17.59 TFLOP forward and 52.77 TFLOP forward
    # plus backward at the pages' 4 + 8 flops per token and head dimension.
    import context_causal_attention_amd as cpa
    S, cp, d, hq = 131072, 8, 128, 32
    n = cpa.cp_pairs(cpa.cp_shard_zigzag(S, cp, 0), None, cpa.cp_unshard_zigzag(S, cp))
    assert n == 1073750016
    fwd = bench.FLOPS_PER_PAIR_HEAD_DIM["fwd"] * d * hq * n
    both = (bench.FLOPS_PER_PAIR_HEAD_DIM["fwd"] + bench.FLOPS_PER_PAIR_HEAD_DIM["bwd"]) * d * hq * n
    assert fwd / 1e12 == pytest.approx(17.59, abs=0.005)
    assert both / 1e12 == pytest.approx(52.77, abs=0.01)
    assert bench.FLOPS_RECOMPUTE_COUNTED["bwd"] == bench.FLOPS_PER_PAIR_HEAD_DIM["bwd"] + 2.0
    assert bench.FLOPS_EXECUTED["bwd"] == 14.0
    assert bench.MFMA_FLOP_PER_CLK * 2.4e9 / 1e12 == pytest.approx(bench.PEAK_BF16_TFLOPS, rel=1e-4)


def test_clock_file_parser(tmp_path):
    f = tmp_path / "pp_dpm_sclk"
    f.write_text("0: 500Mhz\n1: 1900Mhz *\n2: 2400Mhz\n")
    assert bench.ClockSampler._read(str(f)) == 1900
    f.write_text("0: 500Mhz\n1: 2400Mhz\n")
    assert bench.ClockSampler._read(str(f)) is None
    assert bench.ClockSampler._read(str(tmp_path / "missing")) is None


def test_stored_traffic_needs_the_current_sources(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    path = tmp_path / "fwd_traffic_w.txt"
    h = bench.source_hash(bench.KERNEL_SOURCES["fwd"])
    path.write_text(f"# header\nhbm_bytes_per_launch: 1234\nsource_sha256_16: {h}\n")
    assert bench.stored_traffic("fwd", "w") == 1234.0
    path.write_text("hbm_bytes_per_launch: 1234\nsource_sha256_16: 0000000000000000\n")
    assert bench.stored_traffic("fwd", "w") is None
    assert bench.stored_traffic("fwd", "absent") is None
