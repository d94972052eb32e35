"""Host-side logic of bench.py (no GPU): the one-GPU refusal, the algorithmic
byte count of a Stage-1 launch, the roofline bound chosen by arithmetic
intensity, and the traffic record keyed to the kernel sources' code."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_stage1_bytes():
    # W read once, H read once, one 8-byte candidate per (row, vocab tile)
    assert bench.stage1_bytes(64, 4096, 128256, 2, 1002) == 128256 * 4096 * 2 + 64 * 4096 * 2 + 8 * 64 * 1002
    assert bench.stage1_bytes(1, 256, 4096, 4, 16) == 4096 * 256 * 4 + 256 * 4 + 8 * 16


def _rec(B, D, V, esz, n_tiles, us):
    byts = bench.stage1_bytes(B, D, V, esz, n_tiles)
    s1 = us * 1e-3
    return {"flops": 2 * B * V * D, "stage1_bytes": byts, "stage1_ms": s1,
            "stage1_GBps": byts / (s1 * 1e-3) / 1e9, "stage1_TFLOPs": 2 * B * V * D / (s1 * 1e-3) / 1e12}


def test_roofline_bound_follows_arithmetic_intensity():
    # B = 64 bf16: 64 flop/byte, below the 312.5 ridge -> HBM-bound, GB/s
    r = bench.roofline(_rec(64, 4096, 128256, 2, 1002, 158.0), bench.MFMA_BF16_PEAK_TFLOPS, None)
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == bench.HBM_PEAK_GBS
    assert abs(r["frac"] - r["achieved"] / 8000.0) < 1e-12 and 0.8 < r["frac"] < 0.9
    assert abs(r["ridge_flop_per_byte"] - 312.5) < 1e-9
    # B = 1024 bf16: ~1000 flop/byte -> matrix-core bound, TFLOP/s against 2.5 PFLOP/s
    r = bench.roofline(_rec(1024, 7168, 129280, 2, 505, 1700.0), bench.MFMA_BF16_PEAK_TFLOPS, 123)
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s" and r["peak"] == 2500.0 and r["traffic"] == 123
    assert abs(r["achieved"] - 2 * 1024 * 129280 * 7168 / 1.7e-3 / 1e12) < 1e-6
    # fp32 heads: ridge 157.3 / 8 = 19.7 flop/byte (AI = B / 2 for fp32)
    r = bench.roofline(_rec(64, 256, 4096, 4, 32, 20.0), bench.MFMA_F32_PEAK_TFLOPS, None)
    assert r["bound"] == "mfma" and r["peak"] == bench.MFMA_F32_PEAK_TFLOPS
    r = bench.roofline(_rec(8, 256, 4096, 4, 32, 20.0), bench.MFMA_F32_PEAK_TFLOPS, None)
    assert r["bound"] == "hbm"


def test_code_of_ignores_comments_and_layout():
    a = "int x = 1; // one\n/* block\ncomment */ int  y=2;\n"
    b = "int x = 1;\n\n   int y=2; // other words\n"
    assert bench.code_of(a) == "int x = 1; int y=2;"
    assert bench.code_of(b) == "int x = 1; int y=2;"


def test_traffic_record_is_tied_to_the_sources(tmp_path, monkeypatch):
    prof = tmp_path / "profiles"
    prof.mkdir()
    good = {"stage1/w/B8": {"source_hash": bench.source_hash(), "bytes_per_launch": 777}}
    (prof / "traffic.json").write_text(json.dumps(good))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    # source_hash reads the sources under ROOT: point it back at the repository
    monkeypatch.setattr(bench, "source_hash", lambda read=None, _h=good["stage1/w/B8"]["source_hash"]: _h)
    assert bench.traffic_record("stage1", "w", 8) == 777
    assert bench.traffic_record("stage1", "w", 16) is None
    monkeypatch.setattr(bench, "source_hash", lambda read=None: "0000000000000000")
    assert bench.traffic_record("stage1", "w", 8) is None
