"""Host-side parts of bench.py (no GPU): the one-GPU contract, the
algorithmic work it divides by, and the parsers of its profile and
telemetry inputs."""
import json
import os
import subprocess
import sys

import pytest

import moe_inputs as mi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


@pytest.mark.parametrize("n", [2, 8])
def test_more_than_one_gpu_is_refused(n):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", str(n)],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""  # no JSON line


def test_algorithmic_work_of_the_workload_layers():
    den = mi.spec("denoise_1micro")
    # 6 T k H I: gate|up (4 T k H I) and down (2 T k I H)
    assert bench.expert_flops(den) == 6 * 4096 * 8 * 4096 * 1536 == 1236950581248
    assert bench.w13_flops(den) == 4 * 4096 * 8 * 4096 * 1536
    assert bench.expert_flops(mi.spec("denoise_2micro")) == bench.expert_flops(den)
    # the w13 GEMM's least HBM traffic: weights, x and h once, indices
    R = 4096 * 8
    assert bench.w13_algorithmic_bytes(den) == (64 * 3072 * 4096 + 4096 * 4096 + R * 1536) * 2 + R * 4 + 65 * 4
    # decode: each active expert's w13 and down weights (18,874,368 bytes at
    # I = 768), x and out, the router weights
    dec = mi.spec("decode")
    assert (2 * 768 * 4096 + 4096 * 768) * 2 == 18874368
    assert bench.decode_bytes(dec, 42) == 42 * 18874368 + 8 * 4096 * 2 * 2 + 64 * 4096 * 4


def test_traffic_is_reported_only_for_the_profiled_sources(tmp_path):
    """bench reports the counter summary's traffic only while the sha256 it
    records matches the w13 kernel's current sources."""
    def profile(sha):
        return (f"kernel_sources_sha256: `{sha}`\n\nfetch_bytes_per_launch: 2106010180\n\n"
                f"write_bytes_per_launch: 100663296\n")
    good = tmp_path / "good.md"
    good.write_text(profile(bench.kernel_sources_sha256()))
    got = bench.measured_traffic(str(good))
    assert got == {"read": 2106010180, "write": 100663296, "total": 2106010180 + 100663296}
    stale = tmp_path / "stale.md"
    stale.write_text(profile("0" * 64))
    assert bench.measured_traffic(str(stale)) is None
    assert bench.measured_traffic(str(tmp_path / "missing.md")) is None
    # the committed summary has the fields the parser reads
    text = open(os.path.join(ROOT, bench.W13_TRAFFIC_PROFILE)).read()
    for key in ("kernel_sources_sha256:", "fetch_bytes_per_launch:", "write_bytes_per_launch:"):
        assert key in text


def test_engine_clock_parser():
    sample = [{"gpu": 0, "clock": {
        "gfx_0": {"clk": {"value": 2180, "unit": "MHz"}},
        "gfx_1": {"clk": {"value": 2171.5, "unit": "MHz"}},
        "mem_0": {"clk": {"value": 2000, "unit": "MHz"}},
        "gfx_2": {"clk": {"value": "N/A"}}}}]
    assert bench._gfx_clocks_from_json(json.dumps(sample)) == [2180.0, 2171.5]
    assert bench._gfx_clocks_from_json("not json") is None
    assert bench._gfx_clocks_from_json("{}") is None


def test_call_stats():
    s = bench.call_stats([1.0, 2.0, 3.0, 4.0])
    assert s == {"mean": 2.5, "median": 2.5, "min": 1.0, "p90": 3.7, "calls": 4}
