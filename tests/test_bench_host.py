"""CPU checks of bench.py's host-side accounting: the one-GPU refusal, the
algorithmic FLOP and bytes behind every roofline fraction (against the
per-shape figures worked out by hand from the workload definitions), the
traffic record's digest guard, and the CPU-oracle baseline record."""
import json
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


# (m, n, k) -> (GFLOP, algorithmic MB): 2mnk FLOP; bytes = A (m k) + B (n k)
# + both FP32 scale tensors (m KG + NB KG floats) + the BF16 output (2 m n)
HAND = {
    (64, 2112, 7168): (1.9378, 15.886),        # 458752 + 15138816 + 14336 + 3808 + 270336 B
    (64, 7168, 16384): (15.032, 119.468),
    (128, 24576, 1536): (9.6637, 44.252),
    (4096, 7168, 16384): (962.07, 245.395),
    (8192, 8192, 8192): (1099.51, 270.549),
    (16384, 7168, 16384): (3848.29, 629.174),
}


@pytest.mark.parametrize("shape", sorted(HAND))
def test_algorithmic_flop_and_bytes(shape):
    m, n, k = shape
    flop, nbytes = bench.algorithmic(m, n, k)
    gflop, mb = HAND[shape]
    assert abs(flop / 1e9 - gflop) / gflop < 1e-4
    assert abs(nbytes / 1e6 - mb) / mb < 1e-4
    # the bound follows the ridge point (625 FLOP/B for 5.0 PFLOP/s over 8 TB/s)
    assert (flop / nbytes >= bench.RIDGE) == (m > 256)


def test_traffic_record_needs_the_current_kernel_sources(tmp_path, monkeypatch):
    digest = bench.kernel_source_digest()
    assert len(digest) == 16 and digest == bench.kernel_source_digest()
    f = tmp_path / "traffic.md"
    rec = {"shape": [8, 16, 128], "kernel_sources": digest, "hbm_bytes_per_launch": 1234}
    stale = dict(rec, shape=[8, 16, 256], kernel_sources="0" * 16)
    f.write_text("x\ntraffic:" + json.dumps(stale) + "\ntraffic:" + json.dumps(rec) + "\n")
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.measured_traffic(8, 16, 128) == 1234
    assert bench.measured_traffic(8, 16, 256) is None          # recorded for other sources
    assert bench.measured_traffic(8, 32, 128) is None          # no record


def test_cpu_baseline_times_the_whole_small_workload():
    from fp8_block_scaled_04_amd import synth
    shapes = [(8, 16, 256), (4, 24, 128)]
    host = {}
    for (m, n, k) in shapes:
        host[(m, k)] = synth.normal_f32(0, synth.S_LHS, (m, k))
        host[(n, k)] = synth.normal_f32(0, synth.S_RHS, (n, k))
    rec = bench.cpu_baseline(shapes, host, target_s=5.0)
    assert rec["kind"] == "oracle" and rec["unit"] == "TFLOP/s" and rec["value"] > 0
    assert rec["sample"].startswith("the whole workload")
    assert rec["cores"] == rec["threads"] >= 1
    assert rec["nproc"] == os.cpu_count() and isinstance(rec["cpu_model"], str)
    macs = sum(m * n * k for m, n, k in shapes) / 1e9
    assert f"{macs:.1f} G MAC" in rec["sample"]
