"""bench.py's host-side contract, without a GPU: one GPU only, and the HBM traffic figure is
reported only while the attention kernel's sources match the ones the counters were taken on."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


@pytest.mark.parametrize("argv,env", [(["--gpus", "2"], {}), (["--gpus", "8"], {}), ([], {"WORLD_SIZE": "2"})])
def test_more_than_one_gpu_exits_with_a_message(argv, env):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *argv],
                       capture_output=True, text=True, timeout=120, env={**os.environ, **env})
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


def test_traffic_follows_the_kernel_source_hash(tmp_path, monkeypatch):
    f = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    run = ("wan720p-rank-share-bf16", True, "none", True)
    assert bench.measured_traffic(*run) is None                          # no file
    f.write_text("not json")
    assert bench.measured_traffic(*run) is None
    rec = {"workload": "wan720p-rank-share-bf16 (B=1, ...)", "hbm_bytes_per_launch": 123}
    f.write_text(json.dumps(dict(rec, kernel_source_sha256_16="0" * 16)))
    assert bench.measured_traffic(*run) is None                          # counters of another kernel
    f.write_text(json.dumps(dict(rec, kernel_source_sha256_16=bench.kernel_source_hash())))
    assert bench.measured_traffic(*run) == 123


def test_traffic_only_for_the_profiled_launch(tmp_path, monkeypatch):
    f = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    f.write_text(json.dumps({"workload": "wan720p-rank-share-bf16 (B=1, ...)", "hbm_bytes_per_launch": 123,
                             "kernel_source_sha256_16": bench.kernel_source_hash()}))
    assert bench.measured_traffic("wan720p-rank-share-bf16", True, "none", True) == 123
    assert bench.measured_traffic("wan-block-bf16", True, "none", True) is None      # another workload
    assert bench.measured_traffic("wan720p-rank-share-bf16", False, "none", True) is None   # per-chunk calls
    assert bench.measured_traffic("wan720p-rank-share-bf16", True, "all", True) is None     # fallback mode
    assert bench.measured_traffic("wan720p-rank-share-bf16", True, "none", False) is None   # other q_block


def test_committed_traffic_record_is_well_formed():
    with open(bench.TRAFFIC_FILE) as fh:
        t = json.load(fh)
    assert len(t["kernel_source_sha256_16"]) == 16
    assert t["hbm_bytes_per_launch"] > 1.99e9                            # at least the algorithmic bytes


def test_cpu_baseline_stops_after_the_whole_workload():
    """A workload the oracle finishes inside the time budget is timed once, whole: every
    query row of every head exactly once, and a positive rate."""
    from dit_amd import workloads as WL
    inp = WL.generic_inputs(3, "bf16", 1, 2, 64, 300, (100, 50), q_block=64)
    r = bench.cpu_baseline(inp, seconds=1000.0)
    assert r["value"] > 0
    assert r["sample"].startswith(f"{2 * 300} query rows (whole 256-row q-blocks over 2 heads)")
