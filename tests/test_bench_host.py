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
    assert bench.measured_traffic() is None                              # no file
    f.write_text("not json")
    assert bench.measured_traffic() is None
    f.write_text(json.dumps({"kernel_source_sha256_16": "0" * 16, "hbm_bytes_per_launch": 123}))
    assert bench.measured_traffic() is None                              # counters of another kernel
    f.write_text(json.dumps({"kernel_source_sha256_16": bench.kernel_source_hash(), "hbm_bytes_per_launch": 123}))
    assert bench.measured_traffic() == 123


def test_committed_traffic_record_is_well_formed():
    with open(bench.TRAFFIC_FILE) as fh:
        t = json.load(fh)
    assert len(t["kernel_source_sha256_16"]) == 16
    assert t["hbm_bytes_per_launch"] > 1.99e9                            # at least the algorithmic bytes
