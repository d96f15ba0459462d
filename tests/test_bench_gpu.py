"""bench.py end to end on the GPU: one short run prints the one JSON line the benchmark
contract asks for, with the roofline and oracle-baseline objects filled in."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.gpu
def test_bench_prints_the_contract_line():
    print("bench.py --steps 2 --warmup 1 --cpu-seconds 1", flush=True)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "2", "--warmup", "1",
                        "--cpu-seconds", "1"], capture_output=True, text=True, timeout=110)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1, r.stdout
    d = json.loads(lines[0])
    assert d["unit"] == "TFLOP/s" and d["n_gpus"] == 1 and d["steps"] == 2 and d["warmup"] == 1
    assert d["higher_is_better"] is True and d["scaling"] == "weak" and d["vs_baseline"] is None
    assert d["dtype"] == "bf16" and d["data"] == "synthetic"
    assert d["config"]["workload"] == "wan720p-rank-share-bf16"
    assert (d["config"]["heads"], d["config"]["head_dim"], d["config"]["sq"], d["config"]["sk"]) == (40, 128, 18900, 75600)
    assert d["value"] > 0 and d["ms_per_step"] > 0
    flops = 4 * 40 * 18900 * 75600 * 128
    assert abs(d["value"] - flops / (d["ms_per_step"] * 1e-3) / 1e12) <= 1e-3 * d["value"]
    rf = d["roofline"]
    assert rf["bound"] == "mfma" and rf["unit"] == "TFLOP/s" and rf["peak"] == 2516.6
    assert rf["flops_per_launch"] == flops and rf["launch_ms"] > 0
    assert abs(rf["achieved"] - flops / (rf["launch_ms"] * 1e-3) / 1e12) <= 1e-3 * rf["achieved"]
    assert abs(rf["frac"] - rf["achieved"] / rf["peak"]) <= 1e-4
    assert rf["traffic"] is None or rf["traffic"] > 1.99e9
    assert d["bounds"]["ms"] > 0 and d["bounds"]["algorithmic_bytes"] == 2515968000
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["value"] > 0 and cb["cores"] >= 1 and cb["unit"] == "TFLOP/s"
