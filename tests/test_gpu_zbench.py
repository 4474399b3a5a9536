"""bench.py's JSON line on the device: one short run of the default (INMS)
workload, with every field of the line present and the derived figures
consistent with the measured ones."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

KEYS = ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better", "scaling",
        "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline")


@pytest.mark.gpu
def test_bench_line_contract():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "5", "--warmup", "2",
                        "--cpu-agents", "1", "--cpu-heads", "2"],
                       capture_output=True, text=True, timeout=600, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-3000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1, r.stdout[-3000:]
    d = json.loads(lines[0])
    for k in KEYS:
        assert k in d, k
    assert d["n_gpus"] == 1 and d["steps"] == 5 and d["warmup"] == 2
    assert d["higher_is_better"] is True and d["scaling"] == "weak" and d["vs_baseline"] is None
    assert d["unit"] == "agent-tokens/s" and d["dtype"] == "bf16"
    c = d["config"]
    assert c["workload"].startswith("inms:") and c["n_agents"] == 8 and c["physical_blocks"] == 3894
    assert c["unique_kv_bytes_per_step"] == 1020788736
    # value is the throughput of the median timed (cold) step
    assert abs(d["value"] - c["n_agents"] / (d["ms_per_step"] / 1e3)) <= 1e-3 * d["value"] + 0.1
    assert abs(d["step_us"]["median"] - d["ms_per_step"] * 1e3) <= 0.02
    assert d["warm"]["ms_per_step"] > 0
    rf = d["roofline"]
    assert rf["bound"] == "hbm" and rf["unit"] == "GB/s" and rf["peak"] == 8000.0
    assert rf["algorithmic_bytes_per_launch"] == c["unique_kv_bytes_per_step"]
    assert abs(rf["achieved"] - rf["algorithmic_bytes_per_launch"] / rf["avg_launch_us"] / 1e3) <= 1e-2 * rf["achieved"]
    assert abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-3
    assert 0.2 < rf["frac"] < 1.0
    # HBM counters taken on the current kernel and plan
    assert rf["traffic"] is not None and rf["traffic"] >= rf["algorithmic_bytes_per_launch"]
    rc = rf["read_ceiling"]
    assert rc["GBps"] > 0 and abs(rc["frac"] - rf["achieved"] / rc["GBps"]) < 1e-3
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and 1 <= cb["cores"] <= 16 and cb["value"] > 0 and cb["unit"] == d["unit"]
    assert set(cb["split_s"]) == {"table_build", "materialise_cpu_s", "attention_cpu_s"}
