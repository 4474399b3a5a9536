"""bench.py's host-side contract (no GPU): it refuses more than one GPU with a
message, and the pieces of its JSON line that need no device are well formed."""
import json
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""



def test_persist_needs_a_q4_config():
    """--persist defaults to the Q4 workload; a bf16 one is refused with a
    message before anything is allocated."""
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--persist", "--config", "inms"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 1 and "--config q4" in r.stderr and r.stdout.strip() == ""

def test_traffic_fingerprint_and_committed_counters():
    import bench
    h = bench.kernel_source_hash("inms")
    assert len(h) == 16 and h == bench.kernel_source_hash("inms")  # deterministic
    assert h != bench.kernel_source_hash("tokendance")  # the work plan is part of it
    d = json.load(open(os.path.join(ROOT, "profiles", "tile_kernel_inms_hbm_counters.json")))
    # the committed counter runs describe the current kernel and plan
    assert d["source_hash"] == h
    t = bench.measured_traffic("inms")
    assert t == d["hbm_bytes_per_launch"]
    # HBM reads within a few per cent of the unique bytes (each shared block fetched once)
    assert 0.99 < d["hbm_read_bytes_per_launch"] / d["algorithmic_unique_kv_bytes_per_launch"] < 1.05
    assert bench.measured_traffic("no-such-config") is None


def test_source_fingerprint_ignores_comments_only():
    """The kernel fingerprint reads code, not comments: a comment edit keeps it,
    any change to the code (a literal, an operator) changes it, and comment
    markers inside string or character literals are code."""
    import bench
    base = 'int f(int x) {\n  // scale\n  return x * 2; /* twice */\n}\nconst char* s = "a//b";\n'
    same = 'int f(int x) {  /* scale it */\n  return x * 2;   // doubled\n}\nconst char* s = "a//b";'
    assert bench.code_text(base) == bench.code_text(same)
    for other in (base.replace("2;", "3;"), base.replace("*", "+", 1), base.replace('"a//b"', '"a//c"')):
        assert bench.code_text(other) != bench.code_text(base)
    assert bench.code_text("char c = '\\'';  // x") == "char c = '\\'';"


def test_cpu_baseline_sample_is_bounded_and_split():
    """The oracle sample runs in a pool of worker processes over (agent, head
    chunk) jobs covering the requested agents and heads, and reports its wall
    time and the CPU seconds per phase."""
    import bench
    c = bench.cpu_baseline("tiny", 2, 4, workers=3)
    assert c["agents"] == 2 and c["heads"] == 4 and c["workers"] == 3
    # 4 q heads over 2 kv heads: each agent's heads cut into chunks of whole kv-head groups
    assert c["jobs"] == 4
    assert c["seconds"] > 0 and c["os_cpu_count"] >= 1
    assert all(np.isfinite(c[k]) and c[k] >= 0 for k in ("table_build", "materialise", "attention"))
    assert 1 <= bench.CPU_WORKERS <= 16
