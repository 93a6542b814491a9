"""Host-side contract of bench.py (no GPU): the single-GPU guard and the
HBM-traffic lookup."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_more_than_one_gpu_is_refused():
    """--gpus N > 1 exits with status 2 and a JSON line saying why, before
    anything touches a GPU."""
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line["n_gpus"] == 2 and "one GPU" in line["error"]


def test_traffic_only_for_profiled_workload_and_sources(monkeypatch):
    """The committed counters are reported only for the workload they were
    taken on, and only while the pass-1 sources hash the same."""
    import bench
    t = json.load(open(os.path.join(ROOT, "profiles", "traffic.json")))
    cid = t["config_id"]
    if t["source_hash"] == bench.kernel_source_hash():
        assert bench.read_traffic("prop_pass1_kernel", cid) == t["kernels"]["prop_pass1_kernel"]["bytes_per_launch"]
    assert bench.read_traffic("prop_pass1_kernel", cid + 1) is None
    # a different source hash: no traffic
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "0" * 16)
    assert bench.read_traffic("prop_pass1_kernel", cid) is None
