"""Host-side contract of bench.py (no GPU): the single-GPU guard, the
HBM-traffic lookup and the exact baseline's problem at other splits."""
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


def test_exact_baseline_problem_keeps_everything_but_the_split():
    """The exact baseline is timed at other tile lengths on the same tensors:
    only tile_len may differ from the workload's problem."""
    import bench
    import stochastic_sparse_attention_amd as sa
    from stochastic_sparse_attention_amd import synth

    class Dev:                       # the fields bench.exact_problem reads
        pass
    cfg = synth.CONFIGS[4]
    dev = Dev()
    dev.problem = sa.Problem(cfg.batch, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim, cfg.seq_len,
                             dtype=cfg.q_dtype, kv_dtype=cfg.kv_dtype, scale=0.125, tile_len=cfg.tile_len)
    p = bench.exact_problem(sa, dev, cfg, 1024)
    a, b = dev.problem.s, p.s
    for f, _ in a._fields_:
        if f == "tile_len":
            assert (a.tile_len, b.tile_len) == (cfg.tile_len, 1024)
        else:
            assert getattr(a, f) == getattr(b, f), f
