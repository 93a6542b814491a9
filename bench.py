#!/usr/bin/env python3
"""Benchmark of the decode-step S2ANTA-prop path on one MI355X.

One step = one santa_decode_prop call (pass 1, reducer, pass 2) over one
decode step of the Llama-3.1-8B layer shape at 32k context: batch 1, 32 query
heads, 8 KV heads, head dim 128, bf16 KV, S = 128, tiles of 256 tokens
(synthetic inputs with planted high-scoring keys and 4 sinks per KV head).
Inputs are resident in HBM before timing starts; steps rotate over enough
copies of the KV cache (>= 1 GiB) that the 256 MB Infinity Cache cannot hold
them.  `value` comes from plain host calls, one per step (--mode eager, the
default); replay of a captured HIP graph is reported beside it.  The same
GPU's exact split-KV decode (and S2ANTA-flash, where the workload has a flash
budget) is timed the same way, and the fp64 CPU oracle is timed on a bounded
sample on the host.

Prints one JSON line (see the "value"/"roofline"/"cpu_baseline" fields).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "decode-attn µs/step + achieved HBM GB/s (% peak), 32k ctx, S=128, 1×MI355X"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
# the sources of the dominant kernel (prop pass 1), whose HBM counters
# profiles/traffic.json holds
KERNEL_SOURCES = ["santa_prop_pass1.hip", "santa_prop_body.h", "santa_kernels.h", "santa_score.h", "santa_device.h",
                  "santa_launch.h"]


def kernel_source_hash():
    """Hash of the code (comments and blank lines removed) of the sources
    that pass 1 is built from, so that a comment edit keeps the counters."""
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "stochastic_sparse_attention_amd", "csrc", f)) as fh:
            src = fh.read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        src = re.sub(r"//[^\n]*", "", src)
        code = "\n".join(line.rstrip() for line in src.splitlines() if line.strip())
        h.update(code.encode())
    return h.hexdigest()[:16]


def read_traffic(kernel_key, cid):
    """HBM bytes per launch from the committed rocprofv3 --pmc summary, if it
    was taken on the current kernel sources and on workload `cid` (else
    None)."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("source_hash") != kernel_source_hash() or t.get("config_id") != cid:
        return None
    e = t.get("kernels", {}).get(kernel_key)
    return None if e is None else e.get("bytes_per_launch")


# The pages' own figures for this path, as context (not the target): the
# SANTA notes report kernel-latency speedups over FlashInfer and the share of
# V rows read, on hardware they do not name.
PAGES_CONTEXT = {
    "source": "Stochastic Sparse Attention for Memory-Bound Inference (SANTA notes), key designs 2-3 "
              "and the note under Table 1",
    "hardware": "not stated on the pages",
    "prop_speedup_vs_flashinfer": 1.50,
    "prop_setting": "Llama-3.1-8B decode, 32k context, S=128",
    "flash_speedup_vs_flashinfer": 1.51,
    "flash_setting": "same shape, S=2048",
    "v_rows_read_prop": "<1.56% of n_k",
    "sample_budget_fraction": {"prop_S128": 0.0039, "flash_S2048": 0.0625},
    "note": "kernel-level speedups of the pages' own GPU kernels over FlashInfer; this line's "
            "speedup_vs_exact is against this GPU's own exact split-KV decode",
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def time_steps(fn, steps, warmup, events=None):
    """Run fn(i) warmup times untimed, then `steps` times timed with plain
    host calls; with `events`, run the steps once more with the dominant
    kernel bracketed by dispatch-recorded events.  Returns (ms_per_step,
    per-step dominant-kernel ms list or None)."""
    import torch
    import stochastic_sparse_attention_amd as sa
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        fn(warmup + i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    kern = None
    if events:
        # default HIP events, recorded by the dispatch itself: their
        # system-scope fences slow the bracketed kernel, but they time that
        # kernel exactly (events created with hipEventDisableSystemFence
        # leave it alone but then include its dispatch latency)
        pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                 for _ in range(steps)]
        for a, b in pairs:          # create the HIP events (torch creates them on first record)
            a.record()
            b.record()
        torch.cuda.synchronize()
        for i in range(steps):
            sa.santa_set_timing_events(pairs[i][0], pairs[i][1])
            fn(warmup + i)
        torch.cuda.synchronize()
        sa.santa_set_timing_events(None, None)
        kern = [a.elapsed_time(b) for a, b in pairs]
    return (t1 - t0) * 1e3 / steps, kern


def step_spread(fn, steps, warmup):
    """p10/p50/p90 of single-step GPU times: events recorded on the stream
    between consecutive host calls."""
    import torch
    for i in range(warmup):
        fn(i)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    ev[0].record()
    for i in range(steps):
        fn(warmup + i)
        ev[i + 1].record()
    torch.cuda.synchronize()
    per = np.array([ev[i].elapsed_time(ev[i + 1]) for i in range(steps)])
    return {q: round(float(np.percentile(per, q)) * 1e3, 3) for q in (10, 50, 90)}


def time_graph(step_fn, ncopy, steps, warmup):
    """Capture `ncopy` consecutive steps (one per KV copy) into one HIP graph
    and replay it; returns ms per step.  Timed replays cover exactly `steps`
    steps (rounded up to whole graphs)."""
    import torch
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for i in range(ncopy):          # warm the allocator / code paths on the side stream
            step_fn(i)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for i in range(ncopy):
            step_fn(i)
    torch.cuda.synchronize()
    for _ in range(max(1, warmup // ncopy)):
        g.replay()
    torch.cuda.synchronize()
    reps = max(1, -(-steps // ncopy))
    t0 = time.perf_counter()
    for _ in range(reps):
        g.replay()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    # a second pass with events around each replay gives the spread
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, b in evs:
        a.record()
        g.replay()
        b.record()
    torch.cuda.synchronize()
    per = np.array([a.elapsed_time(b) / ncopy for a, b in evs])
    spread = {q: round(float(np.percentile(per, q)) * 1e3, 3) for q in (10, 50, 90)}
    return (t1 - t0) * 1e3 / (reps * ncopy), spread


def torch_read_gbs(torch, dev, nbytes, ncopy, reps=50):
    """Read rate of a torch reduction (a sum over an int64 view, the fastest
    read-bound torch reduction measured on this part) over `nbytes`,
    rotating over `ncopy` buffers so that repeated reads are not served by
    the Infinity Cache.  Bytes read per second."""
    xs = [torch.ones(nbytes // 8, dtype=torch.int64, device=dev) for _ in range(ncopy)]
    for i in range(10):
        xs[i % ncopy].sum()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(reps):
        xs[i % ncopy].sum()
    e1.record()
    torch.cuda.synchronize()
    sec = e0.elapsed_time(e1) * 1e-3 / reps
    del xs
    return nbytes / sec / 1e9


def copy_peak_gbs(torch, dev, nbytes=512 << 20, reps=10):
    """Device-to-device copy rate (read + write bytes per second), the
    measured ceiling beside the 8 TB/s spec."""
    a = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    sec = e0.elapsed_time(e1) * 1e-3 / reps
    del a, b
    return 2 * nbytes / sec / 1e9


def _median_time(fn, seconds, max_reps=50):
    reps, secs = 0, []
    t_start = time.perf_counter()
    while True:
        t0 = time.perf_counter()
        fn()
        secs.append(time.perf_counter() - t0)
        reps += 1
        if time.perf_counter() - t_start >= seconds or reps >= max_reps:
            break
    return float(np.median(secs)), reps


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(inp, S, seconds):
    """The fp64 oracle on the host cores (a reported baseline, not the target):
    prop with OpenMP over the heads at the default thread count, prop on one
    thread, and the exact decode at the default thread count."""
    import oracle as O
    prob = O.Problem.from_inputs(inp)
    u = inp.u(S)
    cores = O.num_threads()
    prop_s, reps = _median_time(lambda: O.santa_prop(prob, inp.q, inp.k, inp.v, S, u), seconds)
    exact_s, ereps = _median_time(lambda: O.exact(prob, inp.q, inp.k, inp.v), seconds / 4, 10)
    O.set_num_threads(1)
    try:
        single_s, sreps = _median_time(lambda: O.santa_prop(prob, inp.q, inp.k, inp.v, S, u), seconds / 2, 5)
    finally:
        O.set_num_threads(cores)
    return {"prop_s": prop_s, "reps": reps, "cores": cores, "exact_s": exact_s, "exact_reps": ereps,
            "single_s": single_s, "single_reps": sreps}


def exact_problem(sa, dev, cfg, tile_len):
    """The device inputs' problem with another tile length (same tensors)."""
    p = dev.problem
    return sa.Problem(cfg.batch, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim, cfg.seq_len,
                      dtype=cfg.q_dtype, kv_dtype=cfg.kv_dtype, scale=p.s.scale, tile_len=tile_len,
                      seq_lens=p.seq_lens, page_size=cfg.page_size, page_table=p.page_table)


def time_exact_best(sa, BM, dev, cfg, ks, vs, ncopy, args, seq):
    """The same GPU's exact split-KV decode at its own best split: tile
    lengths T, 2T and 4T (up to 1024) are timed and the fastest one is the
    reference."""
    import torch
    T = cfg.tile_len
    oute = torch.empty((cfg.batch * cfg.num_q_heads, cfg.head_dim), dtype=torch.float32, device=dev.q.device)
    by_tile = {}
    for TE in sorted({t for t in (T, 2 * T, 4 * T) if t <= 1024}):
        pe = exact_problem(sa, dev, cfg, TE)
        wse = torch.empty(sa.santa_workspace_size(pe, "exact"), dtype=torch.uint8, device=dev.q.device)

        def exact_step(i, pe=pe, wse=wse):
            c = i % ncopy
            sa.exact_decode_ref(pe, dev.q, ks[c], vs[c], oute, workspace=wse)

        tms, tk = time_steps(exact_step, args.steps, args.warmup, events=True)
        by_tile[TE] = (tms, tk, exact_step)
        log(f"bench: exact with T={TE} {tms * 1e3:.2f} us/step (eager), partial {np.mean(tk) * 1e3:.2f} us")
    TE = min(by_tile, key=lambda t: by_tile[t][0])
    ems_eager, ekern, exact_step = by_tile[TE]
    ems_graph, _espread = time_graph(exact_step, ncopy, args.steps, args.warmup)
    ems = ems_eager if args.mode == "eager" else ems_graph
    eb = BM.exact_step_bytes(cfg, TE, seq)
    log(f"bench: exact {ems * 1e3:.2f} us/step (eager {ems_eager * 1e3:.2f}, graph {ems_graph * 1e3:.2f}), "
        f"T={TE}, partial {np.mean(ekern) * 1e3:.2f} us")
    return {
        "tile_len": TE,
        "eager_us_per_step_by_tile_len": {str(t): round(v[0] * 1e3, 3) for t, v in sorted(by_tile.items())},
        "us_per_step": round(ems * 1e3, 3),
        "eager_us_per_step": round(ems_eager * 1e3, 3),
        "graph_us_per_step": round(ems_graph * 1e3, 3),
        "GB/s": round(eb["total"] / (ems * 1e-3) / 1e9, 1),
        "pct_of_hbm_peak": round(100 * eb["total"] / (ems * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
        "partial_kernel_us": round(float(np.mean(ekern)) * 1e3, 3),
        "partial_kernel_GB/s": round(eb["partial"] / (np.mean(ekern) * 1e-3) / 1e9, 1),
    }


def batch16_block(sa, BM, synth, to_device, torch, dev0, args):
    """The 32k layer at batch 16 (the flash comparison workload): prop at
    S = 128, flash at S = 2048 and the exact decode, timed as the headline
    is.  Its 2 GiB of K and V exceed the Infinity Cache, so no copies rotate."""
    cfg = synth.CONFIGS[3]
    log(f"bench: generating workload {cfg.cid} ({cfg.name}) for the batch-16 block")
    inp = synth.make_inputs(cfg, cfg.cid)
    dev = to_device(inp, dev0)
    del inp.k, inp.v
    S, Sf, T = cfg.S, cfg.S_flash, cfg.tile_len
    BH = cfg.batch * cfg.num_q_heads
    ks, vs, ncopy = [dev.k], [dev.v], 1
    out = torch.empty((BH, cfg.head_dim), dtype=torch.float32, device=dev0)
    ws = torch.empty(sa.santa_workspace_size(dev.problem, "prop", S), dtype=torch.uint8, device=dev0)
    u = dev.u(S)

    def prop_step(i):
        sa.santa_decode_prop(dev.problem, dev.q, dev.k, dev.v, S, u, out, workspace=ws)

    pms, pk = time_steps(prop_step, args.steps, args.warmup, events=True)
    pgs, _ = time_graph(prop_step, ncopy, args.steps, args.warmup)
    zms = None
    if not args.no_fused:
        wsz = sa.new_workspace(dev.problem, "prop", S, dev0)

        def fused_step(i):
            sa.santa_decode_prop_fused(dev.problem, dev.q, dev.k, dev.v, S, u, out, workspace=wsz)

        zms, _zk = time_steps(fused_step, args.steps, args.warmup)
        log(f"bench: batch 16 prop in one launch {zms * 1e3:.2f} us/step")
    max_nt = (cfg.seq_len + T - 1) // T
    tb = torch.empty((BH, max_nt), dtype=torch.int32, device=dev0)
    sa.santa_decode_prop(dev.problem, dev.q, dev.k, dev.v, S, u, out, None, tb, workspace=ws)
    torch.cuda.synchronize()
    nb = BM.prop_step_bytes(cfg, S, tb.cpu().numpy(), T, None)
    log(f"bench: batch 16 prop {pms * 1e3:.2f} us/step (graph {pgs * 1e3:.2f}), pass-1 {np.mean(pk) * 1e3:.2f} us")
    wsf = torch.empty(sa.santa_workspace_size(dev.problem, "flash", Sf), dtype=torch.uint8, device=dev0)
    uf = dev.u(Sf)

    def flash_step(i):
        sa.santa_decode_flash(dev.problem, dev.q, dev.k, dev.v, Sf, uf, out, workspace=wsf)

    fms, fk = time_steps(flash_step, args.steps, args.warmup, events=True)
    fb = BM.flash_step_bytes(cfg, Sf, T)
    log(f"bench: batch 16 flash S={Sf} {fms * 1e3:.2f} us/step, tile kernel {np.mean(fk) * 1e3:.2f} us")
    ms = pms if args.mode == "eager" else pgs
    res = {
        "workload": f"{cfg.name}: S2ANTA-prop S={S}, S2ANTA-flash S={Sf}, exact",
        "prop": {"S": S, "us_per_step": round(ms * 1e3, 3), "eager_us_per_step": round(pms * 1e3, 3),
                 "graph_us_per_step": round(pgs * 1e3, 3), "GB/s": round(nb["total"] / (ms * 1e-3) / 1e9, 1),
                 "pct_of_hbm_peak": round(100 * nb["total"] / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
                 "pass1_kernel_us": round(float(np.mean(pk)) * 1e3, 3),
                 "pass1_frac_of_peak": round(nb["pass1"] / (np.mean(pk) * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                 "algorithmic_bytes_per_step": nb},
        "single_launch_us_per_step": None if zms is None else round(zms * 1e3, 3),
        "flash": {"S": Sf, "us_per_step": round(fms * 1e3, 3),
                  "GB/s": round(fb["total"] / (fms * 1e-3) / 1e9, 1),
                  "tile_kernel_us": round(float(np.mean(fk)) * 1e3, 3)},
    }
    if not args.no_exact:
        res["exact_decode_ref"] = time_exact_best(sa, BM, dev, cfg, ks, vs, ncopy, args, None)
        res["prop_speedup_vs_exact"] = round(res["exact_decode_ref"]["us_per_step"] / (ms * 1e3), 3)
    res["prop_speedup_vs_flash"] = round(fms / pms, 3)
    del dev, ks, vs
    torch.cuda.empty_cache()
    return res


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    # about 20 ms of decode work at the headline workload: with 20 warmup
    # steps the first timed block ran up to 8% slow (117 against 108 us per
    # step at 32k batch 16 with e4m3 KV) until the GPU had settled
    ap.add_argument("--warmup", type=int, default=1000)
    ap.add_argument("--config", type=int, default=2, help="workload id (2 = 32k decode layer)")
    ap.add_argument("--kv-bytes-min", type=float, default=1.0, help="GiB of rotated KV copies")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-exact", action="store_true")
    ap.add_argument("--no-samplers", action="store_true",
                    help="skip timing prop with the stratified and i.i.d. threshold generators")
    ap.add_argument("--no-flash", action="store_true",
                    help="skip the S2ANTA-flash leg (run where the workload has a flash budget)")
    ap.add_argument("--no-bernoulli", action="store_true",
                    help="skip prop on Bernoulli qK^T scores (contiguous bf16 and e4m3 workloads)")
    ap.add_argument("--no-fused", action="store_true",
                    help="skip prop in one launch (santa_decode_prop_fused)")
    ap.add_argument("--no-batch16", action="store_true",
                    help="skip the secondary 32k batch-16 block (prop, flash S=2048, exact) that the "
                         "headline run adds")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run 5 device copies of 256 MiB (known traffic: 256 MiB read and "
                         "256 MiB written each) to calibrate the FETCH_SIZE / WRITE_SIZE counters")
    ap.add_argument("--mode", choices=["graph", "eager"], default="eager",
                    help="which timing gives `value`: eager = one host call per step, "
                         "graph = steps replayed from a captured HIP graph (both are reported)")
    args = ap.parse_args(argv)

    if args.gpus != 1:
        print(json.dumps({"error": "the decode path runs on one GPU; --gpus must be 1",
                          "n_gpus": args.gpus}), flush=True)
        log("bench.py: only single-GPU runs are supported (the decode path is not sharded across GPUs)")
        return 2

    import torch
    if args.copy_calibration:
        a = torch.full((256 << 20,), 3, dtype=torch.uint8, device="cuda:0")
        b = torch.empty_like(a)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        log("bench: 5 copies of 256 MiB done")
        return 0
    import stochastic_sparse_attention_amd as sa
    from stochastic_sparse_attention_amd import bytemodel as BM
    from stochastic_sparse_attention_amd import synth
    from stochastic_sparse_attention_amd.device_io import to_device

    sa._lib.load()
    dev0 = torch.device("cuda:0")
    # measured ceilings first (they also bring the GPU out of idle before
    # anything is timed): a device copy and torch's read-bound reduction
    copy_gbs = copy_peak_gbs(torch, dev0)
    read64 = torch_read_gbs(torch, dev0, 64 << 20, 8)
    read1g = torch_read_gbs(torch, dev0, 1 << 30, 1)
    log(f"bench: device copy {copy_gbs:.1f} GB/s (read + write); torch read-bound sum {read64:.1f} GB/s "
        f"at 64 MiB, {read1g:.1f} GB/s at 1 GiB")
    cfg = synth.CONFIGS[args.config]
    S, T = cfg.S, cfg.tile_len
    log(f"bench: generating workload {cfg.cid} ({cfg.name})")
    inp = synth.make_inputs(cfg, cfg.cid)
    dev = to_device(inp, dev0)
    kvb = BM.kv_bytes(cfg)
    ncopy = max(1, int(np.ceil(args.kv_bytes_min * 2 ** 30 / (2 * kvb))))
    ks = [dev.k] + [dev.k.clone() for _ in range(ncopy - 1)]
    vs = [dev.v] + [dev.v.clone() for _ in range(ncopy - 1)]
    BH = cfg.batch * cfg.num_q_heads
    u = dev.u(S)
    out = torch.empty((BH, cfg.head_dim), dtype=torch.float32, device=dev0)
    ws = torch.empty(sa.santa_workspace_size(dev.problem, "prop", S), dtype=torch.uint8, device=dev0)
    log(f"bench: {ncopy} KV copies ({ncopy * 2 * kvb / 2**30:.2f} GiB), S={S}, T={T}")

    def prop_step(i):
        c = i % ncopy
        sa.santa_decode_prop(dev.problem, dev.q, ks[c], vs[c], S, u, out, workspace=ws)

    ms_eager, kern = time_steps(prop_step, args.steps, args.warmup, events=True)
    log(f"bench: prop eager {ms_eager * 1e3:.2f} us/step, pass-1 {np.mean(kern) * 1e3:.2f} us")
    eager_spread = step_spread(prop_step, args.steps, args.warmup)
    ms_graph, spread = time_graph(prop_step, ncopy, args.steps, args.warmup)
    log(f"bench: prop graph {ms_graph * 1e3:.2f} us/step (p10/p50/p90 {spread}); "
        f"eager p10/p50/p90 {eager_spread}")
    ms = ms_eager if args.mode == "eager" else ms_graph

    # one more call with the optional outputs, for the byte count and V-row share
    max_nt = (cfg.seq_len + T - 1) // T
    idx = torch.empty((BH, S), dtype=torch.int32, device=dev0)
    tb = torch.empty((BH, max_nt), dtype=torch.int32, device=dev0)
    sa.santa_decode_prop(dev.problem, dev.q, dev.k, dev.v, S, u, out, idx, tb, workspace=ws)
    torch.cuda.synchronize()
    tb_np, idx_np = tb.cpu().numpy(), idx.cpu().numpy()
    seq = inp.seq_lens if not inp.uniform_len or cfg.page_size else None
    nbytes = BM.prop_step_bytes(cfg, S, tb_np, T, seq)
    pass1_bytes = nbytes["pass1"]
    kern_ms = float(np.mean(kern))
    achieved = pass1_bytes / (kern_ms * 1e-3) / 1e9
    step_gbs = nbytes["total"] / (ms * 1e-3) / 1e9

    kern_sorted = np.sort(np.array(kern))

    result = {
        "metric": METRIC,
        "value": round(step_gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{cfg.name}: S2ANTA-prop", "batch": cfg.batch, "kv_dtype": cfg.kv_dtype,
                   "q_heads": cfg.num_q_heads, "kv_heads": cfg.num_kv_heads,
                   "head_dim": cfg.head_dim, "seq_len": cfg.seq_len, "S": S, "tile_len": T,
                   "kv_copies_rotated": ncopy},
        "us_per_step": round(ms * 1e3, 3),
        "timing_mode": args.mode,
        "eager_us_per_step": round(ms_eager * 1e3, 3),
        "graph_us_per_step": round(ms_graph * 1e3, 3),
        "pct_of_hbm_peak": round(100 * step_gbs / HBM_PEAK_GBS, 2),
        "step_us_p10_p50_p90": spread if args.mode == "graph" else eager_spread,
        "step_spread_note": "eager spread: events recorded between host calls (they add their own overhead); graph spread: per replay of the captured steps",
        "graph_step_us_p10_p50_p90": spread,
        "copy_peak_GB/s": round(copy_gbs, 1),
        "pct_of_copy_peak": round(100 * step_gbs / copy_gbs, 2),
        "torch_read_GB/s": {"64MiB": round(read64, 1), "1GiB": round(read1g, 1),
                            "note": "sum over an int64 view, the fastest torch reduction measured; 64 MiB "
                                    "rotates 8 buffers past the Infinity Cache. Not a hardware ceiling: "
                                    "prop's pass 1 reads faster"},
        "pages_context": PAGES_CONTEXT,
        "algorithmic_bytes_per_step": nbytes,
        "v_row_fraction": round(BM.v_row_fraction(idx_np, cfg, seq), 6),
        "tiles_visited_per_head": round(float((tb_np > 0).sum(1).mean()), 2),
        "roofline": {"kernel": "prop_pass1_kernel", "bound": "hbm", "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": read_traffic("prop_pass1_kernel", cfg.cid),
                     "bytes_per_launch": pass1_bytes, "avg_launch_us": round(kern_ms * 1e3, 3),
                     "launch_us_p10_p50_p90": [round(float(np.percentile(kern_sorted, q)) * 1e3, 3)
                                               for q in (10, 50, 90)],
                     "frac_of_copy_peak": round(achieved / copy_gbs, 4),
                     "vs_torch_read_64MiB": round(achieved / read64, 4)},
    }

    if not args.no_exact:
        result["exact_decode_ref"] = time_exact_best(sa, BM, dev, cfg, ks, vs, ncopy, args, seq)
        result["speedup_vs_exact"] = round(result["exact_decode_ref"]["us_per_step"] / (ms * 1e3), 3)

    if not args.no_samplers:
        uu = dev.uniforms(S)
        result["samplers"] = {"sys": {"us_per_step": round(ms_eager * 1e3, 3)}}
        for smp in ("strat", "iid"):
            def smp_step(i, smp=smp):
                c = i % ncopy
                sa.santa_decode_prop_sampler(dev.problem, dev.q, ks[c], vs[c], S, smp, uu, out, workspace=ws)
            sms, _sk = time_steps(smp_step, args.steps, args.warmup)
            log(f"bench: prop with {smp} thresholds {sms * 1e3:.2f} us/step (eager)")
            result["samplers"][smp] = {"us_per_step": round(sms * 1e3, 3)}

    if not args.no_fused:
        # S2ANTA-prop in one launch (the group's last workgroup samples), on a
        # zeroed workspace (its arrival counters)
        wsz = sa.new_workspace(dev.problem, "prop", S, dev0)

        def fused_step(i):
            c = i % ncopy
            sa.santa_decode_prop_fused(dev.problem, dev.q, ks[c], vs[c], S, u, out, workspace=wsz)

        zms, zk = time_steps(fused_step, args.steps, args.warmup, events=True)
        zgs, _ = time_graph(fused_step, ncopy, args.steps, args.warmup)
        log(f"bench: prop in one launch {zms * 1e3:.2f} us/step (graph {zgs * 1e3:.2f}), kernel {np.mean(zk) * 1e3:.2f} us")
        result["single_launch"] = {
            "us_per_step": round(zms * 1e3, 3), "graph_us_per_step": round(zgs * 1e3, 3),
            "kernel_us": round(float(np.mean(zk)) * 1e3, 3),
            "vs_two_launch": round(ms_eager / zms, 3),
            "note": "santa_decode_prop_fused: pass 1 in every workgroup, reducer and pass 2 in each KV "
                    "group's last-arriving workgroup (agent-scope release + arrival count per workgroup)",
        }

    if cfg.S_flash and not args.no_flash:
        Sf = cfg.S_flash
        wsf = torch.empty(sa.santa_workspace_size(dev.problem, "flash", Sf), dtype=torch.uint8, device=dev0)
        outf = torch.empty_like(out)
        uf = dev.u(Sf)

        def flash_step(i):
            c = i % ncopy
            sa.santa_decode_flash(dev.problem, dev.q, ks[c], vs[c], Sf, uf, outf, workspace=wsf)

        fms_eager, fkern = time_steps(flash_step, args.steps, args.warmup, events=True)
        fms_graph, _fspread = time_graph(flash_step, ncopy, args.steps, args.warmup)
        fms = fms_eager if args.mode == "eager" else fms_graph
        fb = BM.flash_step_bytes(cfg, Sf, T)
        log(f"bench: flash S={Sf} {fms * 1e3:.2f} us/step (eager {fms_eager * 1e3:.2f}, graph {fms_graph * 1e3:.2f}), "
            f"tile kernel {np.mean(fkern) * 1e3:.2f} us")
        result["santa_flash"] = {
            "S": Sf,
            "us_per_step": round(fms * 1e3, 3),
            "eager_us_per_step": round(fms_eager * 1e3, 3),
            "graph_us_per_step": round(fms_graph * 1e3, 3),
            "GB/s": round(fb["total"] / (fms * 1e-3) / 1e9, 1),
            "pct_of_hbm_peak": round(100 * fb["total"] / (fms * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
            "tile_kernel_us": round(float(np.mean(fkern)) * 1e3, 3),
            "tile_kernel_GB/s": round(fb["tile"] / (np.mean(fkern) * 1e-3) / 1e9, 1),
            "prop_speedup_vs_flash": round(fms / ms, 3),
        }
        if not args.no_samplers:
            uuf = dev.uniforms(Sf)
            for smp in ("strat", "iid"):
                def fsmp_step(i, smp=smp):
                    c = i % ncopy
                    sa.santa_decode_flash_sampler(dev.problem, dev.q, ks[c], vs[c], Sf, smp, uuf, outf, workspace=wsf)
                fsms, fk = time_steps(fsmp_step, args.steps, args.warmup, events=True)
                log(f"bench: flash with {smp} thresholds {fsms * 1e3:.2f} us/step (eager), "
                    f"tile kernel {np.mean(fk) * 1e3:.2f} us")
                result["santa_flash"][f"{smp}_us_per_step"] = round(fsms * 1e3, 3)
                result["santa_flash"][f"{smp}_tile_kernel_us"] = round(float(np.mean(fk)) * 1e3, 3)

    if (not args.no_bernoulli and cfg.kv_dtype in ("bf16", "fp8") and cfg.q_dtype == "bf16"
            and not cfg.page_size and cfg.seq_len % 4 == 0):
        # K transposed per KV head (the layout Bernoulli scoring reads), one per rotated copy
        kfs = [kk.transpose(-1, -2).contiguous() for kk in ks]
        fr = torch.empty(cfg.batch * cfg.num_kv_heads, dtype=torch.int32, device=dev0)
        result["bernoulli"] = {"draws": 4, "note": "prop with systematic thresholds on Bernoulli qK^T "
                               "scores; pass 1 reads only the kept features of a feature-major K"}
        for gm, name in ((0, "per_head"), (1, "mean_group_query")):
            ub = dev.bernoulli_uniforms(4, bool(gm))

            def bern_step(i, gm=gm, ub=ub):
                c = i % ncopy
                sa.santa_decode_prop_bernoulli(dev.problem, dev.q, kfs[c], vs[c], S, u, 4, gm, ub, out,
                                               workspace=ws)

            bms, bk = time_steps(bern_step, args.steps, args.warmup, events=True)
            sa.santa_decode_prop_bernoulli(dev.problem, dev.q, kfs[0], vs[0], S, u, 4, gm, ub, out,
                                           features_read=fr, workspace=ws)
            torch.cuda.synchronize()
            fr_np = fr.cpu().numpy()
            bb = BM.bernoulli_pass1_bytes(cfg, fr_np, 4, gm, T, seq)
            bk_ms = float(np.mean(bk))
            log(f"bench: prop on Bernoulli scores ({name}) {bms * 1e3:.2f} us/step (eager), "
                f"pass 1 {bk_ms * 1e3:.2f} us, features read {fr_np.mean() / cfg.head_dim:.3f}")
            result["bernoulli"][name] = {
                "us_per_step": round(bms * 1e3, 3),
                "features_read_frac": round(float(fr_np.mean()) / cfg.head_dim, 4),
                "pass1_kernel_us": round(bk_ms * 1e3, 3),
                "pass1_bytes": bb,
                "pass1_GB/s": round(bb / (bk_ms * 1e-3) / 1e9, 1),
                "speedup_vs_exact_scores": round(ms_eager / bms, 3),
            }
        del kfs

    if args.config == 2 and not args.no_batch16:
        result["batch16"] = batch16_block(sa, BM, synth, to_device, torch, dev0, args)

    if not args.no_cpu_baseline:
        log("bench: timing the CPU oracle")
        cb = cpu_baseline(inp, S, args.cpu_seconds)
        sec = cb["prop_s"]
        result["cpu_baseline"] = {
            "value": round(nbytes["total"] / sec / 1e9, 3), "unit": "GB/s", "cores": cb["cores"],
            "kind": "oracle", "us_per_step": round(sec * 1e6, 1),
            "sample": f"{cb['reps']} full steps of the same workload (all {BH} heads), median",
            "single_thread_us_per_step": round(cb["single_s"] * 1e6, 1),
            "exact_us_per_step": round(cb["exact_s"] * 1e6, 1),
            "cpu_model": cpu_model(),
        }
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
