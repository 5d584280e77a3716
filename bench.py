"""Benchmark one prune-then-graft decode step on one MI355X.

A step is the whole hot path over one batch: graft_build_tree ->
graft_tree_attention -> graft_accept -> graft_update_adjacency, on inputs
already resident in HBM.  Input sets rotate so that the live footprint
exceeds the 256 MB Infinity Cache.  Each set's step is captured once in a
HIP graph and the timed region replays the graphs (the eager time, with the
Python launch path in between, is reported as ms_per_step_eager).  Per-call
durations come from HIP events around replays of a graph that runs the
call on 16 consecutive input sets.  Prints one JSON line.

  python bench.py [--steps K] [--warmup W] [--config NAME] [--gpus 1]

Counter support (HBM traffic of the attention call, see profiles/):
  --copy-calibration   after the timed steps, run a plain elementwise copy of
                       256 MiB three times, so that a rocprofv3 --pmc pass over
                       this process also measures what FETCH_SIZE/WRITE_SIZE
                       report for a known number of bytes;
  --traffic-from-pmc FETCH_DIR WRITE_DIR
                       read two such passes (rocprofv3 --output-format csv) and
                       record the attention call's HBM bytes per launch in
                       profiles/attn_traffic.json (no GPU needed).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "verified tree tokens/s + tree-attn KV-read HBM GB/s (% of peak), 1 MI355X"
HBM_PEAK_GBPS = 8000.0
MFMA_PEAK_TFLOPS = 2500.0         # dense bf16 matrix-core peak
STREAM_BYTES = 2 << 30            # read by the streaming-ceiling reduction
DEFAULT_CONFIG = "llama3_8b_b1"   # the Llama-3-8B verify layer, batch 1
ROTATE_BYTES = 600 << 20          # rotate input sets beyond the 256 MB MALL
ATTN_SRC = os.path.join(ROOT, "tree_attention_verification_graft_amd", "csrc",
                        "tree_attention.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_traffic.json")
CALIBRATION_BYTES = 256 << 20     # size of the counter-calibration copy
CALLS_PER_GRAPH = 16              # calls per graph for the per-call timings
ATTN_KERNELS = ("attn_mfma_kernel", "attn_wave_kernel", "attn_combine_kernel")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def attention_bytes(w, n_nodes):
    """Algorithmic bytes of one attention launch: every prefix K and V row
    once, every tree node's K and V once, q read once, out written once."""
    e = 2 if w.dtype == "bf16" else 4
    kv_prefix = int(w.prefix_len.sum()) * w.Hkv * w.D * 2 * e
    kv_tree = int(np.sum(n_nodes)) * w.Hkv * w.D * 2 * e
    q_out = int(np.sum(n_nodes)) * w.Hq * w.D * 2 * e
    return kv_prefix + kv_tree, q_out


def attention_flops(w, n_nodes, masks):
    """Algorithmic flops of one attention launch: q.k and p.v (2 D each) for
    every (query row, visible key) pair; prefix keys are visible to every
    row, tree keys to the row's ancestors-or-self (mask popcount)."""
    G = w.Hq // w.Hkv
    total = 0
    for b in range(w.B):
        n = int(n_nodes[b])
        vis_tree = sum(bin(int(x)).count("1") for x in masks[b, :n].reshape(-1))
        total += (int(w.prefix_len[b]) * n + vis_tree) * G * w.Hkv * 4 * w.D
    return total


def kernel_source_sha():
    with open(ATTN_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def measured_traffic(name):
    """HBM bytes per attention launch from the committed counter summary,
    or None when none exists for this workload and kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    e = t.get(name)
    if not e or e.get("kernel_source_sha") != kernel_source_sha():
        return None
    return e.get("hbm_bytes_per_launch")


def _pmc_means(run_dir, counter):
    """Mean per-dispatch value of one counter, by kernel, from a rocprofv3
    --output-format csv directory."""
    import csv
    import glob
    files = glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {run_dir}")
    per_kernel = {}
    for f in files:
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] != counter:
                    continue
                per_kernel.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return {k: (sum(v) / len(v), len(v)) for k, v in per_kernel.items()}


def traffic_from_pmc(name, fetch_dir, write_dir):
    """HBM bytes per attention call from FETCH_SIZE and WRITE_SIZE passes,
    each scaled by what the same counter reads for the calibration copy
    (CALIBRATION_BYTES read and written by one elementwise kernel)."""
    out = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        means = _pmc_means(d, counter)
        calib = [v for k, v in means.items() if "neg_kernel" in k or "NegFunctor" in k]
        if not calib:
            raise SystemExit(f"{counter}: no calibration copy kernel in {d}")
        kib_calib = calib[0][0]
        factor = kib_calib * 1024.0 / CALIBRATION_BYTES
        # the plain call's kernels (the fused-RoPE instantiations of the same
        # template, attn_mfma_kernel<NB, true, ...>, are timed beside the
        # step, not here)
        call_kib = sum(v[0] for k, v in means.items()
                       if any(a in k for a in ATTN_KERNELS)
                       and not re.search(r"attn_mfma_kernel<\d+, true", k))
        out[counter] = {"calibration_kib": kib_calib, "factor": factor,
                        "attention_call_kib": call_kib,
                        "bytes_per_call": call_kib * 1024.0 / factor}
    try:
        with open(TRAFFIC_FILE) as f:
            table = json.load(f)
    except (OSError, ValueError):
        table = {}
    table[name] = {
        "kernel_source_sha": kernel_source_sha(),
        "hbm_bytes_per_launch": out["FETCH_SIZE"]["bytes_per_call"] +
                                out["WRITE_SIZE"]["bytes_per_call"],
        "fetch": out["FETCH_SIZE"], "write": out["WRITE_SIZE"],
        "note": ("per graft_tree_attention call (attention kernel plus split combine); "
                 "each counter divided by its reading per byte of a plain 256 MiB copy"),
    }
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(table, f, indent=1, sort_keys=True)
        f.write("\n")
    print(json.dumps(table[name], indent=1))


def cpu_baseline(w, budget_s=20.0):
    """Time the oracle on a bounded sample of the same workload with one
    host thread; scale to tokens/s."""
    import oracle as O
    import workloads as W
    from threadpoolctl import threadpool_limits

    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        m_ids, m_scores = w.m_ids, w.m_scores
        if w.prompt is not None:
            m_ids, m_scores = O.update_adjacency(m_ids, m_scores, w.prompt[None],
                                                 np.array([len(w.prompt) - 2]))
        t1 = time.perf_counter()
        tree = O.build_tree(w.cfg, w.draft_parent, w.draft_token, w.draft_conf, w.n_draft,
                            w.root_token, w.prefix_len, m_ids)
        t_build = time.perf_counter() - t1
        logits = W.plant_path(w.logits, w.dtype, tree["token"], tree["parent"],
                              tree["n_nodes"], w.plant_seed)
        rows = [(b, i, h) for b in range(w.B) for i in range(int(tree["n_nodes"][b]))
                for h in range(w.Hq)]
        # attention: time rows until the budget is half spent, then scale
        f64 = lambda a: O.as_f64(a, w.dtype)
        args = [f64(w.q), f64(w.k_tree), f64(w.v_tree), f64(w.k_cache), f64(w.v_cache)]
        rng = np.random.default_rng(0)
        order = rng.permutation(len(rows))
        done = 0
        t2 = time.perf_counter()
        chunk = 32
        while done < len(rows) and time.perf_counter() - t2 < budget_s / 2:
            sel = [rows[k] for k in order[done:done + chunk]]
            O.tree_attention(*args, w.block_table, w.prefix_len, tree["mask"],
                             tree["n_nodes"], w.scale, rows=sel)
            done += len(sel)
        t_attn = (time.perf_counter() - t2) * len(rows) / done
        t3 = time.perf_counter()
        acc = O.accept(logits, w.dtype, tree["token"], tree["parent"], tree["n_nodes"])
        t_acc = time.perf_counter() - t3
        t4 = time.perf_counter()
        O.update_adjacency(m_ids, m_scores, acc["path_tokens"], acc["accept_len"])
        t_upd = time.perf_counter() - t4
    step = t_build + t_attn + t_acc + t_upd
    tokens = int(tree["n_nodes"].sum())
    return {
        "value": tokens / step, "unit": "tokens/s", "cores": 1, "kind": "oracle",
        "sample": (f"one step of {w.name}: build, accept and update in full; attention on "
                   f"{done} of {len(rows)} (node, head) rows, time scaled to all rows; "
                   f"numpy float64, one thread"),
        "seconds_per_step": step,
        "components_s": {"build": t_build, "attention": t_attn, "accept": t_acc,
                         "update": t_upd},
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default=DEFAULT_CONFIG)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=20.0)
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--traffic-from-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    args = ap.parse_args()
    if args.traffic_from_pmc:
        traffic_from_pmc(args.config, *args.traffic_from_pmc)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch

    import workloads as W
    from tree_attention_verification_graft_amd.pipeline import DeviceStep, to_host

    dev = torch.device("cuda:0")
    log(f"generating workload {args.config}")
    w = W.make(args.config)
    from tree_attention_verification_graft_amd.binding import graft_version
    log(graft_version())

    # First set: seed M from the prompt if the workload has one, build once to
    # plant an acceptable path into the stand-in logits.
    base = DeviceStep(w, device=dev, alloc_update_for_prompt=True)
    if w.prompt is not None:
        base.seed_from_prompt(w.prompt)
    base.build()
    torch.cuda.synchronize()
    t = base.tree_host()
    logits = W.plant_path(w.logits, w.dtype, t["token"], t["parent"], t["n_nodes"],
                          w.plant_seed)
    base.logits.copy_(torch.from_numpy(logits.view(np.int16) if logits.dtype == np.uint16
                                       else logits).to(dev).view(base.logits.dtype))
    # the rotary table of the fused-RoPE variants and the random numbers of
    # sampling acceptance (both timed beside the step)
    base.set_rope(W.workload_rope_table(w))
    ra, rs = W.sampling_uniforms(w.plant_seed, w.B, base.n_max)
    base.rand_accept.copy_(torch.from_numpy(ra).to(dev))
    base.rand_sample.copy_(torch.from_numpy(rs).to(dev))
    per_set = sum(x.numel() * x.element_size() for x in
                  (base.q, base.k_tree, base.v_tree, base.k_cache, base.v_cache, base.logits))
    n_sets = max(1, math.ceil(ROTATE_BYTES / per_set))
    sets = [base]
    for _ in range(n_sets - 1):
        s = DeviceStep.__new__(DeviceStep)
        s.__dict__.update(base.__dict__)
        for k in ("q", "k_tree", "v_tree", "k_cache", "v_cache", "logits"):
            setattr(s, k, getattr(base, k).clone())
        for k in ("tree_token", "tree_parent", "tree_pos", "tree_mask", "n_nodes", "stage",
                  "out", "argmax", "accept_len", "path_nodes", "path_tokens"):
            setattr(s, k, torch.empty_like(getattr(base, k)))
        sets.append(s)
    log(f"{n_sets} rotating input sets of {per_set / 2**20:.1f} MiB")

    stream = torch.cuda.current_stream()
    ev = lambda: torch.cuda.Event(enable_timing=True)

    for k in range(args.warmup):
        sets[k % n_sets].step()
    torch.cuda.synchronize()

    # eager whole-step time (host launch overhead included), for reference
    t0 = time.perf_counter()
    for k in range(args.steps):
        sets[k % n_sets].step()
    torch.cuda.synchronize()
    ms_eager = (time.perf_counter() - t0) * 1e3 / args.steps

    # HIP graphs: one of the whole step per input set (a decode loop replays
    # one step at a time), and, for per-call timing, one graph per call that
    # runs it on CALLS_PER_GRAPH consecutive input sets, so that the graph
    # launch cost does not hide the kernels' own duration.
    calls = ("build", "attention", "accept", "update")
    step_graphs = []
    for s in sets:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            s.step()
        step_graphs.append(g)
    call_graphs = {}
    for c in calls:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for k in range(CALLS_PER_GRAPH):
                getattr(sets[k % n_sets], c)()
        call_graphs[c] = g
    for k in range(args.warmup):
        step_graphs[k % n_sets].replay()
    torch.cuda.synchronize()
    log(f"warmup {args.warmup} done; timing {args.steps} steps")

    # whole-step throughput: graph replays, no events inside the timed region
    t0 = time.perf_counter()
    for k in range(args.steps):
        step_graphs[k % n_sets].replay()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps

    # per-call durations: HIP events on the launch stream around replays of
    # each call's multi-call graph
    reps = max(1, args.steps // CALLS_PER_GRAPH)
    comp = []
    for c in calls:
        call_graphs[c].replay()
        e0, e1 = ev(), ev()
        e0.record(stream)
        for _ in range(reps):
            call_graphs[c].replay()
        e1.record(stream)
        torch.cuda.synchronize()
        comp.append(e0.elapsed_time(e1) / (reps * CALLS_PER_GRAPH))
    comp_ms = np.array(comp)

    # the next rows of the path, measured beside the step: committing the
    # accepted path's K/V to the cache (idempotent: same slots, same values),
    # the all-node update of M, the attention and the commit with the rotary
    # embedding fused in, and sampling acceptance at temperature 1 (last: it
    # overwrites the accepted paths)
    next_us = {}
    for name, call in (("append_kv", lambda s: s.append()),
                       ("update_tree", lambda s: s.update_tree()),
                       ("attention_rope", lambda s: s.attention_rope()),
                       ("append_kv_rope", lambda s: s.append_rope()),
                       ("accept_sample", lambda s: s.accept_sample(1.0))):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for k in range(CALLS_PER_GRAPH):
                call(sets[k % n_sets])
        g.replay()
        e0, e1 = ev(), ev()
        e0.record(stream)
        for _ in range(reps):
            g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        next_us[name] = e0.elapsed_time(e1) * 1e3 / (reps * CALLS_PER_GRAPH)

    n_nodes = np.stack([to_host(s.n_nodes) for s in sets])
    tokens = float(n_nodes.sum(axis=1).mean())
    value = tokens / (ms_per_step / 1e3)
    kv_bytes, qo_bytes = attention_bytes(w, n_nodes[0])
    t_attn_s = comp_ms[1] / 1e3
    achieved = (kv_bytes + qo_bytes) / t_attn_s / 1e9
    kv_gbps = kv_bytes / t_attn_s / 1e9
    flops = attention_flops(w, n_nodes[0], to_host(base.tree_mask).view(np.uint32))
    tflops = flops / t_attn_s / 1e12
    # the dominant kernel's bound: matrix cores above the ridge point
    mfma_bound = flops / (kv_bytes + qo_bytes) > MFMA_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBPS * 1e9)
    e = 2 if w.dtype == "bf16" else 4
    logits_gbps = float(n_nodes[0].sum()) * w.V * e / (comp_ms[2] / 1e3) / 1e9

    # a reference streaming read on this GPU: torch's sum over 2 GiB (a
    # plain reduction kernel; the logits scan of the accept call reads
    # faster at large batches, so this is a reference, not a ceiling)
    big = torch.ones(STREAM_BYTES // 4, dtype=torch.float32, device=dev)
    for _ in range(2):
        big.sum()
    e0, e1 = ev(), ev()
    e0.record(stream)
    for _ in range(5):
        big.sum()
    e1.record(stream)
    torch.cuda.synchronize()
    stream_gbps = 5 * STREAM_BYTES / (e0.elapsed_time(e1) / 1e3) / 1e9
    del big
    traffic = measured_traffic(w.name)
    log("next rows: " + ", ".join(f"{k} {v:.1f} us" for k, v in next_us.items()))
    log(f"step {ms_per_step * 1e3:.1f} us (eager {ms_eager * 1e3:.1f}); build {comp_ms[0] * 1e3:.1f} attn "
        f"{comp_ms[1] * 1e3:.1f} accept {comp_ms[2] * 1e3:.1f} update "
        f"{comp_ms[3] * 1e3:.1f} us; attention {achieved:.0f} GB/s")

    result = {
        "metric": METRIC,
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "ms_per_step_eager": ms_eager,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.B, "q_heads": w.Hq, "kv_heads": w.Hkv,
                   "head_dim": w.D, "prefix_len_total": int(w.prefix_len.sum()),
                   "kmax": w.kmax, "vocab": w.V, "top_s": w.S, "page": w.block,
                   "rotating_sets": n_sets},
        "kv_read_GBps": kv_gbps,
        "kv_read_pct_of_peak": 100.0 * kv_gbps / HBM_PEAK_GBPS,
        "torch_sum_read_GBps": stream_gbps,
        "logits_scan_GBps": logits_gbps,
        "attention_TFLOPs": tflops,
        "components_us": {"build": comp_ms[0] * 1e3, "attention": comp_ms[1] * 1e3,
                          "accept": comp_ms[2] * 1e3, "update": comp_ms[3] * 1e3},
        "roofline": {
            "kernel": "graft_tree_attention",
            "bound": "mfma" if mfma_bound else "hbm",
            "achieved": tflops if mfma_bound else achieved,
            "peak": MFMA_PEAK_TFLOPS if mfma_bound else HBM_PEAK_GBPS,
            "unit": "TFLOP/s" if mfma_bound else "GB/s",
            "frac": tflops / MFMA_PEAK_TFLOPS if mfma_bound else achieved / HBM_PEAK_GBPS,
            "traffic": traffic,
            "algorithmic_bytes_per_launch": kv_bytes + qo_bytes,
            "algorithmic_flops_per_launch": flops,
            "launch_us": comp_ms[1] * 1e3,
        },
        "cpu_baseline": None,
        "next_rows_us": next_us,
    }
    if args.copy_calibration:
        src = torch.ones(CALIBRATION_BYTES // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst
        log("calibration copies done")
    if not args.no_cpu_baseline:
        log("timing the oracle on the host (one thread)")
        result["cpu_baseline"] = cpu_baseline(w, args.cpu_budget)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
