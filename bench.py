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

The default workload is qwen3_235b_share (Qwen3-235B-A22B attention, one
GPU's head share: batch 32, 64/4 heads, prefix 8192, Kmax 64), the largest
that fits one GPU.  The same run also times the attention call alone at the
three bf16 8B-model shapes (llama3_8b_b1, qwen3_8b_b16, llama31_8b_64k) and
reports their KV-read bandwidth against the HBM peak.

  --no-extras          skip the attention-only timings at the other 8B shapes
                       (profiler runs of one workload)

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
DEFAULT_CONFIG = "qwen3_235b_share"  # the largest single-GPU workload
ATTN_8B_SHAPES = ("llama3_8b_b1", "qwen3_8b_b16", "llama31_8b_64k")
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


# Inputs of the oracle's attention, shared with the worker processes: they
# are set before the pool forks (copy-on-write pages, nothing pickled) and
# the pool is forked before this process touches the GPU.
_ORACLE_ARGS = {}


def _oracle_worker_init():
    from threadpoolctl import threadpool_limits
    threadpool_limits(limits=1)


def _oracle_attention_rows(sel):
    import oracle as O
    a = _ORACLE_ARGS
    O.tree_attention(*a["arrays"], a["block_table"], a["prefix_len"], a["mask"], a["n_nodes"],
                     a["scale"], rows=sel)
    return len(sel)


class OracleBaseline:
    """The oracle, as it stands, timed on the host beside the GPU run.

    Build, accept and the update run once in this process (one thread; they
    are a small part of the oracle's step).  Attention, nearly all of it,
    runs on a pool of worker processes (one thread each), one per host core
    up to 16, over randomly drawn (node, head) rows until about half of the
    time budget is spent; its time is scaled to all rows.  The pool is forked
    at construction, before the GPU is used."""

    def __init__(self, w, max_workers=16):
        import multiprocessing as mp

        import oracle as O
        from threadpoolctl import threadpool_limits

        self.w = w
        with threadpool_limits(limits=1):
            m_ids, m_scores = w.m_ids, w.m_scores
            if w.prompt is not None:
                m_ids, m_scores = O.update_adjacency(m_ids, m_scores, w.prompt[None],
                                                     np.array([len(w.prompt) - 2]))
            self.m_ids, self.m_scores = m_ids, m_scores
            t0 = time.perf_counter()
            self.tree = O.build_tree(w.cfg, w.draft_parent, w.draft_token, w.draft_conf,
                                     w.n_draft, w.root_token, w.prefix_len, m_ids)
            self.t_build = time.perf_counter() - t0
        f64 = lambda a: O.as_f64(a, w.dtype)
        _ORACLE_ARGS.update(
            arrays=[f64(w.q), f64(w.k_tree), f64(w.v_tree), f64(w.k_cache), f64(w.v_cache)],
            block_table=w.block_table, prefix_len=w.prefix_len, mask=self.tree["mask"],
            n_nodes=self.tree["n_nodes"], scale=w.scale)
        self.cores = max(1, min(max_workers, len(os.sched_getaffinity(0))))
        self.pool = mp.get_context("fork").Pool(self.cores, initializer=_oracle_worker_init)

    def run(self, budget_s=20.0):
        import oracle as O
        import workloads as W
        from threadpoolctl import threadpool_limits

        w, tree = self.w, self.tree
        rows = [(b, i, h) for b in range(w.B) for i in range(int(tree["n_nodes"][b]))
                for h in range(w.Hq)]
        order = np.random.default_rng(0).permutation(len(rows))
        chunk = 8
        done = 0
        t0 = time.perf_counter()
        while done < len(rows) and time.perf_counter() - t0 < budget_s / 2:
            wave = [[rows[k] for k in order[j:j + chunk]]
                    for j in range(done, min(len(rows), done + chunk * self.cores), chunk)]
            done += sum(self.pool.map(_oracle_attention_rows, wave, chunksize=1))
        t_attn = (time.perf_counter() - t0) * len(rows) / done
        self.pool.close()
        self.pool.join()
        with threadpool_limits(limits=1):
            logits = W.plant_path(w.logits, w.dtype, tree["token"], tree["parent"],
                                  tree["n_nodes"], w.plant_seed)
            t1 = time.perf_counter()
            acc = O.accept(logits, w.dtype, tree["token"], tree["parent"], tree["n_nodes"])
            t_acc = time.perf_counter() - t1
            t2 = time.perf_counter()
            O.update_adjacency(self.m_ids, self.m_scores, acc["path_tokens"], acc["accept_len"])
            t_upd = time.perf_counter() - t2
        step = self.t_build + t_attn + t_acc + t_upd
        tokens = int(tree["n_nodes"].sum())
        return {
            "value": tokens / step, "unit": "tokens/s", "cores": self.cores, "kind": "oracle",
            "sample": (f"one step of {w.name}: build, accept and update in full on one thread; "
                       f"attention on {done} of {len(rows)} randomly drawn (node, head) rows "
                       f"over {self.cores} worker processes (one thread each), its wall time "
                       f"scaled to all rows; numpy float64"),
            "seconds_per_step": step,
            "components_s": {"build": self.t_build, "attention": t_attn, "accept": t_acc,
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
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the attention timings at the other 8B-model shapes")
    ap.add_argument("--traffic-from-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    args = ap.parse_args()
    if args.traffic_from_pmc:
        traffic_from_pmc(args.config, *args.traffic_from_pmc)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import workloads as W

    log(f"generating workload {args.config}")
    w = W.make(args.config)
    # the oracle's worker processes fork here, before anything touches the GPU
    oracle = None if args.no_cpu_baseline else OracleBaseline(w)

    import torch

    from tree_attention_verification_graft_amd.binding import graft_version
    from tree_attention_verification_graft_amd.pipeline import to_host
    log(graft_version())
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()

    sets = make_sets(w, dev)
    n_sets = len(sets)
    log(f"{n_sets} rotating input sets of {set_bytes(sets[0]) / 2**20:.1f} MiB")
    # every set runs one whole step before anything is timed, so that every
    # output the timing reads (the node counts above all) was written
    for s in sets:
        s.step()
    torch.cuda.synchronize()
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
    # the tokens of exactly the steps replayed (every set was stepped above)
    n_nodes = np.stack([to_host(s.n_nodes) for s in sets])
    tokens = float(sum(n_nodes[k % n_sets].sum() for k in range(args.steps))) / args.steps
    value = tokens / (ms_per_step / 1e3)

    reps = max(1, args.steps // CALLS_PER_GRAPH)
    comp_us = {c: time_calls(sets, lambda s, c=c: getattr(s, c)(), reps, stream)
               for c in calls}

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
        next_us[name] = time_calls(sets, call, reps, stream)

    att = attention_figures(w, n_nodes[0], to_host(sets[0].tree_mask).view(np.uint32),
                            comp_us["attention"])
    e = 2 if w.dtype == "bf16" else 4
    logits_gbps = float(n_nodes[0].sum()) * w.V * e / (comp_us["accept"] / 1e6) / 1e9
    stream_gbps = streaming_read_gbps(dev, stream)
    del step_graphs, sets
    torch.cuda.empty_cache()
    log("next rows: " + ", ".join(f"{k} {v:.1f} us" for k, v in next_us.items()))
    log(f"step {ms_per_step * 1e3:.1f} us (eager {ms_eager * 1e3:.1f}); " +
        " ".join(f"{c} {comp_us[c]:.1f}" for c in calls) + " us; plan " + json.dumps(att["plan"]))

    # the attention call alone at the 8B-model shapes, where the KV read is
    # the bound, in the same process
    shapes_8b = {}
    for name in ATTN_8B_SHAPES:
        if name == w.name or args.no_extras:
            continue
        shapes_8b[name] = attention_only(name, dev, stream, reps)
        log(f"{name}: attention {shapes_8b[name]['attention_us']:.1f} us, "
            f"{shapes_8b[name]['achieved_GBps']:.0f} GB/s "
            f"({100 * shapes_8b[name]['frac']:.1f}% of HBM peak)")
    if w.name in ATTN_8B_SHAPES:
        shapes_8b[w.name] = {k: att[k] for k in ("attention_us", "achieved_GBps", "frac",
                                                  "kv_read_GBps", "plan")}

    mfma_bound = att["mfma_bound"]
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
        "tokens_per_step": tokens,
        "kv_read_GBps": att["kv_read_GBps"],
        "kv_read_pct_of_peak": 100.0 * att["kv_read_GBps"] / HBM_PEAK_GBPS,
        "torch_sum_read_GBps": stream_gbps,
        "logits_scan_GBps": logits_gbps,
        "attention_TFLOPs": att["TFLOPs"],
        "attention_plan": att["plan"],
        "components_us": comp_us,
        "roofline": {
            "kernel": ("attn_mfma_kernel" if att["plan"]["matrix_cores"] else "attn_wave_kernel")
                      + ("" if att["plan"]["n_splits"] == 1 else " + attn_combine_kernel"),
            "bound": "mfma" if mfma_bound else "hbm",
            "achieved": att["TFLOPs"] if mfma_bound else att["achieved_GBps"],
            "peak": MFMA_PEAK_TFLOPS if mfma_bound else HBM_PEAK_GBPS,
            "unit": "TFLOP/s" if mfma_bound else "GB/s",
            "frac": att["TFLOPs"] / MFMA_PEAK_TFLOPS if mfma_bound else att["frac"],
            "traffic": measured_traffic(w.name),
            "algorithmic_bytes_per_launch": att["bytes"],
            "algorithmic_flops_per_launch": att["flops"],
            "launch_us": comp_us["attention"],
        },
        "attention_8b_shapes": shapes_8b,
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
    if oracle is not None:
        log(f"timing the oracle on the host ({oracle.cores} worker processes)")
        result["cpu_baseline"] = oracle.run(args.cpu_budget)
    print(json.dumps(result), flush=True)


def set_bytes(s):
    return sum(x.numel() * x.element_size() for x in
               (s.q, s.k_tree, s.v_tree, s.k_cache, s.v_cache, s.logits))


def make_sets(w, dev, attention_only=False):
    """Device buffers of one workload, replicated into enough input sets that
    rotating through them exceeds the 256 MB Infinity Cache.  The first set
    seeds M from the prompt (if the workload has one) and plants an
    acceptable path into the stand-in logits; the copies share its draft
    inputs and M, and have their own q/K/V/logits and outputs."""
    import torch

    import workloads as W
    from tree_attention_verification_graft_amd.pipeline import DeviceStep

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
    rotated = ("q", "k_tree", "v_tree", "k_cache", "v_cache") + (() if attention_only
                                                                   else ("logits",))
    per_set = sum(getattr(base, k).numel() * getattr(base, k).element_size() for k in rotated)
    n_sets = max(1, math.ceil(ROTATE_BYTES / per_set))
    sets = [base]
    for _ in range(n_sets - 1):
        s = DeviceStep.__new__(DeviceStep)
        s.__dict__.update(base.__dict__)
        for k in rotated:
            setattr(s, k, getattr(base, k).clone())
        for k in ("tree_token", "tree_parent", "tree_pos", "tree_mask", "n_nodes", "stage",
                  "out", "argmax", "accept_len", "path_nodes", "path_tokens"):
            setattr(s, k, torch.zeros_like(getattr(base, k)))
        sets.append(s)
    return sets


def time_calls(sets, call, reps, stream):
    """Average duration of one call in microseconds: HIP events on the launch
    stream around `reps` replays of a graph that runs the call on
    CALLS_PER_GRAPH consecutive input sets."""
    import torch
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for k in range(CALLS_PER_GRAPH):
            call(sets[k % len(sets)])
    g.replay()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / (reps * CALLS_PER_GRAPH)


def attention_figures(w, n_nodes, masks, attention_us):
    """Bandwidth, matrix-core rate and roofline fraction of one attention call
    of `attention_us` microseconds."""
    from tree_attention_verification_graft_amd import binding as G
    kv_bytes, qo_bytes = attention_bytes(w, n_nodes)
    flops = attention_flops(w, n_nodes, masks)
    t = attention_us / 1e6
    achieved = (kv_bytes + qo_bytes) / t / 1e9
    dt = G.GRAFT_BF16 if w.dtype == "bf16" else G.GRAFT_F32
    plan = G.graft_tree_attention_plan(dt, w.B, w.n_max, w.Hq, w.Hkv, w.D, w.max_prefix,
                                       int(w.prefix_len.sum()))
    return {"attention_us": attention_us, "bytes": kv_bytes + qo_bytes, "flops": flops,
            "achieved_GBps": achieved, "frac": achieved / HBM_PEAK_GBPS,
            "kv_read_GBps": kv_bytes / t / 1e9, "TFLOPs": flops / t / 1e12,
            # the kernel's bound: matrix cores above the ridge point
            "mfma_bound": flops / (kv_bytes + qo_bytes) >
                          MFMA_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBPS * 1e9),
            "plan": plan}


def attention_only(name, dev, stream, reps):
    """The attention call of one workload, timed like the step's calls."""
    import torch

    import workloads as W
    from tree_attention_verification_graft_amd.pipeline import to_host
    w = W.make(name)
    sets = make_sets(w, dev, attention_only=True)
    for s in sets:
        s.build()
        s.attention()
    torch.cuda.synchronize()
    us = time_calls(sets, lambda s: s.attention(), reps, stream)
    att = attention_figures(w, to_host(sets[0].n_nodes),
                            to_host(sets[0].tree_mask).view(np.uint32), us)
    del sets
    torch.cuda.empty_cache()
    return {k: att[k] for k in ("attention_us", "achieved_GBps", "frac", "kv_read_GBps",
                                "TFLOPs", "plan")}


def streaming_read_gbps(dev, stream):
    """A reference streaming read on this GPU: torch's sum over 2 GiB (a
    plain reduction kernel; the logits scan of the accept call reads faster
    at large batches, so this is a reference, not a ceiling)."""
    import torch
    big = torch.ones(STREAM_BYTES // 4, dtype=torch.float32, device=dev)
    for _ in range(2):
        big.sum()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(5):
        big.sum()
    e1.record(stream)
    torch.cuda.synchronize()
    del big
    torch.cuda.empty_cache()
    return 5 * STREAM_BYTES / (e0.elapsed_time(e1) / 1e3) / 1e9


if __name__ == "__main__":
    main()
