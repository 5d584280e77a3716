"""Seeded synthetic inputs for the prune-then-graft step.

This module only draws random inputs with the shapes and distributions of the
five workloads (and of smaller test variants).  It holds none of the method's
arithmetic: it builds draft trees, the adjacency table's initial contents, KV
pages, queries and logits, and it plants an acceptable path into logits for a
tree that someone else has built.  Both the HIP path's tests and the oracle's
tests take their inputs from here.

Random generation: numpy PCG64; a workload with seed s draws each tensor from
its own child of SeedSequence(s), spawned in a fixed order, so tensors do not
depend on one another's sizes.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

TAU = 0.3            # pruning threshold at every checkpoint
STAGE_DEPTHS = [0, 1, 5]


# ----------------------------------------------------------------------------
# primitive draws
# ----------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (round to nearest even); returns uint16 bits."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounding = ((b >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((b + rounding) >> np.uint32(16)).astype(np.uint16)


def normal_bf16(rng, shape, std=1.0) -> np.ndarray:
    out = np.empty(shape, np.uint16)
    flat = out.reshape(-1)
    step = 1 << 24
    for s in range(0, flat.size, step):
        n = min(step, flat.size - s)
        flat[s:s + n] = f32_to_bf16_bits(
            rng.standard_normal(n, dtype=np.float32) * np.float32(std))
    return out


def normal_f32(rng, shape, std=1.0) -> np.ndarray:
    return (rng.standard_normal(shape, dtype=np.float32) * np.float32(std))


class Zipf:
    """Finite-support Zipf(a) over ids 0..V-1: P(id = k-1) is proportional to
    k^-a; drawn by inverting the cumulative distribution."""

    def __init__(self, V: int, a: float = 1.1):
        w = np.arange(1, V + 1, dtype=np.float64) ** (-a)
        self.cdf = np.cumsum(w) / w.sum()
        self.V = V

    def draw(self, rng, size):
        u = rng.random(size)
        return np.minimum(np.searchsorted(self.cdf, u, side="right"),
                          self.V - 1).astype(np.int32)


def seeded_adjacency(rng, V: int, S: int, zipf: Zipf):
    """Every row gets S distinct Zipf ids (rows with a repeat are redrawn) and
    scores S, S-1, ..., 1, so rows start sorted by descending score."""
    ids = zipf.draw(rng, (V, S))
    while True:
        srt = np.sort(ids, axis=1)
        bad = np.nonzero((srt[:, 1:] == srt[:, :-1]).any(axis=1))[0]
        if bad.size == 0:
            break
        ids[bad] = zipf.draw(rng, (bad.size, S))
    scores = np.tile(np.arange(S, 0, -1, dtype=np.float32), (V, 1))
    return ids.astype(np.int32), scores


def envelope(S: int, kmax: int):
    """Base-tree envelope in breadth-first order: the root gets S children
    (ranks 0..S-1), each of those 2 children (ranks 0, 1), every deeper slot
    one child (rank 0); stops once kmax slots exist.  Returns parent slot
    (-1 = root) and rank lists of length kmax."""
    parent, rank = [], []
    frontier = [-1]
    level = 0
    while len(parent) < kmax:
        fan = S if level == 0 else (2 if level == 1 else 1)
        nxt = []
        for p in frontier:
            for r in range(fan):
                if len(parent) == kmax:
                    break
                parent.append(p)
                rank.append(r)
                nxt.append(len(parent) - 1)
        frontier = nxt
        level += 1
    return parent, rank


def random_draft_tree(rng, n: int, max_tree_depth: int):
    """Parent of node i is uniform over the root (-1) and the earlier nodes
    whose tree depth (root = 0) is below max_tree_depth.  Returns parents and
    each node's tree depth (1 for children of the root)."""
    parent = np.empty(n, np.int32)
    tdepth = np.empty(n, np.int32)
    for i in range(n):
        elig = [-1] + [j for j in range(i) if tdepth[j] < max_tree_depth]
        p = elig[int(rng.integers(len(elig)))]
        parent[i] = p
        tdepth[i] = 1 if p < 0 else tdepth[p] + 1
    return parent, tdepth


def running_product_conf(rng, parent):
    """Confidence of a node = its parent's confidence times U(0,1) (the
    root's confidence is 1): a drafter's cumulative path probability."""
    conf = np.empty(len(parent), np.float32)
    u = rng.random(len(parent)).astype(np.float32)
    for i, p in enumerate(parent):
        conf[i] = u[i] * (np.float32(1.0) if p < 0 else conf[p])
    return conf


def force_outcome(rng, parent, tdepth, conf, outcome):
    """Shape confidences so that checkpoint `outcome` (an index into
    STAGE_DEPTHS, or None) is the first one whose best confidence is below
    TAU.  Levels are draft depths (tree depth - 1)."""
    conf = conf.copy()
    ddepth = tdepth - 1
    stop = len(STAGE_DEPTHS) if outcome is None else outcome
    for s in range(stop):
        at = np.nonzero(ddepth == STAGE_DEPTHS[s])[0]
        if at.size and conf[at].max() < TAU:
            j = at[int(rng.integers(at.size))]
            conf[j] = np.float32(TAU + (1 - TAU) * rng.random())
    if outcome is not None:
        at = np.nonzero(ddepth == STAGE_DEPTHS[outcome])[0]
        conf[at] = conf[at] * np.float32(0.25)
    return conf


# ----------------------------------------------------------------------------
# workloads
# ----------------------------------------------------------------------------

@dataclass
class Workload:
    name: str
    dtype: str                 # "f32" or "bf16" for q/k/v/logits
    B: int
    Hq: int
    Hkv: int
    D: int
    block: int
    kmax: int
    V: int
    S: int
    cfg: dict                  # tree config (kmax, stages, envelope)
    draft_parent: np.ndarray   # [B][n_draft_max] int32
    draft_token: np.ndarray
    draft_conf: np.ndarray     # float32
    n_draft: np.ndarray        # [B] int32
    root_token: np.ndarray     # [B]
    prefix_len: np.ndarray     # [B]
    block_table: np.ndarray    # [B][max_blocks] int32
    num_blocks: int
    m_ids: np.ndarray          # [V][S] int32
    m_scores: np.ndarray       # [V][S] float32
    prompt: np.ndarray | None  # long-context prompt that seeds M, or None
    q: np.ndarray              # [B][n_max][Hq][D] (f32 or bf16 bits)
    k_tree: np.ndarray         # [B][n_max][Hkv][D]
    v_tree: np.ndarray
    k_cache: np.ndarray        # [num_blocks][Hkv][block][D]
    v_cache: np.ndarray        # [num_blocks][Hkv][D][block]
    logits: np.ndarray         # [B][n_max][V] (f32 or bf16 bits), unplanted
    plant_seed: int
    extra: dict = field(default_factory=dict)

    @property
    def n_max(self) -> int:
        return self.kmax + 1

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    @property
    def max_prefix(self) -> int:
        return int(self.prefix_len.max()) if self.B else 0

    @property
    def max_blocks(self) -> int:
        return self.block_table.shape[1]


PRESETS = {
    # Tiny fp32 case.
    "tiny_f32": dict(dtype="f32", B=1, Hq=4, Hkv=1, D=64, prefix=(128, 128),
                     kmax=16, stage_k_ret=[8, 4, 0], V=1000, S=4, n_draft=16,
                     max_tree_depth=5, conf="uniform", logit_std=1.0,
                     table="identity", seed=1001, rope_base=10000.0),
    # Llama-3-8B verify layer, batch 1.
    "llama3_8b_b1": dict(dtype="bf16", B=1, Hq=32, Hkv=8, D=128,
                         prefix=(2048, 2048), kmax=60, stage_k_ret=[32, 16, 0],
                         V=128256, S=8, n_draft=60, max_tree_depth=8,
                         conf="product", logit_std=2.0, table="identity",
                         seed=1002, rope_base=500000.0),
    # Qwen3-8B batched verify: ragged prefixes, permuted pages.
    "qwen3_8b_b16": dict(dtype="bf16", B=16, Hq=32, Hkv=8, D=128,
                         prefix=(512, 4096), kmax=64, stage_k_ret=[32, 16, 0],
                         V=151936, S=8, n_draft=64, max_tree_depth=8,
                         conf="forced", logit_std=2.0, table="permuted",
                         seed=1003, rope_base=1000000.0),
    # Llama-3.1-8B long context; M seeded from the prompt.
    "llama31_8b_64k": dict(dtype="bf16", B=1, Hq=32, Hkv=8, D=128,
                           prefix=(65536, 65536), kmax=64,
                           stage_k_ret=[32, 16, 0], V=128256, S=8, n_draft=64,
                           max_tree_depth=8, conf="product", logit_std=2.0,
                           table="identity", seed=1004, seed_m_from_prompt=True,
                           rope_base=500000.0),
    # Qwen3-235B-A22B attention, one GPU's head share; includes the M update.
    "qwen3_235b_share": dict(dtype="bf16", B=32, Hq=64, Hkv=4, D=128,
                             prefix=(8192, 8192), kmax=64,
                             stage_k_ret=[32, 16, 0], V=151936, S=8,
                             n_draft=64, max_tree_depth=8, conf="product",
                             logit_std=2.0, table="identity", seed=1005,
                             rope_base=1000000.0),
}

# The order of the five workloads as they are listed for this method.
CONFIG_ORDER = ["tiny_f32", "llama3_8b_b1", "qwen3_8b_b16", "llama31_8b_64k",
                "qwen3_235b_share"]


def make(name: str, **overrides) -> Workload:
    """Build a preset workload, optionally with fields overridden (e.g. a
    smaller batch, prefix range or vocabulary for oracle-sized tests)."""
    spec = dict(PRESETS[name])
    spec.update(overrides)
    return make_from_spec(name, spec)


def make_from_spec(name: str, spec: dict) -> Workload:
    ss = np.random.SeedSequence(int(spec["seed"]))
    (r_pref, r_tree, r_tok, r_root, r_table, r_m, r_q, r_kt, r_vt, r_kc, r_vc,
     r_log, r_plant, r_prompt) = [np.random.Generator(np.random.PCG64(c))
                                  for c in ss.spawn(14)]
    dtype = spec["dtype"]
    B, Hq, Hkv, D = spec["B"], spec["Hq"], spec["Hkv"], spec["D"]
    block = spec.get("block", 16)
    kmax, V, S = spec["kmax"], spec["V"], spec["S"]
    n_max = kmax + 1
    zipf = Zipf(V)

    lo, hi = spec["prefix"]
    if lo == hi:
        prefix_len = np.full(B, lo, np.int32)
    else:
        prefix_len = r_pref.integers(lo, hi + 1, size=B).astype(np.int32)
    if "prefix_list" in spec:
        prefix_len = np.asarray(spec["prefix_list"], np.int32)

    # paged layout: each sequence owns the pages of its prefix plus room for
    # the n_max tokens a step can commit after verification
    reserve = int(spec.get("reserve", n_max))
    pages_per_seq = [max(1, -(-(int(p) + reserve) // block)) for p in prefix_len]
    max_blocks = max(pages_per_seq) if B else 1
    num_blocks = int(sum(pages_per_seq))
    phys = np.arange(num_blocks, dtype=np.int32)
    if spec.get("table") == "permuted":
        phys = r_table.permutation(num_blocks).astype(np.int32)
    block_table = np.full((B, max_blocks), -1, np.int32)
    o = 0
    for b in range(B):
        block_table[b, :pages_per_seq[b]] = phys[o:o + pages_per_seq[b]]
        o += pages_per_seq[b]

    # draft trees
    n_draft_max = spec["n_draft"]
    draft_parent = np.full((B, n_draft_max), -1, np.int32)
    draft_token = np.zeros((B, n_draft_max), np.int32)
    draft_conf = np.zeros((B, n_draft_max), np.float32)
    n_draft = np.zeros(B, np.int32)
    n_list = spec.get("n_draft_list")
    for b in range(B):
        n = n_draft_max if n_list is None else int(n_list[b])
        outcome = None
        if spec["conf"] == "forced":
            k = b % (len(STAGE_DEPTHS) + 1)
            outcome = None if k == len(STAGE_DEPTHS) else k
        while True:
            parent, tdepth = random_draft_tree(r_tree, n, spec["max_tree_depth"])
            need = 0 if outcome is None else STAGE_DEPTHS[outcome] + 1
            if n == 0 or tdepth.max() >= need:
                break
        if spec["conf"] == "uniform":
            conf = r_tree.random(n).astype(np.float32)
        else:
            conf = running_product_conf(r_tree, parent)
            if spec["conf"] == "forced":
                conf = force_outcome(r_tree, parent, tdepth, conf, outcome)
        draft_parent[b, :n] = parent
        draft_conf[b, :n] = conf
        draft_token[b, :n] = zipf.draw(r_tok, n)
        n_draft[b] = n

    prompt = None
    if spec.get("seed_m_from_prompt"):
        prompt = zipf.draw(r_prompt, int(prefix_len[0]))
        m_ids = np.full((V, S), -1, np.int32)
        m_scores = np.zeros((V, S), np.float32)
        root_token = np.full(B, prompt[-1], np.int32)
    else:
        m_ids, m_scores = seeded_adjacency(r_m, V, S, zipf)
        root_token = zipf.draw(r_root, B)

    env_parent, env_rank = envelope(S, kmax)
    cfg = dict(kmax=kmax, stage_depth=list(STAGE_DEPTHS),
               stage_tau=[TAU] * len(STAGE_DEPTHS),
               stage_k_ret=list(spec["stage_k_ret"]), k_ret_none=0,
               env_parent=env_parent, env_rank=env_rank)

    if dtype == "bf16":
        draw = normal_bf16
    else:
        draw = normal_f32
    q = draw(r_q, (B, n_max, Hq, D))
    k_tree = draw(r_kt, (B, n_max, Hkv, D))
    v_tree = draw(r_vt, (B, n_max, Hkv, D))
    k_cache = draw(r_kc, (num_blocks, Hkv, block, D))
    v_cache = draw(r_vc, (num_blocks, Hkv, D, block))
    logits = draw(r_log, (B, n_max, V), spec["logit_std"])

    return Workload(name=name, dtype=dtype, B=B, Hq=Hq, Hkv=Hkv, D=D,
                    block=block, kmax=kmax, V=V, S=S, cfg=cfg,
                    draft_parent=draft_parent, draft_token=draft_token,
                    draft_conf=draft_conf, n_draft=n_draft,
                    root_token=root_token, prefix_len=prefix_len,
                    block_table=block_table, num_blocks=num_blocks,
                    m_ids=m_ids, m_scores=m_scores, prompt=prompt, q=q,
                    k_tree=k_tree, v_tree=v_tree, k_cache=k_cache,
                    v_cache=v_cache, logits=logits,
                    plant_seed=int(r_plant.integers(1 << 31)), extra=dict(spec))


# ----------------------------------------------------------------------------
# stand-in target model: plant an acceptable path into the logits
# ----------------------------------------------------------------------------

def plant_path(logits: np.ndarray, dtype: str, tree_token, tree_parent,
               n_nodes, seed: int, boost: float = 1.0) -> np.ndarray:
    """Return a copy of logits in which, for each sequence, a seeded target
    node t is made acceptable: for every edge p -> c on the root path of t,
    row p's entry at token(c) becomes its row maximum plus `boost`.  Random
    logits alone would accept almost nothing; this plants a path of length
    depth(t) without touching how acceptance is decided (under sampling, a
    larger boost makes the planted tokens likely rather than certain)."""
    out = logits.copy()
    rng = np.random.default_rng(seed)
    B = out.shape[0]
    for b in range(B):
        n = int(n_nodes[b])
        if n <= 1:
            continue
        t = int(rng.integers(1, n))
        c = t
        while int(tree_parent[b, c]) >= 0:
            p = int(tree_parent[b, c])
            tok = int(tree_token[b, c])
            if dtype == "bf16":
                row = (out[b, p].astype(np.uint32) << np.uint32(16)).view(np.float32)
                top = np.float32(row.max()) + np.float32(boost)
                out[b, p, tok] = f32_to_bf16_bits(np.array([top], np.float32))[0]
            else:
                out[b, p, tok] = np.float32(out[b, p].max()) + np.float32(boost)
            c = p
    return out


def sampling_uniforms(seed: int, batch: int, n_max: int):
    """The random numbers of sampling acceptance, as float32 in [0, 1):
    rand_accept[b][i] (child i's test) and rand_sample[b][i] (node i's bonus
    draw)."""
    rng = np.random.default_rng(seed)
    ra = rng.random((batch, n_max), dtype=np.float32)
    rs = rng.random((batch, n_max), dtype=np.float32)
    return ra, rs


def rope_table(positions: int, head_dim: int, base: float) -> np.ndarray:
    """The caller-side rotary table [positions][head_dim] float32: row t holds
    cos(t w_i) for i < head_dim / 2, then sin(t w_i), with frequencies
    w_i = base^(-2 i / head_dim) (the published rotary embedding; angles in
    float64, rounded to float32 once).  Llama-3.1's long-context frequency
    rescaling would change only this table's contents."""
    h = head_dim // 2
    w = base ** (-2.0 * np.arange(h, dtype=np.float64) / head_dim)
    ang = np.arange(positions, dtype=np.float64)[:, None] * w[None, :]
    return np.concatenate([np.cos(ang), np.sin(ang)], axis=1).astype(np.float32)


def workload_rope_table(w) -> np.ndarray:
    """The rotary table of a workload: every position up to the longest
    prefix plus a whole tree."""
    base = PRESETS.get(w.name, {}).get("rope_base", 10000.0)
    return rope_table(int(w.max_prefix) + w.kmax + 2, w.D, base)
