"""GPU parity: the HIP path against the oracle on the same seeded inputs.

Bit-exact: hybrid trees (tokens, parents, positions, masks, node counts,
firing stage), argmax, accepted paths, the adjacency table after the
update, and the KV cache after the accepted path is committed.  Attention: max-abs error against the float64 oracle within 1e-2 for
bf16 inputs (fp32 accumulation, bf16 output) and 1e-4 for fp32.
"""
import sys

import numpy as np
import pytest

import oracle as O
import workloads as W

pytestmark = pytest.mark.gpu

# Attention tolerance: 1e-2 (bf16 inputs, fp32 accumulation) or 1e-4 (fp32)
# on top of the rounding of the output itself to its storage type, whose
# relative error is at most half a unit in the last place (2^-9 for bf16,
# 2^-24 for fp32).
TOL = {"bf16": 1e-2, "f32": 1e-4}
OUT_ROUND = {"bf16": 2.0 ** -9, "f32": 2.0 ** -24}


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _f64(a, dtype):
    return O.as_f64(a, dtype)


def oracle_tree(w, m_ids=None):
    return O.build_tree(w.cfg, w.draft_parent, w.draft_token, w.draft_conf, w.n_draft,
                        w.root_token, w.prefix_len, w.m_ids if m_ids is None else m_ids)


def check_tree(gpu, ref):
    nn = ref["n_nodes"]
    np.testing.assert_array_equal(gpu["n_nodes"], nn)
    np.testing.assert_array_equal(gpu["stage"], ref["stage"])
    np.testing.assert_array_equal(gpu["token"], ref["token"])
    np.testing.assert_array_equal(gpu["parent"], ref["parent"])
    np.testing.assert_array_equal(gpu["pos"], ref["pos"])
    np.testing.assert_array_equal(gpu["mask"], ref["mask"])


def check_attention(w, out_gpu, tree, rows=None, raw_bar=True):
    from tree_attention_verification_graft_amd.pipeline import to_host
    got = _f64(to_host(out_gpu), w.dtype)
    ref = O.tree_attention(_f64(w.q, w.dtype), _f64(w.k_tree, w.dtype), _f64(w.v_tree, w.dtype),
                           _f64(w.k_cache, w.dtype), _f64(w.v_cache, w.dtype), w.block_table,
                           w.prefix_len, tree["mask"], tree["n_nodes"], w.scale, rows=rows)
    if rows is None:
        rows = [(b, i, h) for b in range(w.B) for i in range(int(tree["n_nodes"][b]))
                for h in range(w.Hq)]
    err = max(float(np.abs(got[b, i, h] - ref[b, i, h]).max()) for (b, i, h) in rows)
    excess = max(float((np.abs(got[b, i, h] - ref[b, i, h])
                        - OUT_ROUND[w.dtype] * np.abs(ref[b, i, h])).max())
                 for (b, i, h) in rows)
    _say(f"[parity] attention on {len(rows)} rows: max-abs {err:.3e}, "
         f"beyond output rounding {excess:.3e} (bar {TOL[w.dtype]})")
    # the bar on the plain max-abs error, and the same bar on what is left
    # after the output's own rounding to its storage type
    assert np.isfinite(err), f"attention max-abs {err}"
    if raw_bar:
        assert err <= TOL[w.dtype], f"attention max-abs {err}"
    assert excess <= TOL[w.dtype], f"attention error beyond output rounding {excess}"
    return err


def run_full_check(w, attn_rows=None, seed_prompt=False, raw_bar=True):
    """Whole step on the GPU vs the oracle: build, attention, accept (with a
    planted path), update, and the commit of the accepted path to the cache."""
    import torch
    from tree_attention_verification_graft_amd.pipeline import DeviceStep, to_host
    _say(f"[parity] {w.name}: B={w.B} Hq={w.Hq} Hkv={w.Hkv} D={w.D} "
         f"P={w.prefix_len.tolist()[:8]} kmax={w.kmax} V={w.V}")
    m_ids, m_scores = w.m_ids, w.m_scores
    if seed_prompt:
        m_ids, m_scores = O.update_adjacency(m_ids, m_scores, w.prompt[None],
                                             np.array([len(w.prompt) - 2]))
    ref_tree = oracle_tree(w, m_ids)
    logits = W.plant_path(w.logits, w.dtype, ref_tree["token"], ref_tree["parent"],
                          ref_tree["n_nodes"], w.plant_seed)
    ds = DeviceStep(w, logits=logits, alloc_update_for_prompt=seed_prompt)
    if seed_prompt:
        ds.seed_from_prompt(w.prompt)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(to_host(ds.m_ids), m_ids)
        np.testing.assert_array_equal(to_host(ds.m_scores), m_scores)
    ds.build()
    torch.cuda.synchronize()
    check_tree(ds.tree_host(), ref_tree)
    ds.attention()
    torch.cuda.synchronize()
    err = check_attention(w, ds.out, ref_tree, rows=attn_rows, raw_bar=raw_bar)
    ds.accept()
    torch.cuda.synchronize()
    ref_acc = O.accept(logits, w.dtype, ref_tree["token"], ref_tree["parent"],
                       ref_tree["n_nodes"])
    np.testing.assert_array_equal(to_host(ds.argmax), ref_acc["argmax"])
    np.testing.assert_array_equal(to_host(ds.accept_len), ref_acc["accept_len"])
    np.testing.assert_array_equal(to_host(ds.path_nodes), ref_acc["path_nodes"])
    np.testing.assert_array_equal(to_host(ds.path_tokens), ref_acc["path_tokens"])
    ds.update()
    torch.cuda.synchronize()
    ref_ids, ref_sc = O.update_adjacency(m_ids, m_scores, ref_acc["path_tokens"],
                                         ref_acc["accept_len"])
    np.testing.assert_array_equal(to_host(ds.m_ids), ref_ids)
    np.testing.assert_array_equal(to_host(ds.m_scores), ref_sc)
    # commit of the accepted path to the cache (after attention has read it)
    ds.append()
    torch.cuda.synchronize()
    ref_k, ref_v, ref_len = O.append_kv(w.k_cache, w.v_cache, w.block_table, w.prefix_len,
                                        w.k_tree, w.v_tree, ref_acc["path_nodes"],
                                        ref_acc["accept_len"])
    np.testing.assert_array_equal(to_host(ds.new_prefix_len), ref_len)
    assert np.array_equal(to_host(ds.k_cache), ref_k), "k_cache after the commit"
    assert np.array_equal(to_host(ds.v_cache), ref_v), "v_cache after the commit"
    _say(f"[parity] {w.name}: ok, attention max-abs {err:.2e}, "
         f"accept_len {ref_acc['accept_len'].tolist()[:8]}")
    return ds


# ----------------------------------------------------------------------------
# oracle-sized variants of the five workloads (several tiles, ragged tails)
# ----------------------------------------------------------------------------

SMALL = {
    "tiny_f32": dict(),
    "llama3_8b_b1": dict(B=2, Hq=8, Hkv=2, prefix_list=[300, 777], V=4096),
    "qwen3_8b_b16": dict(B=6, Hq=8, Hkv=2, prefix=(40, 700), V=8192),
    "llama31_8b_64k": dict(Hq=8, Hkv=2, prefix=(3000, 3000), V=5000),
    "qwen3_235b_share": dict(B=3, Hq=32, Hkv=2, prefix=(500, 500), V=6000),
}


@pytest.mark.parametrize("name", W.CONFIG_ORDER)
def test_small_variant(name):
    w = W.make(name, **SMALL[name])
    run_full_check(w, seed_prompt=w.prompt is not None)


EDGE = [
    # empty prefixes, a one-token prefix, exact page/tile boundaries
    ("prefix_edges", "qwen3_8b_b16", dict(B=5, Hq=8, Hkv=2, prefix_list=[0, 1, 16, 64, 65],
                                          V=2048)),
    # no drafts at all (pure retrieval) and single-draft sequences
    ("no_drafts", "llama3_8b_b1", dict(B=3, Hq=8, Hkv=2, prefix_list=[100, 200, 5],
                                       n_draft_list=[0, 1, 60], V=1024)),
    # bf16 with head_dim 64 takes the wavefront path at any row count (244
    # query rows per KV head here)
    ("bf16_head_dim_64", "llama3_8b_b1", dict(B=2, Hq=8, Hkv=2, D=64, prefix_list=[300, 1000],
                                              V=2048)),
    # fewer than 16 query rows: bf16 takes the wavefront path
    ("few_rows_bf16", "llama3_8b_b1", dict(B=2, Hq=8, Hkv=2, kmax=2, stage_k_ret=[1, 1, 0],
                                          n_draft=4, prefix_list=[129, 300], V=512)),
    # the largest tree: kmax 127 (4 mask words), 256 drafts, 4-row groups
    ("max_tree", "qwen3_8b_b16", dict(B=2, Hq=8, Hkv=4, kmax=127, stage_k_ret=[64, 32, 0],
                                      n_draft=256, prefix_list=[90, 1000], V=3000)),
    # vocab not a multiple of 8 (scalar argmax loads), fp32 head dim 128
    ("odd_vocab_f32", "tiny_f32", dict(D=128, V=999, prefix=(77, 77))),
    # a long prefix over one KV head: more than 32 prefix splits to combine
    ("many_splits", "llama3_8b_b1", dict(B=1, Hq=4, Hkv=1, kmax=16, stage_k_ret=[8, 4, 0],
                                         n_draft=16, prefix_list=[20000], V=2048)),
    # over 8192 output rows merged from a few splits, a row count that is not
    # a multiple of four, ragged prefixes (some sequences use fewer splits)
    ("combine_rows", "qwen3_8b_b16", dict(B=5, Hq=30, Hkv=6, prefix_list=[1500, 200, 700, 64,
                                                                         1499], V=2048)),
    # GQA group 16 with several row groups and a split prefix
    ("group16_long", "qwen3_235b_share", dict(B=2, Hq=32, Hkv=2, prefix_list=[2500, 4100],
                                              V=3000)),
    # a uniform plan with more work items than compute units and a partial
    # last round: 3 row groups x 7 splits over 12 KV streams pad to 264 items
    # on 256 persistent workgroups, 8 of which run a second item
    ("persistent_partial_round", "qwen3_8b_b16", dict(B=3, Hq=16, Hkv=4, kmax=32,
                                                      stage_k_ret=[16, 8, 0], n_draft=32,
                                                      prefix=(2048, 2048), V=2048)),
    # 65 nodes x group 4 in one row group of 17 blocks (three-block waves) with
    # seven prefix splits: split 0 of the short sequences holds 0, 1 and 2
    # prefix tiles, so their tree tiles go out from the ring's prologue
    ("three_block_short_prefixes", "qwen3_8b_b16", dict(B=6, Hq=32, Hkv=8,
                                                        prefix_list=[3000, 3000, 0, 64, 100,
                                                                     3000], V=2048)),
    # the same with two row groups of 9 and 8 blocks (two-block waves)
    ("two_block_short_prefixes", "qwen3_8b_b16", dict(B=6, Hq=32, Hkv=8,
                                                      prefix_list=[3000, 0, 64, 100, 2000, 130],
                                                      V=2048)),
]


@pytest.mark.parametrize("label,name,over", EDGE, ids=[e[0] for e in EDGE])
def test_edge_case(label, name, over):
    w = W.make(name, **over)
    run_full_check(w)


def test_update_reuses_one_workspace_and_is_deterministic():
    """Updates from the same state give bit-identical tables, and one
    zero-filled workspace serves successive calls of different sizes without
    being cleared (each call matches the oracle).  The sizes cover both the
    per-step path (at most 4096 transitions) and the hash-table path, and the
    Zipf-drawn paths give hub rows with more new successors than one wave
    holds next to the row's S entries."""
    import torch
    from tree_attention_verification_graft_amd import binding as G
    from tree_attention_verification_graft_amd.pipeline import to_device, to_host
    rng = np.random.default_rng(3)
    V, S = 500, 8
    ids, sc = W.synth.seeded_adjacency(rng, V, S, W.Zipf(V))
    ws = torch.zeros(G.graft_update_adjacency_workspace_size(80, 66), dtype=torch.uint8,
                     device="cuda")
    results = {}
    for rep, (n_paths, stride) in enumerate([(40, 66), (40, 66), (7, 20), (80, 66), (40, 66),
                                             (1, 2), (80, 66)]):
        prng = np.random.default_rng(100 + n_paths)
        paths = W.Zipf(V).draw(prng, (n_paths, stride)).astype(np.int32)
        acc = prng.integers(-1, stride - 1, n_paths).astype(np.int32)
        d_ids, d_sc = to_device(ids, "cuda"), to_device(sc, "cuda")
        G.graft_update_adjacency(d_ids, d_sc, to_device(paths, "cuda"), to_device(acc, "cuda"),
                                 ws)
        torch.cuda.synchronize()
        got = (to_host(d_ids), to_host(d_sc))
        ref = O.update_adjacency(ids, sc, paths, acc)
        np.testing.assert_array_equal(got[0], ref[0])
        np.testing.assert_array_equal(got[1], ref[1])
        if (n_paths, stride) in results:
            prev = results[(n_paths, stride)]
            assert (prev[0] == got[0]).all() and (prev[1] == got[1]).all()
        results[(n_paths, stride)] = got


def test_attention_is_deterministic():
    import torch
    from tree_attention_verification_graft_amd.pipeline import DeviceStep
    w = W.make("qwen3_8b_b16", B=4, Hq=8, Hkv=2, prefix=(300, 3000), V=1024)
    ds = DeviceStep(w)
    ds.build()
    ds.attention()
    a = ds.out.clone()
    ds.attention()
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), ds.out.view(torch.int16))


# ----------------------------------------------------------------------------
# full-size workloads, in the launch configuration the benchmark times;
# attention checked on sampled rows
# ----------------------------------------------------------------------------

def plan_rows(w, tree, n_full_seqs, seed):
    """Attention rows for a full-size check, chosen against the launch plan
    the call uses: every row of one KV head (h = b mod Hkv) for n_full_seqs
    sequences spread over the batch, one random row in every (sequence, KV
    head, row group) workgroup set of the plan (each such row's output merges
    every prefix split of its group), and the deepest node of every
    sequence.  Returns the rows and the plan, after asserting the coverage."""
    from tree_attention_verification_graft_amd import binding as G
    dt = G.GRAFT_BF16 if w.dtype == "bf16" else G.GRAFT_F32
    plan = G.graft_tree_attention_plan(dt, w.B, w.n_max, w.Hq, w.Hkv, w.D, w.max_prefix,
                                       int(w.prefix_len.sum()))
    _say(f"[parity] {w.name} plan: {plan}")
    Gq = w.Hq // w.Hkv
    # row groups: runs of 16-row blocks, the first (blocks mod groups) one
    # block longer (matrix-core plans); one group of all rows otherwise
    ng = plan["n_row_groups"]
    if plan["matrix_cores"]:
        blocks = -(-(w.n_max * Gq) // 16)
        lo, rem = divmod(blocks, ng)
        bounds = [16 * (g * lo + min(g, rem)) for g in range(ng + 1)]
    else:
        bounds = [0, plan["rows_per_group"]]
    assert max(b - a for a, b in zip(bounds, bounds[1:])) == plan["rows_per_group"]
    group_of = lambda r: max(g for g in range(ng) if bounds[g] <= r)
    rng = np.random.default_rng(seed)
    nn = [int(x) for x in tree["n_nodes"]]
    rows = set()
    full = sorted({round(k * (w.B - 1) / max(1, n_full_seqs - 1)) for k in range(n_full_seqs)})
    for b in full:
        h = b % w.Hkv
        rows.update((b, i, h * Gq + g) for i in range(nn[b]) for g in range(Gq))
    groups = set()
    for b in range(w.B):
        rows.add((b, nn[b] - 1, int(rng.integers(w.Hq))))
        for h in range(w.Hkv):
            for rg in range(ng):
                lo, hi = bounds[rg], min(bounds[rg + 1], nn[b] * Gq)
                if lo >= hi:
                    continue  # no rows of this sequence in the group
                groups.add((b, h, rg))
                r = int(rng.integers(lo, hi))
                rows.add((b, r // Gq, h * Gq + r % Gq))
    covered = {(b, h // Gq, group_of(i * Gq + h % Gq)) for (b, i, h) in rows}
    assert groups <= covered, "a workgroup set of the plan has no checked row"
    _say(f"[parity] {w.name}: {len(rows)} rows cover all {len(groups)} (sequence, KV head, "
         f"row group) sets x {plan['n_splits']} splits; every row of one KV head of "
         f"sequences {full}")
    return sorted(rows), plan


# sequences whose rows of one KV head are all checked at full size
FULL_SEQS = {"tiny_f32": 1, "llama3_8b_b1": 1, "qwen3_8b_b16": 16, "llama31_8b_64k": 1,
             "qwen3_235b_share": 4}


@pytest.mark.parametrize("name", W.CONFIG_ORDER)
def test_full_size(name):
    w = W.make(name)
    seed = w.prompt is not None
    m_ids = w.m_ids
    if seed:
        m_ids = O.update_adjacency(w.m_ids, w.m_scores, w.prompt[None],
                                   np.array([len(w.prompt) - 2]))[0]
    rows, _ = plan_rows(w, oracle_tree(w, m_ids), FULL_SEQS[name], 7)
    run_full_check(w, attn_rows=rows, seed_prompt=seed)


# The Llama-3-8B workload lists its retrieval budgets for d0/d1/d5 as
# 0/16/32; read literally (d0 -> 0) that contradicts the rule that an earlier
# stage gets more retrieval, so the workloads take (32, 16, 0).  The literal
# order runs here through the same calls: at oracle size with every stage
# outcome forced in turn, and at full size.
LITERAL_K_RET = [0, 16, 32]


def test_literal_k_ret_order_small():
    w = W.make("llama3_8b_b1", B=8, Hq=8, Hkv=2, prefix=(100, 900), V=4096, conf="forced",
               stage_k_ret=LITERAL_K_RET)
    ref = oracle_tree(w)
    assert sorted(set(ref["stage"].tolist())) == [-1, 0, 1, 2]
    run_full_check(w)


def test_literal_k_ret_order_full_size():
    w = W.make("llama3_8b_b1", stage_k_ret=LITERAL_K_RET)
    rows, _ = plan_rows(w, oracle_tree(w), 1, 11)
    run_full_check(w, attn_rows=rows)


UPDATE_TREE = [(n, SMALL[n]) for n in W.CONFIG_ORDER] + [
    # 1040 verified nodes: the per-step path with many rows per workgroup
    ("qwen3_8b_b16", dict(B=16, Hq=8, Hkv=2, prefix=(40, 300), V=4096)),
    # 4160 potential transitions, above the per-step path's 4096: the
    # hash-table path of the update
    ("qwen3_8b_b16", dict(B=64, Hq=4, Hkv=1, prefix=(20, 60), V=4096)),
]


@pytest.mark.parametrize("name,over", UPDATE_TREE,
                         ids=[f"{n}-{i}" for i, (n, _) in enumerate(UPDATE_TREE)])
def test_update_tree_small_variant(name, over):
    run_update_tree_check(W.make(name, **over))


def run_update_tree_check(w):
    """The all-node update on the GPU against the oracle, from the same M:
    every verified node's (token, argmax) transition."""
    import torch
    from tree_attention_verification_graft_amd.pipeline import DeviceStep, to_host
    m_ids, m_scores = w.m_ids, w.m_scores
    if w.prompt is not None:
        m_ids, m_scores = O.update_adjacency(m_ids, m_scores, w.prompt[None],
                                             np.array([len(w.prompt) - 2]))
    ref_tree = oracle_tree(w, m_ids)
    logits = W.plant_path(w.logits, w.dtype, ref_tree["token"], ref_tree["parent"],
                          ref_tree["n_nodes"], w.plant_seed)
    ds = DeviceStep(w, logits=logits, alloc_update_for_prompt=w.prompt is not None)
    if w.prompt is not None:
        ds.seed_from_prompt(w.prompt)
    ds.build()
    ds.accept()
    ds.update_tree()
    torch.cuda.synchronize()
    ref_acc = O.accept(logits, w.dtype, ref_tree["token"], ref_tree["parent"],
                       ref_tree["n_nodes"])
    ref_ids, ref_sc = O.update_adjacency_tree(m_ids, m_scores, ref_tree["token"],
                                              ref_acc["argmax"], ref_tree["n_nodes"])
    np.testing.assert_array_equal(to_host(ds.m_ids), ref_ids)
    np.testing.assert_array_equal(to_host(ds.m_scores), ref_sc)
    _say(f"[parity] {w.name}: all-node update ok "
         f"({int(ref_tree['n_nodes'].sum())} transitions)")


def test_prefix_sum_hint_only_steers_the_plan():
    """The host-side prefix-length sum picks the launch plan (a ragged batch
    gets more splits, launched longest first); any value, right or wrong,
    gives results within the bar."""
    import torch
    from tree_attention_verification_graft_amd import binding as G
    from tree_attention_verification_graft_amd.pipeline import DeviceStep
    w = W.make("qwen3_8b_b16", B=12, Hq=8, Hkv=2, prefix=(64, 2200), V=1024)
    ds = DeviceStep(w)
    ds.build()
    torch.cuda.synchronize()
    tree = ds.tree_host()
    true_sum = int(w.prefix_len.sum())
    for hint in (0, true_sum, 1, 12 * int(w.max_prefix)):
        n = G.graft_tree_attention_workspace_size(G.GRAFT_BF16, w.B, ds.n_max, w.Hq, w.Hkv,
                                                  w.D, w.max_prefix, hint)
        ws = torch.empty(max(n, 256), dtype=torch.uint8, device="cuda")
        ds.out.zero_()
        G.graft_tree_attention(ds.q, ds.k_tree, ds.v_tree, ds.k_cache, ds.v_cache,
                               ds.block_table, ds.prefix_len, w.max_prefix, ds.tree_mask,
                               ds.n_nodes, w.scale, ds.out, ws, sum_prefix=hint)
        torch.cuda.synchronize()
        err = check_attention(w, ds.out, tree)
        _say(f"[parity] prefix-sum hint {hint}: attention max-abs {err:.2e}")
