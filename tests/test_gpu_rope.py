"""GPU parity of the rotary embedding fused into the verification attention
and the commit, against the oracle on the same seeded inputs.

q and k_tree hold unrotated projections; each node is rotated at its tree
position (prefix + depth) with the workload's float32 cos|sin table.
Attention: the same bar as the unrotated call, max(|got - ref| - r |ref|)
within 1e-2 for bf16 and 1e-4 for fp32 (r the output rounding); on the
matrix-core path the rotated bf16 queries and keys are rounded once to bf16
before the dot products, which the bar absorbs.  Commit: values bit-exact,
committed keys within one unit in the last place of the cache type of the
exactly rotated value (the kernel rotates in fp32, then rounds once), every
other slot untouched.
"""
import sys

import numpy as np
import pytest

import oracle as O
import workloads as W

pytestmark = pytest.mark.gpu

TOL = {"bf16": 1e-2, "f32": 1e-4}
OUT_ROUND = {"bf16": 2.0 ** -9, "f32": 2.0 ** -24}

SMALL = {
    "tiny_f32": dict(),
    "llama3_8b_b1": dict(B=2, Hq=8, Hkv=2, prefix_list=[300, 777], V=4096),
    "qwen3_8b_b16": dict(B=6, Hq=8, Hkv=2, prefix=(40, 700), V=8192),
    "llama31_8b_64k": dict(Hq=8, Hkv=2, prefix=(3000, 3000), V=5000),
    "qwen3_235b_share": dict(B=3, Hq=32, Hkv=2, prefix=(500, 500), V=6000),
}
EDGE = {
    "prefix_edges": ("qwen3_8b_b16", dict(B=5, Hq=8, Hkv=2, prefix_list=[0, 1, 16, 64, 65],
                                          V=2048)),
    "few_rows_bf16": ("llama3_8b_b1", dict(B=2, Hq=8, Hkv=2, kmax=2, stage_k_ret=[1, 1, 0],
                                           n_draft=4, prefix_list=[129, 300], V=512)),
    "max_tree": ("qwen3_8b_b16", dict(B=2, Hq=8, Hkv=4, kmax=127, stage_k_ret=[64, 32, 0],
                                      n_draft=256, prefix_list=[90, 1000], V=3000)),
    "f32_d128": ("tiny_f32", dict(D=128, V=999, prefix=(77, 77))),
    "group16_long": ("qwen3_235b_share", dict(B=2, Hq=32, Hkv=2, prefix_list=[2500, 4100],
                                              V=3000)),
    # 264 work items on 256 persistent workgroups (a partial last round)
    "persistent_partial_round": ("qwen3_8b_b16", dict(B=3, Hq=16, Hkv=4, kmax=32,
                                                      stage_k_ret=[16, 8, 0], n_draft=32,
                                                      prefix=(2048, 2048), V=2048)),
    # one row group of 17 blocks, split 0 with 0, 1 and 2 prefix tiles
    "three_block_short_prefixes": ("qwen3_8b_b16", dict(B=6, Hq=32, Hkv=8,
                                                        prefix_list=[3000, 3000, 0, 64, 100,
                                                                     3000], V=2048)),
    # two row groups of 9 and 8 blocks, split 0 with 0 to 3 prefix tiles
    "two_block_short_prefixes": ("qwen3_8b_b16", dict(B=6, Hq=32, Hkv=8,
                                                      prefix_list=[3000, 0, 64, 100, 2000, 130],
                                                      V=2048)),
}


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _f64(a, dtype):
    return O.as_f64(a, dtype)


def _step(w, plant=True):
    """Build the tree on the GPU, set the table, plant an acceptable path."""
    import torch
    from tree_attention_verification_graft_amd.pipeline import DeviceStep, to_device
    ds = DeviceStep(w, alloc_update_for_prompt=w.prompt is not None)
    if w.prompt is not None:
        ds.seed_from_prompt(w.prompt)
    ds.build()
    torch.cuda.synchronize()
    t = ds.tree_host()
    table = W.workload_rope_table(w)
    ds.set_rope(table)
    if plant:
        logits = W.plant_path(w.logits, w.dtype, t["token"], t["parent"], t["n_nodes"],
                              w.plant_seed)
        ds.logits.copy_(to_device(logits, "cuda"))
    return ds, t, table


def _check_attention_rope(w, ds, t, table, rows=None):
    from tree_attention_verification_graft_amd.pipeline import to_host
    got = _f64(to_host(ds.out), w.dtype)
    ref = O.tree_attention_rope(_f64(w.q, w.dtype), _f64(w.k_tree, w.dtype),
                                _f64(w.v_tree, w.dtype), _f64(w.k_cache, w.dtype),
                                _f64(w.v_cache, w.dtype), w.block_table, w.prefix_len,
                                t["mask"], t["n_nodes"], t["pos"], table, w.scale, rows=rows)
    if rows is None:
        rows = [(b, i, h) for b in range(w.B) for i in range(int(t["n_nodes"][b]))
                for h in range(w.Hq)]
    err = max(float(np.abs(got[b, i, h] - ref[b, i, h]).max()) for (b, i, h) in rows)
    excess = max(float((np.abs(got[b, i, h] - ref[b, i, h])
                        - OUT_ROUND[w.dtype] * np.abs(ref[b, i, h])).max())
                 for (b, i, h) in rows)
    assert np.isfinite(err) and excess <= TOL[w.dtype], (
        f"attention max-abs {err} (beyond output rounding: {excess})")
    return err


def _check_commit(w, ds, table):
    """The cache after graft_append_kv_rope against the oracle's commit."""
    from tree_attention_verification_graft_amd.pipeline import to_host
    acc = to_host(ds.accept_len)
    pn = to_host(ds.path_nodes)
    ref_k, ref_v, ref_len = O.append_kv_rope(_f64(w.k_cache, w.dtype), w.v_cache, w.block_table,
                                             w.prefix_len, _f64(w.k_tree, w.dtype), w.v_tree,
                                             pn, acc, table)
    np.testing.assert_array_equal(to_host(ds.new_prefix_len), ref_len)
    assert np.array_equal(to_host(ds.v_cache), ref_v), "v_cache after the commit"
    got_k = _f64(to_host(ds.k_cache), w.dtype)
    blk = w.k_cache.shape[2]
    committed = np.zeros(got_k.shape, bool)
    for b in range(w.B):
        for j in range(int(acc[b]) + 1):
            tok = int(w.prefix_len[b]) + j
            committed[int(w.block_table[b, tok // blk]), :, tok % blk, :] = True
    # untouched slots keep their bits
    assert np.array_equal(got_k[~committed], ref_k[~committed]), "k_cache outside the commit"
    # committed keys: the exact rotation, rounded once (half a unit in the
    # last place), plus the fp32 arithmetic on inputs of magnitude <= ~6
    bits = 8 if w.dtype == "bf16" else 24
    r = ref_k[committed]
    ulp = np.ldexp(1.0, np.frexp(np.abs(r))[1] - bits)
    bad = np.abs(got_k[committed] - r) > ulp + 1e-6
    assert not bad.any(), f"{int(bad.sum())} committed key entries beyond one ulp"
    return int(acc.max())


def _run(w, rows=None):
    import torch
    ds, t, table = _step(w)
    ds.attention_rope()
    torch.cuda.synchronize()
    err = _check_attention_rope(w, ds, t, table, rows)
    ds.accept()
    ds.append_rope()
    torch.cuda.synchronize()
    L = _check_commit(w, ds, table)
    _say(f"[rope] {w.name}: attention max-abs {err:.2e}, commit ok (longest path {L})")


@pytest.mark.parametrize("name", W.CONFIG_ORDER)
def test_small_variant(name):
    _run(W.make(name, **SMALL[name]))


@pytest.mark.parametrize("label", list(EDGE))
def test_edge_case(label):
    name, over = EDGE[label]
    _run(W.make(name, **over))


def _sample_rows(w, n_nodes, n, seed):
    rng = np.random.default_rng(seed)
    rows = set()
    for b in range(w.B):
        rows.add((b, int(n_nodes[b]) - 1, int(rng.integers(w.Hq))))
    while len(rows) < n:
        b = int(rng.integers(w.B))
        rows.add((b, int(rng.integers(int(n_nodes[b]))), int(rng.integers(w.Hq))))
    return sorted(rows)


@pytest.mark.parametrize("name", W.CONFIG_ORDER)
def test_full_size(name):
    """Full sizes, in the launch configuration the benchmark times; attention
    on 48 sampled rows (the deepest node of every sequence among them)."""
    import torch
    w = W.make(name)
    ds, t, table = _step(w)
    ds.attention_rope()
    torch.cuda.synchronize()
    rows = _sample_rows(w, t["n_nodes"], 48, 11)
    err = _check_attention_rope(w, ds, t, table, rows)
    ds.accept()
    ds.append_rope()
    torch.cuda.synchronize()
    L = _check_commit(w, ds, table)
    _say(f"[rope] {name} full size: attention max-abs {err:.2e}, commit ok (longest path {L})")


def test_unit_table_equals_the_unrotated_call():
    """With cos = 1 and sin = 0 everywhere the fused call is the plain one, bit
    for bit (the rotation in fp32 of a bf16 value times 1 is exact)."""
    import torch
    w = W.make("llama3_8b_b1", **SMALL["llama3_8b_b1"])
    ds, t, _ = _step(w, plant=False)
    table = np.zeros((int(w.max_prefix) + w.kmax + 2, w.D), np.float32)
    table[:, :w.D // 2] = 1.0
    ds.set_rope(table)
    ds.out.zero_()  # rows past n_nodes are not written
    ds.attention()
    torch.cuda.synchronize()
    plain = ds.out.clone()
    ds.out.zero_()
    ds.attention_rope()
    torch.cuda.synchronize()
    assert torch.equal(plain.view(torch.int16), ds.out.view(torch.int16))


# ----------------------------------------------------------------------------
# seeded random shapes (tests/random_shapes.py): every third case
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("case", range(0, 24, 3))
def test_random_shape(case):
    import random_shapes as R
    _run(R.make_case(case))
