"""graft_tree_attention_noalloc (library-held scratch, no caller workspace)
against graft_tree_attention (caller workspace) on the same inputs: the same
kernels and launch plan, so the outputs must agree bit for bit.  Two calls in
a row on one GPU, the second with a smaller input, so that the second runs on
scratch the first left behind."""
import sys

import numpy as np
import pytest

import workloads as W

pytestmark = pytest.mark.gpu

CASES = [
    # 64k-token prefix of one sequence: 32 prefix splits, ~4 MB of partials
    ("llama31_8b_64k", dict(Hq=8, Hkv=2, V=2048)),
    # then a smaller, ragged batch with fewer splits
    ("qwen3_8b_b16", dict(B=5, Hq=8, Hkv=2, prefix_list=[300, 1500, 64, 0, 777], V=2048)),
]


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def test_noalloc_matches_workspace_call_twice():
    import torch
    from tree_attention_verification_graft_amd import binding as G
    from tree_attention_verification_graft_amd.pipeline import DeviceStep
    for name, over in CASES:
        w = W.make(name, **over)
        plan = G.graft_tree_attention_plan(G.GRAFT_BF16, w.B, w.n_max, w.Hq, w.Hkv, w.D,
                                           w.max_prefix, int(w.prefix_len.sum()))
        _say(f"[noalloc] {name} B={w.B} P={w.prefix_len.tolist()} plan {plan}")
        assert plan["n_splits"] > 1  # the scratch holds split partials
        ds = DeviceStep(w)
        ds.build()
        ds.out.zero_()
        ds.attention()
        ref = ds.out.clone()
        got = torch.zeros_like(ds.out)
        G.graft_tree_attention_noalloc(ds.q, ds.k_tree, ds.v_tree, ds.k_cache, ds.v_cache,
                                       ds.block_table, ds.prefix_len, w.max_prefix,
                                       ds.tree_mask, ds.n_nodes, w.scale, got,
                                       sum_prefix=ds.sum_prefix)
        torch.cuda.synchronize()
        same = torch.equal(ref.view(torch.int16), got.view(torch.int16))
        _say(f"[noalloc] {name}: bit-identical to the workspace call: {same}")
        assert same
        del ds, ref, got
