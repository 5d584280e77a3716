"""HIP-graph capture of one whole step (the benchmark replays such graphs).

The four calls only launch kernels (no memsets, no allocation, no host
synchronisation), so a step can be captured once and replayed.  Every
replay here starts from the same M and is checked bit for bit against the
eager step, with eager work and synchronisations between the replays.
"""
import numpy as np
import pytest

import workloads as W

pytestmark = pytest.mark.gpu


def _snapshot(ds):
    import torch
    names = ("tree_token", "tree_parent", "tree_pos", "tree_mask", "n_nodes", "stage",
             "argmax", "accept_len", "path_nodes", "path_tokens", "m_ids", "m_scores")
    snap = {k: getattr(ds, k).clone() for k in names}
    snap["out"] = ds.out.view(torch.int16).clone()
    return snap


@pytest.mark.parametrize("name,over", [
    ("qwen3_8b_b16", dict(B=4, Hq=8, Hkv=2, prefix=(300, 1500), V=4096)),
    ("llama31_8b_64k", dict(Hq=8, Hkv=2, prefix=(3000, 3000), V=3000)),
])
def test_step_graph_replays_match_eager(name, over):
    import torch
    from tree_attention_verification_graft_amd.pipeline import DeviceStep, to_device
    w = W.make(name, **over)
    ds = DeviceStep(w, alloc_update_for_prompt=True)
    if w.prompt is not None:
        ds.seed_from_prompt(w.prompt)
    m0 = (ds.m_ids.clone(), ds.m_scores.clone())
    # plant an acceptable path so that the update has transitions to apply
    ds.build()
    torch.cuda.synchronize()
    t = ds.tree_host()
    logits = W.plant_path(w.logits, w.dtype, t["token"], t["parent"], t["n_nodes"],
                          w.plant_seed)
    ds.logits.copy_(to_device(logits, "cuda"))

    def reset_state():
        ds.m_ids.copy_(m0[0])
        ds.m_scores.copy_(m0[1])

    reset_state()
    ds.out.zero_()  # rows past n_nodes are not written: compare them as zeros
    ds.step()
    torch.cuda.synchronize()
    ref = _snapshot(ds)
    assert int(ref["accept_len"].max()) >= 1

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ds.step()
    for rep in range(3):
        reset_state()
        for k in ("tree_token", "tree_parent", "tree_pos", "tree_mask", "argmax",
                  "accept_len", "path_nodes", "path_tokens"):
            getattr(ds, k).fill_(-7)
        ds.out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = _snapshot(ds)
        for k, v in ref.items():
            assert torch.equal(got[k], v), f"replay {rep}: {k} differs from the eager step"


def test_sampling_acceptance_graph_replays_match_eager():
    """Sampling acceptance (two launches, no memsets) captured once and
    replayed: every replay equals the eager call bit for bit."""
    import torch
    from tree_attention_verification_graft_amd.pipeline import DeviceStep, to_device
    w = W.make("qwen3_8b_b16", B=4, Hq=8, Hkv=2, prefix=(300, 900), V=5000)
    ds = DeviceStep(w)
    ds.build()
    torch.cuda.synchronize()
    t = ds.tree_host()
    logits = W.plant_path(w.logits, w.dtype, t["token"], t["parent"], t["n_nodes"],
                          w.plant_seed, boost=4.0)
    ds.logits.copy_(to_device(logits, "cuda"))
    ra, rs = W.sampling_uniforms(9, w.B, ds.n_max)
    ds.rand_accept.copy_(to_device(ra, "cuda"))
    ds.rand_sample.copy_(to_device(rs, "cuda"))
    ds.accept_sample(0.8)
    torch.cuda.synchronize()
    ref = [x.clone() for x in (ds.accept_len, ds.path_nodes, ds.path_tokens)]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ds.accept_sample(0.8)
    for rep in range(3):
        for x in (ds.accept_len, ds.path_nodes, ds.path_tokens):
            x.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(("accept_len", "path_nodes", "path_tokens"), ref,
                              (ds.accept_len, ds.path_nodes, ds.path_tokens)):
            assert torch.equal(a, b), f"replay {rep}: {name} differs from the eager call"
