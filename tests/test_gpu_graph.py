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
    """Sampling acceptance in staged mode (three launches, no memsets)
    captured once and replayed: every replay equals the eager call bit for
    bit."""
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


def test_lazy_sampling_graph_replays_match_eager():
    """Sampling acceptance in lazy mode (a vocabulary past the staging
    area: the root launch, the walk, then the residual and pick launches)
    captured once and replayed.  The batch mixes stops at the root (a
    root-only tree, and root children without mass), where the walk draws
    the bonus token, with deeper stops, which go through the last two
    launches; every replay equals the eager call bit for bit."""
    import torch
    from tree_attention_verification_graft_amd import binding as G
    from tree_attention_verification_graft_amd.pipeline import to_device
    B, n_max, V = 4, 6, 2304 * 4096 + 1
    rng = np.random.default_rng(31)
    x = rng.standard_normal((B, n_max, V), dtype=np.float32)
    parent = np.array([[-1, 0, 1, 2, 3, 0]] * B, np.int32)  # a chain and a root sibling
    token = rng.integers(0, V, (B, n_max)).astype(np.int32)
    n_nodes = np.array([n_max, 1, n_max, 3], np.int32)
    for b in (0, 2, 3):
        # the chain's tokens dominate their rows, except in sequence 3,
        # where the root's children carry no mass
        for c in range(1, int(n_nodes[b])):
            if b != 3 and parent[b, c] >= 0 and c != 5:
                x[b, parent[b, c], token[b, c]] = 60.0
    logits = W.f32_to_bf16_bits(x)
    ra, rs = W.sampling_uniforms(17, B, n_max)
    d = "cuda"
    lg = to_device(logits, d)
    args = [to_device(a, d) for a in (token, parent, n_nodes, ra, rs)]
    i32 = torch.int32
    acc = torch.full((B,), -9, dtype=i32, device=d)
    pn = torch.full((B, n_max), -9, dtype=i32, device=d)
    pt = torch.full((B, n_max + 1), -9, dtype=i32, device=d)
    ws = torch.empty(G.graft_accept_sample_workspace_size("bf16", B, n_max, V),
                     dtype=torch.uint8, device=d)

    def call():
        G.graft_accept_sample(lg, 1.0, *args, acc, pn, pt, ws)

    call()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (acc, pn, pt)]
    # the chain is accepted to its end in sequences 0 and 2, nothing at the
    # root of sequences 1 and 3
    assert ref[0].tolist() == [4, 0, 4, 0], ref[0].tolist()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for rep in range(3):
        for t in (acc, pn, pt):
            t.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(("accept_len", "path_nodes", "path_tokens"), ref, (acc, pn, pt)):
            assert torch.equal(a, b), f"replay {rep}: {name} differs from the eager call"
