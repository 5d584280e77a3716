"""GPU parity of sampling acceptance (temperature > 0) against the oracle.

The oracle works in float64 and reports, per sequence, how close its
decisions came to going the other way: margin_accept, the smallest
|u (1 - removed) - p(x)| over the child tests, and margin_bonus, the
distance of the bonus draw from the nearest boundary of its token's CDF
interval, relative to the residual mass.

The kernels' acceptance probabilities come from float32 exponentials
(relative error below about 1.5e-6, so |u (1 - removed) - p(x)| is off by at
most about 3e-6); the bonus masses are float64 throughout.  Where both
margins exceed MARGIN_ACCEPT and MARGIN_BONUS (an order of magnitude or more
above those errors) the decisions are unique and the outputs must match bit
for bit; otherwise both outcomes are correct, and the GPU's path is checked
for validity (a root path of the tree with its tokens, and a bonus token in
the vocabulary).  Ambiguous sequences must stay rare.
"""
import sys

import numpy as np
import pytest

import oracle as O
import workloads as W

pytestmark = pytest.mark.gpu

MARGIN_ACCEPT = 5e-5
MARGIN_BONUS = 1e-9


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _check_valid(b, parent, token, n_nodes, V, acc_len, path_nodes, path_tokens):
    L = int(acc_len[b])
    n = max(int(n_nodes[b]), 1)
    assert 0 <= L < n
    pn = path_nodes[b]
    assert pn[0] == 0 and (pn[L + 1:] == -1).all()
    for j in range(1, L + 1):
        assert 0 < pn[j] < n and int(parent[b, pn[j]]) == int(pn[j - 1])
    np.testing.assert_array_equal(path_tokens[b, :L + 1], token[b, pn[:L + 1]])
    assert 0 <= int(path_tokens[b, L + 1]) < V
    assert (path_tokens[b, L + 2:] == -1).all()


def compare(ref, got, parent, token, n_nodes, V, max_ambiguous_frac=0.05):
    """Bit-exact where the oracle's margins are above the bounds, valid
    elsewhere."""
    acc_len, path_nodes, path_tokens = got
    B = len(acc_len)
    amb = 0
    for b in range(B):
        _check_valid(b, parent, token, n_nodes, V, acc_len, path_nodes, path_tokens)
        if ref["margin_accept"][b] > MARGIN_ACCEPT and ref["margin_bonus"][b] > MARGIN_BONUS:
            assert int(acc_len[b]) == int(ref["accept_len"][b]), b
            np.testing.assert_array_equal(path_nodes[b], ref["path_nodes"][b])
            np.testing.assert_array_equal(path_tokens[b], ref["path_tokens"][b])
        else:
            amb += 1
            # the decisions before the first close one are certain: the paths
            # agree up to the node where it was taken, and all the way when
            # only the bonus draw is close (then only the bonus may differ)
            close = np.nonzero(ref["margin_by_depth"][b] <= MARGIN_ACCEPT)[0]
            d = int(close[0]) if len(close) else int(ref["accept_len"][b])
            np.testing.assert_array_equal(path_nodes[b, :d + 1], ref["path_nodes"][b, :d + 1])
            if not len(close):
                assert int(acc_len[b]) == int(ref["accept_len"][b]), b
                np.testing.assert_array_equal(path_nodes[b], ref["path_nodes"][b])
                np.testing.assert_array_equal(path_tokens[b, :d + 1],
                                              ref["path_tokens"][b, :d + 1])
    assert amb <= max(1, int(max_ambiguous_frac * B)), f"{amb} of {B} sequences ambiguous"
    return amb


def run_sample(logits, dtype, T, token, parent, n_nodes, ra, rs):
    """One graft_accept_sample call on the GPU; returns host outputs."""
    import torch
    from tree_attention_verification_graft_amd import binding as G
    from tree_attention_verification_graft_amd.pipeline import to_device, to_host
    B, n_max, V = logits.shape
    d = "cuda"
    lg = to_device(logits, d)
    i32 = torch.int32
    acc = torch.full((B,), -9, dtype=i32, device=d)
    pn = torch.full((B, n_max), -9, dtype=i32, device=d)
    pt = torch.full((B, n_max + 1), -9, dtype=i32, device=d)
    ws = torch.empty(max(G.graft_accept_sample_workspace_size(dtype, B, n_max, V), 256),
                     dtype=torch.uint8, device=d)
    G.graft_accept_sample(lg, T, to_device(token.astype(np.int32), d),
                          to_device(parent.astype(np.int32), d),
                          to_device(n_nodes.astype(np.int32), d), to_device(ra, d),
                          to_device(rs, d), acc, pn, pt, ws)
    torch.cuda.synchronize()
    return to_host(acc), to_host(pn), to_host(pt)


def oracle_sample(logits, dtype, T, token, parent, n_nodes, ra, rs):
    return O.accept_sample(logits, dtype, float(np.float32(T)), token, parent, n_nodes,
                           ra.astype(np.float64), rs.astype(np.float64))


# ----------------------------------------------------------------------------
# the five workloads at oracle size, trees from the build call
# ----------------------------------------------------------------------------

SMALL = {
    "tiny_f32": dict(),
    "llama3_8b_b1": dict(B=8, Hq=8, Hkv=2, prefix=(30, 90), V=4096),
    "qwen3_8b_b16": dict(B=16, Hq=8, Hkv=2, prefix=(40, 100), V=8192),
    "llama31_8b_64k": dict(B=4, Hq=8, Hkv=2, prefix=(300, 300), V=5000),
    "qwen3_235b_share": dict(B=6, Hq=32, Hkv=2, prefix=(100, 100), V=6000),
}


def _built_tree(w):
    import torch
    from tree_attention_verification_graft_amd.pipeline import DeviceStep
    ds = DeviceStep(w, alloc_update_for_prompt=w.prompt is not None)
    if w.prompt is not None:
        ds.seed_from_prompt(w.prompt)
    ds.build()
    torch.cuda.synchronize()
    return ds, ds.tree_host()


@pytest.mark.parametrize("name", W.CONFIG_ORDER)
@pytest.mark.parametrize("T", [0.6, 1.0, 1.7])
def test_small_variant(name, T):
    w = W.make(name, **SMALL[name])
    ds, t = _built_tree(w)
    n_max = ds.n_max
    amb = 0
    for rep in range(3):
        logits = W.plant_path(w.logits, w.dtype, t["token"], t["parent"], t["n_nodes"],
                              w.plant_seed + rep, boost=4.0)
        ra, rs = W.sampling_uniforms(100 * rep + int(10 * T), w.B, n_max)
        got = run_sample(logits, w.dtype, T, t["token"], t["parent"], t["n_nodes"], ra, rs)
        ref = oracle_sample(logits, w.dtype, T, t["token"], t["parent"], t["n_nodes"], ra, rs)
        amb += compare(ref, got, t["parent"], t["token"], t["n_nodes"], w.V)
    _say(f"[sample] {name} T={T}: ok, accept_len {got[0].tolist()[:8]}, ambiguous {amb}")


# ----------------------------------------------------------------------------
# random trees: repeated sibling tokens, ragged vocabularies, both dtypes,
# temperatures from near-greedy to flat
# ----------------------------------------------------------------------------

def _random_case(seed, B, n_max, V, dtype, boost, repeat_frac=0.3):
    rng = np.random.default_rng(seed)
    parent = np.full((B, n_max), -1, np.int32)
    token = np.zeros((B, n_max), np.int32)
    n_nodes = rng.integers(1, n_max + 1, B).astype(np.int32)
    n_nodes[0] = n_max
    for b in range(B):
        token[b, 0] = rng.integers(0, V)
        for i in range(1, int(n_nodes[b])):
            parent[b, i] = rng.integers(max(0, i - 6), i)  # deep, bushy trees
            sib = [int(token[b, j]) for j in range(1, i) if parent[b, j] == parent[b, i]]
            if sib and rng.random() < repeat_frac:
                token[b, i] = sib[int(rng.integers(len(sib)))]  # a repeated sibling
            else:
                token[b, i] = rng.integers(0, V)
    x = rng.standard_normal((B, n_max, V)).astype(np.float32) * 2.0
    # high mass on some children's tokens so that walks go deep
    for b in range(B):
        for i in range(1, int(n_nodes[b])):
            if rng.random() < 0.5:
                p = parent[b, i]
                x[b, p, token[b, i]] = x[b, p].max() + boost * rng.random()
    logits = W.f32_to_bf16_bits(x) if dtype == "bf16" else x
    return logits, token, parent, n_nodes


# A tree whose logits take at most 384 MiB (and whose rows' chunk records
# fit the staging area) is sampled in staged mode: statistics of every row,
# then one walk per workgroup.  A larger one, or a vocabulary past 2304
# chunks, takes lazy mode: the root's records, the walk reading each deeper
# row it reaches, and the residual and pick launches after a stop below the
# root.  (dtype, batch, n_max, vocab, temperature)
RANDOM = [
    # staged
    ("bf16", 12, 9, 1000, 1.0), ("bf16", 12, 65, 4103, 0.8), ("bf16", 12, 128, 20000, 1.3),
    ("f32", 12, 9, 999, 1.0), ("f32", 12, 65, 4096, 0.5), ("f32", 12, 128, 9001, 2.5),
    ("bf16", 12, 33, 70001, 0.05), ("f32", 12, 17, 3000, 0.05),
    # ... more than 8192 (row, chunk) pairs: statistics chunks of eight loads
    # per thread (16384 bf16 / 8192 f32 entries), the last one ragged
    ("bf16", 12, 128, 30000, 1.0), ("f32", 12, 128, 12001, 0.9),
    # lazy: rows ragged in the last chunk
    ("bf16", 96, 33, 70001, 1.0), ("f32", 72, 128, 12001, 0.9),
    # ... rows longer than one round of the walk's row pass (131072 bf16 /
    # 65536 f32 entries per round of sixteen 16-byte loads per thread), so
    # that a thread's running sum is rescaled when a later round raises its
    # max; the third takes the entry-at-a-time path over several rounds
    ("bf16", 28, 48, 151936, 0.7), ("f32", 48, 16, 140000, 1.0), ("bf16", 64, 24, 140001, 1.0),
    # ... deep walks at a low temperature
    ("bf16", 48, 65, 70001, 0.05),
    # ... and a vocabulary of more than 2304 chunks of 4096
    ("bf16", 2, 3, 2304 * 4096 + 1, 1.0),
]


def _lazy(dtype, B, n_max, V):
    e, per_chunk = (2, 4096) if dtype == "bf16" else (4, 2048)
    return B * n_max * V * e > 384 << 20 or -(-V // per_chunk) > 2304


@pytest.mark.parametrize("dtype,B,n_max,V,T", RANDOM,
                         ids=[f"{d}-B{b}-n{n}-V{v}-T{t}" for d, b, n, v, t in RANDOM])
def test_random_trees(dtype, B, n_max, V, T):
    amb = 0
    lazy = _lazy(dtype, B, n_max, V)
    for rep in range(1 if lazy else 2):
        logits, token, parent, n_nodes = _random_case(1000 * n_max + V + rep, B, n_max, V,
                                                      dtype, boost=6.0)
        ra, rs = W.sampling_uniforms(7 + rep, B, n_max)
        got = run_sample(logits, dtype, T, token, parent, n_nodes, ra, rs)
        ref = oracle_sample(logits, dtype, T, token, parent, n_nodes, ra, rs)
        amb += compare(ref, got, parent, token, n_nodes, V)
    _say(f"[sample] random {dtype} B={B} n_max={n_max} V={V} T={T} "
         f"{'lazy' if lazy else 'staged'}: ok, ambiguous {amb}")


# -inf logits (a masked vocabulary), staged and lazy
MASKED = [("bf16", 12, 33, 20000, 1.0), ("f32", 12, 17, 9001, 0.3),
          ("bf16", 24, 65, 140001, 1.0)]


@pytest.mark.parametrize("dtype,B,n_max,V,T", MASKED,
                         ids=[f"{d}-B{b}-n{n}-V{v}" for d, b, n, v, t in MASKED])
def test_masked_vocabulary(dtype, B, n_max, V, T):
    """Rows with -inf logits: 30% of the entries at random and a contiguous
    third of the row, so whole vocabulary chunks carry no mass, and some
    children proposing a masked token.  A masked token has probability 0:
    it is never accepted and never drawn as the bonus token."""
    x, token, parent, n_nodes = _random_case(4100 + V, B, n_max, V, "f32", boost=6.0)
    rng = np.random.default_rng(4200 + V)
    x[rng.random(x.shape) < 0.3] = -np.inf
    for b in range(B):
        for i in range(n_max):
            a = int(rng.integers(0, V - V // 3))
            x[b, i, a:a + V // 3] = -np.inf
            x[b, i, int(rng.integers(0, V))] = 1.0  # at least one finite entry
        for i in range(1, int(n_nodes[b])):
            if rng.random() < 0.2:
                x[b, parent[b, i], token[b, i]] = -np.inf
    logits = W.f32_to_bf16_bits(x) if dtype == "bf16" else x
    ra, rs = W.sampling_uniforms(31, B, n_max)
    got = run_sample(logits, dtype, T, token, parent, n_nodes, ra, rs)
    ref = oracle_sample(logits, dtype, T, token, parent, n_nodes, ra, rs)
    compare(ref, got, parent, token, n_nodes, V)
    acc_len, path_nodes, path_tokens = got
    for b in range(B):
        L = int(acc_len[b])
        for j in range(1, L + 1):  # every accepted token had mass in its parent's row
            assert np.isfinite(x[b, path_nodes[b, j - 1], path_tokens[b, j]]), b
        assert np.isfinite(x[b, path_nodes[b, L], path_tokens[b, L + 1]]), b  # the bonus too
    _say(f"[sample] masked {dtype} B={B} n_max={n_max} V={V}: ok, "
         f"{'lazy' if _lazy(dtype, B, n_max, V) else 'staged'}, "
         f"accept_len {acc_len.tolist()[:8]}")


# staged, and lazy by a vocabulary of more than 2304 chunks (then the root
# kernel's residual sums leave the rejected tokens out)
RESIDUAL = [("bf16", 8, 12, 30000), ("f32", 8, 12, 30000),
            ("bf16", 1, 12, 2304 * 4096 + 1), ("f32", 1, 12, 2304 * 2048 + 1)]


@pytest.mark.parametrize("dtype,B,n_max,V", RESIDUAL,
                         ids=[f"{d}-B{b}-V{v}" for d, b, n, v in RESIDUAL])
def test_rejected_mass_leaves_an_exact_residual(dtype, B, n_max, V):
    """The root's children carry almost all the mass and every one is
    rejected: the bonus is drawn from the small residual, whose chunks that
    held the rejected tokens are summed exactly."""
    rng = np.random.default_rng(5)
    parent = np.zeros((B, n_max), np.int32)
    parent[:, 0] = -1
    token = np.zeros((B, n_max), np.int32)
    x = rng.standard_normal((B, n_max, V)).astype(np.float32)
    for b in range(B):
        # spread the children over a few chunks, two sharing one chunk
        token[b, 1:] = rng.choice(V, n_max - 1, replace=False)
        token[b, 2] = token[b, 1] + 1 if token[b, 1] + 1 < V else token[b, 1] - 1
        x[b, 0, token[b, 1:]] = 14.0
    n_nodes = np.full(B, n_max, np.int32)
    ra = np.full((B, n_max), np.float32(0.99999), np.float32)
    _, rs = W.sampling_uniforms(11, B, n_max)
    logits = W.f32_to_bf16_bits(x) if dtype == "bf16" else x
    got = run_sample(logits, dtype, 1.0, token, parent, n_nodes, ra, rs)
    ref = oracle_sample(logits, dtype, 1.0, token, parent, n_nodes, ra, rs)
    assert (ref["accept_len"] == 0).all()
    compare(ref, got, parent, token, n_nodes, V)
    for b in range(B):  # the bonus is never a rejected token
        assert int(got[2][b, 1]) not in set(token[b, 1:].tolist())


@pytest.mark.parametrize("B,V", [(6, 4099), (2, 2304 * 4096 + 1)], ids=["staged", "lazy"])
def test_root_only_and_deterministic(B, V):
    """Root-only trees sample the bonus by inverse CDF; two calls agree."""
    n_max = 5
    logits, token, parent, _ = _random_case(77, B, n_max, V, "bf16", boost=3.0)
    n_nodes = np.ones(B, np.int32)
    ra, rs = W.sampling_uniforms(3, B, n_max)
    a = run_sample(logits, "bf16", 0.9, token, parent, n_nodes, ra, rs)
    b = run_sample(logits, "bf16", 0.9, token, parent, n_nodes, ra, rs)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)
    ref = oracle_sample(logits, "bf16", 0.9, token, parent, n_nodes, ra, rs)
    assert (a[0] == 0).all()
    compare(ref, a, parent, token, n_nodes, V)


# ----------------------------------------------------------------------------
# full-size workloads, in the launch configuration the benchmark times
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("name", W.CONFIG_ORDER)
def test_full_size(name):
    w = W.make(name)
    ds, t = _built_tree(w)
    logits = W.plant_path(w.logits, w.dtype, t["token"], t["parent"], t["n_nodes"],
                          w.plant_seed, boost=5.0)
    ra, rs = W.sampling_uniforms(42, w.B, ds.n_max)
    got = run_sample(logits, w.dtype, 1.0, t["token"], t["parent"], t["n_nodes"], ra, rs)
    ref = oracle_sample(logits, w.dtype, 1.0, t["token"], t["parent"], t["n_nodes"], ra, rs)
    amb = compare(ref, got, t["parent"], t["token"], t["n_nodes"], w.V)
    _say(f"[sample] {name} full size: ok, accept_len {got[0].tolist()[:8]}, ambiguous {amb}")


# ----------------------------------------------------------------------------
# seeded random shapes (tests/random_shapes.py): every third case, from the
# second on, trees from the build call
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("case", range(1, 24, 3))
def test_random_shape(case):
    import random_shapes as R
    w = R.make_case(case)
    ds, t = _built_tree(w)
    logits = W.plant_path(w.logits, w.dtype, t["token"], t["parent"], t["n_nodes"],
                          w.plant_seed, boost=4.0)
    ra, rs = W.sampling_uniforms(500 + case, w.B, ds.n_max)
    got = run_sample(logits, w.dtype, 1.0, t["token"], t["parent"], t["n_nodes"], ra, rs)
    ref = oracle_sample(logits, w.dtype, 1.0, t["token"], t["parent"], t["n_nodes"], ra, rs)
    amb = compare(ref, got, t["parent"], t["token"], t["n_nodes"], w.V)
    _say(f"[sample] random case {case}: ok, accept_len {got[0].tolist()[:8]}, ambiguous {amb}")
