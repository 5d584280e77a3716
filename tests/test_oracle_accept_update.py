"""Pins for the oracle's greedy acceptance and adjacency update (CPU only)."""
import json
import os
import random

import numpy as np
import pytest

import oracle as O
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ----------------------------------------------------------------------------
# acceptance
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_accept_golden(dtype):
    g = _load("accept_example.json")
    lg = np.array([[float(x) for x in row] for row in g["logits"]], np.float32)
    assert np.signbit(lg[5, 0]) and lg[5, 0] == 0.0
    if dtype == "bf16":
        lg = W.f32_to_bf16_bits(lg)  # every value is exact in bf16
    tok = np.array([g["tree_token"]], np.int32)
    par = np.array([g["tree_parent"]], np.int32)
    a = O.accept(lg[None], dtype, tok, par, np.array([6]))
    e = g["expect"]
    assert a["argmax"][0].tolist() == e["argmax"]
    assert int(a["accept_len"][0]) == e["accept_len"]
    assert a["path_nodes"][0, :4].tolist() == e["path_nodes"]
    assert (a["path_nodes"][0, 4:] == -1).all()
    assert a["path_tokens"][0, :5].tolist() == e["path_tokens"]
    assert (a["path_tokens"][0, 5:] == -1).all()


class TinyModel:
    """Deterministic random next-token model: logits depend on the last two
    tokens of the context."""

    def __init__(self, rng, V):
        self.A = rng.standard_normal((V, V)).astype(np.float32)
        self.B = rng.standard_normal((V + 1, V)).astype(np.float32)
        self.V = V

    def logits(self, ctx):
        prev2 = ctx[-2] if len(ctx) >= 2 else self.V
        return (self.A[ctx[-1]] + np.float32(0.5) * self.B[prev2]).astype(np.float32)

    def greedy(self, ctx, steps):
        ctx = list(ctx)
        out = []
        for _ in range(steps):
            t = int(np.argmax(self.logits(ctx)))
            out.append(t)
            ctx.append(t)
        return out


@pytest.mark.parametrize("seed", range(25))
def test_accept_equals_greedy_decoding_of_tiny_model(seed):
    """The emitted tokens equal what the target alone emits when decoding
    greedily step by step, and no tree path matches the greedy continuation
    deeper than the accepted length."""
    rng = np.random.default_rng(seed)
    V = 6
    model = TinyModel(rng, V)
    prefix = rng.integers(0, V, 5).tolist()
    n = int(rng.integers(1, 20))
    parent = [-1]
    token = [prefix[-1]]
    for i in range(1, n):
        p = int(rng.integers(0, i))
        parent.append(p)
        # walk the path of p to build its context
        path = []
        j = p
        while j > 0:
            path.append(token[j])
            j = parent[j]
        ctx = prefix + path[::-1]
        if rng.random() < 0.6:
            token.append(int(np.argmax(model.logits(ctx))))
        else:
            token.append(int(rng.integers(V)))
    logits = np.zeros((1, n, V), np.float32)
    paths = []
    for i in range(n):
        path = []
        j = i
        while j > 0:
            path.append(token[j])
            j = parent[j]
        path = path[::-1]
        paths.append(path)
        logits[0, i] = model.logits(prefix + path)
    a = O.accept(logits, "f32", np.array([token]), np.array([parent]), np.array([n]))
    L = int(a["accept_len"][0])
    greedy = model.greedy(prefix, L + 1)
    assert a["path_tokens"][0, 1:L + 2].tolist() == greedy
    assert a["path_tokens"][0, 0] == prefix[-1]
    # brute force: deepest node whose path equals the greedy continuation
    g_long = model.greedy(prefix, 25)
    best = max(len(p) for p in paths if p == g_long[:len(p)])
    assert L == best


@pytest.mark.parametrize("seed", range(25))
def test_accept_brute_force_over_paths(seed):
    """Random trees with planted matches: the accepted node is the deepest
    node all of whose path edges match the argmax of the parent row, ties to
    the lowest index."""
    rng = np.random.default_rng(50 + seed)
    V, n = 5, int(rng.integers(1, 30))
    parent = [-1] + [int(rng.integers(0, i)) for i in range(1, n)]
    logits = rng.standard_normal((1, n, V)).astype(np.float32)
    am = logits[0].argmax(1)
    token = [int(rng.integers(V))]
    for i in range(1, n):
        token.append(int(am[parent[i]]) if rng.random() < 0.7 else int(rng.integers(V)))
    a = O.accept(logits, "f32", np.array([token]), np.array([parent]), np.array([n]))
    best = None
    for i in range(n):
        j, ok, d = i, True, 0
        while parent[j] >= 0:
            ok &= token[j] == int(am[parent[j]])
            j = parent[j]
            d += 1
        if ok and (best is None or d > best[0]):
            best = (d, i)
    assert int(a["accept_len"][0]) == best[0]
    assert int(a["path_nodes"][0, best[0]]) == best[1]


def test_accept_chain_accepts_matched_prefix():
    V = 8
    tok = [3, 1, 2, 7, 4]
    logits = np.full((1, 5, V), -1.0, np.float32)
    for i, nxt in enumerate([1, 2, 0, 4, 5]):  # row 2 predicts 0, not 7
        logits[0, i, nxt] = 1.0
    a = O.accept(logits, "f32", np.array([tok]), np.array([[-1, 0, 1, 2, 3]]),
                 np.array([5]))
    assert int(a["accept_len"][0]) == 2
    assert a["path_tokens"][0, :4].tolist() == [3, 1, 2, 0]


def test_accept_lowest_index_ties_in_bf16():
    """Distinct fp32 values that round to the same bf16 value tie; the lower
    index wins.  Also -0 vs +0."""
    x = np.array([1.0, 1.00390625, 1.001953125, 0.5], np.float32)  # all -> 1.0 in bf16
    bits = W.f32_to_bf16_bits(x)
    assert len(set(bits.tolist()[:3])) == 1
    a = O.accept(bits[None, None], "bf16", np.array([[0]]), np.array([[-1]]), np.array([1]))
    assert int(a["argmax"][0, 0]) == 0
    z = np.array([0x8000, 0x0000, 0x8000], np.uint16)
    a = O.accept(z[None, None], "bf16", np.array([[0]]), np.array([[-1]]), np.array([1]))
    assert int(a["argmax"][0, 0]) == 0


# ----------------------------------------------------------------------------
# adjacency update
# ----------------------------------------------------------------------------

def test_update_golden():
    g = _load("update_example.json")
    ids, sc = O.update_adjacency(np.array(g["m_ids"], np.int32),
                                 np.array(g["m_scores"], np.float32),
                                 np.array(g["path_tokens"], np.int32),
                                 np.array(g["accept_len"], np.int32))
    assert ids.tolist() == g["expect_ids"]
    assert sc.tolist() == g["expect_scores"]


def _brute_update(ids, scores, paths, acc):
    """Independent formulation: literal list of transitions, list.count for
    multiplicities, repeated extraction of the best remaining candidate."""
    trans = []
    for p, L in zip(paths, acc):
        for k in range(int(L) + 1):
            trans.append((int(p[k]), int(p[k + 1])))
    ids = ids.copy()
    scores = scores.copy()
    V, S = ids.shape
    for u in sorted({t[0] for t in trans}):
        succ = [t[1] for t in trans if t[0] == u]
        cand = []
        for v in sorted(set(succ) | {int(x) for x in ids[u] if x >= 0}):
            old = [float(scores[u, s]) for s in range(S) if ids[u, s] == v]
            cand.append([v, (old[0] if old else 0.0) + succ.count(v)])
        chosen = []
        while cand and len(chosen) < S:
            top = cand[0]
            for c in cand[1:]:
                if c[1] > top[1] or (c[1] == top[1] and c[0] < top[0]):
                    top = c
            chosen.append(top)
            cand.remove(top)
        ids[u] = -1
        scores[u] = 0.0
        for s, (v, sc) in enumerate(chosen):
            ids[u, s] = v
            scores[u, s] = sc
    return ids, scores


@pytest.mark.parametrize("seed", range(20))
def test_update_matches_brute_force_and_is_order_free(seed):
    rng = np.random.default_rng(seed)
    V, S = 12, 3
    ids = np.full((V, S), -1, np.int32)
    scores = np.zeros((V, S), np.float32)
    for u in range(V):
        k = int(rng.integers(0, S + 1))
        ids[u, :k] = rng.permutation(V)[:k]
        scores[u, :k] = np.sort(rng.integers(1, 5, k))[::-1]
        # keep rows in the (score desc, id asc) order the table maintains
        order = sorted(range(k), key=lambda s: (-scores[u, s], ids[u, s]))
        ids[u, :k] = ids[u, order]
        scores[u, :k] = scores[u, order]
    n_paths, stride = 5, 8
    paths = rng.integers(0, V, (n_paths, stride)).astype(np.int32)
    acc = rng.integers(-1, stride - 1, n_paths).astype(np.int32)
    got = O.update_adjacency(ids, scores, paths, acc)
    ref = _brute_update(ids, scores, paths, acc)
    np.testing.assert_array_equal(got[0], ref[0])
    np.testing.assert_array_equal(got[1], ref[1])
    # the transitions of one call may come in any order
    trans = O.transitions(paths, acc)
    random.Random(seed).shuffle(trans)
    as_paths = np.array([[u, v] for u, v in trans] or np.zeros((0, 2)), np.int32)
    got2 = O.update_adjacency(ids, scores, as_paths, np.zeros(len(trans), np.int32))
    np.testing.assert_array_equal(got2[0], got[0])
    np.testing.assert_array_equal(got2[1], got[1])
    # rows stay sorted, ids distinct, untouched rows unchanged
    touched = {u for u, _ in trans}
    for u in range(V):
        row = [(float(s), int(i)) for i, s in zip(got[0][u], got[1][u]) if i >= 0]
        assert row == sorted(row, key=lambda x: (-x[0], x[1]))
        assert len({i for _, i in row}) == len(row)
        if u not in touched:
            assert (got[0][u] == ids[u]).all() and (got[1][u] == scores[u]).all()


def test_prompt_seeding_is_exact_top_bigrams():
    """Seeding an empty table from a prompt (as one path) yields, per token,
    the S most frequent next tokens with their exact counts (numpy unique)."""
    rng = np.random.default_rng(11)
    V, S, L = 300, 8, 5000
    prompt = W.Zipf(V).draw(rng, L)
    ids0 = np.full((V, S), -1, np.int32)
    sc0 = np.zeros((V, S), np.float32)
    ids, sc = O.update_adjacency(ids0, sc0, prompt[None], np.array([L - 2]))
    pairs = prompt[:-1].astype(np.int64) * V + prompt[1:]
    uniq, cnt = np.unique(pairs, return_counts=True)
    for u in range(V):
        sel = (uniq // V) == u
        vs, cs = uniq[sel] % V, cnt[sel]
        order = np.lexsort((vs, -cs))[:S]
        k = len(order)
        assert ids[u, :k].tolist() == vs[order].tolist()
        assert sc[u, :k].tolist() == cs[order].astype(np.float32).tolist()
        assert (ids[u, k:] == -1).all() and (sc[u, k:] == 0).all()
