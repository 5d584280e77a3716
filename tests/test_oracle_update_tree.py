"""Pins for the all-node update of M (every verified node's transition).

* A hand-worked example (four nodes, empty M, S = 2).
* The transitions are recomputed independently: numpy's argmax over each
  verified node's logits row, paired with the node's token.
* The accepted path's transitions (the default update) are a sub-multiset of
  the all-node transitions.
"""
from collections import Counter

import numpy as np
import pytest

import oracle as O


def test_hand_worked_example():
    token = np.array([[5, 7, 9, 7, 0]], np.int32)
    argmax = np.array([[7, 3, 3, 1, -1]], np.int32)
    n_nodes = np.array([4])
    assert O.tree_transitions(token, argmax, n_nodes) == [(5, 7), (7, 3), (9, 3), (7, 1)]
    V, S = 10, 2
    ids = np.full((V, S), -1, np.int32)
    sc = np.zeros((V, S), np.float32)
    new_ids, new_sc = O.update_adjacency_tree(ids, sc, token, argmax, n_nodes)
    # row 5: {7: 1}; row 7: {3: 1, 1: 1} -> equal counts, lower id first;
    # row 9: {3: 1}; every other row untouched
    exp_ids = ids.copy()
    exp_sc = sc.copy()
    exp_ids[5] = [7, -1]
    exp_sc[5] = [1, 0]
    exp_ids[7] = [1, 3]
    exp_sc[7] = [1, 1]
    exp_ids[9] = [3, -1]
    exp_sc[9] = [1, 0]
    np.testing.assert_array_equal(new_ids, exp_ids)
    np.testing.assert_array_equal(new_sc, exp_sc)


def _random_verified_tree(rng, B, n_max, V):
    parent = np.full((B, n_max), -1, np.int32)
    token = np.zeros((B, n_max), np.int32)
    n_nodes = rng.integers(1, n_max + 1, B)
    for b in range(B):
        for i in range(1, int(n_nodes[b])):
            parent[b, i] = rng.integers(0, i)
        token[b, :n_nodes[b]] = rng.integers(0, V, n_nodes[b])
    logits = rng.standard_normal((B, n_max, V)).astype(np.float32)
    # make some children match their parent's argmax so paths are accepted
    for b in range(B):
        for i in range(1, int(n_nodes[b])):
            if rng.random() < 0.6:
                p = parent[b, i]
                logits[b, p, token[b, i]] = logits[b, p].max() + 1.0
    return parent, token, n_nodes, logits


@pytest.mark.parametrize("seed", range(10))
def test_transitions_against_numpy_argmax_and_path(seed):
    rng = np.random.default_rng(300 + seed)
    B, n_max, V = 3, 12, 9
    parent, token, n_nodes, logits = _random_verified_tree(rng, B, n_max, V)
    acc = O.accept(logits, "f32", token, parent, n_nodes)
    pairs = O.tree_transitions(token, acc["argmax"], n_nodes)
    # independent: numpy argmax of each verified row (first maximum)
    ref = [(int(token[b, i]), int(np.argmax(logits[b, i])))
           for b in range(B) for i in range(int(n_nodes[b]))]
    assert pairs == ref
    # the accepted path's transitions are among them
    path = Counter(O.transitions(acc["path_tokens"], acc["accept_len"]))
    assert not path - Counter(pairs)


@pytest.mark.parametrize("seed", range(6))
def test_update_tree_is_the_update_of_its_pairs(seed):
    rng = np.random.default_rng(400 + seed)
    B, n_max, V, S = 2, 10, 7, 3
    parent, token, n_nodes, logits = _random_verified_tree(rng, B, n_max, V)
    argmax = np.argmax(logits, axis=2).astype(np.int32)
    ids = np.full((V, S), -1, np.int32)
    sc = np.zeros((V, S), np.float32)
    for u in range(V):
        k = int(rng.integers(0, S + 1))
        ids[u, :k] = rng.choice(V, k, replace=False)
        sc[u, :k] = np.sort(rng.integers(1, 5, k))[::-1]
    got = O.update_adjacency_tree(ids, sc, token, argmax, n_nodes)
    # brute force: count the pairs, merge into each row, keep the best S
    cnt = Counter((int(token[b, i]), int(argmax[b, i]))
                  for b in range(B) for i in range(int(n_nodes[b])))
    exp_ids, exp_sc = ids.copy(), sc.copy()
    for u in {u for (u, _) in cnt}:
        cand = {int(v): float(s) for v, s in zip(ids[u], sc[u]) if v >= 0}
        for (uu, v), c in cnt.items():
            if uu == u:
                cand[v] = cand.get(v, 0.0) + c
        best = sorted(cand.items(), key=lambda kv: (-kv[1], kv[0]))[:S]
        exp_ids[u] = -1
        exp_sc[u] = 0
        for s_, (v, x) in enumerate(best):
            exp_ids[u, s_] = v
            exp_sc[u, s_] = x
    np.testing.assert_array_equal(got[0], exp_ids)
    np.testing.assert_array_equal(got[1], exp_sc)
