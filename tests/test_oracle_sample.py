"""Pins for the oracle's sampling acceptance (temperature > 0).

* Losslessness, by Monte Carlo on a tiny vocabulary: the first emitted token
  is distributed as softmax(root logits / T), and, given that it is the
  token of a child c, the second emitted token as softmax(logits_c / T)
  (a chi-square bound on 40000 draws).
* The low-temperature limit is greedy acceptance (the O3 pins), on trees
  whose siblings carry distinct tokens.
* A root-only tree samples by inverse CDF: numpy's cumsum + searchsorted.
* A repeated sibling token is never accepted.
"""
import numpy as np
import pytest

import oracle as O


def _softmax(z):
    e = np.exp(z - z.max())
    return e / e.sum()


def _tree():
    # root 0; children 1 (tok 2), 2 (tok 0), 3 (tok 4); grandchildren under 1
    parent = np.array([[-1, 0, 0, 0, 1, 1, 2]], np.int32)
    token = np.array([[3, 2, 0, 4, 1, 3, 2]], np.int32)
    return parent, token


def test_lossless_first_and_second_token():
    rng = np.random.default_rng(11)
    V, T = 5, 0.8
    parent, token = _tree()
    n = parent.shape[1]
    logits = rng.standard_normal((1, n, V)).astype(np.float32) * 1.5
    N = 40000
    first = np.zeros(V)
    second = {c: np.zeros(V) for c in (1, 2, 3)}
    child_of_tok = {2: 1, 0: 2, 4: 3}
    for _ in range(N):
        ra = rng.random((1, n))
        rs = rng.random((1, n))
        r = O.accept_sample(logits, "f32", T, token, parent, np.array([n]), ra, rs)
        x1 = int(r["path_tokens"][0, 1])
        first[x1] += 1
        if x1 in child_of_tok:
            second[child_of_tok[x1]][int(r["path_tokens"][0, 2])] += 1
    p_root = _softmax(logits[0, 0].astype(np.float64) / T)

    def chi2_ok(counts, p):
        tot = counts.sum()
        exp = p * tot
        chi2 = float(((counts - exp) ** 2 / np.maximum(exp, 1e-12)).sum())
        # 4 degrees of freedom: P(chi2 > 30) < 1e-5
        return chi2 < 30.0, chi2

    ok, chi = chi2_ok(first, p_root)
    assert ok, (chi, first / N, p_root)
    for c, cnt in second.items():
        if cnt.sum() < 2000:
            continue
        ok, chi = chi2_ok(cnt, _softmax(logits[0, c].astype(np.float64) / T))
        assert ok, (c, chi)


@pytest.mark.parametrize("seed", range(10))
def test_low_temperature_is_greedy(seed):
    rng = np.random.default_rng(600 + seed)
    B, n_max, V = 2, 9, 7
    parent = np.full((B, n_max), -1, np.int32)
    token = np.zeros((B, n_max), np.int32)
    n_nodes = rng.integers(1, n_max + 1, B)
    for b in range(B):
        token[b, 0] = rng.integers(0, V)
        for i in range(1, int(n_nodes[b])):
            parent[b, i] = rng.integers(0, i)
            # siblings carry distinct tokens: with a repeated token, greedy
            # acceptance may pick the deeper of the two subtrees while
            # sampling follows the first sibling
            taken = {int(token[b, j]) for j in range(1, i) if parent[b, j] == parent[b, i]}
            token[b, i] = rng.choice([t for t in range(V) if t not in taken])
    # distinct logits per row, some children made the parent's argmax
    logits = np.stack([np.stack([rng.permutation(V).astype(np.float32) for _ in range(n_max)])
                       for _ in range(B)])
    for b in range(B):
        for i in range(1, int(n_nodes[b])):
            if rng.random() < 0.6:
                p = parent[b, i]
                logits[b, p, token[b, i]] = logits[b, p].max() + 1.0
    greedy = O.accept(logits, "f32", token, parent, n_nodes)
    r = O.accept_sample(logits, "f32", 1e-3, token, parent, n_nodes,
                        rng.uniform(0.01, 0.99, (B, n_max)), rng.uniform(0.01, 0.99, (B, n_max)))
    np.testing.assert_array_equal(r["accept_len"], greedy["accept_len"])
    np.testing.assert_array_equal(r["path_nodes"], greedy["path_nodes"])
    np.testing.assert_array_equal(r["path_tokens"], greedy["path_tokens"])


def test_root_only_is_inverse_cdf_sampling():
    rng = np.random.default_rng(3)
    V, T = 11, 1.3
    logits = rng.standard_normal((1, 1, V)).astype(np.float32)
    p = _softmax(logits[0, 0].astype(np.float64) / T)
    cdf = np.cumsum(p)
    for u in rng.random(50):
        r = O.accept_sample(logits, "f32", T, np.array([[4]]), np.array([[-1]]), np.array([1]),
                            np.zeros((1, 1)), np.array([[u]]))
        assert r["accept_len"][0] == 0
        assert r["path_tokens"][0, 1] == int(np.searchsorted(cdf, u * cdf[-1], side="right"))


def test_repeated_sibling_token_never_accepted():
    V, T = 4, 1.0
    parent = np.array([[-1, 0, 0]], np.int32)
    token = np.array([[0, 2, 2]], np.int32)
    logits = np.zeros((1, 3, V), np.float32)
    logits[0, 0, 2] = 3.0  # token 2 likely at the root
    # reject child 1 (u just above p(2)), offer child 2 with u = 0: still
    # rejected, since token 2's mass is gone
    p2 = _softmax(logits[0, 0].astype(np.float64) / T)[2]
    ra = np.array([[0.0, p2 + 1e-3, 0.0]])
    r = O.accept_sample(logits, "f32", T, token, parent, np.array([3]), ra,
                        np.array([[0.5, 0.5, 0.5]]))
    assert r["accept_len"][0] == 0
    assert r["path_tokens"][0, 1] != 2


def test_margins_on_a_hand_worked_case():
    """Root with children of tokens 0 and 1 under p = (0.5, 0.3, 0.15, 0.05):
    u = 0.55 rejects token 0 (margin 0.05); with 0.5 removed, u = 0.56 gives
    0.56 * 0.5 - 0.3 = -0.02, so token 1 is accepted (margin 0.02).  Node 2
    has no children; its uniform row and draw 0.6 pick token 2, whose CDF
    interval [0.5, 0.75) lies 0.1 from the target at its nearer end."""
    p_root = np.array([0.5, 0.3, 0.15, 0.05])
    logits = np.zeros((1, 3, 4), np.float32)
    logits[0, 0] = np.log(p_root)
    parent = np.array([[-1, 0, 0]], np.int32)
    token = np.array([[3, 0, 1]], np.int32)
    ra = np.array([[0.0, 0.55, 0.56]])
    rs = np.array([[0.0, 0.0, 0.6]])
    r = O.accept_sample(logits, "f32", 1.0, token, parent, np.array([3]), ra, rs)
    assert r["accept_len"][0] == 1
    assert list(r["path_nodes"][0]) == [0, 2, -1]
    assert list(r["path_tokens"][0]) == [3, 1, 2, -1]
    # float32 logits of log(p) carry ~1e-8 relative error
    assert abs(r["margin_accept"][0] - 0.02) < 1e-6
    assert abs(r["margin_bonus"][0] - 0.1) < 1e-6
    # both child tests are made at the root (depth 0); node 2 makes none
    md = r["margin_by_depth"][0]
    assert abs(md[0] - 0.02) < 1e-6 and np.isinf(md[1:]).all()


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_margin_by_depth_places_each_test_on_the_path(seed):
    """The per-depth margins cover exactly the nodes of the path that made a
    child test, and their minimum is the sequence's margin_accept."""
    rng = np.random.default_rng(seed)
    B, n, V = 6, 12, 7
    parent = np.full((B, n), -1, np.int32)
    for b in range(B):
        for i in range(1, n):
            parent[b, i] = int(rng.integers(0, i))
    token = rng.integers(0, V, (B, n)).astype(np.int32)
    logits = (rng.standard_normal((B, n, V)) * 2.0).astype(np.float32)
    ra = rng.random((B, n))
    rs = rng.random((B, n))
    r = O.accept_sample(logits, "f32", 0.7, token, parent, np.full(B, n), ra, rs)
    for b in range(B):
        L = int(r["accept_len"][b])
        md = r["margin_by_depth"][b]
        path = r["path_nodes"][b, :L + 1]
        for d in range(n):
            has_child = d <= L and any(int(parent[b, c]) == int(path[d]) for c in range(n))
            assert np.isfinite(md[d]) == has_child, (b, d)
        assert np.min(md) == r["margin_accept"][b]

