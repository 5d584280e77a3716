"""Pins for the oracle's tree attention (CPU only).

The oracle is checked against torch's scaled_dot_product_attention (float64,
CPU) -- a library routine that knows nothing of trees or pages -- and against
closed forms.  Tree visibility is given to the library as a walk up the
parent array, never as the mask the oracle reads.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle as O


def _paged(rng, K, V, block, permute=True):
    """Scatter contiguous per-sequence K/V [B][P][Hkv][D] into pages: K pages
    token-major [blk][Hkv][block][D], V pages dim-major [blk][Hkv][D][block]."""
    B, P, Hkv, D = K.shape
    npg = max(1, -(-P // block))
    nblocks = B * npg
    phys = rng.permutation(nblocks) if permute else np.arange(nblocks)
    kc = rng.standard_normal((nblocks, Hkv, block, D))  # junk where unused
    vc = rng.standard_normal((nblocks, Hkv, D, block))
    table = np.zeros((B, npg), np.int32)
    for b in range(B):
        for pg in range(npg):
            table[b, pg] = phys[b * npg + pg]
        for t in range(P):
            blk = table[b, t // block]
            for h in range(Hkv):
                kc[blk, h, t % block, :] = K[b, t, h, :]
                vc[blk, h, :, t % block] = V[b, t, h, :]
    return kc, vc, table


def _mask_from_parents(parent, n_max):
    W = O.mask_words(n_max)
    m = np.zeros((n_max, W), np.uint32)
    for i in range(len(parent)):
        j = i
        while j >= 0:
            m[i, j // 32] |= np.uint32(1 << (j % 32))
            j = parent[j]
    return m


def _sdpa(q, k, v, scale, causal=False):
    return F.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
        is_causal=causal, scale=scale).numpy()


@pytest.mark.parametrize("P", [0, 1, 16, 37])
def test_chain_equals_causal_attention(P):
    """A chain tree on top of a prefix is ordinary causal attention over
    prefix || chain (torch SDPA with is_causal over the full length)."""
    rng = np.random.default_rng(P)
    N, Hq, Hkv, D, block = 7, 4, 2, 16, 8
    G = Hq // Hkv
    Kall = rng.standard_normal((1, P + N, Hkv, D))
    Vall = rng.standard_normal((1, P + N, Hkv, D))
    Qall = rng.standard_normal((1, P + N, Hq, D))
    kc, vc, table = _paged(rng, Kall[:, :P], Vall[:, :P], block)
    parent = [-1] + list(range(N - 1))
    mask = _mask_from_parents(parent, N)[None]
    scale = 0.3
    out = O.tree_attention(Qall[:, P:], Kall[:, P:], Vall[:, P:], kc, vc, table,
                           np.array([P]), mask, np.array([N]), scale)
    # library: [B, H, L, D] with K/V heads repeated per query group
    q = Qall.transpose(0, 2, 1, 3)
    k = np.repeat(Kall.transpose(0, 2, 1, 3), G, axis=1)
    v = np.repeat(Vall.transpose(0, 2, 1, 3), G, axis=1)
    ref = _sdpa(q, k, v, scale, causal=True)[:, :, P:, :].transpose(0, 2, 1, 3)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("seed", range(12))
def test_each_row_is_dense_attention_over_its_path(seed):
    """Brute force on random trees of up to 12 nodes and ragged prefixes: row
    i equals plain attention over prefix || (root-to-i path), the path taken
    by walking parents."""
    rng = np.random.default_rng(1000 + seed)
    B, Hq, Hkv, D, block = 2, 6, 3, 8, 4
    G = Hq // Hkv
    n_max = 12
    n_nodes = rng.integers(1, n_max + 1, B)
    P = rng.integers(0, 23, B)
    Pm = int(P.max())
    Kp = rng.standard_normal((B, Pm, Hkv, D))
    Vp = rng.standard_normal((B, Pm, Hkv, D))
    kc, vc, table = _paged(rng, Kp, Vp, block)
    q = rng.standard_normal((B, n_max, Hq, D))
    kt = rng.standard_normal((B, n_max, Hkv, D))
    vt = rng.standard_normal((B, n_max, Hkv, D))
    parents = []
    mask = np.zeros((B, n_max, 1), np.uint32)
    for b in range(B):
        par = [-1] + [int(rng.integers(0, i)) for i in range(1, int(n_nodes[b]))]
        parents.append(par)
        mask[b, :len(par)] = _mask_from_parents(par, n_max)[:len(par)]
    scale = 1 / np.sqrt(D)
    out = O.tree_attention(q, kt, vt, kc, vc, table, P, mask, n_nodes, scale)
    for b in range(B):
        for i in range(int(n_nodes[b])):
            path = []
            j = i
            while j >= 0:
                path.append(j)
                j = parents[b][j]
            path = path[::-1]
            for hq in range(Hq):
                h = hq // G
                k = np.concatenate([Kp[b, :P[b], h], kt[b, path, h]])[None, None]
                v = np.concatenate([Vp[b, :P[b], h], vt[b, path, h]])[None, None]
                ref = _sdpa(q[b, i, hq][None, None, None], k, v, scale)[0, 0, 0]
                np.testing.assert_allclose(out[b, i, hq], ref, rtol=0, atol=1e-12)
        # rows past n_nodes are not produced
        assert np.isnan(out[b, int(n_nodes[b]):]).all()


def test_uniform_keys_give_mean_of_values():
    """Identical keys make the softmax uniform: the output is the mean of the
    visible values (closed form)."""
    rng = np.random.default_rng(5)
    Hq, Hkv, D, block, P, N = 2, 1, 4, 4, 9, 5
    kvec = rng.standard_normal(D)
    Kp = np.broadcast_to(kvec, (1, P, Hkv, D)).copy()
    Vp = rng.standard_normal((1, P, Hkv, D))
    kc, vc, table = _paged(rng, Kp, Vp, block)
    kt = np.broadcast_to(kvec, (1, N, Hkv, D)).copy()
    vt = rng.standard_normal((1, N, Hkv, D))
    q = rng.standard_normal((1, N, Hq, D))
    parent = [-1, 0, 1, 0, 3]
    mask = _mask_from_parents(parent, N)[None]
    out = O.tree_attention(q, kt, vt, kc, vc, table, np.array([P]), mask,
                           np.array([N]), 0.7)
    for i, path in enumerate([[0], [0, 1], [0, 1, 2], [0, 3], [0, 3, 4]]):
        ref = (Vp[0, :, 0].sum(0) + vt[0, path, 0].sum(0)) / (P + len(path))
        for hq in range(Hq):
            np.testing.assert_allclose(out[0, i, hq], ref, rtol=0, atol=1e-12)


def test_single_node_is_decode_attention_and_shift_invariant():
    """A tree with only the root is plain decode attention over prefix||root;
    shifting every key along q leaves the output unchanged."""
    rng = np.random.default_rng(9)
    Hq, Hkv, D, block, P = 4, 4, 8, 16, 40
    Kp = rng.standard_normal((1, P, Hkv, D))
    Vp = rng.standard_normal((1, P, Hkv, D))
    kc, vc, table = _paged(rng, Kp, Vp, block, permute=False)
    q = rng.standard_normal((1, 1, Hq, D))
    kt = rng.standard_normal((1, 1, Hkv, D))
    vt = rng.standard_normal((1, 1, Hkv, D))
    mask = np.ones((1, 1, 1), np.uint32)
    out = O.tree_attention(q, kt, vt, kc, vc, table, np.array([P]), mask,
                           np.array([1]), 0.25)
    for h in range(Hq):
        k = np.concatenate([Kp[0, :, h], kt[0, :, h]])[None, None]
        v = np.concatenate([Vp[0, :, h], vt[0, :, h]])[None, None]
        ref = _sdpa(q[0, 0, h][None, None, None], k, v, 0.25)[0, 0, 0]
        np.testing.assert_allclose(out[0, 0, h], ref, rtol=0, atol=1e-12)
    # shift: adding the same vector to every key adds q.delta to every score
    delta = rng.standard_normal(D)
    out2 = O.tree_attention(q, kt + delta, vt, kc + delta, vc, table,
                            np.array([P]), mask, np.array([1]), 0.25)
    # only the query whose head matches a shifted key sees a uniform shift;
    # with one query per head every score of that head moves by q.delta
    np.testing.assert_allclose(out2, out, rtol=0, atol=1e-10)


def test_gather_prefix_layouts():
    """The page gather reads K token-major and V dim-major through the table."""
    rng = np.random.default_rng(3)
    Kp = rng.standard_normal((1, 21, 2, 5))
    Vp = rng.standard_normal((1, 21, 2, 5))
    kc, vc, table = _paged(rng, Kp, Vp, 4)
    for h in range(2):
        K, V = O.gather_prefix(kc, vc, table[0], 21, h)
        np.testing.assert_array_equal(K, Kp[0, :, h])
        np.testing.assert_array_equal(V, Vp[0, :, h])
