"""Pins for the oracle's KV-cache commit of the accepted path (CPU only).

* The cache layout is checked through numpy views: with each sequence's
  pages contiguous, a reshape of its pages is the token-ordered K (token-major
  pages) or V (dim-major pages), independent of the oracle's page arithmetic.
* Semantics: the accepted node's verification row (tree attention over the
  prefix and its root path) must equal plain decode attention (torch SDPA,
  float64) over the committed cache alone.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle as O


def _setup(rng, prefixes, n_max, Hkv=2, D=8, block=4, permute=False):
    B = len(prefixes)
    pages = [-(-(int(p) + n_max) // block) for p in prefixes]
    nblocks = sum(pages)
    phys = rng.permutation(nblocks) if permute else np.arange(nblocks)
    table = np.full((B, max(pages)), -1, np.int32)
    o = 0
    for b in range(B):
        table[b, :pages[b]] = phys[o:o + pages[b]]
        o += pages[b]
    kc = rng.standard_normal((nblocks, Hkv, block, D))
    vc = rng.standard_normal((nblocks, Hkv, D, block))
    kt = rng.standard_normal((B, n_max, Hkv, D))
    vt = rng.standard_normal((B, n_max, Hkv, D))
    return kc, vc, table, kt, vt, pages


def _token_views(kc, vc, first_page, n_pages):
    """Token-ordered [Hkv][tokens][D] views of one sequence's contiguous pages."""
    k = kc[first_page:first_page + n_pages]              # [pg][Hkv][blk][D]
    v = vc[first_page:first_page + n_pages]              # [pg][Hkv][D][blk]
    Hkv, D = k.shape[1], k.shape[3]
    kv = k.transpose(1, 0, 2, 3).reshape(Hkv, -1, D)
    vv = v.transpose(1, 0, 3, 2).reshape(Hkv, -1, D)
    return kv, vv


@pytest.mark.parametrize("seed", range(8))
def test_append_identity_layout(seed):
    rng = np.random.default_rng(50 + seed)
    n_max = 9
    prefixes = np.array(rng.integers(0, 14, 3), np.int32)
    kc, vc, table, kt, vt, pages = _setup(rng, prefixes, n_max)
    L = rng.integers(0, n_max, len(prefixes)).astype(np.int32)
    path = np.full((len(prefixes), n_max), -1, np.int32)
    for b in range(len(prefixes)):
        path[b, :L[b] + 1] = np.concatenate([[0], rng.choice(np.arange(1, n_max), L[b],
                                                             replace=False)])
    k2, v2, new_len = O.append_kv(kc, vc, table, prefixes, kt, vt, path, L)
    np.testing.assert_array_equal(new_len, prefixes + L + 1)
    first = 0
    for b in range(len(prefixes)):
        kv0, vv0 = _token_views(kc, vc, first, pages[b])
        kv1, vv1 = _token_views(k2, v2, first, pages[b])
        P = int(prefixes[b])
        written = np.zeros(kv0.shape[1], bool)
        for j in range(int(L[b]) + 1):
            node = path[b, j]
            np.testing.assert_array_equal(kv1[:, P + j, :], kt[b, node])
            np.testing.assert_array_equal(vv1[:, P + j, :], vt[b, node])
            written[P + j] = True
        np.testing.assert_array_equal(kv1[:, ~written], kv0[:, ~written])
        np.testing.assert_array_equal(vv1[:, ~written], vv0[:, ~written])
        first += pages[b]
    # the inputs are not modified
    assert not np.shares_memory(k2, kc) and not np.shares_memory(v2, vc)


@pytest.mark.parametrize("seed", range(6))
def test_committed_cache_decodes_like_the_verified_row(seed):
    """The accepted node saw the prefix and its root path during verification;
    after the commit, decoding it against the cache alone gives the same
    output."""
    rng = np.random.default_rng(70 + seed)
    n_max, Hq, Hkv, D, block = 10, 4, 2, 8, 4
    G = Hq // Hkv
    prefixes = np.array(rng.integers(0, 19, 2), np.int32)
    kc, vc, table, kt, vt, _ = _setup(rng, prefixes, n_max, Hkv, D, block, permute=True)
    B = len(prefixes)
    q = rng.standard_normal((B, n_max, Hq, D))
    parents, mask = [], np.zeros((B, n_max, 1), np.uint32)
    path = np.full((B, n_max), -1, np.int32)
    L = np.zeros(B, np.int32)
    acc = np.zeros(B, np.int64)
    for b in range(B):
        par = [-1] + [int(rng.integers(0, i)) for i in range(1, n_max)]
        parents.append(par)
        for i in range(n_max):
            j = i
            while j >= 0:
                mask[b, i, 0] |= np.uint32(1 << j)
                j = par[j]
        a = int(rng.integers(0, n_max))
        chain = []
        j = a
        while j >= 0:
            chain.append(j)
            j = par[j]
        chain = chain[::-1]
        path[b, :len(chain)] = chain
        L[b] = len(chain) - 1
        acc[b] = a
    scale = 1 / np.sqrt(D)
    verified = O.tree_attention(q, kt, vt, kc, vc, table, prefixes, mask,
                                np.full(B, n_max), scale)
    k2, v2, new_len = O.append_kv(kc, vc, table, prefixes, kt, vt, path, L)
    for b in range(B):
        for hq in range(Hq):
            h = hq // G
            Kp, Vp = O.gather_prefix(k2, v2, table[b], int(new_len[b]), h)
            ref = F.scaled_dot_product_attention(
                torch.from_numpy(q[b, acc[b], hq])[None, None, None],
                torch.from_numpy(Kp)[None, None], torch.from_numpy(Vp)[None, None],
                scale=scale).numpy()[0, 0, 0]
            np.testing.assert_allclose(verified[b, acc[b], hq], ref, rtol=0, atol=1e-12)


def test_root_only_and_capacity():
    rng = np.random.default_rng(7)
    kc, vc, table, kt, vt, pages = _setup(rng, np.array([5], np.int32), 3)
    path = np.array([[2, -1, -1]], np.int32)
    k2, v2, new_len = O.append_kv(kc, vc, table, np.array([5]), kt, vt, path,
                                  np.array([0], np.int32))
    assert new_len[0] == 6
    kv, vv = _token_views(k2, v2, 0, pages[0])
    np.testing.assert_array_equal(kv[:, 5], kt[0, 2])
    np.testing.assert_array_equal(vv[:, 5], vt[0, 2])
    # a negative accept length leaves the sequence untouched
    k3, v3, n3 = O.append_kv(kc, vc, table, np.array([5]), kt, vt, path,
                             np.array([-1], np.int32))
    assert n3[0] == 5 and np.array_equal(k3, kc) and np.array_equal(v3, vc)
    # pages for 5 + 3 tokens: committing 4 tokens after a prefix of 5 overflows
    with pytest.raises(ValueError):
        O.append_kv(kc, vc, table, np.array([5]), kt, vt,
                    np.array([[0, 1, 2, 0]], np.int32), np.array([3], np.int32))
