"""Pins for the oracle's rotary position embedding by tree position.

* rope is complex multiplication: (x_i + j x_{i+D/2}) (c + j s), computed by
  numpy's complex arithmetic on an arbitrary table of unit phasors.
* With a table built from angles t w_i, attention scores depend only on the
  offset between query and key positions (shifting both changes nothing),
  and position 0 is the identity; rotation keeps norms.
* tree_attention_rope equals a brute-force dense attention over the root
  path in which every key and query is rotated through the complex route at
  its own position (prefix keys at 0 .. P-1 already in the cache rotated,
  tree nodes at prefix + depth).
* append_kv_rope commits rotated keys at the cache positions prefix + j and
  copies the values.
"""
import numpy as np
import pytest

import oracle as O


def _complex_rotate(x, pos, cos_sin):
    """The same rotation by an independent route: complex products."""
    x = np.asarray(x, np.float64)
    h = x.shape[-1] // 2
    tab = np.asarray(cos_sin, np.float64)[np.asarray(pos)]
    z = x[..., :h] + 1j * x[..., h:]
    w = tab[..., :h] + 1j * tab[..., h:]
    y = z * w
    return np.concatenate([y.real, y.imag], axis=-1)


def _angle_table(positions, D, base=10000.0):
    w = base ** (-2.0 * np.arange(D // 2) / D)
    ang = np.arange(positions)[:, None] * w[None, :]
    return np.concatenate([np.cos(ang), np.sin(ang)], axis=1)


@pytest.mark.parametrize("D", [2, 16, 128])
def test_rope_is_complex_multiplication(D):
    rng = np.random.default_rng(D)
    theta = rng.uniform(-np.pi, np.pi, (40, D // 2))
    table = np.concatenate([np.cos(theta), np.sin(theta)], axis=1)
    x = rng.standard_normal((7, 3, D))
    pos = rng.integers(0, 40, (7, 3))
    np.testing.assert_allclose(O.rope(x, pos, table), _complex_rotate(x, pos, table),
                               rtol=0, atol=1e-13)


def test_rope_relative_positions_identity_and_norm():
    rng = np.random.default_rng(1)
    D = 64
    table = _angle_table(400, D)
    q = rng.standard_normal(D)
    k = rng.standard_normal(D)
    for m, n, s in [(5, 3, 100), (0, 17, 250), (33, 33, 7), (120, 2, 90)]:
        a = O.rope(q, m, table) @ O.rope(k, n, table)
        b = O.rope(q, m + s, table) @ O.rope(k, n + s, table)
        assert abs(a - b) < 1e-10
    np.testing.assert_allclose(O.rope(q, 0, table), q, atol=0)
    for t in (1, 77, 399):
        y = O.rope(q, t, table)
        # each (i, i + D/2) pair keeps its length
        np.testing.assert_allclose(y[:D // 2] ** 2 + y[D // 2:] ** 2,
                                   q[:D // 2] ** 2 + q[D // 2:] ** 2, rtol=1e-12)


def _random_case(seed, B=2, n_max=9, Hq=4, Hkv=2, D=16, blk=4):
    rng = np.random.default_rng(seed)
    parent = np.full((B, n_max), -1, np.int32)
    depth = np.zeros((B, n_max), np.int32)
    n_nodes = rng.integers(1, n_max + 1, B)
    mask = np.zeros((B, n_max, 1), np.uint32)
    for b in range(B):
        mask[b, 0, 0] = 1
        for i in range(1, int(n_nodes[b])):
            p = int(rng.integers(0, i))
            parent[b, i] = p
            depth[b, i] = depth[b, p] + 1
            mask[b, i, 0] = mask[b, p, 0] | np.uint32(1 << i)
    prefix = rng.integers(0, 20, B).astype(np.int32)
    tree_pos = (prefix[:, None] + depth).astype(np.int32)
    table = _angle_table(64, D)
    max_blocks = (int(prefix.max()) + n_max + blk - 1) // blk
    nblk = B * max_blocks
    block_table = rng.permutation(nblk).reshape(B, max_blocks).astype(np.int32)
    k_raw_prefix = rng.standard_normal((B, int(prefix.max()) + 1, Hkv, D))
    k_cache = np.zeros((nblk, Hkv, blk, D))
    v_cache = np.zeros((nblk, Hkv, D, blk))
    v_prefix = rng.standard_normal((B, int(prefix.max()) + 1, Hkv, D))
    for b in range(B):
        for t in range(int(prefix[b])):
            page = block_table[b, t // blk]
            k_cache[page, :, t % blk, :] = _complex_rotate(k_raw_prefix[b, t], t, table)
            v_cache[page, :, :, t % blk] = v_prefix[b, t]
    q = rng.standard_normal((B, n_max, Hq, D))
    k_tree = rng.standard_normal((B, n_max, Hkv, D))
    v_tree = rng.standard_normal((B, n_max, Hkv, D))
    return dict(q=q, k_tree=k_tree, v_tree=v_tree, k_cache=k_cache, v_cache=v_cache,
                block_table=block_table, prefix=prefix, mask=mask, n_nodes=n_nodes,
                tree_pos=tree_pos, table=table, parent=parent, k_raw_prefix=k_raw_prefix,
                v_prefix=v_prefix)


@pytest.mark.parametrize("seed", range(8))
def test_tree_attention_rope_brute_force(seed):
    c = _random_case(seed)
    scale = 0.3
    got = O.tree_attention_rope(c["q"], c["k_tree"], c["v_tree"], c["k_cache"], c["v_cache"],
                                c["block_table"], c["prefix"], c["mask"], c["n_nodes"],
                                c["tree_pos"], c["table"], scale)
    B, n_max, Hq, D = c["q"].shape
    G = Hq // c["k_tree"].shape[2]
    for b in range(B):
        P = int(c["prefix"][b])
        for i in range(int(c["n_nodes"][b])):
            path = [i]
            while c["parent"][b, path[-1]] >= 0:
                path.append(int(c["parent"][b, path[-1]]))
            for hq in range(Hq):
                h = hq // G
                keys = [_complex_rotate(c["k_raw_prefix"][b, t, h], t, c["table"])
                        for t in range(P)]
                keys += [_complex_rotate(c["k_tree"][b, j, h], P + len(_anc(c, b, j)) - 1,
                                         c["table"]) for j in sorted(path)]
                vals = [c["v_prefix"][b, t, h] for t in range(P)]
                vals += [c["v_tree"][b, j, h] for j in sorted(path)]
                qv = _complex_rotate(c["q"][b, i, hq], P + len(path) - 1, c["table"])
                s = np.array([kk @ qv for kk in keys]) * scale
                wgt = np.exp(s - s.max())
                ref = (wgt @ np.array(vals)) / wgt.sum()
                np.testing.assert_allclose(got[b, i, hq], ref, rtol=0, atol=1e-12)


def _anc(c, b, j):
    out = [j]
    while c["parent"][b, out[-1]] >= 0:
        out.append(int(c["parent"][b, out[-1]]))
    return out


def test_append_kv_rope_commits_rotated_keys_at_cache_positions():
    c = _random_case(3)
    B = len(c["prefix"])
    path_nodes = np.full(c["parent"].shape, -1, np.int32)
    accept_len = np.zeros(B, np.int32)
    for b in range(B):
        # the deepest node's root path
        i = int(c["n_nodes"][b]) - 1
        path = _anc(c, b, i)[::-1]
        path_nodes[b, :len(path)] = path
        accept_len[b] = len(path) - 1
    k, v, new_len = O.append_kv_rope(c["k_cache"], c["v_cache"], c["block_table"], c["prefix"],
                                     c["k_tree"], c["v_tree"], path_nodes, accept_len,
                                     c["table"])
    k0, v0, len0 = O.append_kv(c["k_cache"], c["v_cache"], c["block_table"], c["prefix"],
                               c["k_tree"], c["v_tree"], path_nodes, accept_len)
    np.testing.assert_array_equal(v, v0)
    np.testing.assert_array_equal(new_len, len0)
    blk = k.shape[2]
    touched = np.zeros(k.shape[:1] + k.shape[2:3], bool)
    for b in range(B):
        P = int(c["prefix"][b])
        for j in range(int(accept_len[b]) + 1):
            t = P + j
            page = c["block_table"][b, t // blk]
            touched[page, t % blk] = True
            want = _complex_rotate(c["k_tree"][b, path_nodes[b, j]], t, c["table"])
            np.testing.assert_allclose(k[page, :, t % blk, :], want, rtol=0, atol=1e-13)
    # every other slot is as before
    for page in range(k.shape[0]):
        for slot in range(blk):
            if not touched[page, slot]:
                np.testing.assert_array_equal(k[page, :, slot, :], c["k_cache"][page, :, slot, :])
