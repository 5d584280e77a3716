"""GPU parity of the per-node argmax inside graft_accept on crafted bf16 rows.

The argmax is the lowest index among the maxima, with -0 equal to +0
(greedy acceptance, lossless verification in the architecture paragraph of
the "Draft Less, Retrieve More" summary).  Random logits almost never tie,
so these rows plant the cases that decide ties: repeated maxima in one chunk
and across chunks, signed zeros as the maximum, all-negative rows, the
extreme finite values, constant rows, maxima at the first and last
vocabulary entries, and equal maxima on both sides of a chunk edge.  Both chunk sizes of the argmax launch are covered
(a small grid, and one above 8192 workgroups).
"""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from tree_attention_verification_graft_amd import binding as G

pytestmark = pytest.mark.gpu


def _rows(n_rows, V, seed):
    """Crafted bf16 bit patterns, one case per row, cycling over the cases."""
    rng = np.random.default_rng(seed)
    out = np.empty((n_rows, V), np.uint16)
    for r in range(n_rows):
        case = r % 10
        x = rng.standard_normal(V).astype(np.float32)
        bits = W.f32_to_bf16_bits(x)
        if case == 0:  # one maximum, planted three times (two near, one far)
            m = W.f32_to_bf16_bits(np.array([9.5], np.float32))[0]
            pos = sorted({int(rng.integers(V)), int(rng.integers(V))})
            p0 = pos[0]
            for p in (p0, min(p0 + 1, V - 1), pos[-1]):
                bits[p] = m
        elif case == 1:  # all negative, then -0 before +0: -0 wins
            bits = W.f32_to_bf16_bits(-np.abs(x) - 0.25)
            a, b = sorted(rng.choice(V, 2, replace=False).tolist())
            bits[a], bits[b] = 0x8000, 0x0000
        elif case == 2:  # all negative, +0 before -0: +0 wins
            bits = W.f32_to_bf16_bits(-np.abs(x) - 0.25)
            a, b = sorted(rng.choice(V, 2, replace=False).tolist())
            bits[a], bits[b] = 0x0000, 0x8000
        elif case == 3:  # all negative; the maximum is the least negative
            bits = W.f32_to_bf16_bits(-np.abs(x) - 1.0)
        elif case == 4:  # the maximum at the last entry
            bits[V - 1] = W.f32_to_bf16_bits(np.array([20.0], np.float32))[0]
        elif case == 5:  # the maximum at entry 0, repeated later
            bits[0] = bits[V // 2] = W.f32_to_bf16_bits(np.array([20.0], np.float32))[0]
        elif case == 6:  # extreme finite values: -max everywhere but one +max
            bits[:] = 0xFF7F
            bits[int(rng.integers(V))] = 0x7F7F
        elif case == 9:  # one maximum on both sides of each chunk edge (4096- and
            # 6144-entry chunks): the lower index, in the earlier chunk, wins
            m = W.f32_to_bf16_bits(np.array([15.0], np.float32))[0]
            for edge in (6144, 4096):
                if edge < V:
                    bits[edge - 1] = bits[edge] = m
        elif case == 7:  # a constant negative row: entry 0
            bits[:] = W.f32_to_bf16_bits(np.array([-3.0], np.float32))[0]
        else:  # only -max: entry 0
            bits[:] = 0xFF7F
        out[r] = bits
    return out


def _chain_accept(logits_h, dtype):
    """graft_accept on one chain per sequence (node i's parent is i - 1), and
    the oracle's greedy verification of the same rows."""
    dev = torch.device("cuda:0")
    B, n_max, V = logits_h.shape
    n_nodes = np.full(B, n_max, np.int32)
    parent = np.tile(np.arange(-1, n_max - 1, dtype=np.int32), (B, 1))
    token = np.zeros((B, n_max), np.int32)
    words = G.mask_words(n_max)
    mask = np.zeros((B, n_max, words), np.uint32)
    for i in range(n_max):
        for j in range(i + 1):
            mask[:, i, j // 32] |= np.uint32(1 << (j % 32))
    ref = O.accept(logits_h, dtype, token, parent, n_nodes)

    i32 = torch.int32
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    if dtype == "bf16":
        logits = t(logits_h.view(np.int16)).view(torch.bfloat16)
    else:
        logits = t(logits_h.astype(np.float32))
    argmax = torch.empty((B, n_max), dtype=i32, device=dev)
    accept_len = torch.empty(B, dtype=i32, device=dev)
    path_nodes = torch.empty((B, n_max), dtype=i32, device=dev)
    path_tokens = torch.empty((B, n_max + 1), dtype=i32, device=dev)
    ws = torch.empty(max(G.graft_accept_workspace_size(B, n_max, V), 256),
                     dtype=torch.uint8, device=dev)
    G.graft_accept(logits, t(token), t(parent), t(mask.view(np.int32)), t(n_nodes), argmax,
                   accept_len, path_nodes, path_tokens, ws)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(argmax.cpu().numpy(), ref["argmax"])
    np.testing.assert_array_equal(accept_len.cpu().numpy(), ref["accept_len"])
    np.testing.assert_array_equal(path_tokens.cpu().numpy(), ref["path_tokens"])
    return ref


@pytest.mark.parametrize("B,n_max,V", [(2, 5, 32768), (4, 65, 128256), (3, 7, 1000),
                                       (3, 7, 999)],
                         ids=["small_grid", "large_grid", "vocab_1000", "vocab_999_scalar"])
def test_argmax_crafted_rows(B, n_max, V):
    rows = _rows(B * n_max, V, seed=B * 1000 + V)
    _chain_accept(rows.reshape(B, n_max, V), "bf16")


def _masked_rows(n_rows, V, seed):
    """Rows of a masked vocabulary (-inf logits), as float32 values, one case
    per row, cycling over the cases."""
    rng = np.random.default_rng(seed)
    ninf, pinf = np.float32(-np.inf), np.float32(np.inf)
    lowest = np.float32(-3.3895314e38)  # the most negative finite bf16, also finite in f32
    out = np.empty((n_rows, V), np.float32)
    for r in range(n_rows):
        case = r % 6
        x = rng.standard_normal(V).astype(np.float32)
        if case == 0:  # a few finite entries among -inf: the largest finite one
            row = np.full(V, ninf)
            keep = rng.choice(V, max(V // 100, 2), replace=False)
            row[keep] = x[keep]
        elif case == 1:  # every entry -inf: all equal, entry 0
            row = np.full(V, ninf)
        elif case == 2:  # -inf everywhere but the lowest finite value once
            row = np.full(V, ninf)
            row[int(rng.integers(V))] = lowest
        elif case == 3:  # -inf everywhere but the last entry
            row = np.full(V, ninf)
            row[V - 1] = np.float32(-7.0)
        elif case == 4:  # half masked, entry 0 masked, one maximum on both sides of
            # each chunk edge (4096- and 6144-entry chunks): the lower index wins
            row = x.copy()
            row[rng.random(V) < 0.5] = ninf
            row[0] = ninf
            for edge in (6144, 4096):
                if edge < V:
                    row[edge - 1] = row[edge] = np.float32(12.0)
        else:  # +inf twice among -inf and finite entries: the first +inf
            row = x.copy()
            row[rng.random(V) < 0.5] = ninf
            a, b = sorted(rng.choice(V, 2, replace=False).tolist())
            row[a] = row[b] = pinf
        out[r] = row
    return out


@pytest.mark.parametrize("dtype,B,n_max,V", [("bf16", 2, 6, 32768), ("bf16", 4, 65, 128256),
                                             ("bf16", 3, 7, 999), ("f32", 2, 6, 32768),
                                             ("f32", 3, 7, 999), ("f32", 2, 33, 151936)],
                         ids=["bf16_small_grid", "bf16_large_grid", "bf16_vocab_999",
                              "f32_small_grid", "f32_vocab_999", "f32_large"])
def test_argmax_masked_vocabulary(dtype, B, n_max, V):
    """-inf logits (a masked vocabulary) order below every finite value and tie
    with each other; a row of -inf only takes entry 0, and +inf orders above
    every finite value."""
    rows = _masked_rows(B * n_max, V, seed=B * 77 + V).reshape(B, n_max, V)
    logits_h = W.f32_to_bf16_bits(rows) if dtype == "bf16" else rows
    ref = _chain_accept(logits_h, dtype)
    # the oracle's argmax itself on the crafted cases it decides
    am = ref["argmax"].reshape(-1)
    for r in range(B * n_max):
        if r % 6 == 1:
            assert am[r] == 0
        elif r % 6 == 3:
            assert am[r] == V - 1
