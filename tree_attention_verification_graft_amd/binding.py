"""ctypes binding of libgraft with the same function names as the C ABI.

Argument marshalling only: every function takes torch tensors that already
live on the GPU, checks dtype/shape/contiguity on the host, and passes raw
device pointers plus torch's current HIP stream to the library.  Nothing here
computes any part of the step.  If libgraft.so is missing the import fails;
there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgraft.so")

GRAFT_F32 = 0
GRAFT_BF16 = 1
MAX_STAGES = 8
MAX_NODES = 128
MAX_TOP_S = 32

EXPORTED = [
    "graft_build_tree", "graft_tree_attention_workspace_size",
    "graft_tree_attention_plan", "graft_tree_attention", "graft_tree_attention_noalloc",
    "graft_accept_workspace_size", "graft_accept",
    "graft_accept_sample_workspace_size", "graft_accept_sample",
    "graft_update_adjacency_workspace_size", "graft_update_adjacency",
    "graft_update_adjacency_tree_workspace_size", "graft_update_adjacency_tree",
    "graft_append_kv", "graft_tree_attention_rope", "graft_append_kv_rope",
    "graft_last_error", "graft_version",
]


class GraftError(RuntimeError):
    pass


class AttentionPlan(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "matrix_cores", "n_row_groups", "rows_per_group", "n_splits", "tiles_per_split",
        "tree_shift", "key_pairs", "longest_first", "workgroups")]


class TreeConfig(ctypes.Structure):
    _fields_ = [
        ("kmax", ctypes.c_int32),
        ("n_stages", ctypes.c_int32),
        ("k_ret_none", ctypes.c_int32),
        ("stage_depth", ctypes.c_int32 * MAX_STAGES),
        ("stage_tau", ctypes.c_float * MAX_STAGES),
        ("stage_k_ret", ctypes.c_int32 * MAX_STAGES),
        ("env_len", ctypes.c_int32),
        ("env_parent", ctypes.c_int32 * (MAX_NODES - 1)),
        ("env_rank", ctypes.c_int32 * (MAX_NODES - 1)),
    ]


def make_config(cfg: dict) -> TreeConfig:
    """Pack a tree-config dict (kmax, stage_depth, stage_tau, stage_k_ret,
    k_ret_none, env_parent, env_rank) into the C struct."""
    c = TreeConfig()
    c.kmax = int(cfg["kmax"])
    depth = list(cfg["stage_depth"])
    if len(depth) > MAX_STAGES:
        raise GraftError("too many pruning stages")
    c.n_stages = len(depth)
    c.k_ret_none = int(cfg.get("k_ret_none", 0))
    for s, d in enumerate(depth):
        c.stage_depth[s] = int(d)
        c.stage_tau[s] = float(cfg["stage_tau"][s])
        c.stage_k_ret[s] = int(cfg["stage_k_ret"][s])
    env_p, env_r = list(cfg["env_parent"]), list(cfg["env_rank"])
    if len(env_p) > MAX_NODES - 1 or len(env_p) != len(env_r):
        raise GraftError("bad envelope")
    c.env_len = len(env_p)
    for j, (pp, rr) in enumerate(zip(env_p, env_r)):
        c.env_parent[j] = int(pp)
        c.env_rank[j] = int(rr)
    return c


def _load(path=LIB_PATH):
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built; run __graft_entry__.build()")
    lib = ctypes.CDLL(path)
    P, I, SZ, I64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t, ctypes.c_int64
    sig = {
        "graft_build_tree": [ctypes.POINTER(TreeConfig), I, I, P, P, P, P, P, P, P, I, I,
                             P, P, P, P, P, P, P],
        "graft_tree_attention_workspace_size": [I, I, I, I, I, I, I, I64],
        "graft_tree_attention_plan": [I, I, I, I, I, I, I, I64, ctypes.POINTER(AttentionPlan)],
        "graft_tree_attention": [I, I, I, I, I, I, P, P, P, P, P, I, P, I, P, I, I64, P, P,
                                 ctypes.c_float, P, P, SZ, P],
        "graft_tree_attention_noalloc": [I, I, I, I, I, I, P, P, P, P, P, I, P, I, P, I, I64, P,
                                         P, ctypes.c_float, P, P],
        "graft_accept_workspace_size": [I, I, I],
        "graft_accept": [I, I, I, I, P, P, P, P, P, P, P, P, P, P, SZ, P],
        "graft_accept_sample_workspace_size": [I, I, I, I],
        "graft_accept_sample": [I, I, I, I, P, ctypes.c_float, P, P, P, P, P, P, P, P, P, SZ,
                                P],
        "graft_update_adjacency_workspace_size": [I, I],
        "graft_update_adjacency": [P, P, I, I, I, I, P, P, P, SZ, P],
        "graft_update_adjacency_tree_workspace_size": [I, I],
        "graft_update_adjacency_tree": [P, P, I, I, I, I, P, P, P, P, SZ, P],
        "graft_append_kv": [I, I, I, I, I, P, P, P, P, I, I, P, I, P, P, P, P, P],
        "graft_tree_attention_rope": [I, I, I, I, I, I, P, P, P, P, P, I, P, I, P, I, I64, P, P,
                                      P, P, I, ctypes.c_float, P, P, SZ, P],
        "graft_append_kv_rope": [I, I, I, I, I, P, P, P, P, I, I, P, I, P, P, P, P, P, I, P],
        "graft_last_error": [],
        "graft_version": [],
    }
    for name, args in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        if name.endswith("_workspace_size"):
            f.restype = SZ
        elif name in ("graft_last_error", "graft_version"):
            f.restype = ctypes.c_char_p
        else:
            f.restype = ctypes.c_int32
    return lib


_lib = _load()


def lib():
    return _lib


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise GraftError("tensor arguments must be on the GPU")
    if not t.is_contiguous():
        raise GraftError("tensor arguments must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _check(status, what):
    if status != 0:
        msg = _lib.graft_last_error().decode()
        raise GraftError(f"{what} failed ({status}): {msg}")


def _expect(t, dtype, shape, name):
    if t.dtype != dtype:
        raise GraftError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise GraftError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")


def _dtype_code(t):
    if t.dtype == torch.bfloat16:
        return GRAFT_BF16
    if t.dtype == torch.float32:
        return GRAFT_F32
    raise GraftError(f"unsupported dtype {t.dtype}")


def mask_words(n_max: int) -> int:
    return (n_max + 31) // 32


# --------------------------------------------------------------- the calls

def graft_build_tree(cfg, draft_parent, draft_token, draft_conf, n_draft, root_token,
                     prefix_len, m_ids, tree_token, tree_parent, tree_pos, tree_mask,
                     n_nodes, stage_out, stream=None):
    c = cfg if isinstance(cfg, TreeConfig) else make_config(cfg)
    B, nd = draft_parent.shape
    V, S = m_ids.shape
    n_max = c.kmax + 1
    i32 = torch.int32
    for t, n in ((draft_parent, "draft_parent"), (draft_token, "draft_token")):
        _expect(t, i32, (B, nd), n)
    _expect(draft_conf, torch.float32, (B, nd), "draft_conf")
    for t, n in ((n_draft, "n_draft"), (root_token, "root_token"), (prefix_len, "prefix_len"),
                 (n_nodes, "n_nodes"), (stage_out, "stage_out")):
        _expect(t, i32, (B,), n)
    _expect(m_ids, i32, (V, S), "m_ids")
    for t, n in ((tree_token, "tree_token"), (tree_parent, "tree_parent"),
                 (tree_pos, "tree_pos")):
        _expect(t, i32, (B, n_max), n)
    _expect(tree_mask, i32, (B, n_max, mask_words(n_max)), "tree_mask")
    st = _lib.graft_build_tree(ctypes.byref(c), B, nd, _ptr(draft_parent), _ptr(draft_token),
                               _ptr(draft_conf), _ptr(n_draft), _ptr(root_token),
                               _ptr(prefix_len), _ptr(m_ids), V, S, _ptr(tree_token),
                               _ptr(tree_parent), _ptr(tree_pos), _ptr(tree_mask),
                               _ptr(n_nodes), _ptr(stage_out), _stream(stream))
    _check(st, "graft_build_tree")


def graft_tree_attention_workspace_size(dtype_code, batch, n_max, hq, hkv, head_dim,
                                        max_prefix, sum_prefix=0):
    return int(_lib.graft_tree_attention_workspace_size(dtype_code, batch, n_max, hq, hkv,
                                                        head_dim, max_prefix, int(sum_prefix)))


def graft_tree_attention_plan(dtype_code, batch, n_max, hq, hkv, head_dim, max_prefix,
                              sum_prefix=0) -> dict:
    """The attention launch plan for these shapes, as a dict of the
    graft_attention_plan fields."""
    pl = AttentionPlan()
    _check(_lib.graft_tree_attention_plan(dtype_code, batch, n_max, hq, hkv, head_dim,
                                          int(max_prefix), int(sum_prefix), ctypes.byref(pl)),
           "graft_tree_attention_plan")
    return {n: int(getattr(pl, n)) for n, _ in AttentionPlan._fields_}


def graft_tree_attention(q, k_tree, v_tree, k_cache, v_cache, block_table, prefix_len,
                         max_prefix, tree_mask, n_nodes, scale, out, workspace,
                         stream=None, sum_prefix=0):
    B, n_max, hq, D = q.shape
    hkv = k_tree.shape[2]
    nblk, _, blk, _ = k_cache.shape
    dt = _dtype_code(q)
    for t, n in ((k_tree, "k_tree"), (v_tree, "v_tree")):
        _expect(t, q.dtype, (B, n_max, hkv, D), n)
    _expect(k_cache, q.dtype, (nblk, hkv, blk, D), "k_cache")
    _expect(v_cache, q.dtype, (nblk, hkv, D, blk), "v_cache")
    _expect(out, q.dtype, (B, n_max, hq, D), "out")
    _expect(tree_mask, torch.int32, (B, n_max, mask_words(n_max)), "tree_mask")
    if block_table.dtype != torch.int32 or block_table.dim() != 2 or block_table.shape[0] != B:
        raise GraftError("block_table: expected int32 [batch][max_blocks]")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = _lib.graft_tree_attention(dt, B, n_max, hq, hkv, D, _ptr(q), _ptr(k_tree),
                                   _ptr(v_tree), _ptr(k_cache), _ptr(v_cache), blk,
                                   _ptr(block_table), block_table.shape[1], _ptr(prefix_len),
                                   int(max_prefix), int(sum_prefix), _ptr(tree_mask),
                                   _ptr(n_nodes),
                                   float(scale), _ptr(out), _ptr(workspace), ws_bytes,
                                   _stream(stream))
    _check(st, "graft_tree_attention")


def graft_tree_attention_noalloc(q, k_tree, v_tree, k_cache, v_cache, block_table,
                                 prefix_len, max_prefix, tree_mask, n_nodes, scale, out,
                                 stream=None, sum_prefix=0):
    """graft_tree_attention with the library's own device scratch in place of
    a caller workspace."""
    B, n_max, hq, D = q.shape
    hkv = k_tree.shape[2]
    nblk, _, blk, _ = k_cache.shape
    dt = _dtype_code(q)
    for t, n in ((k_tree, "k_tree"), (v_tree, "v_tree")):
        _expect(t, q.dtype, (B, n_max, hkv, D), n)
    _expect(k_cache, q.dtype, (nblk, hkv, blk, D), "k_cache")
    _expect(v_cache, q.dtype, (nblk, hkv, D, blk), "v_cache")
    _expect(out, q.dtype, (B, n_max, hq, D), "out")
    _expect(tree_mask, torch.int32, (B, n_max, mask_words(n_max)), "tree_mask")
    if block_table.dtype != torch.int32 or block_table.dim() != 2 or block_table.shape[0] != B:
        raise GraftError("block_table: expected int32 [batch][max_blocks]")
    st = _lib.graft_tree_attention_noalloc(dt, B, n_max, hq, hkv, D, _ptr(q), _ptr(k_tree),
                                           _ptr(v_tree), _ptr(k_cache), _ptr(v_cache), blk,
                                           _ptr(block_table), block_table.shape[1],
                                           _ptr(prefix_len), int(max_prefix), int(sum_prefix),
                                           _ptr(tree_mask), _ptr(n_nodes), float(scale),
                                           _ptr(out), _stream(stream))
    _check(st, "graft_tree_attention_noalloc")


def graft_tree_attention_rope(q, k_tree, v_tree, k_cache, v_cache, block_table, prefix_len,
                              max_prefix, tree_mask, n_nodes, tree_pos, rope_cos_sin, scale,
                              out, workspace, stream=None, sum_prefix=0):
    B, n_max, hq, D = q.shape
    hkv = k_tree.shape[2]
    nblk, _, blk, _ = k_cache.shape
    dt = _dtype_code(q)
    for t, n in ((k_tree, "k_tree"), (v_tree, "v_tree")):
        _expect(t, q.dtype, (B, n_max, hkv, D), n)
    _expect(k_cache, q.dtype, (nblk, hkv, blk, D), "k_cache")
    _expect(v_cache, q.dtype, (nblk, hkv, D, blk), "v_cache")
    _expect(out, q.dtype, (B, n_max, hq, D), "out")
    _expect(tree_mask, torch.int32, (B, n_max, mask_words(n_max)), "tree_mask")
    _expect(tree_pos, torch.int32, (B, n_max), "tree_pos")
    if rope_cos_sin.dtype != torch.float32 or rope_cos_sin.dim() != 2 or \
            rope_cos_sin.shape[1] != D:
        raise GraftError("rope_cos_sin: expected float32 [positions][head_dim]")
    if block_table.dtype != torch.int32 or block_table.dim() != 2 or block_table.shape[0] != B:
        raise GraftError("block_table: expected int32 [batch][max_blocks]")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = _lib.graft_tree_attention_rope(dt, B, n_max, hq, hkv, D, _ptr(q), _ptr(k_tree),
                                        _ptr(v_tree), _ptr(k_cache), _ptr(v_cache), blk,
                                        _ptr(block_table), block_table.shape[1],
                                        _ptr(prefix_len), int(max_prefix), int(sum_prefix),
                                        _ptr(tree_mask),
                                        _ptr(n_nodes), _ptr(tree_pos), _ptr(rope_cos_sin),
                                        rope_cos_sin.shape[0], float(scale), _ptr(out),
                                        _ptr(workspace), ws_bytes, _stream(stream))
    _check(st, "graft_tree_attention_rope")


def graft_accept_workspace_size(batch, n_max, vocab):
    return int(_lib.graft_accept_workspace_size(batch, n_max, vocab))


def graft_accept(logits, tree_token, tree_parent, tree_mask, n_nodes, argmax, accept_len,
                 path_nodes, path_tokens, workspace, stream=None):
    B, n_max, V = logits.shape
    dt = _dtype_code(logits)
    i32 = torch.int32
    for t, n in ((tree_token, "tree_token"), (tree_parent, "tree_parent"),
                 (argmax, "argmax"), (path_nodes, "path_nodes")):
        _expect(t, i32, (B, n_max), n)
    _expect(tree_mask, i32, (B, n_max, mask_words(n_max)), "tree_mask")
    _expect(path_tokens, i32, (B, n_max + 1), "path_tokens")
    _expect(accept_len, i32, (B,), "accept_len")
    _expect(n_nodes, i32, (B,), "n_nodes")
    ws_bytes = workspace.numel() * workspace.element_size()
    st = _lib.graft_accept(dt, B, n_max, V, _ptr(logits), _ptr(tree_token), _ptr(tree_parent),
                           _ptr(tree_mask), _ptr(n_nodes), _ptr(argmax), _ptr(accept_len),
                           _ptr(path_nodes), _ptr(path_tokens), _ptr(workspace), ws_bytes,
                           _stream(stream))
    _check(st, "graft_accept")


def graft_accept_sample_workspace_size(dtype, batch, n_max, vocab):
    code = GRAFT_BF16 if dtype in ("bf16", torch.bfloat16) else GRAFT_F32
    return int(_lib.graft_accept_sample_workspace_size(code, batch, n_max, vocab))


def graft_accept_sample(logits, temperature, tree_token, tree_parent, n_nodes, rand_accept,
                        rand_sample, accept_len, path_nodes, path_tokens, workspace,
                        stream=None):
    B, n_max, V = logits.shape
    dt = _dtype_code(logits)
    i32 = torch.int32
    for t, n in ((tree_token, "tree_token"), (tree_parent, "tree_parent"),
                 (path_nodes, "path_nodes")):
        _expect(t, i32, (B, n_max), n)
    _expect(rand_accept, torch.float32, (B, n_max), "rand_accept")
    _expect(rand_sample, torch.float32, (B, n_max), "rand_sample")
    _expect(path_tokens, i32, (B, n_max + 1), "path_tokens")
    _expect(accept_len, i32, (B,), "accept_len")
    _expect(n_nodes, i32, (B,), "n_nodes")
    ws_bytes = workspace.numel() * workspace.element_size()
    st = _lib.graft_accept_sample(dt, B, n_max, V, _ptr(logits), float(temperature),
                                  _ptr(tree_token), _ptr(tree_parent), _ptr(n_nodes),
                                  _ptr(rand_accept), _ptr(rand_sample), _ptr(accept_len),
                                  _ptr(path_nodes), _ptr(path_tokens), _ptr(workspace),
                                  ws_bytes, _stream(stream))
    _check(st, "graft_accept_sample")


def graft_update_adjacency_workspace_size(n_paths, path_stride):
    return int(_lib.graft_update_adjacency_workspace_size(n_paths, path_stride))


def graft_update_adjacency(m_ids, m_scores, path_tokens, accept_len, workspace, stream=None):
    V, S = m_ids.shape
    n_paths, stride = path_tokens.shape
    _expect(m_ids, torch.int32, (V, S), "m_ids")
    _expect(m_scores, torch.float32, (V, S), "m_scores")
    _expect(path_tokens, torch.int32, (n_paths, stride), "path_tokens")
    _expect(accept_len, torch.int32, (n_paths,), "accept_len")
    ws_bytes = workspace.numel() * workspace.element_size()
    st = _lib.graft_update_adjacency(_ptr(m_ids), _ptr(m_scores), V, S, n_paths, stride,
                                     _ptr(path_tokens), _ptr(accept_len), _ptr(workspace),
                                     ws_bytes, _stream(stream))
    _check(st, "graft_update_adjacency")


def graft_update_adjacency_tree_workspace_size(batch, n_max):
    return int(_lib.graft_update_adjacency_tree_workspace_size(batch, n_max))


def graft_update_adjacency_tree(m_ids, m_scores, tree_token, argmax, n_nodes, workspace,
                                stream=None):
    V, S = m_ids.shape
    B, n_max = tree_token.shape
    i32 = torch.int32
    _expect(m_ids, i32, (V, S), "m_ids")
    _expect(m_scores, torch.float32, (V, S), "m_scores")
    _expect(argmax, i32, (B, n_max), "argmax")
    _expect(tree_token, i32, (B, n_max), "tree_token")
    _expect(n_nodes, i32, (B,), "n_nodes")
    ws_bytes = workspace.numel() * workspace.element_size()
    st = _lib.graft_update_adjacency_tree(_ptr(m_ids), _ptr(m_scores), V, S, B, n_max,
                                          _ptr(tree_token), _ptr(argmax), _ptr(n_nodes),
                                          _ptr(workspace), ws_bytes, _stream(stream))
    _check(st, "graft_update_adjacency_tree")


def graft_append_kv(k_tree, v_tree, k_cache, v_cache, block_table, prefix_len, path_nodes,
                    accept_len, new_prefix_len, stream=None):
    B, n_max, hkv, D = k_tree.shape
    nblk, _, blk, _ = k_cache.shape
    dt = _dtype_code(k_tree)
    i32 = torch.int32
    _expect(v_tree, k_tree.dtype, (B, n_max, hkv, D), "v_tree")
    _expect(k_cache, k_tree.dtype, (nblk, hkv, blk, D), "k_cache")
    _expect(v_cache, k_tree.dtype, (nblk, hkv, D, blk), "v_cache")
    _expect(path_nodes, i32, (B, n_max), "path_nodes")
    for t, n in ((prefix_len, "prefix_len"), (accept_len, "accept_len"),
                 (new_prefix_len, "new_prefix_len")):
        _expect(t, i32, (B,), n)
    if block_table.dtype != i32 or block_table.dim() != 2 or block_table.shape[0] != B:
        raise GraftError("block_table: expected int32 [batch][max_blocks]")
    st = _lib.graft_append_kv(dt, B, n_max, hkv, D, _ptr(k_tree), _ptr(v_tree), _ptr(k_cache),
                              _ptr(v_cache), nblk, blk, _ptr(block_table), block_table.shape[1],
                              _ptr(prefix_len), _ptr(path_nodes), _ptr(accept_len),
                              _ptr(new_prefix_len), _stream(stream))
    _check(st, "graft_append_kv")


def graft_append_kv_rope(k_tree, v_tree, k_cache, v_cache, block_table, prefix_len, path_nodes,
                         accept_len, new_prefix_len, rope_cos_sin, stream=None):
    B, n_max, hkv, D = k_tree.shape
    nblk, _, blk, _ = k_cache.shape
    dt = _dtype_code(k_tree)
    i32 = torch.int32
    _expect(v_tree, k_tree.dtype, (B, n_max, hkv, D), "v_tree")
    _expect(k_cache, k_tree.dtype, (nblk, hkv, blk, D), "k_cache")
    _expect(v_cache, k_tree.dtype, (nblk, hkv, D, blk), "v_cache")
    _expect(path_nodes, i32, (B, n_max), "path_nodes")
    for t, n in ((prefix_len, "prefix_len"), (accept_len, "accept_len"),
                 (new_prefix_len, "new_prefix_len")):
        _expect(t, i32, (B,), n)
    if block_table.dtype != i32 or block_table.dim() != 2 or block_table.shape[0] != B:
        raise GraftError("block_table: expected int32 [batch][max_blocks]")
    if rope_cos_sin.dtype != torch.float32 or rope_cos_sin.dim() != 2 or \
            rope_cos_sin.shape[1] != D:
        raise GraftError("rope_cos_sin: expected float32 [positions][head_dim]")
    st = _lib.graft_append_kv_rope(dt, B, n_max, hkv, D, _ptr(k_tree), _ptr(v_tree),
                                   _ptr(k_cache), _ptr(v_cache), nblk, blk, _ptr(block_table),
                                   block_table.shape[1], _ptr(prefix_len), _ptr(path_nodes),
                                   _ptr(accept_len), _ptr(new_prefix_len), _ptr(rope_cos_sin),
                                   rope_cos_sin.shape[0], _stream(stream))
    _check(st, "graft_append_kv_rope")


def graft_last_error():
    return _lib.graft_last_error().decode()


def graft_version():
    return _lib.graft_version().decode()
