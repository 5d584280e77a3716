"""Device-side driver for one decode step: uploads a workload's host arrays,
allocates outputs and workspaces with torch, and issues the four libgraft
calls on the current stream.  Plumbing only -- all of the step's arithmetic
runs in the HIP kernels behind the binding.
"""
from __future__ import annotations

import numpy as np
import torch

from . import binding as G


def to_device(a: np.ndarray, device) -> torch.Tensor:
    """Upload a numpy array; uint16 arrays are bf16 bit patterns."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    if a.dtype == np.uint32:
        return torch.from_numpy(a.view(np.int32)).to(device)
    return torch.from_numpy(a).to(device)


def to_host(t: torch.Tensor) -> np.ndarray:
    """Download a tensor; bf16 comes back as uint16 bit patterns."""
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


class DeviceStep:
    """Holds one workload's device buffers and runs the step's four calls.

    `w` is any object with the workload attributes (see workloads.synth)."""

    def __init__(self, w, device="cuda:0", logits=None, alloc_update_for_prompt=False):
        self.w = w
        self.dev = torch.device(device)
        d = self.dev
        i32 = torch.int32
        self.cfg = G.make_config(w.cfg)
        self.n_max = w.kmax + 1
        self.words = G.mask_words(self.n_max)
        B = w.B
        self.draft_parent = to_device(w.draft_parent, d)
        self.draft_token = to_device(w.draft_token, d)
        self.draft_conf = to_device(w.draft_conf, d)
        self.n_draft = to_device(w.n_draft, d)
        self.root_token = to_device(w.root_token, d)
        self.prefix_len = to_device(w.prefix_len, d)
        self.block_table = to_device(w.block_table, d)
        self.m_ids = to_device(w.m_ids, d)
        self.m_scores = to_device(w.m_scores, d)
        self.q = to_device(w.q, d)
        self.k_tree = to_device(w.k_tree, d)
        self.v_tree = to_device(w.v_tree, d)
        self.k_cache = to_device(w.k_cache, d)
        self.v_cache = to_device(w.v_cache, d)
        self.logits = to_device(w.logits if logits is None else logits, d)
        # outputs
        self.tree_token = torch.zeros((B, self.n_max), dtype=i32, device=d)
        self.tree_parent = torch.empty_like(self.tree_token)
        self.tree_pos = torch.empty_like(self.tree_token)
        self.tree_mask = torch.zeros((B, self.n_max, self.words), dtype=i32, device=d)
        self.n_nodes = torch.zeros((B,), dtype=i32, device=d)
        self.stage = torch.zeros((B,), dtype=i32, device=d)
        self.out = torch.empty_like(self.q)
        self.argmax = torch.empty((B, self.n_max), dtype=i32, device=d)
        self.accept_len = torch.empty((B,), dtype=i32, device=d)
        self.path_nodes = torch.empty((B, self.n_max), dtype=i32, device=d)
        self.path_tokens = torch.empty((B, self.n_max + 1), dtype=i32, device=d)
        self.new_prefix_len = torch.empty((B,), dtype=i32, device=d)
        # workspaces
        dt = G.GRAFT_BF16 if w.dtype == "bf16" else G.GRAFT_F32
        # the host-side sum of the prefix lengths steers the attention plan
        self.sum_prefix = int(np.asarray(w.prefix_len, np.int64).sum())
        n = G.graft_tree_attention_workspace_size(dt, B, self.n_max, w.Hq, w.Hkv, w.D,
                                                  w.max_prefix, self.sum_prefix)
        self.attn_ws = torch.empty(max(n, 256), dtype=torch.uint8, device=d)
        n = G.graft_accept_workspace_size(B, self.n_max, w.V)
        self.accept_ws = torch.empty(max(n, 256), dtype=torch.uint8, device=d)
        n = G.graft_accept_sample_workspace_size(w.dtype, B, self.n_max, w.V)
        self.sample_ws = torch.empty(max(n, 256), dtype=torch.uint8, device=d)
        # the random numbers of sampling acceptance (set by the caller)
        self.rand_accept = torch.zeros((B, self.n_max), dtype=torch.float32, device=d)
        self.rand_sample = torch.zeros((B, self.n_max), dtype=torch.float32, device=d)
        n = G.graft_update_adjacency_workspace_size(B, self.n_max + 1)
        if alloc_update_for_prompt and w.prompt is not None:
            n = max(n, G.graft_update_adjacency_workspace_size(1, len(w.prompt)))
        self.update_ws = torch.zeros(n, dtype=torch.uint8, device=d)
        n = G.graft_update_adjacency_tree_workspace_size(B, self.n_max)
        self.update_tree_ws = torch.zeros(n, dtype=torch.uint8, device=d)

    # ---- the four calls
    def build(self):
        G.graft_build_tree(self.cfg, self.draft_parent, self.draft_token, self.draft_conf,
                           self.n_draft, self.root_token, self.prefix_len, self.m_ids,
                           self.tree_token, self.tree_parent, self.tree_pos, self.tree_mask,
                           self.n_nodes, self.stage)

    def attention(self):
        G.graft_tree_attention(self.q, self.k_tree, self.v_tree, self.k_cache, self.v_cache,
                               self.block_table, self.prefix_len, self.w.max_prefix,
                               self.tree_mask, self.n_nodes, self.w.scale, self.out,
                               self.attn_ws, sum_prefix=self.sum_prefix)

    def accept(self):
        G.graft_accept(self.logits, self.tree_token, self.tree_parent, self.tree_mask,
                       self.n_nodes, self.argmax, self.accept_len, self.path_nodes,
                       self.path_tokens, self.accept_ws)

    def accept_sample(self, temperature: float):
        """Sampling acceptance at `temperature` > 0 in place of the greedy
        one, with the random numbers in rand_accept / rand_sample."""
        G.graft_accept_sample(self.logits, temperature, self.tree_token, self.tree_parent,
                              self.n_nodes, self.rand_accept, self.rand_sample,
                              self.accept_len, self.path_nodes, self.path_tokens,
                              self.sample_ws)

    def update(self):
        G.graft_update_adjacency(self.m_ids, self.m_scores, self.path_tokens, self.accept_len,
                                 self.update_ws)

    def update_tree(self):
        """The all-node variant of the update (every verified node's
        transition) in place of the accepted-path update."""
        G.graft_update_adjacency_tree(self.m_ids, self.m_scores, self.tree_token, self.argmax,
                                      self.n_nodes, self.update_tree_ws)

    def set_rope(self, table):
        """The rotary table [positions][head_dim] float32 for the fused
        variants (q, k_tree then hold unrotated projections)."""
        self.rope = torch.from_numpy(np.ascontiguousarray(table, np.float32)).to(self.dev)

    def attention_rope(self):
        G.graft_tree_attention_rope(self.q, self.k_tree, self.v_tree, self.k_cache, self.v_cache,
                                    self.block_table, self.prefix_len, self.w.max_prefix,
                                    self.tree_mask, self.n_nodes, self.tree_pos, self.rope,
                                    self.w.scale, self.out, self.attn_ws,
                                    sum_prefix=self.sum_prefix)

    def append_rope(self):
        G.graft_append_kv_rope(self.k_tree, self.v_tree, self.k_cache, self.v_cache,
                               self.block_table, self.prefix_len, self.path_nodes,
                               self.accept_len, self.new_prefix_len, self.rope)

    def append(self):
        G.graft_append_kv(self.k_tree, self.v_tree, self.k_cache, self.v_cache,
                          self.block_table, self.prefix_len, self.path_nodes, self.accept_len,
                          self.new_prefix_len)

    def step(self):
        self.build()
        self.attention()
        self.accept()
        self.update()

    def seed_from_prompt(self, prompt: np.ndarray):
        """Prompt evidence: the prompt as one path through the update call."""
        path = torch.from_numpy(np.ascontiguousarray(prompt, np.int32)[None]).to(self.dev)
        acc = torch.tensor([len(prompt) - 2], dtype=torch.int32, device=self.dev)
        G.graft_update_adjacency(self.m_ids, self.m_scores, path, acc, self.update_ws)

    def tree_host(self):
        return {"token": to_host(self.tree_token), "parent": to_host(self.tree_parent),
                "pos": to_host(self.tree_pos),
                "mask": to_host(self.tree_mask).view(np.uint32),
                "n_nodes": to_host(self.n_nodes), "stage": to_host(self.stage)}
