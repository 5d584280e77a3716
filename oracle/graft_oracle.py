"""Plain CPU oracle for one prune-then-graft speculative-decoding step.

TEST INFRASTRUCTURE ONLY.  This module is the correctness reference for the
HIP library.  Only the test suite, the smoke check and the CPU-baseline leg of
the benchmark may import it; the library and its Python binding never do, and
this module imports nothing from them.  It is deliberately slow and literal:
Python loops over tree nodes, numpy for the dense arithmetic, float64
throughout for attention.

Sources (cited below by tag; the pages carry no section numbers, so the
paragraph is named by its content):
  [AT]        "Draft Less, Retrieve More: hybrid tree construction for
              speculative decoding", Korean summary article on aitrends.kr.
  [AT-steps]  its three-point summary paragraph (pruning caps acceptance;
              retrieval from an on-GPU adjacency matrix starting at the root
              refills the released slots; verification budget unchanged).
  [AT-method] its five-step method paragraph (c_d per depth, per-stage split
              Kmax = K_draft_s + K_ret_s, templates G_ret_s filled from M
              starting at the root, gate g_s, hybrid merge, online update).
  [AT-arch]   its architecture paragraph (four axes; pruning at d0/d1/d5 with
              thresholds tau_d; smaller stage index gives retrieval more
              budget; per-stage template prefixes of a base-tree envelope;
              T_s = T_draft_s U G_ret_s with |T_s| = Kmax; one target forward
              with tree attention; retrieval nodes are proposals; lossless).
  [CP]        the paper's English abstract on chatpaper.ai (draft-then-verify,
              pruned positions filled with retrieved tokens, lossless).

Where the pages leave a step open, the reading taken is stated in the function
that implements it; the full list of readings lives with the design notes.

O5 (append_kv) commits the accepted path to the KV cache, the step that
follows verification when decoding continues; O6 (accept_sample) is the
temperature > 0 acceptance; O7 (rope, tree_attention_rope, append_kv_rope)
rotates queries and keys by their tree positions inside those two steps.

Conventions shared with the C header (by specification, not by code):
  * draft arrays  [B][n_draft_max]: parent (-1 = child of the root; otherwise
    an earlier index), token, conf (float32);
  * hybrid tree   [B][n_max] with n_max = kmax + 1: token, parent, pos,
    mask [B][n_max][W] uint32 (bit j of word j // 32), W = ceil(n_max / 32);
  * adjacency M   ids int32 [V][S], scores float32 [V][S];
  * K cache pages [blocks][Hkv][block][D] (token-major), V cache pages
    [blocks][Hkv][D][block] (dim-major);
  * q, out        [B][n_max][Hq][D]; k_tree, v_tree [B][n_max][Hkv][D].
"""

from __future__ import annotations

from collections import Counter

import numpy as np

NO_NODE = -1


# ----------------------------------------------------------------------------
# dtype helpers (bf16 is carried as raw uint16 bit patterns)
# ----------------------------------------------------------------------------

def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to float64."""
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def as_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 view of an input given as fp32 values or bf16 bits."""
    if dtype == "bf16":
        return bf16_bits_to_f64(x)
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


def mask_words(n_max: int) -> int:
    return (n_max + 31) // 32


# ----------------------------------------------------------------------------
# O1: hybrid tree construction  ([AT-steps], [AT-method], [AT-arch], [CP])
# ----------------------------------------------------------------------------

def _draft_depths(parent: np.ndarray) -> list[int]:
    """Draft depth index: a child of the root has depth 0 (so 'd0' is the
    first drafted level), a child of a depth-d node has depth d + 1."""
    depth: list[int] = []
    for i, p in enumerate(parent):
        if p < 0:
            depth.append(0)
        else:
            if p >= i:
                raise ValueError("draft parent must precede its child")
            depth.append(depth[p] + 1)
    return depth


def _firing_stage(depth, conf, stage_depth, stage_tau):
    """[AT-method]/[AT-arch]: at each pruning checkpoint d_s the depth
    confidence c_d is compared with tau_s and the gate g_s decides whether the
    draft is cut there.  Readings: c_d is the largest confidence among the
    nodes at depth d; the gate fires when c_d < tau_s (strict); a checkpoint
    with no node at its depth does not fire; the first firing checkpoint (in
    ascending depth) wins.  Returns the stage index or None."""
    for s, (d, tau) in enumerate(zip(stage_depth, stage_tau)):
        at_d = [np.float32(conf[i]) for i in range(len(depth)) if depth[i] == d]
        if not at_d:
            continue
        c_d = max(at_d)
        if c_d < np.float32(tau):
            return s
    return None


def build_tree_one(cfg: dict, parent, token, conf, root_token: int,
                   prefix_len: int, m_ids: np.ndarray):
    """Build one hybrid tree.  Returns a dict with the compact node lists
    (before padding) plus the firing stage and the number of kept drafts.

    Steps, in the pages' order:
      1. pruning releases budget ([AT-method] first step): find the firing
         stage s*, keep drafts no deeper than its checkpoint, capped at
         K_draft = Kmax - K_ret_{s*} ([AT-method] budget split; [AT-arch]
         smaller s => larger K_ret).  With no firing stage the cap is
         Kmax - k_ret_none.
      2. retrieval fills the template ([AT-method] second step, [AT-arch]
         template prefixes): the first Kmax - n_kept slots of the base-tree
         envelope are filled by M lookups that start at the root token
         ([AT-steps]).  Reading: the released budget is filled back so that
         drafts + retrieval proposals total Kmax ([AT-steps] budget unchanged,
         [AT-arch] |T_s| = Kmax).
      3. merge into one tree ([AT-method] third step): root, then kept drafts
         in input order, then valid retrieval slots in envelope order.
    """
    kmax = int(cfg["kmax"])
    stage_depth = list(cfg["stage_depth"])
    stage_tau = [np.float32(t) for t in cfg["stage_tau"]]
    stage_k_ret = list(cfg["stage_k_ret"])
    k_ret_none = int(cfg.get("k_ret_none", 0))
    env_parent = list(cfg["env_parent"])
    env_rank = list(cfg["env_rank"])
    if len(env_parent) < kmax:
        raise ValueError("envelope must hold at least kmax slots")

    n = len(parent)
    depth = _draft_depths(parent)
    stage = _firing_stage(depth, conf, stage_depth, stage_tau)

    # Step 1: candidates and the K_draft cap.  Reading: a firing checkpoint
    # at depth d keeps the drafted levels 0..d and stops drafting below.
    if stage is None:
        candidates = list(range(n))
        k_ret = k_ret_none
    else:
        candidates = [i for i in range(n) if depth[i] <= stage_depth[stage]]
        k_ret = stage_k_ret[stage]
    k_draft = kmax - k_ret

    # Reading: the drafts that survive the cap are those with the highest
    # path confidence (minimum confidence along the root path), ties to the
    # lower index.  A parent's path confidence is never below its child's and
    # a parent precedes its child, so the kept set is closed under ancestors.
    path_min = []
    for i in range(n):
        c = np.float32(conf[i])
        path_min.append(c if parent[i] < 0 else min(c, path_min[parent[i]]))
    ranked = sorted(candidates, key=lambda i: (-float(path_min[i]), i))
    kept = sorted(ranked[:max(0, min(k_draft, len(candidates)))])
    n_kept = len(kept)

    # Step 2: retrieval slots of the envelope prefix.  Slot j hangs below the
    # root (env_parent < 0) or below an earlier slot; its token is column
    # env_rank[j] of M's row for the parent's token.  Reading: an empty M
    # entry (-1) drops the slot and every slot below it.
    k_fill = kmax - n_kept
    slot_valid: list[bool] = []
    slot_token: list[int] = []
    for j in range(k_fill):
        p = env_parent[j]
        if p < 0:
            parent_ok, parent_tok = True, int(root_token)
        else:
            if p >= j:
                raise ValueError("envelope parent must precede its slot")
            parent_ok, parent_tok = slot_valid[p], slot_token[p]
        if parent_ok:
            tok = int(m_ids[parent_tok][env_rank[j]])
            ok = tok >= 0
        else:
            tok, ok = -1, False
        slot_valid.append(ok)
        slot_token.append(tok)

    # Step 3: merge.  Node 0 is the root (already verified, not part of Kmax).
    out_token = [int(root_token)]
    out_parent = [NO_NODE]
    draft_new = {}
    for i in kept:
        draft_new[i] = len(out_token)
        out_token.append(int(token[i]))
        out_parent.append(0 if parent[i] < 0 else draft_new[parent[i]])
    slot_new = {}
    for j in range(k_fill):
        if not slot_valid[j]:
            continue
        slot_new[j] = len(out_token)
        out_token.append(slot_token[j])
        out_parent.append(0 if env_parent[j] < 0 else slot_new[env_parent[j]])

    # Tree depth (root = 0), position ids and ancestor-or-self sets.
    n_nodes = len(out_token)
    tdepth = []
    anc = []
    for i in range(n_nodes):
        p = out_parent[i]
        tdepth.append(0 if p < 0 else tdepth[p] + 1)
        anc.append({i} if p < 0 else anc[p] | {i})
    pos = [int(prefix_len) + d for d in tdepth]
    return {
        "token": out_token, "parent": out_parent, "pos": pos, "anc": anc,
        "n_nodes": n_nodes, "stage": -1 if stage is None else stage,
        "n_kept": n_kept,
    }


def build_tree(cfg: dict, draft_parent, draft_token, draft_conf, n_draft,
               root_token, prefix_len, m_ids):
    """Batched O1 with the padded output layout of the C header.

    Returns dict of numpy arrays: token/parent/pos int32 [B][n_max],
    mask uint32 [B][n_max][W], n_nodes int32 [B], stage int32 [B],
    n_kept int32 [B].  Rows at or beyond n_nodes hold -1 (mask 0)."""
    kmax = int(cfg["kmax"])
    n_max = kmax + 1
    W = mask_words(n_max)
    B = len(n_draft)
    tok = np.full((B, n_max), -1, np.int32)
    par = np.full((B, n_max), -1, np.int32)
    pos = np.full((B, n_max), -1, np.int32)
    mask = np.zeros((B, n_max, W), np.uint32)
    n_nodes = np.zeros(B, np.int32)
    stage = np.zeros(B, np.int32)
    n_kept = np.zeros(B, np.int32)
    for b in range(B):
        n = int(n_draft[b])
        t = build_tree_one(cfg, [int(x) for x in draft_parent[b][:n]],
                           [int(x) for x in draft_token[b][:n]],
                           np.asarray(draft_conf[b][:n], np.float32),
                           int(root_token[b]), int(prefix_len[b]), m_ids)
        nn = t["n_nodes"]
        tok[b, :nn] = t["token"]
        par[b, :nn] = t["parent"]
        pos[b, :nn] = t["pos"]
        for i in range(nn):
            for j in t["anc"][i]:
                mask[b, i, j // 32] |= np.uint32(1) << np.uint32(j % 32)
        n_nodes[b] = nn
        stage[b] = t["stage"]
        n_kept[b] = t["n_kept"]
    return {"token": tok, "parent": par, "pos": pos, "mask": mask,
            "n_nodes": n_nodes, "stage": stage, "n_kept": n_kept}


# ----------------------------------------------------------------------------
# O2: tree-masked verification attention  ([AT-arch] one target forward over
# the existing tree-attention path; [CP] draft-then-verify)
# ----------------------------------------------------------------------------

def gather_prefix(k_cache, v_cache, block_table_row, prefix_len: int, h: int):
    """Prefix keys/values of one sequence and KV head, in token order, read
    through the page table.  K pages are token-major, V pages dim-major."""
    blk = k_cache.shape[2]
    t = np.arange(prefix_len)
    pages = np.asarray(block_table_row)[t // blk]
    K = k_cache[pages, h, t % blk, :]
    V = v_cache[pages, h, :, t % blk]
    return K, V


def tree_attention(q, k_tree, v_tree, k_cache, v_cache, block_table,
                   prefix_len, tree_mask, n_nodes, scale, rows=None):
    """Standard tree attention of the verification pass.

    For sequence b, query head hq (KV head hq // G with G = Hq / Hkv) and tree
    node i < n_nodes[b]: the visible keys are every prefix token of b and the
    tree nodes j whose bit is set in mask[b][i]; the output is
    sum_j softmax_j(scale * q.k_j) v_j.  All arrays are float64 (the caller
    widens bf16 exactly).  Reading: q and k are already rotated by the caller;
    the tree's own K/V live outside the cache.

    rows: optional iterable of (b, i, hq) to evaluate; others stay NaN.
    Returns out [B][n_max][Hq][D] float64."""
    B, n_max, Hq, D = q.shape
    Hkv = k_tree.shape[2]
    G = Hq // Hkv
    out = np.full(q.shape, np.nan)
    if rows is None:
        rows = [(b, i, hq) for b in range(B) for i in range(int(n_nodes[b]))
                for hq in range(Hq)]
    by_group: dict = {}
    for (b, i, hq) in rows:
        by_group.setdefault((b, hq // G), []).append((i, hq))
    for (b, h), items in sorted(by_group.items()):
        Kp, Vp = gather_prefix(k_cache, v_cache, block_table[b], int(prefix_len[b]), h)
        for (i, hq) in items:
            if i >= int(n_nodes[b]):
                continue
            vis = [j for j in range(int(n_nodes[b]))
                   if (int(tree_mask[b, i, j // 32]) >> (j % 32)) & 1]
            K = np.concatenate([Kp, k_tree[b, vis, h, :]], axis=0)
            V = np.concatenate([Vp, v_tree[b, vis, h, :]], axis=0)
            s = (K @ q[b, i, hq, :]) * scale
            w = np.exp(s - s.max())
            out[b, i, hq, :] = (w @ V) / w.sum()
    return out


# ----------------------------------------------------------------------------
# O7: rotary position embedding by tree position, fused into the verification
# attention and the commit ([AT-arch] one target forward with tree attention;
# positions prefix + depth, reading D13).  The pages do not name the target's
# positional scheme; the workloads' targets (Llama 3, Qwen3) use rotary
# embeddings (RoFormer, Su et al. 2021) with the "rotate half" pairing of dim
# i with dim i + D/2.  The caller supplies the table of cosines and sines.
# ----------------------------------------------------------------------------

def rope(x, pos, cos_sin):
    """Rotate the last axis of x (float64, even length D) by positions pos.

    cos_sin is the caller's table [positions][D]: row t holds cos(t w_i) in
    its first D/2 entries and sin(t w_i) in the last D/2.  For i < D/2 the
    pair (x_i, x_{i+D/2}) becomes (x_i c - x_{i+D/2} s, x_{i+D/2} c + x_i s)
    with (c, s) from row pos.  pos broadcasts against x's leading axes."""
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    h = D // 2
    tab = np.asarray(cos_sin, dtype=np.float64)[np.asarray(pos)]
    c, s = tab[..., :h], tab[..., h:]
    x1, x2 = x[..., :h], x[..., h:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def tree_attention_rope(q, k_tree, v_tree, k_cache, v_cache, block_table, prefix_len,
                        tree_mask, n_nodes, tree_pos, cos_sin, scale, rows=None):
    """Tree attention whose queries and tree keys arrive unrotated: node i's
    query and key are rotated by its position tree_pos[b][i] first; the
    cached prefix keys were rotated when they were written.  Then exactly
    `tree_attention`.  All arrays float64 (bf16 widened exactly)."""
    pos = np.asarray(tree_pos)[:, :, None]  # broadcast over heads
    qr = rope(q, pos, cos_sin)
    kr = rope(k_tree, pos, cos_sin)
    return tree_attention(qr, kr, v_tree, k_cache, v_cache, block_table, prefix_len,
                          tree_mask, n_nodes, scale, rows=rows)


def append_kv_rope(k_cache, v_cache, block_table, prefix_len, k_tree, v_tree,
                   path_nodes, accept_len, cos_sin):
    """`append_kv` for unrotated tree keys: the committed key of cache token
    t = prefix_len + j is rope(k_tree[node], t); values are copied.

    k_cache, k_tree float64 (bf16 widened exactly); v arrays of any dtype.
    Returns (k float64 with the committed rows exact, v, new prefix_len)."""
    k, v, new_len = append_kv(k_cache, v_cache, block_table, prefix_len, k_tree, v_tree,
                              path_nodes, accept_len)
    k = np.asarray(k, dtype=np.float64)
    blk = k.shape[2]
    for b in range(len(prefix_len)):
        L = int(accept_len[b])
        P = int(prefix_len[b])
        for j in range(L + 1):
            node = int(path_nodes[b][j])
            t = P + j
            page = int(block_table[b][t // blk])
            k[page, :, t % blk, :] = rope(k_tree[b, node, :, :], t, cos_sin)
    return k, v, new_len


# ----------------------------------------------------------------------------
# O3: lossless greedy acceptance  ([AT-arch] lossless verification with
# retrieval nodes as proposals; [CP] training-free and lossless)
# ----------------------------------------------------------------------------

def accept(logits, dtype: str, tree_token, tree_parent, n_nodes):
    """Greedy verification of the hybrid tree.

    Readings: the target decodes greedily, so a node is accepted when every
    node on its root path carries the target's argmax after its parent; the
    argmax takes the lowest vocabulary index among equal maxima (-0 equals
    +0); the accepted node is the deepest fully matched node, ties to the
    lower node index; the emitted tokens are the path's tokens after the root
    plus the target's argmax after the accepted node (the bonus token).

    Returns argmax [B][n_max] (-1 past n_nodes), accept_len [B],
    path_nodes [B][n_max] and path_tokens [B][n_max + 1] (-1 padded);
    path_tokens[b][0] is the root token."""
    B, n_max = tree_token.shape
    am = np.full((B, n_max), -1, np.int32)
    acc_len = np.zeros(B, np.int32)
    path_nodes = np.full((B, n_max), -1, np.int32)
    path_tokens = np.full((B, n_max + 1), -1, np.int32)
    for b in range(B):
        n = int(n_nodes[b])
        for i in range(n):
            row = as_f64(logits[b, i], dtype)
            am[b, i] = int(np.argmax(row))  # first index among maxima
        depth = [0] * n
        full = [False] * n
        for i in range(n):
            p = int(tree_parent[b, i])
            if p < 0:
                depth[i], full[i] = 0, True
            else:
                depth[i] = depth[p] + 1
                full[i] = full[p] and int(tree_token[b, i]) == int(am[b, p])
        best = max((i for i in range(n) if full[i]), key=lambda i: (depth[i], -i))
        path = []
        x = best
        while x >= 0:
            path.append(x)
            x = int(tree_parent[b, x])
        path.reverse()
        acc_len[b] = depth[best]
        path_nodes[b, :len(path)] = path
        toks = [int(tree_token[b, x]) for x in path] + [int(am[b, best])]
        path_tokens[b, :len(toks)] = toks
    return {"argmax": am, "accept_len": acc_len, "path_nodes": path_nodes,
            "path_tokens": path_tokens}


# ----------------------------------------------------------------------------
# O4: online update of the adjacency table M  ([AT-method] fourth step,
# [AT-arch] online update from the verified tree)
# ----------------------------------------------------------------------------

def transitions(path_tokens, accept_len):
    """Consecutive token pairs of each accepted path including the bonus
    token: accept_len + 1 pairs per path; a negative accept_len skips it."""
    pairs = []
    for p in range(len(accept_len)):
        L = int(accept_len[p])
        for k in range(L + 1):
            pairs.append((int(path_tokens[p][k]), int(path_tokens[p][k + 1])))
    return pairs


def update_adjacency(m_ids, m_scores, path_tokens, accept_len):
    """Batch-synchronous count update of M from verified transitions.

    Readings: M row u is a top-S list of successor tokens with float32
    scores.  Every transition u -> v of the call adds 1 to v's score in row u;
    a successor not yet in the row enters with its count; the row keeps the S
    best entries by (score descending, id ascending) and pads with (-1, 0).
    All transitions of one call are applied together, so the result does not
    depend on their order.  Prompt evidence for long contexts ([AT-method]
    fifth step) is the same update applied to the prompt as one path.

    Returns new (ids, scores) arrays; inputs are not modified."""
    ids = np.array(m_ids, dtype=np.int32, copy=True)
    scores = np.array(m_scores, dtype=np.float32, copy=True)
    V, S = ids.shape
    counts = Counter(transitions(path_tokens, accept_len))
    by_row: dict = {}
    for (u, v), c in counts.items():
        if not (0 <= u < V and 0 <= v < V):
            raise ValueError("transition token out of range")
        by_row.setdefault(u, {})[v] = c
    for u, new in by_row.items():
        cand: dict = {}
        for s in range(S):
            if ids[u, s] >= 0:
                cand[int(ids[u, s])] = float(scores[u, s])
        for v, c in new.items():
            cand[v] = cand.get(v, 0.0) + float(c)
        best = sorted(cand.items(), key=lambda kv: (-kv[1], kv[0]))[:S]
        ids[u, :] = -1
        scores[u, :] = 0.0
        for s, (v, sc) in enumerate(best):
            ids[u, s] = v
            scores[u, s] = np.float32(sc)
    return ids, scores


# ----------------------------------------------------------------------------
# O5: committing the accepted path to the KV cache  ([AT-arch] one target
# forward verifies the tree and decoding continues from the accepted tokens)
# ----------------------------------------------------------------------------

def append_kv(k_cache, v_cache, block_table, prefix_len, k_tree, v_tree,
              path_nodes, accept_len):
    """Write the K/V of each sequence's accepted path into its paged cache.

    Reading: the verified tokens that decoding keeps are the root and the
    accepted nodes, path_nodes[b][0 .. accept_len[b]]; node path_nodes[b][j]
    sits at tree depth j, so its K/V (computed in the verification pass at
    position prefix_len + j) becomes cache token prefix_len + j.  The bonus
    token is not part of the tree: its K/V comes from the next step, where it
    is the root.  K pages are token-major [blocks][Hkv][block][D], V pages
    dim-major [blocks][Hkv][D][block].

    Returns new (k_cache, v_cache, prefix_len); inputs are not modified.
    Raises ValueError if a sequence's pages cannot hold the new tokens."""
    k = np.array(k_cache, copy=True)
    v = np.array(v_cache, copy=True)
    blk = k.shape[2]
    B = len(prefix_len)
    new_len = np.array(prefix_len, dtype=np.int32, copy=True)
    for b in range(B):
        L = int(accept_len[b])
        P = int(prefix_len[b])
        if L < 0:
            continue
        if P + L + 1 > len(block_table[b]) * blk:
            raise ValueError("the page table cannot hold the accepted tokens")
        for j in range(L + 1):
            node = int(path_nodes[b][j])
            t = P + j
            page = int(block_table[b][t // blk])
            k[page, :, t % blk, :] = k_tree[b, node, :, :]
            v[page, :, :, t % blk] = v_tree[b, node, :, :]
        new_len[b] = P + L + 1
    return k, v, new_len


def tree_transitions(tree_token, argmax, n_nodes):
    """Every verified node's transition: (token(i), argmax(i)) for i < n_nodes.

    Reading of the literal wording that M learns from the logits of the
    verified tree ([AT-method] fourth step): each verified node contributes
    the target's greedy continuation after its token, accepted or not.  The
    accepted path's transitions are among them (each accepted node's token is
    its parent's argmax, and the bonus is the last node's argmax)."""
    pairs = []
    for b in range(len(n_nodes)):
        for i in range(int(n_nodes[b])):
            pairs.append((int(tree_token[b][i]), int(argmax[b][i])))
    return pairs


def update_adjacency_tree(m_ids, m_scores, tree_token, argmax, n_nodes):
    """The update of O4 applied to every verified node's transition, as one
    length-2 path per node."""
    pairs = tree_transitions(tree_token, argmax, n_nodes)
    paths = np.array(pairs, dtype=np.int64).reshape(-1, 2)
    return update_adjacency(m_ids, m_scores, paths, np.zeros(len(paths), np.int64))


# ----------------------------------------------------------------------------
# O6: lossless sampling acceptance  ([AT-arch] retrieval nodes are proposals
# like drafts and verification preserves the target distribution; [CP]
# lossless), the temperature > 0 counterpart of O3
# ----------------------------------------------------------------------------

def accept_sample(logits, dtype: str, temperature: float, tree_token, tree_parent,
                  n_nodes, rand_accept, rand_sample):
    """Recursive rejection sampling over the verified tree.

    Reading: every child of a node is a deterministic proposal of its token,
    tried in index order against the node's target distribution
    p = softmax(logits / T).  With residual r (initially p), a proposal of
    token x is accepted iff rand_accept[b][child] < r(x); on rejection x's
    mass is removed and r renormalised (r(x) = 0 afterwards, so a repeated
    token is always rejected).  An accepted child becomes the current node;
    when no child is accepted, the bonus token is the smallest y whose
    cumulative residual mass exceeds rand_sample[b][node] (inverse CDF over
    token ids in increasing order).  The emitted tokens are distributed as
    the target's own samples, whatever the proposals (lossless).

    All arithmetic is float64 from the exact logits.  Returns accept_len,
    path_nodes, path_tokens like `accept`, plus two diagnostics per
    sequence that say how close each decision came to going the other way:
    `margin_accept`, the smallest |u * (1 - removed) - p(x)| over the child
    tests (the test u < r(x) in absolute probability units), and
    `margin_bonus`, the distance of the bonus draw's target from the nearest
    boundary of the sampled token's CDF interval, relative to the residual
    mass.  An implementation whose probabilities carry an error below a
    margin takes the same decision.  `margin_by_depth[b][d]` is the smallest
    child-test margin among the tests at the path's node of depth d (inf
    where none was made): decisions before the first close one are certain."""
    lg = as_f64(np.asarray(logits), dtype)
    B, n_max, V = lg.shape
    T = float(temperature)
    accept_len = np.zeros(B, np.int32)
    path_nodes = np.full((B, n_max), -1, np.int32)
    path_tokens = np.full((B, n_max + 1), -1, np.int32)
    margin_accept = np.full(B, np.inf)
    margin_bonus = np.full(B, np.inf)
    margin_by_depth = np.full((B, n_max), np.inf)
    for b in range(B):
        n = int(n_nodes[b])
        node = 0
        path = [0]
        while True:
            z = lg[b, node] / T
            p = np.exp(z - z.max())
            p /= p.sum()
            removed = 0.0
            gone = set()
            nxt = -1
            for c in range(node + 1, n):
                if int(tree_parent[b, c]) != node:
                    continue
                x = int(tree_token[b, c])
                if x in gone:
                    continue
                thr = p[x] / (1.0 - removed) if removed < 1.0 else 0.0
                u = float(rand_accept[b, c])
                margin_accept[b] = min(margin_accept[b], abs(u * (1.0 - removed) - p[x]))
                d = len(path) - 1
                margin_by_depth[b, d] = min(margin_by_depth[b, d], abs(u * (1.0 - removed) - p[x]))
                if u < thr:
                    nxt = c
                    break
                gone.add(x)
                removed += p[x]
            if nxt < 0:
                r = p.copy()
                for x in gone:
                    r[x] = 0.0
                cdf = np.cumsum(r)
                target = float(rand_sample[b, node]) * cdf[-1]
                y = int(np.searchsorted(cdf, target, side="right"))
                y = min(y, V - 1)
                lo = cdf[y - 1] if y > 0 else 0.0
                m = min(abs(target - lo), abs(cdf[y] - target))
                margin_bonus[b] = min(margin_bonus[b], m / max(cdf[-1], 1e-300))
                bonus = y
                break
            node = nxt
            path.append(node)
        accept_len[b] = len(path) - 1
        path_nodes[b, :len(path)] = path
        path_tokens[b, :len(path)] = [int(tree_token[b, x]) for x in path]
        path_tokens[b, len(path)] = bonus
    return {"accept_len": accept_len, "path_nodes": path_nodes,
            "path_tokens": path_tokens, "margin_accept": margin_accept,
            "margin_bonus": margin_bonus, "margin_by_depth": margin_by_depth}
