"""The oracle's pins must catch plausible mistakes.

Each case plants one mistake into a private copy of the oracle's source (CPU
only; the real module is untouched), points the pin tests at the copy, and
requires at least one pin to fail.
"""
import importlib.util
import inspect
import os
import types

import pytest

import oracle.graft_oracle as real
import test_oracle_accept_update as T_au
import test_oracle_append as T_ap
import test_oracle_rope as T_ro
import test_oracle_sample as T_sa
import test_oracle_update_tree as T_ut
import test_oracle_attention as T_at
import test_oracle_build_tree as T_bt

SRC = inspect.getsource(real)

MUTANTS = [
    ("gate not strict", "if c_d < np.float32(tau):", "if c_d <= np.float32(tau):"),
    ("c_d mean for max", "c_d = max(at_d)", "c_d = np.float32(sum(at_d) / len(at_d))"),
    ("c_d min for max", "c_d = max(at_d)", "c_d = min(at_d)"),
    ("c_d sum for max", "c_d = max(at_d)", "c_d = np.float32(sum(at_d))"),
    ("c_d from the first node", "c_d = max(at_d)", "c_d = at_d[0]"),
    ("K_ret order reversed", "k_ret = stage_k_ret[stage]", "k_ret = stage_k_ret[len(stage_k_ret) - 1 - stage]"),
    ("firing level dropped", "if depth[i] <= stage_depth[stage]]", "if depth[i] < stage_depth[stage]]"),
    ("cap keeps worst drafts", "key=lambda i: (-float(path_min[i]), i)", "key=lambda i: (float(path_min[i]), i)"),
    ("cap by own conf", "path_min.append(c if parent[i] < 0 else min(c, path_min[parent[i]]))", "path_min.append(c)"),
    ("no fill back", "k_fill = kmax - n_kept", "k_fill = min(k_ret, kmax - n_kept)"),
    ("wrong M column", "tok = int(m_ids[parent_tok][env_rank[j]])", "tok = int(m_ids[parent_tok][0])"),
    ("no cascade", "parent_ok, parent_tok = slot_valid[p], slot_token[p]", "parent_ok, parent_tok = True, slot_token[p]"),
    ("slots under root", "out_parent.append(0 if env_parent[j] < 0 else slot_new[env_parent[j]])", "out_parent.append(0)"),
    ("position off by one", "pos = [int(prefix_len) + d for d in tdepth]", "pos = [int(prefix_len) + d + 1 for d in tdepth]"),
    ("mask without self", "anc.append({i} if p < 0 else anc[p] | {i})", "anc.append({i} if p < 0 else set(anc[p]))"),
    ("scale dropped", "s = (K @ q[b, i, hq, :]) * scale", "s = (K @ q[b, i, hq, :])"),
    ("wrong kv head", "by_group.setdefault((b, hq // G), [])", "by_group.setdefault((b, hq % Hkv), [])"),
    ("V read token-major", "V = v_cache[pages, h, :, t % blk]", "V = v_cache[pages, h, t % blk, :]"),
    ("tree keys ignore mask", "if (int(tree_mask[b, i, j // 32]) >> (j % 32)) & 1]", "]"),
    ("partial match accepted", "full[i] = full[p] and int(tree_token[b, i]) == int(am[b, p])", "full[i] = int(tree_token[b, i]) == int(am[b, p])"),
    ("ties to higher node", "key=lambda i: (depth[i], -i))", "key=lambda i: (depth[i], i))"),
    ("bonus from parent", "toks = [int(tree_token[b, x]) for x in path] + [int(am[b, best])]", "toks = [int(tree_token[b, x]) for x in path] + [int(am[b, path[-2] if len(path) > 1 else best])]"),
    ("argmax last index", "am[b, i] = int(np.argmax(row))", "am[b, i] = int(len(row) - 1 - np.argmax(row[::-1]))"),
    ("update ties by id desc", "key=lambda kv: (-kv[1], kv[0]))[:S]", "key=lambda kv: (-kv[1], -kv[0]))[:S]"),
    ("update forgets old score", "cand[v] = cand.get(v, 0.0) + float(c)", "cand[v] = float(c)"),
    ("update ignores repeated transitions", "counts = Counter(transitions(path_tokens, accept_len))", "counts = Counter(set(transitions(path_tokens, accept_len)))"),
    ("bonus transition dropped", "for k in range(L + 1):", "for k in range(L):"),
    ("commit one slot late", "            t = P + j\n            page = int(block_table[b][t // blk])\n            k[page, :, t % blk, :] = k_tree", "            t = P + j + 1\n            page = int(block_table[b][t // blk])\n            k[page, :, t % blk, :] = k_tree"),
    ("commit drops the deepest node", "        for j in range(L + 1):\n            node = int(path_nodes[b][j])\n            t = P + j\n            page = int(block_table[b][t // blk])\n            k[page, :, t % blk, :] = k_tree", "        for j in range(L):\n            node = int(path_nodes[b][j])\n            t = P + j\n            page = int(block_table[b][t // blk])\n            k[page, :, t % blk, :] = k_tree"),
    ("commit length short", "new_len[b] = P + L + 1", "new_len[b] = P + L"),
    ("commit V from K", "v[page, :, :, t % blk] = v_tree[b, node, :, :]", "v[page, :, :, t % blk] = k_tree[b, node, :, :]"),
    ("tree update skips the root", "        for i in range(int(n_nodes[b])):\n            pairs.append", "        for i in range(1, int(n_nodes[b])):\n            pairs.append"),
    ("tree update pairs reversed", "pairs.append((int(tree_token[b][i]), int(argmax[b][i])))", "pairs.append((int(argmax[b][i]), int(tree_token[b][i])))"),
    ("sampling test against p, not the residual", "thr = p[x] / (1.0 - removed) if removed < 1.0 else 0.0", "thr = p[x]"),
    ("bonus keeps rejected mass", "                    r[x] = 0.0\n", "                    r[x] = r[x]\n"),
    ("sampling accepts on u > r(x)", "                if u < thr:\n", "                if u > thr:\n"),
    ("bonus from the root's row", "                r = p.copy()\n", "                r = np.exp(lg[b, 0] / T - (lg[b, 0] / T).max()); r /= r.sum()\n"),
    ("rope sine sign flipped", "[x1 * c - x2 * s, x2 * c + x1 * s]", "[x1 * c + x2 * s, x2 * c - x1 * s]"),
    ("rope pairs adjacent dims", "    x1, x2 = x[..., :h], x[..., h:]\n", "    x1, x2 = x[..., 0::2], x[..., 1::2]\n"),
    ("query not rotated", "    qr = rope(q, pos, cos_sin)\n", "    qr = np.asarray(q, dtype=np.float64)\n"),
    ("tree keys rotated by node index", "    kr = rope(k_tree, pos, cos_sin)\n", "    kr = rope(k_tree, np.arange(k_tree.shape[1])[None, :, None], cos_sin)\n"),
    ("commit rotated at tree depth", "rope(k_tree[b, node, :, :], t, cos_sin)", "rope(k_tree[b, node, :, :], j, cos_sin)"),
]


def _mutant_module(old, new):
    assert SRC.count(old) == 1, old
    src = SRC.replace(old, new)
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src, "oracle_mutant", "exec"), mod.__dict__)
    return mod


def _pin_calls():
    """Every pin test with its parameter values, as zero-arg callables."""
    calls = []
    for idx in range(6):
        calls.append(lambda idx=idx: T_bt.test_golden_examples(idx))
    for s in range(40):
        calls.append(lambda s=s: T_bt.test_invariants_random(s))
    for s in range(30):
        calls.append(lambda s=s: T_bt.test_kept_set_is_best_by_path_confidence(s))
    calls += [T_bt.test_stage_gate_readings, T_bt.test_no_retrieval_mode_is_topk_drafts]
    for order in sorted(T_bt.K_RET_ORDERS):
        calls.append(lambda order=order: T_bt.test_k_ret_orders_on_the_llama3_8b_shape(order))
    for P in [0, 1, 16, 37]:
        calls.append(lambda P=P: T_at.test_chain_equals_causal_attention(P))
    for s in range(12):
        calls.append(lambda s=s: T_at.test_each_row_is_dense_attention_over_its_path(s))
    calls += [T_at.test_uniform_keys_give_mean_of_values,
              T_at.test_single_node_is_decode_attention_and_shift_invariant,
              T_at.test_gather_prefix_layouts]
    for d in ["f32", "bf16"]:
        calls.append(lambda d=d: T_au.test_accept_golden(d))
    for s in range(25):
        calls.append(lambda s=s: T_au.test_accept_equals_greedy_decoding_of_tiny_model(s))
        calls.append(lambda s=s: T_au.test_accept_brute_force_over_paths(s))
    calls += [T_au.test_accept_chain_accepts_matched_prefix,
              T_au.test_accept_lowest_index_ties_in_bf16, T_au.test_update_golden,
              T_au.test_prompt_seeding_is_exact_top_bigrams]
    for s in range(20):
        calls.append(lambda s=s: T_au.test_update_matches_brute_force_and_is_order_free(s))
    for s in range(8):
        calls.append(lambda s=s: T_ap.test_append_identity_layout(s))
    for s in range(6):
        calls.append(lambda s=s: T_ap.test_committed_cache_decodes_like_the_verified_row(s))
    calls.append(T_ap.test_root_only_and_capacity)
    calls.append(T_ut.test_hand_worked_example)
    for s in range(10):
        calls.append(lambda s=s: T_ut.test_transitions_against_numpy_argmax_and_path(s))
    for s in range(6):
        calls.append(lambda s=s: T_ut.test_update_tree_is_the_update_of_its_pairs(s))
    for D in [2, 16, 128]:
        calls.append(lambda D=D: T_ro.test_rope_is_complex_multiplication(D))
    calls.append(T_ro.test_rope_relative_positions_identity_and_norm)
    for s in range(8):
        calls.append(lambda s=s: T_ro.test_tree_attention_rope_brute_force(s))
    calls.append(T_ro.test_append_kv_rope_commits_rotated_keys_at_cache_positions)
    calls += [T_sa.test_root_only_is_inverse_cdf_sampling,
              T_sa.test_repeated_sibling_token_never_accepted,
              T_sa.test_margins_on_a_hand_worked_case]
    for s in range(10):
        calls.append(lambda s=s: T_sa.test_low_temperature_is_greedy(s))
    calls.append(T_sa.test_lossless_first_and_second_token)
    return calls


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(name, old, new, monkeypatch):
    mod = _mutant_module(old, new)
    for t in (T_bt, T_at, T_au, T_ap, T_ut, T_ro, T_sa):
        monkeypatch.setattr(t, "O", mod)
    failed = 0
    for call in _pin_calls():
        try:
            call()
        except Exception:
            failed += 1
            break
    assert failed, f"no pin caught the planted mistake: {name}"
