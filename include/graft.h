/*
 * libgraft -- the hot path of one prune-then-graft speculative-decoding step
 * on one AMD Instinct MI355X (gfx950), as a C ABI.
 *
 * The method is the one described in "Draft Less, Retrieve More: hybrid tree
 * construction for speculative decoding" (summary article on aitrends.kr and
 * the paper's abstract on chatpaper.ai).  Citations below name the article's
 * paragraphs by content: the three-point summary, the five-step method
 * paragraph and the architecture paragraph.
 *
 * One decode step is four calls, enqueued on the caller's HIP stream:
 *   graft_build_tree        prune the draft tree and refill it from M
 *   graft_tree_attention    verify the hybrid tree with tree-masked attention
 *   graft_accept            greedy (lossless) longest-path acceptance
 *   graft_accept_sample     sampling (temperature > 0) lossless acceptance
 *   graft_update_adjacency  online update of the successor table M
 *   graft_update_adjacency_tree  the same update from every verified node
 *   graft_append_kv         commit of the accepted path to the KV cache
 *   graft_tree_attention_rope, graft_append_kv_rope
 *                           the same two with the rotary position embedding
 *                           fused into their key/query loads
 *
 * Conventions for every call
 *   - Every array argument is DEVICE memory owned by the caller.  The library
 *     never allocates, frees or synchronises; scratch memory comes from a
 *     caller workspace whose size the matching *_workspace_size query gives.
 *   - Calls are asynchronous: they validate host-side scalars, enqueue
 *     kernels on `stream` and return.  A non-zero status means nothing was
 *     enqueued (GRAFT_ERR_INVALID_ARG, GRAFT_ERR_UNSUPPORTED,
 *     GRAFT_ERR_WORKSPACE) or a launch failed (GRAFT_ERR_HIP);
 *     graft_last_error() then returns a message (thread-local).
 *   - Device-side contents are preconditions, not checked: parents precede
 *     children, token ids lie in [0, vocab), counts lie within their bounds.
 *     Out-of-range ids read by a kernel are skipped rather than dereferenced
 *     where noted.
 *   - Hybrid-tree arrays are [batch][n_max] with n_max = kmax + 1 (the root
 *     is node 0 and is not counted in kmax).  Ancestor masks are
 *     [batch][n_max][GRAFT_MASK_WORDS(n_max)] uint32, bit j of word j/32 set
 *     when node j is the node itself or one of its ancestors.
 *   - bf16 tensors are raw 16-bit brain-float values.
 *   - The library is stateless and thread-safe; M is caller state.
 */
#ifndef GRAFT_H
#define GRAFT_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t graft_status;
enum {
  GRAFT_OK = 0,
  GRAFT_ERR_INVALID_ARG = -1,  /* bad scalar, null pointer or shape */
  GRAFT_ERR_UNSUPPORTED = -2,  /* valid but outside what the kernels cover */
  GRAFT_ERR_WORKSPACE = -3,    /* workspace missing or too small */
  GRAFT_ERR_HIP = -4           /* a HIP call or kernel launch failed */
};

typedef enum { GRAFT_F32 = 0, GRAFT_BF16 = 1 } graft_dtype;

enum {
  GRAFT_MAX_STAGES = 8,        /* pruning checkpoints per config */
  GRAFT_MAX_NODES = 128,       /* n_max = kmax + 1 <= 128 */
  GRAFT_MAX_DRAFT = 256,       /* draft nodes per sequence */
  GRAFT_MAX_TOP_S = 32,        /* successors per row of M */
  GRAFT_MAX_KV_HEADS = 65536,  /* hkv: per-page and per-node byte offsets fit 32 bits */
  GRAFT_MAX_VOCAB = 2147418112 /* 2^31 - 2^16: vocabulary chunks index in int32 */
};

#define GRAFT_MASK_WORDS(n_max) (((n_max) + 31) / 32)

/*
 * Tree configuration (HOST memory; copied into the kernel arguments).
 *
 * Pruning checkpoints (method paragraph, first step; architecture paragraph:
 * pruning at d0, d1, d5 with thresholds tau_d): at checkpoint s the largest
 * confidence among draft nodes at draft depth stage_depth[s] (children of
 * the root have depth 0) is compared with stage_tau[s]; the first checkpoint
 * whose value is strictly below its threshold fires.  A checkpoint with no
 * node at its depth does not fire.  stage_depth must be ascending.
 *
 * Budget split (method paragraph: Kmax = K_draft_s + K_ret_s; architecture
 * paragraph: earlier stages give retrieval more): when stage s fires, drafts
 * deeper than stage_depth[s] are dropped and at most kmax - stage_k_ret[s]
 * drafts are kept (those with the highest minimum confidence along their
 * root path, ties to the lower index).  With no firing stage the cap is
 * kmax - k_ret_none.  The released budget is filled back to kmax proposals.
 *
 * Retrieval template (architecture paragraph: per-stage prefixes of a
 * base-tree envelope filled by lookups in M; three-point summary: retrieval
 * starts at the root): slot j of the envelope hangs below the root
 * (env_parent[j] < 0) or below an earlier slot, and takes column
 * env_rank[j] of M's row for its parent's token.  A stage uses the first
 * kmax - n_kept slots.  An empty entry (-1) drops the slot and the slots
 * below it.  env_len >= kmax.
 */
typedef struct {
  int32_t kmax;                               /* 1 .. GRAFT_MAX_NODES - 1 */
  int32_t n_stages;                           /* 0 .. GRAFT_MAX_STAGES */
  int32_t k_ret_none;                         /* 0 .. kmax */
  int32_t stage_depth[GRAFT_MAX_STAGES];
  float stage_tau[GRAFT_MAX_STAGES];
  int32_t stage_k_ret[GRAFT_MAX_STAGES];      /* 0 .. kmax */
  int32_t env_len;                            /* kmax .. GRAFT_MAX_NODES - 1 */
  int32_t env_parent[GRAFT_MAX_NODES - 1];
  int32_t env_rank[GRAFT_MAX_NODES - 1];      /* 0 .. top_s - 1 */
} graft_tree_config;

/*
 * graft_build_tree -- prune the draft tree and graft retrieved tokens.
 * Method paragraph, first to third steps; architecture paragraph
 * (T_s = T_draft_s U G_ret_s, |T_s| = Kmax).
 *
 * Inputs (device):
 *   draft_parent, draft_token  int32 [batch][n_draft_max]; parent -1 means a
 *                              child of the root, otherwise an earlier index
 *   draft_conf                 float [batch][n_draft_max]
 *   n_draft                    int32 [batch], 0 .. n_draft_max
 *   root_token                 int32 [batch], the last verified token
 *   prefix_len                 int32 [batch], tokens already in the KV cache
 *   m_ids                      int32 [vocab][top_s], -1 = empty entry
 * Outputs (device, n_max = cfg->kmax + 1):
 *   tree_token, tree_parent, tree_pos  int32 [batch][n_max]; node 0 is the
 *       root; then the kept drafts in input order; then the valid retrieval
 *       slots in envelope order.  pos = prefix_len + depth (root depth 0).
 *       Rows at or past n_nodes hold -1.
 *   tree_mask   uint32 [batch][n_max][GRAFT_MASK_WORDS(n_max)], 0 past n_nodes
 *   n_nodes     int32 [batch], 1 .. n_max
 *   stage_out   int32 [batch], index of the firing checkpoint or -1
 * One workgroup per sequence.  n_draft_max <= GRAFT_MAX_DRAFT.
 */
graft_status graft_build_tree(const graft_tree_config *cfg, int32_t batch,
                              int32_t n_draft_max, const int32_t *draft_parent,
                              const int32_t *draft_token, const float *draft_conf,
                              const int32_t *n_draft, const int32_t *root_token,
                              const int32_t *prefix_len, const int32_t *m_ids,
                              int32_t vocab, int32_t top_s, int32_t *tree_token,
                              int32_t *tree_parent, int32_t *tree_pos,
                              uint32_t *tree_mask, int32_t *n_nodes,
                              int32_t *stage_out, hipStream_t stream);

/*
 * graft_tree_attention -- verification attention of the hybrid tree in one
 * pass (architecture paragraph: one target forward over the tree-attention
 * path; abstract: draft-then-verify).
 *
 * For sequence b, query head hq (KV head hq / (hq_count / hkv)) and tree
 * node i < n_nodes[b], the visible keys are all prefix tokens
 * 0 .. prefix_len[b]-1 of b and the tree nodes j whose bit is set in
 * tree_mask[b][i]; out = softmax(scale * q.k) weighted sum of v, with a
 * finite scale > 0 (1/sqrt(head_dim) for standard attention).  q and the
 * keys are expected already position-rotated.  Rows i >= n_nodes[b] of out
 * are left untouched.
 *
 * Layouts (device):
 *   q, out           [batch][n_max][hq][head_dim]   (dtype)
 *   k_tree, v_tree   [batch][n_max][hkv][head_dim]  (dtype), this step's
 *                    tree tokens, not yet in the cache
 *   k_cache          [num_blocks][hkv][block_size][head_dim]  token-major pages
 *   v_cache          [num_blocks][hkv][head_dim][block_size]  dim-major pages
 *   block_table      int32 [batch][max_blocks_per_seq]; entries past
 *                    ceil(prefix_len/block_size) are never read
 *   prefix_len       int32 [batch], each <= max_prefix (host bound) and
 *                    <= max_blocks_per_seq * block_size
 *   sum_prefix       host-side sum of prefix_len (<= 0 when unknown): it
 *                    only steers the launch plan (a ragged batch gets more
 *                    prefix splits and its longest work launched first);
 *                    any value gives the same results.  Pass the same value
 *                    to the workspace query.
 * Arithmetic: fp32 accumulation; bf16 output rounded to nearest even.
 * Supported: block_size 16; head_dim 64 or 128 (bf16 with head_dim 128 takes
 * the matrix-core path when n_nodes * group >= 16 rows); hkv <=
 * GRAFT_MAX_KV_HEADS, else GRAFT_ERR_UNSUPPORTED.
 * workspace: >= graft_tree_attention_workspace_size(...) bytes, any contents.
 */
size_t graft_tree_attention_workspace_size(graft_dtype dtype, int32_t batch,
                                           int32_t n_max, int32_t hq, int32_t hkv,
                                           int32_t head_dim, int32_t max_prefix,
                                           int64_t sum_prefix);
/*
 * graft_tree_attention_plan -- the launch plan graft_tree_attention (and
 * graft_tree_attention_rope) uses for these shapes: which kernel runs and how
 * its work is cut.  Host-only, enqueues nothing; the arguments mean what they
 * mean for graft_tree_attention.  Returns GRAFT_ERR_INVALID_ARG for a null
 * `plan` and the call's own shape errors otherwise.
 *   matrix_cores     1: the matrix-core kernel (bf16, head_dim 128, at least
 *                    16 query rows per KV head); 0: one wave per query row
 *   n_row_groups     workgroups along the query rows of one KV head
 *   rows_per_group   query rows (node x group + head-in-group) of the largest
 *                    row group.  Matrix-core plans cut the rows of a KV head
 *                    into 16-row blocks, nb = ceil(n_max * group / 16), and
 *                    give the first (nb mod n_row_groups) groups one block
 *                    more than the others; the wavefront plan has one group
 *   n_splits         prefix splits; above 1 a combine launch merges them
 *   tiles_per_split  64-key prefix tiles per split
 *   tree_shift       split s covers prefix tiles [s tps - shift, (s+1) tps -
 *                    shift): the tree's own tiles count as split 0's first
 *   key_pairs        1: two waves share each 16-row block, one half of each
 *                    64-key tile each
 *   longest_first    1: ragged batch, (sequence, split) work started longest
 *                    first
 *   workgroups       workgroups of the attention launch.  A matrix-core
 *                    launch has one work item per (sequence, KV head, row
 *                    group, split), rounded up to a multiple of 8; without
 *                    longest_first it has at most 256 workgroups (one per
 *                    compute unit), each running its items back to back,
 *                    with longest_first one workgroup per item
 */
typedef struct {
  int32_t matrix_cores, n_row_groups, rows_per_group, n_splits, tiles_per_split,
      tree_shift, key_pairs, longest_first, workgroups;
} graft_attention_plan;
graft_status graft_tree_attention_plan(graft_dtype dtype, int32_t batch, int32_t n_max,
                                       int32_t hq, int32_t hkv, int32_t head_dim,
                                       int32_t max_prefix, int64_t sum_prefix,
                                       graft_attention_plan *plan);
graft_status graft_tree_attention(graft_dtype dtype, int32_t batch, int32_t n_max,
                                  int32_t hq, int32_t hkv, int32_t head_dim,
                                  const void *q, const void *k_tree,
                                  const void *v_tree, const void *k_cache,
                                  const void *v_cache, int32_t block_size,
                                  const int32_t *block_table,
                                  int32_t max_blocks_per_seq,
                                  const int32_t *prefix_len, int32_t max_prefix,
                                  int64_t sum_prefix, const uint32_t *tree_mask,
                                  const int32_t *n_nodes, float scale, void *out,
                                  void *workspace, size_t workspace_bytes,
                                  hipStream_t stream);

/*
 * graft_tree_attention_noalloc -- graft_tree_attention without a caller
 * workspace, for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation).
 * Same arguments, layouts, results and launch plan as graft_tree_attention;
 * the split partials go to a scratch array that the library holds in device
 * memory, GRAFT_NOALLOC_SCRATCH_BYTES on each GPU it runs on, from the
 * first call on that GPU until the process ends.  The call allocates and
 * frees nothing (the first call on a device looks up that device's copy of
 * the array).  A plan whose partials need more than the array holds is
 * rejected with GRAFT_ERR_WORKSPACE before any launch
 * (graft_tree_attention_workspace_size gives the need).  Every call on one
 * GPU shares that GPU's array: calls that overlap on one GPU (concurrent
 * streams, or threads) race and must be ordered by the caller.
 */
#define GRAFT_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
graft_status graft_tree_attention_noalloc(graft_dtype dtype, int32_t batch, int32_t n_max,
                                          int32_t hq, int32_t hkv, int32_t head_dim,
                                          const void *q, const void *k_tree,
                                          const void *v_tree, const void *k_cache,
                                          const void *v_cache, int32_t block_size,
                                          const int32_t *block_table,
                                          int32_t max_blocks_per_seq,
                                          const int32_t *prefix_len, int32_t max_prefix,
                                          int64_t sum_prefix, const uint32_t *tree_mask,
                                          const int32_t *n_nodes, float scale, void *out,
                                          hipStream_t stream);

/*
 * graft_tree_attention_rope -- graft_tree_attention for unrotated queries
 * and tree keys: the rotary position embedding at each node's tree position
 * is fused into their loads (architecture paragraph: the tree-attention
 * verify forward; positions prefix_len + depth as written by
 * graft_build_tree).  The pages do not name the target's positional scheme;
 * this is the published rotary embedding with the rotate-half pairing used
 * by Llama 3 and Qwen3: for i < head_dim/2 the pair (x_i, x_{i+head_dim/2})
 * becomes (x_i c - x_{i+head_dim/2} s, x_{i+head_dim/2} c + x_i s).
 *
 * Node i's query (every head) and key are rotated at position
 * p = tree_pos[b][i]; the cached prefix keys are used as they are (rotated
 * when they were written, e.g. by graft_append_kv_rope).
 *   tree_pos       int32 [batch][n_max] (from graft_build_tree)
 *   rope_cos_sin   float [rope_positions][head_dim], 16-byte aligned: row p
 *                  holds cos(p w_i) for i < head_dim/2, then sin(p w_i)
 *                  (any frequencies w_i, including rescaled ones)
 * Positions outside [0, rope_positions) are a precondition violation; the
 * kernels clamp them into the table.  The rotation is computed in fp32; on
 * the matrix-core path the rotated bf16 inputs are rounded once to bf16
 * before the dot products.  Everything else, workspace included, as
 * graft_tree_attention.
 */
graft_status graft_tree_attention_rope(graft_dtype dtype, int32_t batch, int32_t n_max,
                                       int32_t hq, int32_t hkv, int32_t head_dim,
                                       const void *q, const void *k_tree,
                                       const void *v_tree, const void *k_cache,
                                       const void *v_cache, int32_t block_size,
                                       const int32_t *block_table,
                                       int32_t max_blocks_per_seq,
                                       const int32_t *prefix_len, int32_t max_prefix,
                                       int64_t sum_prefix, const uint32_t *tree_mask,
                                       const int32_t *n_nodes, const int32_t *tree_pos,
                                       const float *rope_cos_sin,
                                       int32_t rope_positions, float scale, void *out,
                                       void *workspace, size_t workspace_bytes,
                                       hipStream_t stream);

/*
 * graft_accept -- lossless greedy acceptance (architecture paragraph:
 * retrieval nodes are proposals like drafts and the output distribution is
 * preserved; abstract: lossless), read for greedy decoding.
 *
 *   argmax[b][i]    lowest vocabulary index among the maxima of logits[b][i]
 *                   (-0 equals +0); -1 for i >= n_nodes[b]
 *   a node is accepted when every node on its root path carries the argmax
 *   of its parent's row; the deepest accepted node wins, ties to the lower
 *   index.
 *   accept_len[b]   depth of the accepted node (0 = only the root)
 *   path_nodes      int32 [batch][n_max]: root .. accepted node, -1 padded
 *   path_tokens     int32 [batch][n_max + 1]: the path's tokens (root token
 *                   first) followed by the accepted node's argmax (bonus),
 *                   -1 padded; accept_len + 2 valid entries
 * Inputs: logits [batch][n_max][vocab] (dtype), vocab <= GRAFT_MAX_VOCAB
 * (else GRAFT_ERR_UNSUPPORTED); tree arrays as produced by graft_build_tree.
 * workspace: >= graft_accept_workspace_size(...) bytes, any contents (one
 * packed value/index key per node row and vocabulary chunk; chunks hold
 * 2048 to 16384 entries).
 * Calls that share one workspace must not overlap.
 */
size_t graft_accept_workspace_size(int32_t batch, int32_t n_max, int32_t vocab);
graft_status graft_accept(graft_dtype dtype, int32_t batch, int32_t n_max,
                          int32_t vocab, const void *logits,
                          const int32_t *tree_token, const int32_t *tree_parent,
                          const uint32_t *tree_mask, const int32_t *n_nodes,
                          int32_t *argmax, int32_t *accept_len,
                          int32_t *path_nodes, int32_t *path_tokens,
                          void *workspace, size_t workspace_bytes,
                          hipStream_t stream);

/*
 * graft_accept_sample -- lossless acceptance when the target samples at
 * temperature T > 0 (architecture paragraph: retrieval nodes are proposals
 * like drafts and verification keeps the target distribution; abstract:
 * lossless), by recursive rejection sampling.
 *
 * Each node's target distribution is p = softmax(logits[b][i] / T).  From
 * the root, the children of the current node are tried in index order, each
 * as a deterministic proposal of its token x: with r the residual
 * distribution (initially p), the child is accepted iff
 * rand_accept[b][child] < r(x); otherwise x's mass is removed from r and r
 * renormalised (so a token repeated among siblings is never accepted).  An
 * accepted child becomes the current node.  When no child is accepted, the
 * bonus token is the smallest y whose cumulative residual mass, over token
 * ids in increasing order, exceeds rand_sample[b][node] * (total residual
 * mass).  The emitted tokens are distributed as samples of the target.
 *
 *   accept_len, path_nodes, path_tokens  as graft_accept (the last valid
 *                   path_tokens entry is the sampled bonus token)
 * Inputs: logits [batch][n_max][vocab] (dtype), finite or -inf;
 * temperature finite and > 0; tree_token, tree_parent int32 [batch][n_max]
 * and n_nodes int32 [batch] as produced by graft_build_tree; rand_accept,
 * rand_sample float32 [batch][n_max] in [0, 1), drawn by the caller (entry
 * [b][i] of rand_accept is child i's test, of rand_sample node i's bonus
 * draw).  Precision: the acceptance tests use probabilities from float32
 * exponentials (relative error below about 1.5e-6), so a test can differ
 * from exact arithmetic only when |u (1 - removed) - p(x)| is below a few
 * 1e-6; the bonus draw uses float64 masses and sums, so it can differ only
 * when rand_sample * (residual mass) lies within about 1e-13 (relative) of
 * a token's cumulative boundary.
 * workspace: >= graft_accept_sample_workspace_size(...) bytes, any contents
 * (chunk statistics, the stop row's residual mass per chunk and a
 * per-sequence record between the launches).  Calls that share one
 * workspace must not overlap.  Trees of at most 384 MiB of logits (and at
 * most 2304 vocabulary chunks of 4096 bf16 or 2048 f32 entries) read every
 * row once, at a cost independent of how deep the walks go; larger ones
 * read the root row and then only the rows a walk reaches, one workgroup
 * per sequence, at a cost that grows with the deepest walk of the batch.
 * vocab <= GRAFT_MAX_VOCAB, else GRAFT_ERR_UNSUPPORTED.
 */
size_t graft_accept_sample_workspace_size(graft_dtype dtype, int32_t batch, int32_t n_max,
                                          int32_t vocab);
graft_status graft_accept_sample(graft_dtype dtype, int32_t batch, int32_t n_max,
                                 int32_t vocab, const void *logits, float temperature,
                                 const int32_t *tree_token, const int32_t *tree_parent,
                                 const int32_t *n_nodes, const float *rand_accept,
                                 const float *rand_sample, int32_t *accept_len,
                                 int32_t *path_nodes, int32_t *path_tokens,
                                 void *workspace, size_t workspace_bytes,
                                 hipStream_t stream);

/*
 * graft_update_adjacency -- online update of M (method paragraph, fourth
 * step: M keeps learning from the verified tree; fifth step: prompt evidence
 * for long contexts, which is this call with the prompt as one path).
 *
 * Path p contributes the transitions (path_tokens[p][k], path_tokens[p][k+1])
 * for k = 0 .. accept_len[p] (the bonus token included); a negative
 * accept_len skips the path; transitions with a token outside [0, vocab)
 * are skipped.  Requires accept_len[p] + 2 <= path_stride.  All transitions
 * of one call are applied together: each adds 1 to its successor's score in
 * the predecessor's row, a successor not yet present enters with its count,
 * and every touched row keeps its top_s best entries by (score descending,
 * id ascending), padded with (-1, 0.0).  Scores are counts: exact while
 * below 2^24.  Rows no transition touches are not written.
 *
 * m_ids int32 [vocab][top_s], m_scores float [vocab][top_s] (updated in
 * place); path_tokens int32 [n_paths][path_stride]; accept_len int32 [n_paths].
 * workspace: >= graft_update_adjacency_workspace_size(n_paths, path_stride)
 * bytes.  It must be zero-filled before its first use.  Every call leaves
 * its hash tables and counters cleared again (the rest of the workspace is
 * scratch that is written before it is read), so one workspace can be
 * reused across calls of any size it covers without clearing.  Its layout
 * depends only on workspace_bytes.  Calls that share one workspace must not
 * overlap.
 */
size_t graft_update_adjacency_workspace_size(int32_t n_paths, int32_t path_stride);
graft_status graft_update_adjacency(int32_t *m_ids, float *m_scores, int32_t vocab,
                                    int32_t top_s, int32_t n_paths,
                                    int32_t path_stride, const int32_t *path_tokens,
                                    const int32_t *accept_len, void *workspace,
                                    size_t workspace_bytes, hipStream_t stream);

/*
 * graft_update_adjacency_tree -- the all-node variant of the online update
 * (method paragraph, fourth step, read literally: M learns from the logits
 * of the whole verified tree).  Every verified node i < n_nodes[b]
 * contributes the transition (tree_token[b][i], argmax[b][i]); the update
 * rule is that of graft_update_adjacency (counts, batch-synchronous, top_s
 * by score descending then id ascending).  The accepted path's transitions
 * are among these.
 *
 * tree_token, argmax int32 [batch][n_max] (from graft_build_tree and
 * graft_accept); n_nodes int32 [batch]; m_ids / m_scores as in
 * graft_update_adjacency.
 * workspace: >= graft_update_adjacency_tree_workspace_size(batch, n_max)
 * bytes, zero-filled before its first use; like graft_update_adjacency,
 * every call leaves it ready for the next.  Calls that share one workspace
 * must not overlap.
 */
size_t graft_update_adjacency_tree_workspace_size(int32_t batch, int32_t n_max);
graft_status graft_update_adjacency_tree(int32_t *m_ids, float *m_scores, int32_t vocab,
                                         int32_t top_s, int32_t batch, int32_t n_max,
                                         const int32_t *tree_token, const int32_t *argmax,
                                         const int32_t *n_nodes, void *workspace,
                                         size_t workspace_bytes, hipStream_t stream);

/*
 * graft_append_kv -- commit the accepted path to the paged KV cache, the
 * step after verification (architecture paragraph: one target forward
 * verifies the hybrid tree and decoding continues from the accepted tokens).
 *
 * For sequence b with L = accept_len[b] >= 0: tree node path_nodes[b][j]
 * (j = 0 .. L: the root, then the accepted nodes, as written by
 * graft_accept) sits at tree depth j, so its K/V (computed in the
 * verification pass at position prefix_len[b] + j) is written to cache
 * token prefix_len[b] + j for every KV head.  new_prefix_len[b] =
 * prefix_len[b] + L + 1, or prefix_len[b] when L < 0.  The bonus token is
 * not in the tree: its K/V comes from the next step, where it is the root.
 *
 * Layouts as graft_tree_attention: k_tree, v_tree [batch][n_max][hkv]
 * [head_dim]; k_cache [num_blocks][hkv][block_size][head_dim] (token-major
 * pages), v_cache [num_blocks][hkv][head_dim][block_size] (dim-major);
 * block_table int32 [batch][max_blocks_per_seq]; path_nodes int32
 * [batch][n_max]; prefix_len, accept_len, new_prefix_len int32 [batch].
 * Precondition: the table maps every position below prefix_len[b] + L + 1
 * to a page in [0, num_blocks).  Positions past max_blocks_per_seq *
 * block_size, pages outside [0, num_blocks) and path entries outside
 * [0, n_max) are skipped (never written).  new_prefix_len must not alias
 * prefix_len.  Only the committed slots of the caches are written.
 */
graft_status graft_append_kv(graft_dtype dtype, int32_t batch, int32_t n_max, int32_t hkv,
                             int32_t head_dim, const void *k_tree, const void *v_tree,
                             void *k_cache, void *v_cache, int32_t num_blocks,
                             int32_t block_size, const int32_t *block_table,
                             int32_t max_blocks_per_seq, const int32_t *prefix_len,
                             const int32_t *path_nodes, const int32_t *accept_len,
                             int32_t *new_prefix_len, hipStream_t stream);

/*
 * graft_append_kv_rope -- graft_append_kv for unrotated tree keys: the key
 * committed to cache token t = prefix_len[b] + j is rotated at position t
 * (the rotary embedding of graft_tree_attention_rope, computed in fp32 and
 * rounded once to the cache dtype); values are copied.  rope_cos_sin and
 * rope_positions as in graft_tree_attention_rope; head_dim even.
 * Everything else as graft_append_kv.
 */
graft_status graft_append_kv_rope(graft_dtype dtype, int32_t batch, int32_t n_max,
                                  int32_t hkv, int32_t head_dim, const void *k_tree,
                                  const void *v_tree, void *k_cache, void *v_cache,
                                  int32_t num_blocks, int32_t block_size,
                                  const int32_t *block_table, int32_t max_blocks_per_seq,
                                  const int32_t *prefix_len, const int32_t *path_nodes,
                                  const int32_t *accept_len, int32_t *new_prefix_len,
                                  const float *rope_cos_sin, int32_t rope_positions,
                                  hipStream_t stream);

/* Message for the last non-OK status returned on this thread. */
const char *graft_last_error(void);

/* Library version string. */
const char *graft_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GRAFT_H */
