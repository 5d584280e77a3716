// Host side of the C ABI: argument validation, launch planning, workspace
// carving.  No allocation, no synchronisation: every call only enqueues
// kernels on the caller's stream.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "graft_internal.h"

#include <algorithm>
#include <mutex>

namespace graft {

static thread_local char g_error[512] = "";

graft_status set_error(graft_status code, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_error, sizeof(g_error), fmt, ap);
  va_end(ap);
  return code;
}

graft_status check_launch(const char *what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return set_error(GRAFT_ERR_HIP, "%s: kernel launch failed: %s", what, hipGetErrorString(e));
  return GRAFT_OK;
}

SampleLayout sample_layout(graft_dtype dtype, int32_t batch, int32_t n_max, int32_t vocab) {
  const size_t wchunks = (size_t)sample_walk_chunks(dtype, vocab);
  // staged: the statistics of every row, sized for the smaller chunks (the
  // most per row); lazy: the root rows' chunk records
  const size_t recs =
      sample_lazy(dtype, batch, n_max, vocab)
          ? (size_t)batch * wchunks * sizeof(RootChunk)
          : (size_t)batch * n_max * sample_stat_chunks(dtype, 2, vocab) * sizeof(ChunkStat);
  SampleLayout l{};
  l.off_chunk_w = align_up(recs, 256);
  l.off_rec = l.off_chunk_w + align_up((size_t)batch * wchunks * sizeof(double), 256);
  l.total = l.off_rec + align_up((size_t)batch * sizeof(SampleRec), 256);
  return l;
}

// Scratch of graft_tree_attention_noalloc (its split partials): one copy on
// each device, looked up once per device with that device current.  Host
// code uses only the looked-up address: the array's own name is a host-side
// stand-in, not a device address.
static __device__ __align__(256) unsigned char scratch[GRAFT_NOALLOC_SCRATCH_BYTES];
namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];

graft_status noalloc_scratch(void **out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess)
    return set_error(GRAFT_ERR_HIP, "graft_tree_attention_noalloc: hipGetDevice: %s",
                     hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return set_error(GRAFT_ERR_UNSUPPORTED, "graft_tree_attention_noalloc: device %d above %d",
                     dev, kMaxDevices - 1);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return set_error(GRAFT_ERR_HIP,
                       "graft_tree_attention_noalloc: scratch lookup on device %d: %s", dev,
                       hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return GRAFT_OK;
}
}  // namespace

}  // namespace graft

using namespace graft;

#define REQUIRE(cond, code, ...)               \
  do {                                         \
    if (!(cond)) return set_error(code, __VA_ARGS__); \
  } while (0)

extern "C" {

const char *graft_last_error(void) { return g_error; }

const char *graft_version(void) { return "libgraft 0.1 (gfx950)"; }

// --------------------------------------------------------------- build tree
graft_status graft_build_tree(const graft_tree_config *cfg, int32_t batch,
                              int32_t n_draft_max, const int32_t *draft_parent,
                              const int32_t *draft_token, const float *draft_conf,
                              const int32_t *n_draft, const int32_t *root_token,
                              const int32_t *prefix_len, const int32_t *m_ids,
                              int32_t vocab, int32_t top_s, int32_t *tree_token,
                              int32_t *tree_parent, int32_t *tree_pos,
                              uint32_t *tree_mask, int32_t *n_nodes,
                              int32_t *stage_out, hipStream_t stream) {
  g_error[0] = 0;
  REQUIRE(cfg, GRAFT_ERR_INVALID_ARG, "graft_build_tree: cfg is null");
  REQUIRE(batch >= 0, GRAFT_ERR_INVALID_ARG, "graft_build_tree: batch < 0");
  REQUIRE(cfg->kmax >= 1 && cfg->kmax <= GRAFT_MAX_NODES - 1, GRAFT_ERR_INVALID_ARG,
          "graft_build_tree: kmax %d outside 1..%d", cfg->kmax, GRAFT_MAX_NODES - 1);
  REQUIRE(cfg->n_stages >= 0 && cfg->n_stages <= GRAFT_MAX_STAGES, GRAFT_ERR_INVALID_ARG,
          "graft_build_tree: n_stages %d outside 0..%d", cfg->n_stages, GRAFT_MAX_STAGES);
  REQUIRE(cfg->k_ret_none >= 0 && cfg->k_ret_none <= cfg->kmax, GRAFT_ERR_INVALID_ARG,
          "graft_build_tree: k_ret_none outside 0..kmax");
  for (int s = 0; s < cfg->n_stages; ++s) {
    REQUIRE(cfg->stage_k_ret[s] >= 0 && cfg->stage_k_ret[s] <= cfg->kmax, GRAFT_ERR_INVALID_ARG,
            "graft_build_tree: stage_k_ret[%d] outside 0..kmax", s);
    REQUIRE(cfg->stage_depth[s] >= 0, GRAFT_ERR_INVALID_ARG,
            "graft_build_tree: stage_depth[%d] < 0", s);
    REQUIRE(s == 0 || cfg->stage_depth[s] > cfg->stage_depth[s - 1], GRAFT_ERR_INVALID_ARG,
            "graft_build_tree: stage_depth must be ascending");
    REQUIRE(!std::isnan(cfg->stage_tau[s]), GRAFT_ERR_INVALID_ARG,
            "graft_build_tree: stage_tau[%d] is NaN", s);
  }
  REQUIRE(cfg->env_len >= cfg->kmax && cfg->env_len <= GRAFT_MAX_NODES - 1,
          GRAFT_ERR_INVALID_ARG, "graft_build_tree: env_len must be in kmax..%d",
          GRAFT_MAX_NODES - 1);
  REQUIRE(top_s >= 1 && top_s <= GRAFT_MAX_TOP_S, GRAFT_ERR_INVALID_ARG,
          "graft_build_tree: top_s outside 1..%d", GRAFT_MAX_TOP_S);
  REQUIRE(vocab >= 1, GRAFT_ERR_INVALID_ARG, "graft_build_tree: vocab < 1");
  for (int j = 0; j < cfg->env_len; ++j) {
    REQUIRE(cfg->env_parent[j] < j, GRAFT_ERR_INVALID_ARG,
            "graft_build_tree: env_parent[%d] must precede its slot", j);
    REQUIRE(cfg->env_rank[j] >= 0 && cfg->env_rank[j] < top_s, GRAFT_ERR_INVALID_ARG,
            "graft_build_tree: env_rank[%d] outside 0..top_s-1", j);
  }
  REQUIRE(n_draft_max >= 0 && n_draft_max <= GRAFT_MAX_DRAFT, GRAFT_ERR_UNSUPPORTED,
          "graft_build_tree: n_draft_max %d outside 0..%d", n_draft_max, GRAFT_MAX_DRAFT);
  if (batch == 0) return GRAFT_OK;
  REQUIRE((n_draft_max == 0 || (draft_parent && draft_token && draft_conf)) && n_draft &&
              root_token && prefix_len && m_ids && tree_token && tree_parent && tree_pos &&
              tree_mask && n_nodes && stage_out,
          GRAFT_ERR_INVALID_ARG, "graft_build_tree: null device pointer");

  BuildParams p{};
  p.cfg = *cfg;
  for (int j = cfg->env_len; j < GRAFT_MAX_NODES - 1; ++j) {
    p.cfg.env_parent[j] = -1;
    p.cfg.env_rank[j] = 0;
  }
  // envelope levels (parents precede their slots, checked above)
  p.env_levels = 0;
  for (int j = 0; j < GRAFT_MAX_NODES - 1; ++j) {
    const int par = j < cfg->env_len ? cfg->env_parent[j] : -1;
    p.env_level[j] = (int8_t)(j >= cfg->env_len ? -1 : par < 0 ? 0 : p.env_level[par] + 1);
    if (j < cfg->env_len) p.env_levels = std::max(p.env_levels, p.env_level[j] + 1);
  }
  p.batch = batch;
  p.n_draft_max = n_draft_max;
  p.vocab = vocab;
  p.top_s = top_s;
  p.n_max = cfg->kmax + 1;
  p.words = GRAFT_MASK_WORDS(p.n_max);
  p.draft_parent = draft_parent;
  p.draft_token = draft_token;
  p.draft_conf = draft_conf;
  p.n_draft = n_draft;
  p.root_token = root_token;
  p.prefix_len = prefix_len;
  p.m_ids = m_ids;
  p.tree_token = tree_token;
  p.tree_parent = tree_parent;
  p.tree_pos = tree_pos;
  p.tree_mask = tree_mask;
  p.n_nodes = n_nodes;
  p.stage_out = stage_out;
  launch_build_tree(p, stream);
  return check_launch("graft_build_tree");
}

// ---------------------------------------------------------------- attention
static graft_status check_attn_shape(graft_dtype dtype, int32_t batch, int32_t n_max,
                                     int32_t hq, int32_t hkv, int32_t head_dim,
                                     int32_t max_prefix) {
  REQUIRE(dtype == GRAFT_F32 || dtype == GRAFT_BF16, GRAFT_ERR_INVALID_ARG,
          "graft_tree_attention: unknown dtype %d", (int)dtype);
  REQUIRE(batch >= 0 && n_max >= 1 && n_max <= GRAFT_MAX_NODES, GRAFT_ERR_INVALID_ARG,
          "graft_tree_attention: batch/n_max out of range");
  REQUIRE(hq >= 1 && hkv >= 1 && hq % hkv == 0, GRAFT_ERR_INVALID_ARG,
          "graft_tree_attention: hq must be a positive multiple of hkv");
  REQUIRE(hkv <= GRAFT_MAX_KV_HEADS, GRAFT_ERR_UNSUPPORTED,
          "graft_tree_attention: hkv %d above %d", hkv, (int)GRAFT_MAX_KV_HEADS);
  REQUIRE(head_dim == 64 || head_dim == 128, GRAFT_ERR_UNSUPPORTED,
          "graft_tree_attention: head_dim %d not supported (64 or 128)", head_dim);
  REQUIRE(max_prefix >= 0, GRAFT_ERR_INVALID_ARG, "graft_tree_attention: max_prefix < 0");
  REQUIRE((long long)batch * hkv * (hq / hkv) < (1LL << 24), GRAFT_ERR_UNSUPPORTED,
          "graft_tree_attention: too many heads x sequences");
  return GRAFT_OK;
}

size_t graft_tree_attention_workspace_size(graft_dtype dtype, int32_t batch, int32_t n_max,
                                           int32_t hq, int32_t hkv, int32_t head_dim,
                                           int32_t max_prefix, int64_t sum_prefix) {
  if (check_attn_shape(dtype, batch, n_max, hq, hkv, head_dim, max_prefix) != GRAFT_OK)
    return 0;
  const AttnPlan pl =
      plan_attention(dtype, batch, n_max, hq, hkv, head_dim, max_prefix, sum_prefix);
  return align_up(pl.part_o_bytes, 256) + align_up(pl.part_ml_bytes, 256);
}

graft_status graft_tree_attention_plan(graft_dtype dtype, int32_t batch, int32_t n_max,
                                       int32_t hq, int32_t hkv, int32_t head_dim,
                                       int32_t max_prefix, int64_t sum_prefix,
                                       graft_attention_plan *plan) {
  g_error[0] = 0;
  REQUIRE(plan, GRAFT_ERR_INVALID_ARG, "graft_tree_attention_plan: plan is null");
  const graft_status st = check_attn_shape(dtype, batch, n_max, hq, hkv, head_dim, max_prefix);
  if (st != GRAFT_OK) return st;
  const AttnPlan pl =
      plan_attention(dtype, batch, n_max, hq, hkv, head_dim, max_prefix, sum_prefix);
  plan->matrix_cores = pl.mfma ? 1 : 0;
  plan->n_row_groups = pl.n_row_groups;
  plan->rows_per_group = pl.rows_per_group;
  plan->n_splits = pl.n_splits;
  plan->tiles_per_split = pl.tiles_per_split;
  plan->tree_shift = pl.mfma ? pl.tree_shift : 0;
  plan->key_pairs = pl.mfma && pl.key_pairs ? 1 : 0;
  plan->longest_first = pl.mfma && pl.lpt ? 1 : 0;
  plan->workgroups = (int32_t)attention_workgroups(pl, batch, hkv);
  return GRAFT_OK;
}

static graft_status attention_impl(graft_dtype dtype, int32_t batch, int32_t n_max, int32_t hq,
                                   int32_t hkv, int32_t head_dim, const void *q,
                                   const void *k_tree, const void *v_tree, const void *k_cache,
                                   const void *v_cache, int32_t block_size,
                                   const int32_t *block_table, int32_t max_blocks_per_seq,
                                   const int32_t *prefix_len, int32_t max_prefix,
                                   int64_t sum_prefix, const uint32_t *tree_mask,
                                   const int32_t *n_nodes,
                                   const int32_t *tree_pos, const float *rope,
                                   int32_t rope_positions, float scale, void *out,
                                   void *workspace, size_t workspace_bytes,
                                   hipStream_t stream) {
  graft_status st = check_attn_shape(dtype, batch, n_max, hq, hkv, head_dim, max_prefix);
  if (st != GRAFT_OK) return st;
  REQUIRE(block_size == 16, GRAFT_ERR_UNSUPPORTED,
          "graft_tree_attention: block_size %d not supported (16)", block_size);
  REQUIRE(max_blocks_per_seq >= 1 &&
              (long long)max_blocks_per_seq * block_size >= (long long)max_prefix,
          GRAFT_ERR_INVALID_ARG,
          "graft_tree_attention: max_blocks_per_seq * block_size < max_prefix");
  REQUIRE(std::isfinite(scale) && scale > 0.f, GRAFT_ERR_INVALID_ARG,
          "graft_tree_attention: scale must be finite and > 0");
  if (batch == 0) return GRAFT_OK;
  REQUIRE(q && k_tree && v_tree && k_cache && v_cache && block_table && prefix_len &&
              tree_mask && n_nodes && out,
          GRAFT_ERR_INVALID_ARG, "graft_tree_attention: null device pointer");

  const AttnPlan pl =
      plan_attention(dtype, batch, n_max, hq, hkv, head_dim, max_prefix, sum_prefix);
  const size_t need = align_up(pl.part_o_bytes, 256) + align_up(pl.part_ml_bytes, 256);
  REQUIRE(need == 0 || (workspace && workspace_bytes >= need), GRAFT_ERR_WORKSPACE,
          "graft_tree_attention: workspace of %zu bytes needed, %zu given", need,
          workspace_bytes);

  AttnParams p{};
  p.batch = batch;
  p.n_max = n_max;
  p.hq = hq;
  p.hkv = hkv;
  p.group = hq / hkv;
  p.head_dim = head_dim;
  p.words = GRAFT_MASK_WORDS(n_max);
  p.q = q;
  p.k_tree = k_tree;
  p.v_tree = v_tree;
  p.k_cache = k_cache;
  p.v_cache = v_cache;
  p.block_table = block_table;
  p.max_blocks = max_blocks_per_seq;
  p.prefix_len = prefix_len;
  p.tree_mask = tree_mask;
  p.n_nodes = n_nodes;
  p.scale_log2 = scale * 1.4426950408889634f;
  p.tree_pos = tree_pos;
  p.rope = rope;
  p.rope_positions = rope_positions;
  p.out = out;
  p.n_splits = pl.n_splits;
  p.tiles_per_split = pl.tiles_per_split;
  p.n_row_groups = pl.n_row_groups;
  p.rows_per_group = pl.rows_per_group;
  p.group_blocks_lo = pl.group_blocks_lo;
  p.group_blocks_rem = pl.group_blocks_rem;
  p.lpt = pl.mfma && pl.lpt ? 1 : 0;
  p.key_pairs = pl.mfma && pl.key_pairs ? 1 : 0;
  p.tree_shift = pl.mfma ? pl.tree_shift : 0;
  char *ws = static_cast<char *>(workspace);
  p.part_o = pl.n_splits > 1 ? reinterpret_cast<float *>(ws) : nullptr;
  p.part_ml = pl.n_splits > 1
                  ? reinterpret_cast<float *>(ws + align_up(pl.part_o_bytes, 256))
                  : nullptr;
  if (pl.mfma)
    launch_attention_bf16_mfma(p, stream);
  else
    launch_attention_wave(dtype, p, stream);
  if ((st = check_launch("graft_tree_attention")) != GRAFT_OK) return st;
  if (pl.n_splits > 1) {
    launch_attention_combine(dtype, p, stream);
    if ((st = check_launch("graft_tree_attention (combine)")) != GRAFT_OK) return st;
  }
  return GRAFT_OK;
}

graft_status graft_tree_attention(graft_dtype dtype, int32_t batch, int32_t n_max,
                                  int32_t hq, int32_t hkv, int32_t head_dim,
                                  const void *q, const void *k_tree, const void *v_tree,
                                  const void *k_cache, const void *v_cache,
                                  int32_t block_size, const int32_t *block_table,
                                  int32_t max_blocks_per_seq, const int32_t *prefix_len,
                                  int32_t max_prefix, int64_t sum_prefix,
                                  const uint32_t *tree_mask, const int32_t *n_nodes,
                                  float scale, void *out,
                                  void *workspace, size_t workspace_bytes,
                                  hipStream_t stream) {
  g_error[0] = 0;
  return attention_impl(dtype, batch, n_max, hq, hkv, head_dim, q, k_tree, v_tree, k_cache,
                        v_cache, block_size, block_table, max_blocks_per_seq, prefix_len,
                        max_prefix, sum_prefix, tree_mask, n_nodes, nullptr, nullptr, 0, scale,
                        out,
                        workspace, workspace_bytes, stream);
}

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
                                          hipStream_t stream) {
  g_error[0] = 0;
  graft_status st = check_attn_shape(dtype, batch, n_max, hq, hkv, head_dim, max_prefix);
  if (st != GRAFT_OK) return st;
  const AttnPlan pl =
      plan_attention(dtype, batch, n_max, hq, hkv, head_dim, max_prefix, sum_prefix);
  const size_t need = align_up(pl.part_o_bytes, 256) + align_up(pl.part_ml_bytes, 256);
  REQUIRE(need <= GRAFT_NOALLOC_SCRATCH_BYTES, GRAFT_ERR_WORKSPACE,
          "graft_tree_attention_noalloc: the plan needs %zu bytes of scratch, the library "
          "holds %zu", need, (size_t)GRAFT_NOALLOC_SCRATCH_BYTES);
  void *ws = nullptr;
  if ((st = noalloc_scratch(&ws)) != GRAFT_OK) return st;
  return attention_impl(dtype, batch, n_max, hq, hkv, head_dim, q, k_tree, v_tree, k_cache,
                        v_cache, block_size, block_table, max_blocks_per_seq, prefix_len,
                        max_prefix, sum_prefix, tree_mask, n_nodes, nullptr, nullptr, 0, scale,
                        out, ws, GRAFT_NOALLOC_SCRATCH_BYTES, stream);
}

graft_status graft_tree_attention_rope(graft_dtype dtype, int32_t batch, int32_t n_max,
                                       int32_t hq, int32_t hkv, int32_t head_dim,
                                       const void *q, const void *k_tree, const void *v_tree,
                                       const void *k_cache, const void *v_cache,
                                       int32_t block_size, const int32_t *block_table,
                                       int32_t max_blocks_per_seq, const int32_t *prefix_len,
                                       int32_t max_prefix, int64_t sum_prefix,
                                       const uint32_t *tree_mask, const int32_t *n_nodes,
                                       const int32_t *tree_pos,
                                       const float *rope_cos_sin, int32_t rope_positions,
                                       float scale, void *out, void *workspace,
                                       size_t workspace_bytes, hipStream_t stream) {
  g_error[0] = 0;
  REQUIRE(rope_positions >= 1, GRAFT_ERR_INVALID_ARG,
          "graft_tree_attention_rope: rope_positions < 1");
  REQUIRE(batch == 0 || (tree_pos && rope_cos_sin), GRAFT_ERR_INVALID_ARG,
          "graft_tree_attention_rope: null device pointer");
  REQUIRE(((uintptr_t)rope_cos_sin & 15) == 0, GRAFT_ERR_INVALID_ARG,
          "graft_tree_attention_rope: the table must be 16-byte aligned");
  return attention_impl(dtype, batch, n_max, hq, hkv, head_dim, q, k_tree, v_tree, k_cache,
                        v_cache, block_size, block_table, max_blocks_per_seq, prefix_len,
                        max_prefix, sum_prefix, tree_mask, n_nodes, tree_pos, rope_cos_sin,
                        rope_positions,
                        scale, out, workspace, workspace_bytes, stream);
}

// ------------------------------------------------------------------- accept
size_t graft_accept_workspace_size(int32_t batch, int32_t n_max, int32_t vocab) {
  if (batch < 0 || n_max < 1 || n_max > GRAFT_MAX_NODES || vocab < 1) return 0;
  // sized for the largest chunk count any launch uses
  return align_up(
      (size_t)batch * n_max * accept_chunks_max(vocab) * sizeof(unsigned long long), 256);
}

graft_status graft_accept(graft_dtype dtype, int32_t batch, int32_t n_max, int32_t vocab,
                          const void *logits, const int32_t *tree_token,
                          const int32_t *tree_parent, const uint32_t *tree_mask,
                          const int32_t *n_nodes, int32_t *argmax, int32_t *accept_len,
                          int32_t *path_nodes, int32_t *path_tokens, void *workspace,
                          size_t workspace_bytes, hipStream_t stream) {
  g_error[0] = 0;
  REQUIRE(dtype == GRAFT_F32 || dtype == GRAFT_BF16, GRAFT_ERR_INVALID_ARG,
          "graft_accept: unknown dtype %d", (int)dtype);
  REQUIRE(batch >= 0 && batch <= 65535 && n_max >= 1 && n_max <= GRAFT_MAX_NODES,
          GRAFT_ERR_INVALID_ARG, "graft_accept: batch/n_max out of range");
  REQUIRE(vocab >= 1, GRAFT_ERR_INVALID_ARG, "graft_accept: vocab < 1");
  REQUIRE(vocab <= GRAFT_MAX_VOCAB, GRAFT_ERR_UNSUPPORTED, "graft_accept: vocab above %d",
          (int)GRAFT_MAX_VOCAB);
  REQUIRE((long long)batch * n_max <= 65535, GRAFT_ERR_UNSUPPORTED,
          "graft_accept: batch * n_max above 65535");
  if (batch == 0) return GRAFT_OK;
  REQUIRE(logits && tree_token && tree_parent && tree_mask && n_nodes && argmax &&
              accept_len && path_nodes && path_tokens,
          GRAFT_ERR_INVALID_ARG, "graft_accept: null device pointer");
  const size_t need = graft_accept_workspace_size(batch, n_max, vocab);
  REQUIRE(workspace && workspace_bytes >= need, GRAFT_ERR_WORKSPACE,
          "graft_accept: workspace of %zu bytes needed, %zu given", need, workspace_bytes);
  AcceptParams p{};
  p.batch = batch;
  p.n_max = n_max;
  p.vocab = vocab;
  p.words = GRAFT_MASK_WORDS(n_max);
  p.chunks = accept_chunks(dtype, batch * n_max, vocab);
  p.logits = logits;
  p.tree_token = tree_token;
  p.tree_parent = tree_parent;
  p.tree_mask = tree_mask;
  p.n_nodes = n_nodes;
  p.argmax = argmax;
  p.accept_len = accept_len;
  p.path_nodes = path_nodes;
  p.path_tokens = path_tokens;
  p.partial = static_cast<unsigned long long *>(workspace);
  launch_accept(dtype, p, stream);
  return check_launch("graft_accept");
}

// ------------------------------------------------------ sampling acceptance
size_t graft_accept_sample_workspace_size(graft_dtype dtype, int32_t batch, int32_t n_max,
                                          int32_t vocab) {
  if ((dtype != GRAFT_F32 && dtype != GRAFT_BF16) || batch < 0 || n_max < 1 ||
      n_max > GRAFT_MAX_NODES || vocab < 1)
    return 0;
  return sample_layout(dtype, batch, n_max, vocab).total;
}

graft_status graft_accept_sample(graft_dtype dtype, int32_t batch, int32_t n_max, int32_t vocab,
                                 const void *logits, float temperature,
                                 const int32_t *tree_token, const int32_t *tree_parent,
                                 const int32_t *n_nodes, const float *rand_accept,
                                 const float *rand_sample, int32_t *accept_len,
                                 int32_t *path_nodes, int32_t *path_tokens, void *workspace,
                                 size_t workspace_bytes, hipStream_t stream) {
  g_error[0] = 0;
  REQUIRE(dtype == GRAFT_F32 || dtype == GRAFT_BF16, GRAFT_ERR_INVALID_ARG,
          "graft_accept_sample: unknown dtype %d", (int)dtype);
  REQUIRE(batch >= 0 && batch <= 65535 && n_max >= 1 && n_max <= GRAFT_MAX_NODES,
          GRAFT_ERR_INVALID_ARG, "graft_accept_sample: batch/n_max out of range");
  REQUIRE(vocab >= 1, GRAFT_ERR_INVALID_ARG, "graft_accept_sample: vocab < 1");
  REQUIRE(vocab <= GRAFT_MAX_VOCAB, GRAFT_ERR_UNSUPPORTED,
          "graft_accept_sample: vocab above %d", (int)GRAFT_MAX_VOCAB);
  REQUIRE(std::isfinite(temperature) && temperature > 0.f, GRAFT_ERR_INVALID_ARG,
          "graft_accept_sample: temperature must be finite and > 0");
  const double k_log2 = 1.4426950408889634 / (double)temperature;
  REQUIRE(k_log2 < 1e37, GRAFT_ERR_UNSUPPORTED, "graft_accept_sample: temperature below 1e-37");
  REQUIRE((long long)batch * n_max <= 65535, GRAFT_ERR_UNSUPPORTED,
          "graft_accept_sample: batch * n_max above 65535");
  if (batch == 0) return GRAFT_OK;
  REQUIRE(logits && tree_token && tree_parent && n_nodes && rand_accept && rand_sample &&
              accept_len && path_nodes && path_tokens,
          GRAFT_ERR_INVALID_ARG, "graft_accept_sample: null device pointer");
  const size_t need = graft_accept_sample_workspace_size(dtype, batch, n_max, vocab);
  REQUIRE(workspace && workspace_bytes >= need, GRAFT_ERR_WORKSPACE,
          "graft_accept_sample: workspace of %zu bytes needed, %zu given", need,
          workspace_bytes);
  SampleParams p{};
  p.batch = batch;
  p.n_max = n_max;
  p.vocab = vocab;
  p.lazy = sample_lazy(dtype, batch, n_max, vocab) ? 1 : 0;
  p.stat_loads = sample_stat_loads(dtype, batch * n_max, vocab);
  p.chunks = sample_stat_chunks(dtype, p.stat_loads, vocab);
  p.wchunks = sample_walk_chunks(dtype, vocab);
  p.k_log2 = k_log2;
  p.k_hi = (float)k_log2;
  p.k_lo = (float)(k_log2 - (double)p.k_hi);
  p.logits = logits;
  p.tree_token = tree_token;
  p.tree_parent = tree_parent;
  p.n_nodes = n_nodes;
  p.rand_accept = rand_accept;
  p.rand_sample = rand_sample;
  p.accept_len = accept_len;
  p.path_nodes = path_nodes;
  p.path_tokens = path_tokens;
  const SampleLayout lay = sample_layout(dtype, batch, n_max, vocab);
  p.stats = static_cast<ChunkStat *>(workspace);
  p.root = static_cast<RootChunk *>(workspace);
  p.chunk_w = reinterpret_cast<double *>(static_cast<char *>(workspace) + lay.off_chunk_w);
  p.rec = reinterpret_cast<SampleRec *>(static_cast<char *>(workspace) + lay.off_rec);
  launch_accept_sample(dtype, p, stream);
  return check_launch("graft_accept_sample");
}

// ---------------------------------------------------------------- adjacency
static uint32_t update_capacity(long long max_transitions) {
  uint32_t c = 64;
  while ((long long)c < 2 * max_transitions) c <<= 1;
  return c;
}

size_t graft_update_adjacency_workspace_size(int32_t n_paths, int32_t path_stride) {
  if (n_paths < 0 || path_stride < 2) return update_layout(64).total;
  const long long t = (long long)n_paths * (path_stride - 1);
  if (t > (1LL << 28)) return 0;
  return update_layout(update_capacity(t)).total;
}

static graft_status update_impl(int32_t *m_ids, float *m_scores, int32_t vocab, int32_t top_s,
                                int32_t n_paths, int32_t path_stride,
                                const int32_t *path_tokens, const int32_t *accept_len,
                                void *workspace, size_t workspace_bytes, hipStream_t stream) {
  g_error[0] = 0;
  REQUIRE(vocab >= 1, GRAFT_ERR_INVALID_ARG, "graft_update_adjacency: vocab < 1");
  REQUIRE(top_s >= 1 && top_s <= GRAFT_MAX_TOP_S, GRAFT_ERR_INVALID_ARG,
          "graft_update_adjacency: top_s outside 1..%d", GRAFT_MAX_TOP_S);
  REQUIRE(n_paths >= 0 && path_stride >= 0, GRAFT_ERR_INVALID_ARG,
          "graft_update_adjacency: negative n_paths or path_stride");
  const long long t = path_stride >= 2 ? (long long)n_paths * (path_stride - 1) : 0;
  REQUIRE(t <= (1LL << 28), GRAFT_ERR_UNSUPPORTED,
          "graft_update_adjacency: more than 2^28 transitions");
  if (t == 0) return GRAFT_OK;
  REQUIRE(m_ids && m_scores && path_tokens && accept_len, GRAFT_ERR_INVALID_ARG,
          "graft_update_adjacency: null device pointer");
  REQUIRE(workspace, GRAFT_ERR_WORKSPACE, "graft_update_adjacency: workspace is null");
  // The layout depends only on the workspace size, so one zero-filled
  // buffer stays valid across calls of different sizes.
  uint32_t cap = 64;
  while (update_layout(cap * 2).total <= workspace_bytes && cap < (1u << 30)) cap *= 2;
  REQUIRE(update_layout(cap).total <= workspace_bytes && (long long)cap >= 2 * t,
          GRAFT_ERR_WORKSPACE, "graft_update_adjacency: workspace of %zu bytes needed, %zu given",
          graft_update_adjacency_workspace_size(n_paths, path_stride), workspace_bytes);
  UpdateParams p{};
  p.m_ids = m_ids;
  p.m_scores = m_scores;
  p.vocab = vocab;
  p.top_s = top_s;
  p.n_paths = n_paths;
  p.path_stride = path_stride;
  p.max_transitions = (int32_t)t;
  p.path_tokens = path_tokens;
  p.accept_len = accept_len;
  p.ws = static_cast<char *>(workspace);
  p.lay = update_layout(cap);
  launch_update(p, stream);
  return check_launch("graft_update_adjacency");
}

graft_status graft_update_adjacency(int32_t *m_ids, float *m_scores, int32_t vocab,
                                    int32_t top_s, int32_t n_paths, int32_t path_stride,
                                    const int32_t *path_tokens, const int32_t *accept_len,
                                    void *workspace, size_t workspace_bytes,
                                    hipStream_t stream) {
  return update_impl(m_ids, m_scores, vocab, top_s, n_paths, path_stride, path_tokens,
                     accept_len, workspace, workspace_bytes, stream);
}

// ------------------------------------------------------- all-node update
static size_t tree_pairs_bytes(int32_t batch, int32_t n_max) {
  const size_t rows = (size_t)batch * n_max;
  return align_up(rows * 2 * sizeof(int32_t), 256) + align_up(rows * sizeof(int32_t), 256);
}

size_t graft_update_adjacency_tree_workspace_size(int32_t batch, int32_t n_max) {
  if (batch < 0 || n_max < 1 || n_max > GRAFT_MAX_NODES) return 0;
  return tree_pairs_bytes(batch, n_max) +
         graft_update_adjacency_workspace_size(batch * n_max, 2);
}

graft_status graft_update_adjacency_tree(int32_t *m_ids, float *m_scores, int32_t vocab,
                                         int32_t top_s, int32_t batch, int32_t n_max,
                                         const int32_t *tree_token, const int32_t *argmax,
                                         const int32_t *n_nodes, void *workspace,
                                         size_t workspace_bytes, hipStream_t stream) {
  g_error[0] = 0;
  REQUIRE(batch >= 0 && n_max >= 1 && n_max <= GRAFT_MAX_NODES, GRAFT_ERR_INVALID_ARG,
          "graft_update_adjacency_tree: batch/n_max out of range");
  REQUIRE((long long)batch * n_max <= (1LL << 28), GRAFT_ERR_UNSUPPORTED,
          "graft_update_adjacency_tree: batch * n_max too large");
  REQUIRE(vocab >= 1 && top_s >= 1 && top_s <= GRAFT_MAX_TOP_S, GRAFT_ERR_INVALID_ARG,
          "graft_update_adjacency_tree: vocab/top_s out of range");
  if (batch == 0) return GRAFT_OK;
  REQUIRE(m_ids && m_scores && tree_token && argmax && n_nodes, GRAFT_ERR_INVALID_ARG,
          "graft_update_adjacency_tree: null device pointer");
  const size_t need = graft_update_adjacency_tree_workspace_size(batch, n_max);
  REQUIRE(workspace && workspace_bytes >= need, GRAFT_ERR_WORKSPACE,
          "graft_update_adjacency_tree: workspace of %zu bytes needed, %zu given", need,
          workspace_bytes);
  char *ws = static_cast<char *>(workspace);
  int32_t *pairs = reinterpret_cast<int32_t *>(ws);
  int32_t *lens = reinterpret_cast<int32_t *>(
      ws + align_up((size_t)batch * n_max * 2 * sizeof(int32_t), 256));
  launch_tree_pairs(batch, n_max, tree_token, argmax, n_nodes, pairs, lens, stream);
  const graft_status st = check_launch("graft_update_adjacency_tree");
  if (st != GRAFT_OK) return st;
  const size_t head = tree_pairs_bytes(batch, n_max);
  // nearly every row is a valid transition here; the per-step path, whose
  // workgroups each sort only the transitions of their own rows, stays
  // ahead of the hash-table path up to its capacity (measured at 1040 and
  // 2080 transitions)
  return update_impl(m_ids, m_scores, vocab, top_s, batch * n_max, 2, pairs, lens, ws + head,
                     workspace_bytes - head, stream);
}

// ---------------------------------------------------------------- KV append
static graft_status append_impl(graft_dtype dtype, int32_t batch, int32_t n_max, int32_t hkv,
                                int32_t head_dim, const void *k_tree, const void *v_tree,
                                void *k_cache, void *v_cache, int32_t num_blocks,
                                int32_t block_size, const int32_t *block_table,
                                int32_t max_blocks_per_seq, const int32_t *prefix_len,
                                const int32_t *path_nodes, const int32_t *accept_len,
                                int32_t *new_prefix_len, const float *rope,
                                int32_t rope_positions, hipStream_t stream) {
  REQUIRE(dtype == GRAFT_F32 || dtype == GRAFT_BF16, GRAFT_ERR_INVALID_ARG,
          "graft_append_kv: unknown dtype %d", (int)dtype);
  REQUIRE(batch >= 0 && n_max >= 1 && n_max <= GRAFT_MAX_NODES && hkv >= 1 && head_dim >= 1,
          GRAFT_ERR_INVALID_ARG, "graft_append_kv: bad shape");
  REQUIRE((long long)batch * hkv <= (1LL << 31) - 1, GRAFT_ERR_UNSUPPORTED,
          "graft_append_kv: batch * hkv too large");
  REQUIRE(num_blocks >= 0 && block_size >= 1 && max_blocks_per_seq >= 1, GRAFT_ERR_INVALID_ARG,
          "graft_append_kv: bad cache geometry");
  if (batch == 0) return GRAFT_OK;
  REQUIRE(k_tree && v_tree && k_cache && v_cache && block_table && prefix_len && path_nodes &&
              accept_len && new_prefix_len,
          GRAFT_ERR_INVALID_ARG, "graft_append_kv: null device pointer");
  REQUIRE((const void *)new_prefix_len != (const void *)prefix_len, GRAFT_ERR_INVALID_ARG,
          "graft_append_kv: new_prefix_len must not alias prefix_len");
  AppendParams p{};
  p.batch = batch;
  p.n_max = n_max;
  p.hkv = hkv;
  p.head_dim = head_dim;
  p.block_size = block_size;
  p.max_blocks = max_blocks_per_seq;
  p.num_blocks = num_blocks;
  p.k_tree = k_tree;
  p.v_tree = v_tree;
  p.k_cache = k_cache;
  p.v_cache = v_cache;
  p.block_table = block_table;
  p.prefix_len = prefix_len;
  p.path_nodes = path_nodes;
  p.accept_len = accept_len;
  p.new_prefix_len = new_prefix_len;
  p.rope = rope;
  p.rope_positions = rope_positions;
  launch_append_kv(dtype, p, stream);
  return check_launch("graft_append_kv");
}

graft_status graft_append_kv(graft_dtype dtype, int32_t batch, int32_t n_max, int32_t hkv,
                             int32_t head_dim, const void *k_tree, const void *v_tree,
                             void *k_cache, void *v_cache, int32_t num_blocks,
                             int32_t block_size, const int32_t *block_table,
                             int32_t max_blocks_per_seq, const int32_t *prefix_len,
                             const int32_t *path_nodes, const int32_t *accept_len,
                             int32_t *new_prefix_len, hipStream_t stream) {
  g_error[0] = 0;
  return append_impl(dtype, batch, n_max, hkv, head_dim, k_tree, v_tree, k_cache, v_cache,
                     num_blocks, block_size, block_table, max_blocks_per_seq, prefix_len,
                     path_nodes, accept_len, new_prefix_len, nullptr, 0, stream);
}

graft_status graft_append_kv_rope(graft_dtype dtype, int32_t batch, int32_t n_max, int32_t hkv,
                                  int32_t head_dim, const void *k_tree, const void *v_tree,
                                  void *k_cache, void *v_cache, int32_t num_blocks,
                                  int32_t block_size, const int32_t *block_table,
                                  int32_t max_blocks_per_seq, const int32_t *prefix_len,
                                  const int32_t *path_nodes, const int32_t *accept_len,
                                  int32_t *new_prefix_len, const float *rope_cos_sin,
                                  int32_t rope_positions, hipStream_t stream) {
  g_error[0] = 0;
  REQUIRE(head_dim % 2 == 0, GRAFT_ERR_INVALID_ARG, "graft_append_kv_rope: odd head_dim");
  REQUIRE(rope_positions >= 1, GRAFT_ERR_INVALID_ARG, "graft_append_kv_rope: rope_positions < 1");
  REQUIRE(batch == 0 || rope_cos_sin, GRAFT_ERR_INVALID_ARG,
          "graft_append_kv_rope: null device pointer");
  return append_impl(dtype, batch, n_max, hkv, head_dim, k_tree, v_tree, k_cache, v_cache,
                     num_blocks, block_size, block_table, max_blocks_per_seq, prefix_len,
                     path_nodes, accept_len, new_prefix_len, rope_cos_sin, rope_positions,
                     stream);
}

}  // extern "C"
