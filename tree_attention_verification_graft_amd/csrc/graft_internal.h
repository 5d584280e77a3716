// Internal declarations shared by the library's translation units.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "../../include/graft.h"

namespace graft {

// ---- wave-wide exchanges that stay in the vector ALU.  lane_pair gives
// lane l's value and the value of lane l ^ stride (stride 1, 2, 4, ..., 32)
// as an unordered pair {a, b}, which is all a maximum, a sum or a
// compare-exchange needs.  Strides up to 8 move the partner's value with DPP
// lane permutes within rows of 16 (xor 1 and 2 are quad permutes; xor 4 is
// the half-row mirror then the quad reversal, xor 8 the row mirror then the
// half-row mirror); 16 and 32 use the gfx950 row-swap permutes, whose two
// results hold the lane's own value and its partner's.  All 64 lanes must be
// active.
__device__ inline uint32_t dpp_lane_xor(uint32_t v, int stride) {
  constexpr int kQuadXor1 = 0xB1, kQuadXor2 = 0x4E, kQuadRev = 0x1B;
  constexpr int kHalfMirror = 0x141, kMirror = 0x140;
  const int x = (int)v;
  switch (stride) {
    case 1: return (uint32_t)__builtin_amdgcn_update_dpp(x, x, kQuadXor1, 0xF, 0xF, false);
    case 2: return (uint32_t)__builtin_amdgcn_update_dpp(x, x, kQuadXor2, 0xF, 0xF, false);
    case 4: {
      const int t = __builtin_amdgcn_update_dpp(x, x, kHalfMirror, 0xF, 0xF, false);
      return (uint32_t)__builtin_amdgcn_update_dpp(t, t, kQuadRev, 0xF, 0xF, false);
    }
    default: {  // 8
      const int t = __builtin_amdgcn_update_dpp(x, x, kMirror, 0xF, 0xF, false);
      return (uint32_t)__builtin_amdgcn_update_dpp(t, t, kHalfMirror, 0xF, 0xF, false);
    }
  }
}
__device__ inline void lane_pair(uint32_t v, int stride, uint32_t &a, uint32_t &b) {
  if (stride <= 8) {
    a = v;
    b = dpp_lane_xor(v, stride);
  } else {
    const auto r = stride == 16 ? __builtin_amdgcn_permlane16_swap(v, v, false, false)
                                : __builtin_amdgcn_permlane32_swap(v, v, false, false);
    a = r[0];
    b = r[1];
  }
}
__device__ inline void lane_pair(unsigned long long v, int stride, unsigned long long &a,
                                 unsigned long long &b) {
  uint32_t al, bl, ah, bh;
  lane_pair((uint32_t)v, stride, al, bl);
  lane_pair((uint32_t)(v >> 32), stride, ah, bh);
  a = ((unsigned long long)ah << 32) | al;
  b = ((unsigned long long)bh << 32) | bl;
}


// Order-preserving int16 keys of the two bf16 values in a word, by packed
// 16-bit integer ops: a negative value flips its magnitude bits (so larger
// magnitudes order lower) and moves up by one, which folds -0 onto +0.  A
// key of -32768 is below every value's (the most negative finite value maps
// to -32639), so it marks entries outside the chunk.
typedef short short2v __attribute__((ext_vector_type(2)));
__device__ inline short2v okey2(uint32_t w) {
  const short2v x = __builtin_bit_cast(short2v, w);
  const short2v s = x >> (short2v){15, 15};  // 0 or -1 per half
  return (x ^ (s & (short2v){0x7fff, 0x7fff})) - s;
}
// The bf16 bits of a key (either zero for key 0).
__device__ inline uint32_t key_bf16(int key) {
  return key >= 0 ? (uint32_t)key : (uint32_t)(((key - 1) ^ 0x7fff) & 0xffff);
}

// Thread-local error message behind graft_last_error().
graft_status set_error(graft_status code, const char *fmt, ...);

// Map the last HIP launch error (if any) to a status.
graft_status check_launch(const char *what);

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// ---------------------------------------------------------------- tree build
struct BuildParams {
  graft_tree_config cfg;
  int8_t env_level[GRAFT_MAX_NODES - 1];  // envelope depth of each slot (root children 0)
  int32_t env_levels;                     // 1 + the deepest slot's level (0 if no slots)
  int32_t batch, n_draft_max, vocab, top_s, n_max, words;
  const int32_t *draft_parent;
  const int32_t *draft_token;
  const float *draft_conf;
  const int32_t *n_draft;
  const int32_t *root_token;
  const int32_t *prefix_len;
  const int32_t *m_ids;
  int32_t *tree_token;
  int32_t *tree_parent;
  int32_t *tree_pos;
  uint32_t *tree_mask;
  int32_t *n_nodes;
  int32_t *stage_out;
};
void launch_build_tree(const BuildParams &p, hipStream_t stream);

// ----------------------------------------------------------------- attention
struct AttnParams {
  int32_t batch, n_max, hq, hkv, group, head_dim, words;
  const void *q;
  const void *k_tree;
  const void *v_tree;
  const void *k_cache;
  const void *v_cache;
  const int32_t *block_table;
  int32_t max_blocks;
  const int32_t *prefix_len;
  const uint32_t *tree_mask;
  const int32_t *n_nodes;
  float scale_log2;  // scale * log2(e)
  // rotary embedding of queries and tree keys on load (rope == nullptr: the
  // inputs arrive rotated): table [rope_positions][head_dim] of cos | sin
  const int32_t *tree_pos;
  const float *rope;
  int32_t rope_positions;
  void *out;
  // split-K plan
  int32_t n_splits;        // prefix splits per (sequence, kv head, row group)
  int32_t tiles_per_split; // 64-key prefix tiles per split
  int32_t n_row_groups;    // row groups per (sequence, kv head)
  int32_t rows_per_group;  // query rows of the largest row group (multiple of 16)
  // matrix-core path: row groups are runs of 16-row blocks, the first
  // group_blocks_rem of them group_blocks_lo + 1 blocks long, the rest
  // group_blocks_lo (the wavefront path has one group of rows_per_group rows)
  int32_t group_blocks_lo, group_blocks_rem;
  int32_t lpt;             // rank (sequence, split) pairs longest first on the device
  int32_t key_pairs;       // waves w and w + 4 share rows, one 32-key half of each tile each
  int32_t tree_shift;      // split s covers prefix tiles [s tps - shift, (s + 1) tps - shift)
  float *part_o;           // [batch][hkv][groups][splits][rows][D]
  float *part_ml;          // [batch][hkv][groups][splits][rows][2]
};
struct AttnPlan {
  bool mfma;
  bool lpt;  // ragged batch: launch the longest (sequence, split) work first
  bool key_pairs;  // at most 4 row blocks per group: waves pair up on the keys of each tile
  int32_t tree_shift;  // tree tiles counted at the front of split 0 (0: none)
  int32_t n_splits, tiles_per_split, n_row_groups, rows_per_group;
  int32_t group_blocks_lo, group_blocks_rem;  // see AttnParams
  size_t part_o_bytes, part_ml_bytes;
};
// sum_prefix: the caller's sum of prefix lengths (<= 0: unknown, every
// sequence is taken at max_prefix); it only steers the plan.
AttnPlan plan_attention(graft_dtype dtype, int32_t batch, int32_t n_max, int32_t hq,
                        int32_t hkv, int32_t head_dim, int32_t max_prefix, int64_t sum_prefix);
// Workgroups of the attention launch of a plan.
long attention_workgroups(const AttnPlan &pl, int32_t batch, int32_t hkv);
void launch_attention_bf16_mfma(const AttnParams &p, hipStream_t stream);
void launch_attention_wave(graft_dtype dtype, const AttnParams &p, hipStream_t stream);
void launch_attention_combine(graft_dtype dtype, const AttnParams &p,
                              hipStream_t stream);

// -------------------------------------------------------------------- accept
struct AcceptParams {
  int32_t batch, n_max, vocab, words, chunks;
  const void *logits;
  const int32_t *tree_token;
  const int32_t *tree_parent;
  const uint32_t *tree_mask;
  const int32_t *n_nodes;
  int32_t *argmax;
  int32_t *accept_len;
  int32_t *path_nodes;
  int32_t *path_tokens;
  unsigned long long *partial;  // [batch * n_max][chunks] packed (value, ~index)
};
// Vocabulary chunks per row of one launch, and the most any launch uses.
int32_t accept_chunks(graft_dtype dtype, int32_t rows, int32_t vocab);
int32_t accept_chunks_max(int32_t vocab);
void launch_accept(graft_dtype dtype, const AcceptParams &p, hipStream_t stream);

// ---------------------------------------------------------------- adjacency
struct UpdateLayout {
  uint32_t capacity;        // hash slots (power of two)
  size_t off_pair_key, off_pair_cnt, off_row_key, off_row_nnew, off_row_off,
      off_row_fill, off_pair_list, off_row_list, off_bucket_v, off_bucket_c,
      off_counters, total;
};
UpdateLayout update_layout(uint32_t capacity);
struct UpdateParams {
  int32_t *m_ids;
  float *m_scores;
  int32_t vocab, top_s, n_paths, path_stride, max_transitions;
  const int32_t *path_tokens;
  const int32_t *accept_len;
  char *ws;
  UpdateLayout lay;
};
// Calls of at most 4096 potential transitions take the single-pass LDS path
// (each workgroup gathers and sorts the transitions of its own rows), larger
// ones the hash-table path.
void launch_update(const UpdateParams &p, hipStream_t stream);
void launch_tree_pairs(int32_t batch, int32_t n_max, const int32_t *tree_token,
                       const int32_t *argmax, const int32_t *n_nodes, int32_t *pairs,
                       int32_t *lens, hipStream_t stream);

// ------------------------------------------------------ sampling acceptance
struct ChunkStat {
  float m;    // chunk max
  float pad;
  double z;   // chunk sum of exp2((l - m) * log2(e) / temperature)
};
// What the walk hands to the bonus draw, per sequence.
struct alignas(16) SampleRec {
  int32_t stop, len, ngone, pad;
  float row_max;  // max logit of the stop node's row
  float u;        // rand_sample of the stop node
  int32_t pad2[2];
  int32_t gone[GRAFT_MAX_NODES];  // tokens rejected at the stop node
};
constexpr int kSampleStage = 2304;  // chunk records one workgroup stages in LDS (36 KB)
// Statistics of one vocabulary chunk of a root row, relative to the chunk's
// own max: z sums the float64 masses of all entries, r those of the entries
// that are not a root child's token (the residual mass when the walk stops
// at the root).
struct alignas(16) RootChunk {
  double z, r;
  float m;  // chunk max (-inf: no mass)
  int32_t pad[3];
};
struct SampleParams {
  int32_t batch, n_max, vocab;
  int32_t lazy;                // 0: staged mode, 1: lazy mode
  int32_t chunks, stat_loads;  // staged statistics chunks per row, loads per thread of one
  int32_t wchunks;             // chunks of the stop row's float64 masses
  double k_log2;   // log2(e) / temperature
  float k_hi, k_lo;  // k_log2 split into a float and the float of the rest
  const void *logits;
  const int32_t *tree_token;
  const int32_t *tree_parent;
  const int32_t *n_nodes;
  const float *rand_accept;
  const float *rand_sample;
  int32_t *accept_len;
  int32_t *path_nodes;
  int32_t *path_tokens;
  ChunkStat *stats;  // staged: [batch * n_max][chunks]
  RootChunk *root;   // lazy: [batch][wchunks] chunk records of the root rows
  double *chunk_w;   // [batch][wchunks] residual mass of the stop row per chunk
  SampleRec *rec;    // [batch]
};
// Chunks of the stop row's float64 masses (4096 bf16 or 2048 f32 entries).
int32_t sample_walk_chunks(graft_dtype dtype, int32_t vocab);
// Staged statistics chunks: loads per thread for a launch over `rows` node
// rows, and chunks per row at that many loads (2048 or 1024 entries per
// load).
int32_t sample_stat_loads(graft_dtype dtype, int32_t rows, int32_t vocab);
int32_t sample_stat_chunks(graft_dtype dtype, int32_t loads, int32_t vocab);
// Whether a call takes lazy mode (the root's records, deeper rows read by
// the walk) rather than staged mode (statistics of every row).
bool sample_lazy(graft_dtype dtype, int32_t batch, int32_t n_max, int32_t vocab);
struct SampleLayout {
  size_t off_chunk_w, off_rec, total;  // the records (stats or root) at offset 0
};
SampleLayout sample_layout(graft_dtype dtype, int32_t batch, int32_t n_max, int32_t vocab);
void launch_accept_sample(graft_dtype dtype, const SampleParams &p, hipStream_t stream);

// ------------------------------------------------------------ KV append
struct AppendParams {
  int32_t batch, n_max, hkv, head_dim, block_size, max_blocks, num_blocks;
  const void *k_tree;
  const void *v_tree;
  void *k_cache;
  void *v_cache;
  const int32_t *block_table;
  const int32_t *prefix_len;
  const int32_t *path_nodes;
  const int32_t *accept_len;
  int32_t *new_prefix_len;
  const float *rope;       // nullptr: keys arrive rotated
  int32_t rope_positions;
};
void launch_append_kv(graft_dtype dtype, const AppendParams &p, hipStream_t stream);

}  // namespace graft
