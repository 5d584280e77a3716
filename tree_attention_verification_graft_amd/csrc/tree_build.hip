// Hybrid tree assembly: prune the draft tree, fill the released budget from
// the successor table M starting at the root, merge, and emit ancestor masks
// and position ids.  One workgroup per sequence; every step is a
// workgroup-parallel pass over at most 256 draft nodes / 127 slots in LDS.
//
// Method: "Draft Less, Retrieve More" (aitrends.kr summary), method paragraph
// steps one to three and the architecture paragraph; readings as documented
// in include/graft.h.
#include "graft_internal.h"

namespace graft {
namespace {

constexpr int kThreads = 256;  // == GRAFT_MAX_DRAFT

// Order-preserving map of a float onto uint32 (larger float -> larger uint).
__device__ inline uint32_t float_key(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ inline float key_float(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
  return __uint_as_float(u);
}

__global__ __launch_bounds__(kThreads) void build_tree_kernel(BuildParams p) {
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const graft_tree_config &cfg = p.cfg;

  __shared__ int32_t s_parent[kThreads];
  __shared__ int32_t s_jump[kThreads];
  __shared__ int32_t s_cnt[kThreads];
  __shared__ float s_pm[kThreads];
  __shared__ int32_t s_newidx[kThreads];
  __shared__ uint8_t s_kept[kThreads];
  __shared__ uint32_t s_cmax[GRAFT_MAX_STAGES];
  __shared__ int32_t s_cexist[GRAFT_MAX_STAGES];
  __shared__ int32_t s_slot_tok[GRAFT_MAX_NODES];
  __shared__ int32_t s_slot_level[GRAFT_MAX_NODES];
  __shared__ uint8_t s_slot_valid[GRAFT_MAX_NODES];
  __shared__ int32_t s_slot_new[GRAFT_MAX_NODES];
  __shared__ int32_t s_out_tok[GRAFT_MAX_NODES];
  __shared__ int32_t s_out_par[GRAFT_MAX_NODES];
  __shared__ int32_t s_stage, s_kdraft, s_nkept, s_nvalid, s_maxlevel;

  const int n = min(max(p.n_draft[b], 0), p.n_draft_max);
  const size_t drow = (size_t)b * p.n_draft_max;
  const int root = p.root_token[b];
  const bool root_ok = root >= 0 && root < p.vocab;

  int32_t my_parent = -1, my_token = 0;
  float my_conf = 0.f;
  if (tid < n) {
    my_parent = p.draft_parent[drow + tid];
    my_token = p.draft_token[drow + tid];
    my_conf = p.draft_conf[drow + tid];
    if (my_parent >= tid) my_parent = -1;  // precondition guard: parent < child
  }
  s_parent[tid] = my_parent;
  s_jump[tid] = my_parent;
  s_cnt[tid] = 1;
  s_pm[tid] = my_conf;
  s_newidx[tid] = 0;
  if (tid < GRAFT_MAX_STAGES) {
    s_cmax[tid] = 0u;
    s_cexist[tid] = 0;
  }
  if (tid == 0) s_maxlevel = 0;
  __syncthreads();

  // Draft depth (children of the root are depth 0) and the minimum confidence
  // along the root path, by pointer jumping: after round r each node covers
  // the 2^r nearest nodes of its chain.
  for (int r = 0; r < 8; ++r) {
    int j = s_jump[tid];
    int cnt = s_cnt[tid];
    float pm = s_pm[tid];
    int nj = j;
    if (j >= 0) {
      cnt += s_cnt[j];
      pm = fminf(pm, s_pm[j]);
      nj = s_jump[j];
    }
    __syncthreads();
    s_jump[tid] = nj;
    s_cnt[tid] = cnt;
    s_pm[tid] = pm;
    __syncthreads();
  }
  const int my_depth = s_cnt[tid] - 1;
  const float my_pm = s_pm[tid];

  // Depth confidence c_d = max confidence at each checkpoint depth.
  if (tid < n) {
    for (int s = 0; s < cfg.n_stages; ++s) {
      if (my_depth == cfg.stage_depth[s]) {
        atomicMax(&s_cmax[s], float_key(my_conf));
        s_cexist[s] = 1;
      }
    }
  }
  __syncthreads();
  if (tid == 0) {
    int stage = -1;
    for (int s = 0; s < cfg.n_stages; ++s) {
      if (s_cexist[s] && key_float(s_cmax[s]) < cfg.stage_tau[s]) {
        stage = s;
        break;
      }
    }
    s_stage = stage;
    s_kdraft = cfg.kmax - (stage < 0 ? cfg.k_ret_none : cfg.stage_k_ret[stage]);
  }
  __syncthreads();
  const int stage = s_stage;
  const int k_draft = s_kdraft;

  // Candidates: every draft if nothing fires, else drafts no deeper than the
  // firing checkpoint.  Keep the k_draft best by (path-min desc, index asc).
  s_pm[tid] = my_pm;
  const bool cand = tid < n && (stage < 0 || my_depth <= cfg.stage_depth[stage]);
  s_kept[tid] = cand ? 1 : 0;
  __syncthreads();
  bool kept = false;
  if (cand) {
    int rank = 0;
    for (int j = 0; j < n; ++j) {
      if (!s_kept[j] || j == tid) continue;
      float pj = s_pm[j];
      rank += (pj > my_pm) || (pj == my_pm && j < tid);
    }
    kept = rank < k_draft;
  }
  __syncthreads();
  s_kept[tid] = kept ? 1 : 0;
  __syncthreads();

  // Compaction of kept drafts, in input order, after the root.
  if (kept) {
    int before = 0;
    for (int j = 0; j < tid; ++j) before += s_kept[j];
    s_newidx[tid] = 1 + before;
  }
  if (tid == 0) {
    int c = 0;
    for (int j = 0; j < n; ++j) c += s_kept[j];
    s_nkept = c;
  }
  __syncthreads();
  const int n_kept = s_nkept;
  const int k_fill = cfg.kmax - n_kept;

  // Retrieval: the first k_fill envelope slots, resolved level by level from
  // the root downwards (a slot's token is a lookup in its parent's row).
  int my_level = 0;
  if (tid < k_fill) {
    int j = cfg.env_parent[tid];
    while (j >= 0) {
      ++my_level;
      j = cfg.env_parent[j];
    }
    s_slot_level[tid] = my_level;
    s_slot_valid[tid] = 0;
    s_slot_tok[tid] = -1;
    atomicMax(&s_maxlevel, my_level);
  }
  __syncthreads();
  const int max_level = s_maxlevel;
  for (int lv = 0; lv <= max_level; ++lv) {
    if (tid < k_fill && my_level == lv) {
      const int ps = cfg.env_parent[tid];
      const bool pok = ps < 0 ? root_ok : (s_slot_valid[ps] != 0);
      const int ptok = ps < 0 ? root : s_slot_tok[ps];
      int tok = -1;
      bool ok = false;
      if (pok) {
        tok = p.m_ids[(size_t)ptok * p.top_s + cfg.env_rank[tid]];
        ok = tok >= 0 && tok < p.vocab;
      }
      s_slot_tok[tid] = tok;
      s_slot_valid[tid] = ok ? 1 : 0;
    }
    __syncthreads();
  }
  if (tid < k_fill && s_slot_valid[tid]) {
    int before = 0;
    for (int j = 0; j < tid; ++j) before += s_slot_valid[j];
    s_slot_new[tid] = 1 + n_kept + before;
  }
  if (tid == 0) {
    int c = 0;
    for (int j = 0; j < k_fill; ++j) c += s_slot_valid[j];
    s_nvalid = c;
  }
  __syncthreads();
  const int n_nodes = 1 + n_kept + s_nvalid;

  // Merge: root, kept drafts, valid retrieval slots.
  if (tid == 0) {
    s_out_tok[0] = root;
    s_out_par[0] = -1;
  }
  if (kept) {
    const int ni = s_newidx[tid];
    s_out_tok[ni] = my_token;
    s_out_par[ni] = my_parent < 0 ? 0 : s_newidx[my_parent];
  }
  if (tid < k_fill && s_slot_valid[tid]) {
    const int ni = s_slot_new[tid];
    const int ps = cfg.env_parent[tid];
    s_out_tok[ni] = s_slot_tok[tid];
    s_out_par[ni] = ps < 0 ? 0 : s_slot_new[ps];
  }
  __syncthreads();

  // Per output node: depth, position and ancestor-or-self mask.
  if (tid < p.n_max) {
    const size_t o = (size_t)b * p.n_max + tid;
    uint32_t m[GRAFT_MAX_NODES / 32] = {0u, 0u, 0u, 0u};
    if (tid < n_nodes) {
      // Parents precede children, so the walk takes at most tid steps; the
      // bound also holds on inputs that break the documented preconditions.
      int d = 0;
      int j = tid;
      for (int steps = 0; j >= 0 && j <= tid && steps <= tid; ++steps) {
        m[j >> 5] |= 1u << (j & 31);
        const int pj = s_out_par[j];
        j = pj < j ? pj : -1;
        d += (j >= 0);
      }
      p.tree_token[o] = s_out_tok[tid];
      p.tree_parent[o] = s_out_par[tid];
      p.tree_pos[o] = p.prefix_len[b] + d;
    } else {
      p.tree_token[o] = -1;
      p.tree_parent[o] = -1;
      p.tree_pos[o] = -1;
    }
    for (int w = 0; w < p.words; ++w) p.tree_mask[o * p.words + w] = m[w];
  }
  if (tid == 0) {
    p.n_nodes[b] = n_nodes;
    p.stage_out[b] = stage;
  }
}

}  // namespace

void launch_build_tree(const BuildParams &p, hipStream_t stream) {
  hipLaunchKernelGGL(build_tree_kernel, dim3(p.batch), dim3(kThreads), 0, stream, p);
}

}  // namespace graft
