// Hybrid tree assembly: prune the draft tree, fill the released budget from
// the successor table M starting at the root, merge, and emit ancestor masks
// and position ids.  One workgroup per sequence.
//
// Retrieval only needs the root token (the three-point summary of "Draft
// Less, Retrieve More" has it start from the root in parallel with
// drafting), so every envelope slot is resolved speculatively from the start
// of the kernel, one envelope level per phase; each level's M lookups are in
// flight while the workgroup does one phase of the pruning work in LDS.  The
// merge then takes the first kmax - n_kept slots.
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
  __shared__ float s_pm[kThreads];
  __shared__ uint8_t s_flag[kThreads];  // candidate, then kept
  __shared__ int32_t s_newidx[kThreads];
  __shared__ uint32_t s_cmax[GRAFT_MAX_STAGES];
  __shared__ int32_t s_cexist[GRAFT_MAX_STAGES];
  __shared__ int32_t s_slot_tok[GRAFT_MAX_NODES];
  __shared__ uint8_t s_slot_valid[GRAFT_MAX_NODES];
  __shared__ int32_t s_slot_new[GRAFT_MAX_NODES];
  __shared__ int32_t s_out_tok[GRAFT_MAX_NODES];
  __shared__ int32_t s_out_par[GRAFT_MAX_NODES];
  __shared__ int32_t s_nkept, s_nvalid, s_maxlevel;

  const int n = min(max(p.n_draft[b], 0), p.n_draft_max);
  const size_t drow = (size_t)b * p.n_draft_max;
  const int root = p.root_token[b];
  const bool root_ok = root >= 0 && root < p.vocab;
  const int env = cfg.env_len;

  int32_t my_parent = -1, my_token = 0;
  float my_conf = 0.f;
  if (tid < n) {
    my_parent = p.draft_parent[drow + tid];
    my_token = p.draft_token[drow + tid];
    my_conf = p.draft_conf[drow + tid];
    if (my_parent >= tid) my_parent = -1;  // precondition guard: parent < child
  }
  // envelope level of slot tid (root children are level 0)
  int my_level = -1;
  if (tid < env) {
    my_level = 0;
    for (int j = cfg.env_parent[tid]; j >= 0; j = cfg.env_parent[j]) ++my_level;
  }
  s_parent[tid] = my_parent;
  s_pm[tid] = my_conf;
  s_newidx[tid] = 0;
  if (tid < GRAFT_MAX_STAGES) {
    s_cmax[tid] = 0u;
    s_cexist[tid] = 0;
  }
  if (tid < GRAFT_MAX_NODES) {
    s_slot_valid[tid] = 0;
    s_slot_tok[tid] = -1;
  }
  if (tid == 0) s_maxlevel = 0;
  __syncthreads();
  if (tid < env) atomicMax(&s_maxlevel, my_level);

  // One envelope level: slots of level lv look up their parent's row of M.
  // The load is issued here and its value stored by `finish` after the
  // caller's phase of pruning work, so the two overlap.
  int pending_tok = -1;
  bool pending = false;
  auto issue_level = [&](int lv) {
    pending = tid < env && my_level == lv;
    if (pending) {
      const int ps = cfg.env_parent[tid];
      const bool pok = ps < 0 ? root_ok : (s_slot_valid[ps] != 0);
      const int ptok = ps < 0 ? root : s_slot_tok[ps];
      pending_tok = pok ? p.m_ids[(size_t)ptok * p.top_s + cfg.env_rank[tid]] : -1;
    }
  };
  auto finish_level = [&]() {
    if (pending) {
      const bool ok = pending_tok >= 0 && pending_tok < p.vocab;
      s_slot_tok[tid] = pending_tok;
      s_slot_valid[tid] = ok ? 1 : 0;
    }
  };

  // ---- phase 1: level 0 lookups || draft depth and path-minimum confidence
  issue_level(0);
  int my_depth = 0;  // children of the root have draft depth 0
  float my_pm = my_conf;
  if (tid < n) {
    // parents precede children, so the walk has at most tid steps
    int j = my_parent;
    for (int steps = 0; j >= 0 && steps < tid; ++steps) {
      ++my_depth;
      my_pm = fminf(my_pm, s_pm[j]);
      j = s_parent[j];
    }
  }
  finish_level();
  __syncthreads();
  const int max_level = s_maxlevel;

  // ---- phase 2: level 1 || depth confidence c_d = max at each checkpoint
  issue_level(1);
  if (tid < n) {
    for (int s = 0; s < cfg.n_stages; ++s) {
      if (my_depth == cfg.stage_depth[s]) {
        atomicMax(&s_cmax[s], float_key(my_conf));
        s_cexist[s] = 1;
      }
    }
  }
  finish_level();
  __syncthreads();
  // every thread takes the (uniform) stage decision from LDS
  int stage = -1;
  for (int s = 0; s < cfg.n_stages; ++s) {
    if (s_cexist[s] && key_float(s_cmax[s]) < cfg.stage_tau[s]) {
      stage = s;
      break;
    }
  }
  const int k_draft = cfg.kmax - (stage < 0 ? cfg.k_ret_none : cfg.stage_k_ret[stage]);
  const bool cand = tid < n && (stage < 0 || my_depth <= cfg.stage_depth[stage]);

  // ---- phase 3: level 2 || candidates; keep the k_draft best by
  // (path-min desc, index asc)
  issue_level(2);
  s_pm[tid] = my_pm;
  s_flag[tid] = cand ? 1 : 0;
  finish_level();
  __syncthreads();
  issue_level(3);
  bool kept = false;
  if (cand) {
    int rank = 0;
    for (int j = 0; j < n; ++j) {
      if (!s_flag[j] || j == tid) continue;
      const float pj = s_pm[j];
      rank += (pj > my_pm) || (pj == my_pm && j < tid);
    }
    kept = rank < k_draft;
  }
  finish_level();
  __syncthreads();
  s_flag[tid] = kept ? 1 : 0;
  __syncthreads();

  // ---- phase 4: level 4 || compaction of kept drafts after the root
  issue_level(4);
  if (kept) {
    int before = 0;
    for (int j = 0; j < tid; ++j) before += s_flag[j];
    s_newidx[tid] = 1 + before;
  }
  if (tid == 0) {
    int cnt = 0;
    for (int j = 0; j < n; ++j) cnt += s_flag[j];
    s_nkept = cnt;
  }
  finish_level();
  __syncthreads();
  // remaining envelope levels, if the envelope is deeper
  for (int lv = 5; lv <= max_level; ++lv) {
    issue_level(lv);
    finish_level();
    __syncthreads();
  }
  const int n_kept = s_nkept;
  const int k_fill = cfg.kmax - n_kept;

  // valid slots among the first k_fill, compacted after the kept drafts
  const bool slot_ok = tid < k_fill && s_slot_valid[tid];
  if (slot_ok) {
    int before = 0;
    for (int j = 0; j < tid; ++j) before += s_slot_valid[j];
    s_slot_new[tid] = 1 + n_kept + before;
  }
  if (tid == 0) {
    int cnt = 0;
    for (int j = 0; j < k_fill; ++j) cnt += s_slot_valid[j];
    s_nvalid = cnt;
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
  if (slot_ok) {
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
