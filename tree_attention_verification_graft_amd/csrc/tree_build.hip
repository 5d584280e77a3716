// Hybrid tree assembly: prune the draft tree, fill the released budget from
// the successor table M starting at the root, merge, and emit ancestor masks
// and position ids.  One workgroup per sequence.
//
// Retrieval only needs the root token (the three-point summary of "Draft
// Less, Retrieve More" has it start from the root in parallel with
// drafting), so every envelope slot is resolved speculatively from the start
// of the kernel, one envelope level per phase; each level's M lookups are in
// flight while the workgroup does one phase of the pruning work in LDS.  The
// merge then takes the first kmax - n_kept slots.  The chain of dependent
// M lookups (one per envelope level) is the kernel's critical path, so every
// other step is kept to a few LDS operations: counts and compactions are
// wave ballots, and the best-K_draft selection only ranks when the
// candidates exceed the budget.
//
// Method: "Draft Less, Retrieve More" (aitrends.kr summary), method paragraph
// steps one to three and the architecture paragraph; readings as documented
// in include/graft.h.
#include "graft_internal.h"

namespace graft {
namespace {

constexpr int kThreads = 256;  // == GRAFT_MAX_DRAFT
constexpr int kWaves = kThreads / 64;

// Order-preserving map of a float onto uint32 (larger float -> larger uint).
__device__ inline uint32_t float_key(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ inline float key_float(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
  return __uint_as_float(u);
}

// Block-wide exclusive count of `flag` over thread index, and the total.
// `cnt` is a per-call LDS array of kWaves words; the call contains one
// barrier.
struct Count {
  int before, total;
};
__device__ inline Count block_count(bool flag, uint32_t *cnt) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const unsigned long long bal = __ballot(flag);
  if (lane == 0) cnt[wave] = (uint32_t)__popcll(bal);
  __syncthreads();
  Count r;
  r.before = __popcll(bal & ((1ull << lane) - 1ull));
  r.total = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const int c = (int)cnt[w];
    r.before += w < wave ? c : 0;
    r.total += c;
  }
  return r;
}

__global__ __launch_bounds__(kThreads) void build_tree_kernel(BuildParams p) {
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const graft_tree_config &cfg = p.cfg;

  __shared__ int32_t s_parent[kThreads];
  __shared__ float s_pm[kThreads];
  __shared__ unsigned long long s_key[kThreads];  // candidate keys, compacted
  __shared__ int32_t s_newidx[kThreads];
  __shared__ uint32_t s_cmax[GRAFT_MAX_STAGES];
  __shared__ int32_t s_cexist[GRAFT_MAX_STAGES];
  __shared__ int32_t s_slot_tok[GRAFT_MAX_NODES];
  __shared__ uint8_t s_slot_valid[GRAFT_MAX_NODES];
  __shared__ int32_t s_slot_new[GRAFT_MAX_NODES];
  __shared__ int32_t s_out_tok[GRAFT_MAX_NODES];
  __shared__ int32_t s_out_par[GRAFT_MAX_NODES];
  __shared__ uint32_t s_cnt[4][kWaves];

  // ---- every input load is issued up front; none depends on another
  const int n_raw = p.n_draft[b];
  const int root = p.root_token[b];
  const int prefix = p.prefix_len[b];
  const size_t drow = (size_t)b * p.n_draft_max;
  int32_t my_parent = -1, my_token = 0;
  float my_conf = 0.f;
  if (tid < p.n_draft_max) {
    my_parent = p.draft_parent[drow + tid];
    my_token = p.draft_token[drow + tid];
    my_conf = p.draft_conf[drow + tid];
  }
  const int env = cfg.env_len;
  int env_par = -1, env_rank = 0, env_lvl = -1;
  if (tid < env) {
    env_par = cfg.env_parent[tid];
    env_rank = cfg.env_rank[tid];
    env_lvl = p.env_level[tid];
  }
  const int n = min(max(n_raw, 0), p.n_draft_max);
  const bool is_draft = tid < n;
  if (!is_draft || my_parent >= tid) my_parent = -1;  // precondition guard: parent < child
  const bool root_ok = root >= 0 && root < p.vocab;

  // One envelope level: slots of level lv look up their parent's row of M.
  // The load is issued by `issue_level` and its value stored by
  // `finish_level` after the caller's phase of pruning work, so the two
  // overlap.
  int pending_tok = -1;
  bool pending = false;
  auto issue_level = [&](int lv) {
    pending = tid < env && env_lvl == lv;
    if (pending) {
      const bool pok = env_par < 0 ? root_ok : (s_slot_valid[env_par] != 0);
      const int ptok = env_par < 0 ? root : s_slot_tok[env_par];
      pending_tok = pok ? p.m_ids[(size_t)ptok * p.top_s + env_rank] : -1;
    }
  };
  auto finish_level = [&]() {
    if (pending) {
      s_slot_tok[tid] = pending_tok;
      s_slot_valid[tid] = (pending_tok >= 0 && pending_tok < p.vocab) ? 1 : 0;
    }
  };

  // ---- level 0 || draft depth and path-minimum confidence
  issue_level(0);
  s_parent[tid] = my_parent;
  s_pm[tid] = my_conf;
  if (tid < GRAFT_MAX_STAGES) {
    s_cmax[tid] = 0u;
    s_cexist[tid] = 0;
  }
  if (tid < GRAFT_MAX_NODES) {
    s_slot_valid[tid] = 0;
    s_slot_tok[tid] = -1;
  }
  __syncthreads();
  int my_depth = 0;  // children of the root have draft depth 0
  float my_pm = my_conf;
  if (is_draft) {
    // parents precede children, so the walk has at most tid steps
    int j = my_parent;
    for (int steps = 0; j >= 0 && steps < tid; ++steps) {
      ++my_depth;
      my_pm = fminf(my_pm, s_pm[j]);
      j = s_parent[j];
    }
  }
  // depth confidence c_d = max over the drafts at each checkpoint depth
  if (is_draft) {
    for (int s = 0; s < cfg.n_stages; ++s) {
      if (my_depth == cfg.stage_depth[s]) {
        atomicMax(&s_cmax[s], float_key(my_conf));
        s_cexist[s] = 1;
      }
    }
  }
  finish_level();
  __syncthreads();

  // ---- level 1 || stage decision (uniform) and the candidate count
  issue_level(1);
  int stage = -1;
  for (int s = 0; s < cfg.n_stages; ++s) {
    if (s_cexist[s] && key_float(s_cmax[s]) < cfg.stage_tau[s]) {
      stage = s;
      break;
    }
  }
  const int k_draft = cfg.kmax - (stage < 0 ? cfg.k_ret_none : cfg.stage_k_ret[stage]);
  const bool cand = is_draft && (stage < 0 || my_depth <= cfg.stage_depth[stage]);
  const Count cc = block_count(cand, s_cnt[0]);
  bool kept = cand;
  if (cc.total > k_draft) {
    // keep the k_draft best by (path-min desc, index asc): a candidate's
    // rank is the number of candidate keys above its own
    const unsigned long long key =
        ((unsigned long long)float_key(my_pm) << 32) | (uint32_t)(kThreads - 1 - tid);
    if (cand) s_key[cc.before] = key;
    __syncthreads();
    if (cand) {
      int rank = 0;
      for (int j = 0; j < cc.total; ++j) rank += s_key[j] > key;
      kept = rank < k_draft;
    }
  }
  finish_level();
  __syncthreads();

  // ---- level 2 || compaction of the kept drafts after the root
  issue_level(2);
  const Count ck = block_count(kept, s_cnt[1]);
  s_newidx[tid] = kept ? 1 + ck.before : 0;
  const int n_kept = ck.total;
  finish_level();
  __syncthreads();
  // remaining envelope levels
  for (int lv = 3; lv < p.env_levels; ++lv) {
    issue_level(lv);
    finish_level();
    __syncthreads();
  }

  // valid slots among the first k_fill, compacted after the kept drafts
  const int k_fill = cfg.kmax - n_kept;
  const bool slot_ok = tid < k_fill && tid < env && s_slot_valid[tid];
  const Count cs = block_count(slot_ok, s_cnt[2]);
  if (slot_ok) s_slot_new[tid] = 1 + n_kept + cs.before;
  const int n_nodes = 1 + n_kept + cs.total;
  __syncthreads();

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
    s_out_tok[ni] = s_slot_tok[tid];
    s_out_par[ni] = env_par < 0 ? 0 : s_slot_new[env_par];
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
      p.tree_pos[o] = prefix + d;
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
