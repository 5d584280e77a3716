// Online update of the successor table M from verified transitions.
//
// Every transition (u, v) of a call is scattered with atomics into two
// open-addressing hash tables in the caller's workspace: one keyed by the
// pair (counting its multiplicity), one keyed by the row u (counting its
// distinct successors).  A single-workgroup scan turns per-row counts into
// bucket offsets, the pairs are placed into their row's bucket, and one wave
// per touched row merges the row's current entries with its bucket and
// re-selects the top S by (score descending, id ascending).  The selection
// order is a total order and the counts are integers, so the result does not
// depend on the order in which atomics land.  Each kernel clears the
// workspace entries it consumed, so the workspace is all-zero between calls.
//
// Method: "Draft Less, Retrieve More" (aitrends.kr summary), method paragraph
// (fourth step: online update of M from the verified tree; fifth step:
// prompt evidence for long contexts, which is the same update over the
// prompt) and architecture paragraph.
#include "graft_internal.h"

namespace graft {
namespace {

constexpr int kThreads = 256;

enum { kNPairs = 0, kNRows = 1, kSavedPairs = 2, kSavedRows = 3 };

__device__ inline uint32_t hash32(uint64_t x) {
  x ^= x >> 33;
  x *= 0xff51afd7ed558ccdull;
  x ^= x >> 33;
  x *= 0xc4ceb9fe1a85ec53ull;
  x ^= x >> 33;
  return (uint32_t)x;
}

struct Tables {
  unsigned long long *pair_key;
  uint32_t *pair_cnt;
  int32_t *row_key;  // u + 1, 0 = empty
  uint32_t *row_nnew;
  uint32_t *row_off;
  uint32_t *row_fill;
  uint32_t *pair_list;
  uint32_t *row_list;
  int32_t *bucket_v;
  uint32_t *bucket_c;
  uint32_t *counters;
  uint32_t mask;  // capacity - 1
};

__device__ inline Tables tables(const UpdateParams &p) {
  Tables t;
  char *w = p.ws;
  t.pair_key = reinterpret_cast<unsigned long long *>(w + p.lay.off_pair_key);
  t.pair_cnt = reinterpret_cast<uint32_t *>(w + p.lay.off_pair_cnt);
  t.row_key = reinterpret_cast<int32_t *>(w + p.lay.off_row_key);
  t.row_nnew = reinterpret_cast<uint32_t *>(w + p.lay.off_row_nnew);
  t.row_off = reinterpret_cast<uint32_t *>(w + p.lay.off_row_off);
  t.row_fill = reinterpret_cast<uint32_t *>(w + p.lay.off_row_fill);
  t.pair_list = reinterpret_cast<uint32_t *>(w + p.lay.off_pair_list);
  t.row_list = reinterpret_cast<uint32_t *>(w + p.lay.off_row_list);
  t.bucket_v = reinterpret_cast<int32_t *>(w + p.lay.off_bucket_v);
  t.bucket_c = reinterpret_cast<uint32_t *>(w + p.lay.off_bucket_c);
  t.counters = reinterpret_cast<uint32_t *>(w + p.lay.off_counters);
  t.mask = p.lay.capacity - 1;
  return t;
}

// Find the row slot of u (it is present once the scatter kernel has run).
__device__ inline uint32_t find_row(const Tables &t, int u) {
  uint32_t s = hash32((uint64_t)u) & t.mask;
  for (uint32_t probe = 0; probe <= t.mask; ++probe) {
    if (t.row_key[s] == u + 1) return s;
    s = (s + 1) & t.mask;
  }
  return 0xffffffffu;
}

// 1) scatter: one thread per potential transition.
__global__ __launch_bounds__(kThreads) void scatter_kernel(UpdateParams p) {
  const int t_id = blockIdx.x * kThreads + threadIdx.x;
  if (t_id >= p.max_transitions) return;
  const int per = p.path_stride - 1;
  const int path = t_id / per;
  const int k = t_id % per;
  const int L = p.accept_len[path];
  if (L < 0 || k > L || L + 2 > p.path_stride) return;
  const int u = p.path_tokens[(size_t)path * p.path_stride + k];
  const int v = p.path_tokens[(size_t)path * p.path_stride + k + 1];
  if (u < 0 || u >= p.vocab || v < 0 || v >= p.vocab) return;
  Tables t = tables(p);

  // row table
  uint32_t rs = hash32((uint64_t)u) & t.mask;
  for (uint32_t probe = 0; probe <= t.mask; ++probe) {
    const int old = atomicCAS(&t.row_key[rs], 0, u + 1);
    if (old == 0) {
      const uint32_t idx = atomicAdd(&t.counters[kNRows], 1u);
      t.row_list[idx] = rs;
      break;
    }
    if (old == u + 1) break;
    rs = (rs + 1) & t.mask;
  }
  // pair table
  const unsigned long long key = ((unsigned long long)(uint32_t)(u + 1) << 32) | (uint32_t)v;
  uint32_t ps = hash32(key) & t.mask;
  for (uint32_t probe = 0; probe <= t.mask; ++probe) {
    const unsigned long long old = atomicCAS(&t.pair_key[ps], 0ull, key);
    if (old == 0ull) {
      atomicAdd(&t.pair_cnt[ps], 1u);
      const uint32_t idx = atomicAdd(&t.counters[kNPairs], 1u);
      t.pair_list[idx] = ps;
      atomicAdd(&t.row_nnew[rs], 1u);
      break;
    }
    if (old == key) {
      atomicAdd(&t.pair_cnt[ps], 1u);
      break;
    }
    ps = (ps + 1) & t.mask;
  }
}

// 2) scan: bucket offsets per touched row (one workgroup).
__global__ __launch_bounds__(1024) void scan_kernel(UpdateParams p) {
  Tables t = tables(p);
  __shared__ uint32_t s_n_rows, s_carry;
  __shared__ uint32_t s_wave[16];
  if (threadIdx.x == 0) {
    s_n_rows = t.counters[kNRows];
    s_carry = 0;
    t.counters[kSavedRows] = t.counters[kNRows];
    t.counters[kSavedPairs] = t.counters[kNPairs];
  }
  __syncthreads();
  const uint32_t n_rows = s_n_rows;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (uint32_t base = 0; base < n_rows; base += 1024) {
    const uint32_t i = base + threadIdx.x;
    const uint32_t rs = i < n_rows ? t.row_list[i] : 0u;
    const uint32_t c = i < n_rows ? t.row_nnew[rs] : 0u;
    // inclusive scan within the wave
    uint32_t x = c;
    for (int off = 1; off < 64; off <<= 1) {
      const uint32_t y = __shfl_up(x, off);
      if (lane >= off) x += y;
    }
    if (lane == 63) s_wave[wave] = x;
    __syncthreads();
    if (threadIdx.x == 0) {
      uint32_t acc = 0;
      for (int w = 0; w < 16; ++w) {
        const uint32_t v = s_wave[w];
        s_wave[w] = acc;
        acc += v;
      }
    }
    __syncthreads();
    if (i < n_rows) t.row_off[rs] = s_carry + s_wave[wave] + x - c;
    __syncthreads();
    if (threadIdx.x == 1023) s_carry += s_wave[15] + x;
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    t.counters[kNRows] = 0;
    t.counters[kNPairs] = 0;
  }
}

// 3) place every distinct pair into its row's bucket; clear the pair table.
__global__ __launch_bounds__(kThreads) void place_kernel(UpdateParams p) {
  Tables t = tables(p);
  const uint32_t idx = blockIdx.x * kThreads + threadIdx.x;
  if (idx >= t.counters[kSavedPairs]) return;
  const uint32_t ps = t.pair_list[idx];
  const unsigned long long key = t.pair_key[ps];
  const int u = (int)(key >> 32) - 1;
  const int v = (int)(key & 0xffffffffull);
  const uint32_t cnt = t.pair_cnt[ps];
  const uint32_t rs = find_row(t, u);
  if (rs == 0xffffffffu) return;  // cannot happen: the scatter inserted u
  const uint32_t pos = t.row_off[rs] + atomicAdd(&t.row_fill[rs], 1u);
  t.bucket_v[pos] = v;
  t.bucket_c[pos] = cnt;
  t.pair_key[ps] = 0ull;
  t.pair_cnt[ps] = 0u;
}

__device__ inline uint32_t score_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ inline unsigned long long cand_key(float score, int id) {
  return ((unsigned long long)score_key(score) << 32) | (uint32_t)(~(uint32_t)id);
}

// 4) per touched row: merge and re-select the top S (one wave per row).
__global__ __launch_bounds__(kThreads) void reselect_kernel(UpdateParams p) {
  Tables t = tables(p);
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const uint32_t idx = blockIdx.x * (kThreads / 64) + wave;
  __shared__ int32_t s_id[kThreads / 64][GRAFT_MAX_TOP_S];
  __shared__ float s_sc[kThreads / 64][GRAFT_MAX_TOP_S];
  __shared__ uint32_t s_add[kThreads / 64][GRAFT_MAX_TOP_S];
  if (idx >= t.counters[kSavedRows]) return;  // whole wave leaves together
  const int S = p.top_s;
  const uint32_t rs = t.row_list[idx];
  const int u = t.row_key[rs] - 1;
  const uint32_t n = t.row_nnew[rs];
  const uint32_t off = t.row_off[rs];
  int32_t *ids = p.m_ids + (size_t)u * S;
  float *sc = p.m_scores + (size_t)u * S;

  if (lane < S) {
    s_id[wave][lane] = ids[lane];
    s_sc[wave][lane] = sc[lane];
    s_add[wave][lane] = 0u;
  }
  __builtin_amdgcn_wave_barrier();
  // bucket entries that are already in the row add to that entry
  for (uint32_t e = lane; e < n; e += 64) {
    const int v = t.bucket_v[off + e];
    for (int s = 0; s < S; ++s)
      if (s_id[wave][s] == v) s_add[wave][s] = t.bucket_c[off + e];
  }
  __builtin_amdgcn_wave_barrier();

  // S rounds of "best candidate strictly below the previous pick"
  unsigned long long last = ~0ull;
  for (int r = 0; r < S; ++r) {
    unsigned long long best = 0ull;
    for (int s = lane; s < S; s += 64) {
      const int id = s_id[wave][s];
      if (id < 0) continue;
      const float score = s_sc[wave][s] + (float)s_add[wave][s];
      const unsigned long long k = cand_key(score, id);
      if (k < last && k > best) best = k;
    }
    for (uint32_t e = lane; e < n; e += 64) {
      const int v = t.bucket_v[off + e];
      bool resident = false;
      for (int s = 0; s < S; ++s) resident |= (s_id[wave][s] == v);
      if (resident) continue;
      const unsigned long long k = cand_key((float)t.bucket_c[off + e], v);
      if (k < last && k > best) best = k;
    }
    for (int o = 32; o > 0; o >>= 1) {
      const unsigned long long y = __shfl_xor(best, o);
      best = y > best ? y : best;
    }
    // write after all lanes have read the old row (s_id/s_sc live in LDS)
    if (lane == r) {
      if (best == 0ull) {
        ids[r] = -1;
        sc[r] = 0.f;
      } else {
        const uint32_t sk = (uint32_t)(best >> 32);
        const uint32_t bits = (sk & 0x80000000u) ? (sk & 0x7fffffffu) : ~sk;
        ids[r] = (int)(~(uint32_t)(best & 0xffffffffull));
        sc[r] = __uint_as_float(bits);
      }
    }
    last = best == 0ull ? 0ull : best;
    if (best == 0ull) {
      for (int s = r + 1 + lane; s < S; s += 64) {
        ids[s] = -1;
        sc[s] = 0.f;
      }
      break;
    }
  }
  // clear this row's table entries
  if (lane == 0) {
    t.row_key[rs] = 0;
    t.row_nnew[rs] = 0u;
    t.row_off[rs] = 0u;
    t.row_fill[rs] = 0u;
  }
}

}  // namespace

UpdateLayout update_layout(uint32_t capacity) {
  UpdateLayout l{};
  l.capacity = capacity;
  const size_t C = capacity, T = capacity / 2;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o = align_up(o + bytes, 256);
    return at;
  };
  l.off_pair_key = take(C * 8);
  l.off_pair_cnt = take(C * 4);
  l.off_row_key = take(C * 4);
  l.off_row_nnew = take(C * 4);
  l.off_row_off = take(C * 4);
  l.off_row_fill = take(C * 4);
  l.off_pair_list = take(T * 4);
  l.off_row_list = take(T * 4);
  l.off_bucket_v = take(T * 4);
  l.off_bucket_c = take(T * 4);
  l.off_counters = take(64);
  l.total = o;
  return l;
}

void launch_update(const UpdateParams &p, hipStream_t stream) {
  const uint32_t half = p.lay.capacity / 2;
  const int g1 = (p.max_transitions + kThreads - 1) / kThreads;
  hipLaunchKernelGGL(scatter_kernel, dim3(g1), dim3(kThreads), 0, stream, p);
  hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(1024), 0, stream, p);
  hipLaunchKernelGGL(place_kernel, dim3((half + kThreads - 1) / kThreads), dim3(kThreads), 0,
                     stream, p);
  hipLaunchKernelGGL(reselect_kernel, dim3((half + 3) / 4), dim3(kThreads), 0, stream, p);
}

}  // namespace graft
