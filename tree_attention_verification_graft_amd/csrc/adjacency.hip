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
// Calls with at most 4096 potential transitions (one decode step; callers
// whose transitions are nearly all valid lower that limit) take a path that
// sorts the pairs in LDS instead and needs no workspace; both paths give the
// same table.
//
// Method: "Draft Less, Retrieve More" (aitrends.kr summary), method paragraph
// (fourth step: online update of M from the verified tree; fifth step:
// prompt evidence for long contexts, which is the same update over the
// prompt) and architecture paragraph.
#include "graft_internal.h"

#include <algorithm>

namespace graft {
namespace {

constexpr int kThreads = 256;

enum { kNPairs = 0, kNRows = 1, kSavedPairs = 2, kSavedRows = 3 };

// Hash of a 64-bit key for the open-addressing tables: the 64-bit finalizer
// ("fmix64") of Austin Appleby's public-domain MurmurHash3, with its published
// shift amounts and multipliers.
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
__device__ inline float key_score(unsigned long long k) {
  const uint32_t sk = (uint32_t)(k >> 32);
  return __uint_as_float((sk & 0x80000000u) ? (sk & 0x7fffffffu) : ~sk);
}
__device__ inline int key_id(unsigned long long k) { return (int)(~(uint32_t)(k & 0xffffffffull)); }

// Per-wave LDS scratch of the row merge.
// One bitonic step at position i of lane-held keys, partner i ^ stride in
// the same wave: the lower position keeps the min when the block sorts up.
__device__ inline unsigned long long bitonic_step(unsigned long long x, int i, int size,
                                                  int stride) {
  unsigned long long a, b;
  lane_pair(x, stride, a, b);
  const unsigned long long mn = a < b ? a : b, mx = a < b ? b : a;
  const bool up = (i & size) == 0, lower = (i & stride) == 0;
  return lower == up ? mn : mx;
}

struct RowScratch {
  int32_t id[GRAFT_MAX_TOP_S];
  float sc[GRAFT_MAX_TOP_S];
  uint32_t add[GRAFT_MAX_TOP_S];
  unsigned long long key[64];
};

// Merge row u of M (ids/sc, S entries) with n new successor entries and
// re-select the top S by (score descending, id ascending); one wave.
// get(e) returns {v, count, first}: entries with first == false repeat an
// earlier entry and are ignored.  Distinct ids per row make the candidate
// keys distinct, so ranks are a permutation.
struct NewEntry {
  int v;
  uint32_t count;
  bool first;
};
template <class Get>
__device__ void merge_row(int32_t *ids, float *sc, int S, int n, const Get &get, RowScratch &w) {
  const int lane = threadIdx.x & 63;
  int my_id = -1;
  float my_sc = 0.f;
  if (lane < S) {
    my_id = ids[lane];
    my_sc = sc[lane];
    w.id[lane] = my_id;
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  if (S + n <= 64) {
    // One candidate per lane: lanes < S hold the row's entries, lanes S ..
    // S + n - 1 the new entries; each candidate's output slot is its rank.
    bool valid = false;
    int id = -1;
    float score = 0.f;
    if (lane < S) {
      id = my_id;
      valid = id >= 0;
      uint32_t add = 0u;
      for (int e = 0; e < n; ++e) {
        const NewEntry x = get(e);
        if (x.first && x.v == id) add = x.count;
      }
      score = my_sc + (float)add;
    } else if (lane < S + n) {
      const NewEntry x = get(lane - S);
      bool resident = false;
      for (int q = 0; q < S; ++q) resident |= (w.id[q] == x.v);
      valid = x.first && !resident;
      id = x.v;
      score = (float)x.count;
    }
    const unsigned long long key = valid ? cand_key(score, id) : 0ull;
    w.key[lane] = key;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    int rank = 0;
    for (int k = 0; k < S + n; ++k) rank += (w.key[k] > key);
    const int n_valid = __popcll(__ballot(valid));
    if (valid && rank < S) {
      ids[rank] = id;
      sc[rank] = score;
    }
    if (lane >= n_valid && lane < S) {
      ids[lane] = -1;
      sc[lane] = 0.f;
    }
    return;
  }

  // Many new entries (a frequent token): S rounds of "best candidate
  // strictly below the previous pick".
  if (lane < S) {
    w.sc[lane] = my_sc;
    w.add[lane] = 0u;
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  constexpr int kRegEntries = 16;  // new entries per lane held in registers
  if (n <= 64 * kRegEntries) {
    // Each lane reads its entries once: a resident successor's count goes
    // to w.add (first entries carry distinct tokens, so no two lanes write
    // one slot), any other successor becomes a candidate key kept in
    // registers, and the rounds scan only those.
    unsigned long long ck[kRegEntries];
#pragma unroll
    for (int t = 0; t < kRegEntries; ++t) {
      ck[t] = 0ull;
      const int e = lane + 64 * t;
      if (e < n) {
        const NewEntry x = get(e);
        if (x.first) {
          bool resident = false;
          for (int q = 0; q < S; ++q) {
            if (w.id[q] == x.v) {
              w.add[q] = x.count;
              resident = true;
            }
          }
          if (!resident) ck[t] = cand_key((float)x.count, x.v);
        }
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    unsigned long long last = ~0ull;
    for (int r = 0; r < S; ++r) {
      unsigned long long best = 0ull;
      if (lane < S && w.id[lane] >= 0) {
        const unsigned long long k = cand_key(w.sc[lane] + (float)w.add[lane], w.id[lane]);
        if (k < last) best = k;
      }
#pragma unroll
      for (int t = 0; t < kRegEntries; ++t)
        if (ck[t] < last && ck[t] > best) best = ck[t];
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) {
        unsigned long long a, b;
        lane_pair(best, o, a, b);
        best = a > b ? a : b;
      }
      // the old row lives in LDS, so writing slot r cannot disturb the reads
      if (lane == 0) {
        ids[r] = best ? key_id(best) : -1;
        sc[r] = best ? key_score(best) : 0.f;
      }
      if (best == 0ull) {
        for (int q = r + 1 + lane; q < S; q += 64) {
          ids[q] = -1;
          sc[q] = 0.f;
        }
        break;
      }
      last = best;
    }
    return;
  }
  // Longer rows read their entries again in every round.
  for (int e = lane; e < n; e += 64) {
    const NewEntry x = get(e);
    if (!x.first) continue;
    for (int q = 0; q < S; ++q)
      if (w.id[q] == x.v) w.add[q] = x.count;
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  unsigned long long last = ~0ull;
  for (int r = 0; r < S; ++r) {
    unsigned long long best = 0ull;
    if (lane < S && w.id[lane] >= 0) {
      const unsigned long long k = cand_key(w.sc[lane] + (float)w.add[lane], w.id[lane]);
      if (k < last) best = k;
    }
    for (int e = lane; e < n; e += 64) {
      const NewEntry x = get(e);
      if (!x.first) continue;
      bool resident = false;
      for (int q = 0; q < S; ++q) resident |= (w.id[q] == x.v);
      if (resident) continue;
      const unsigned long long k = cand_key((float)x.count, x.v);
      if (k < last && k > best) best = k;
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      unsigned long long a, b;
      lane_pair(best, o, a, b);
      best = a > b ? a : b;
    }
    // the old row lives in LDS, so writing slot r cannot disturb the reads
    if (lane == 0) {
      ids[r] = best ? key_id(best) : -1;
      sc[r] = best ? key_score(best) : 0.f;
    }
    if (best == 0ull) {
      for (int q = r + 1 + lane; q < S; q += 64) {
        ids[q] = -1;
        sc[q] = 0.f;
      }
      break;
    }
    last = best;
  }
}

// 4) per touched row: merge and re-select the top S (one wave per row).
__global__ __launch_bounds__(kThreads) void reselect_kernel(UpdateParams p) {
  Tables t = tables(p);
  const int wave = threadIdx.x >> 6;
  const uint32_t idx = blockIdx.x * (kThreads / 64) + wave;
  __shared__ RowScratch s_w[kThreads / 64];
  if (idx >= t.counters[kSavedRows]) return;  // whole wave leaves together
  const int S = p.top_s;
  const uint32_t rs = t.row_list[idx];
  const int u = t.row_key[rs] - 1;
  const uint32_t n = t.row_nnew[rs];
  const uint32_t off = t.row_off[rs];
  const int32_t *bv = t.bucket_v + off;
  const uint32_t *bc = t.bucket_c + off;
  merge_row(p.m_ids + (size_t)u * S, p.m_scores + (size_t)u * S, S, (int)n,
            [&](int e) { return NewEntry{bv[e], bc[e], true}; }, s_w[wave]);
  // clear this row's table entries
  if ((threadIdx.x & 63) == 0) {
    t.row_key[rs] = 0;
    t.row_nnew[rs] = 0u;
    t.row_off[rs] = 0u;
    t.row_fill[rs] = 0u;
  }
}

// ---------------------------------------------------------------------------
// Small calls (at most kSmallT potential transitions, the per-step case).
// Rows are partitioned over the workgroups by source token: workgroup g owns
// the rows u with u mod G = g.  Each workgroup gathers the valid (u, v) keys
// of its own rows into LDS, sorts them (equal pairs form runs whose length
// is the count; each row is one segment), numbers its rows in sorted order
// and merges them with one wave per row.  No two workgroups touch the same
// row, so they need no agreement, and the table needs no workspace.
constexpr int kSmallT = 4096;
constexpr int kSmallThreads = 1024;
constexpr int kSmallWaves = kSmallThreads / 64;

__device__ inline void cas_pair(unsigned long long &a, unsigned long long &b, bool up) {
  if ((a > b) == up) {
    const unsigned long long t = a;
    a = b;
    b = t;
  }
}

__global__ __launch_bounds__(kSmallThreads) void update_small_kernel(UpdateParams p) {
  __shared__ unsigned long long s_key[kSmallT];
  __shared__ uint16_t s_row_beg[kSmallT + 1];  // row r spans [beg[r], beg[r + 1])
  __shared__ uint32_t s_wave_cnt[kSmallWaves];
  __shared__ RowScratch s_w[kSmallWaves];
  __shared__ int s_nv;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const unsigned long long kNone = ~0ull;

  // 1) gather the valid (u, v) keys of this workgroup's rows (in any order:
  // they are sorted next)
  if (tid == 0) s_nv = 0;
  __syncthreads();
  // kGather transitions per thread per round, every load of a round issued
  // before any is used: for t < max_transitions = n_paths * (path_stride -
  // 1), the path index is below n_paths and k + 1 below path_stride, so the
  // token reads stay inside the path array whatever accept_len holds
  constexpr int kGather = 4;
  const int per = p.path_stride - 1;
  for (int t0 = 0; t0 < p.max_transitions; t0 += kSmallThreads * kGather) {
    int L[kGather], u[kGather], v[kGather], k[kGather];
#pragma unroll
    for (int j = 0; j < kGather; ++j) {
      const int t = t0 + j * kSmallThreads + tid;
      L[j] = -1;
      u[j] = v[j] = k[j] = 0;
      if (t < p.max_transitions) {
        const int path = t / per;
        k[j] = t % per;
        L[j] = p.accept_len[path];
        u[j] = p.path_tokens[(size_t)path * p.path_stride + k[j]];
        v[j] = p.path_tokens[(size_t)path * p.path_stride + k[j] + 1];
      }
    }
#pragma unroll
    for (int j = 0; j < kGather; ++j) {
      if (L[j] >= 0 && k[j] <= L[j] && L[j] + 2 <= p.path_stride && u[j] >= 0 &&
          u[j] < p.vocab && v[j] >= 0 && v[j] < p.vocab &&
          (uint32_t)u[j] % gridDim.x == blockIdx.x)
        s_key[atomicAdd(&s_nv, 1)] =
            ((unsigned long long)(uint32_t)u[j] << 32) | (uint32_t)v[j];
    }
  }
  __syncthreads();
  const int nv = s_nv;
  if (nv == 0) return;
  int n2 = 1;
  while (n2 < nv) n2 <<= 1;

  // 2) ascending bitonic sort of the n2 >= nv keys (padding sorts last)
  if (n2 <= 64) {
    if (wave == 0) {
      unsigned long long x = lane < nv ? s_key[lane] : kNone;
#pragma unroll
      for (int size = 2; size <= 64; size <<= 1)
#pragma unroll
        for (int stride = size >> 1; stride > 0; stride >>= 1)
          x = bitonic_step(x, lane, size, stride);
      if (lane < nv) s_key[lane] = x;
    }
  } else if (n2 <= kSmallThreads) {
    // one key per thread: strides below 64 within the wave's lanes, larger
    // ones through LDS (n2 is a multiple of 64, so a wave is wholly inside
    // or wholly past the keys)
    const bool own = tid < n2;
    unsigned long long x = own && tid < nv ? s_key[tid] : kNone;
    for (int size = 2; size <= n2; size <<= 1) {
      int stride = size >> 1;
      for (; stride >= 64; stride >>= 1) {
        __syncthreads();  // earlier reads of s_key are done
        if (own) s_key[tid] = x;
        __syncthreads();
        if (own) {
          const unsigned long long y = s_key[tid ^ stride];
          const unsigned long long mn = x < y ? x : y, mx = x < y ? y : x;
          x = ((tid & stride) == 0) == ((tid & size) == 0) ? mn : mx;
        }
      }
      if (own) {
#pragma unroll
        for (int st = 32; st > 0; st >>= 1)
          if (st <= stride) x = bitonic_step(x, tid, size, st);
      }
    }
    __syncthreads();
    if (own) s_key[tid] = x;
  } else {
    for (int i = nv + tid; i < n2; i += kSmallThreads) s_key[i] = kNone;
    __syncthreads();
    for (int size = 2; size <= n2; size <<= 1) {
      for (int stride = size >> 1; stride > 0; stride >>= 1) {
        for (int i = tid; i < n2 / 2; i += kSmallThreads) {
          const int lo = 2 * i - (i & (stride - 1));
          unsigned long long a = s_key[lo], b = s_key[lo + stride];
          cas_pair(a, b, (lo & size) == 0);
          s_key[lo] = a;
          s_key[lo + stride] = b;
        }
        __syncthreads();
      }
    }
  }
  __syncthreads();

  // 3) number the rows: row r starts at the r-th position whose u differs
  // from its predecessor (a block-wide scan of the start flags)
  int carry = 0;
  for (int base = 0; base < nv; base += kSmallThreads) {
    const int i = base + tid;
    const bool start = i < nv && (i == 0 || (s_key[i] >> 32) != (s_key[i - 1] >> 32));
    const unsigned long long bal = __ballot(start);
    const int below = __popcll(bal & ((1ull << lane) - 1ull));
    if (lane == 0) s_wave_cnt[wave] = (uint32_t)__popcll(bal);
    __syncthreads();
    int before = carry;
    for (int w = 0; w < wave; ++w) before += (int)s_wave_cnt[w];
    if (start) s_row_beg[before + below] = (uint16_t)i;
    int total = 0;
    for (int w = 0; w < kSmallWaves; ++w) total += (int)s_wave_cnt[w];
    carry += total;
    __syncthreads();
  }
  const int n_rows = carry;
  if (tid == 0) s_row_beg[n_rows] = (uint16_t)nv;
  __syncthreads();

  // 4) this workgroup's rows, one wave each
  const int S = p.top_s;
  for (int r = wave; r < n_rows; r += kSmallWaves) {
    const int beg = s_row_beg[r];
    const int end = s_row_beg[r + 1];
    const int u = (int)(s_key[beg] >> 32);
    auto get = [&](int e) {
      const int i = beg + e;
      const unsigned long long k = s_key[i];
      NewEntry x;
      x.v = (int)(k & 0xffffffffull);
      x.first = i == beg || s_key[i - 1] != k;
      int j = i + 1;
      if (x.first)
        while (j < end && s_key[j] == k) ++j;
      x.count = (uint32_t)(j - i);
      return x;
    };
    merge_row(p.m_ids + (size_t)u * S, p.m_scores + (size_t)u * S, S, end - beg, get,
              s_w[wave]);
  }
}

// The all-node variant: every verified node's (token, argmax) as one
// length-2 path; rows past n_nodes get accept length -1 (skipped).
__global__ __launch_bounds__(kThreads) void tree_pairs_kernel(int32_t batch, int32_t n_max,
                                                             const int32_t *tree_token,
                                                             const int32_t *argmax,
                                                             const int32_t *n_nodes,
                                                             int32_t *pairs, int32_t *lens) {
  const long r = (long)blockIdx.x * kThreads + threadIdx.x;
  if (r >= (long)batch * n_max) return;
  const int b = (int)(r / n_max), i = (int)(r % n_max);
  const bool live = i < min(n_nodes[b], n_max);
  pairs[2 * r] = live ? tree_token[r] : -1;
  pairs[2 * r + 1] = live ? argmax[r] : -1;
  lens[r] = live ? 0 : -1;
}

}  // namespace

void launch_tree_pairs(int32_t batch, int32_t n_max, const int32_t *tree_token,
                       const int32_t *argmax, const int32_t *n_nodes, int32_t *pairs,
                       int32_t *lens, hipStream_t stream) {
  const long rows = (long)batch * n_max;
  hipLaunchKernelGGL(tree_pairs_kernel, dim3((unsigned)((rows + kThreads - 1) / kThreads)),
                     dim3(kThreads), 0, stream, batch, n_max, tree_token, argmax, n_nodes, pairs,
                     lens);
}

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
  if (p.max_transitions <= kSmallT) {
    // enough workgroups that every touched row (at most one per transition)
    // gets a wave of its own (at most 256 at kSmallT transitions; a cap of 64
    // left two rows per wave at 2,080 transitions, one more round trip)
    const int groups = std::max(1, (p.max_transitions + kSmallWaves - 1) / kSmallWaves);
    hipLaunchKernelGGL(update_small_kernel, dim3(groups), dim3(kSmallThreads), 0, stream, p);
    return;
  }
  const uint32_t half = p.lay.capacity / 2;
  const int g1 = (p.max_transitions + kThreads - 1) / kThreads;
  hipLaunchKernelGGL(scatter_kernel, dim3(g1), dim3(kThreads), 0, stream, p);
  hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(1024), 0, stream, p);
  // distinct pairs and touched rows are both at most max_transitions
  const uint32_t most = std::min<uint32_t>(half, (uint32_t)p.max_transitions);
  hipLaunchKernelGGL(place_kernel, dim3((most + kThreads - 1) / kThreads), dim3(kThreads), 0,
                     stream, p);
  hipLaunchKernelGGL(reselect_kernel, dim3((most + 3) / 4), dim3(kThreads), 0, stream, p);
}

}  // namespace graft
