// Greedy (lossless) acceptance of the verified hybrid tree, in two launches.
//
// argmax_chunks_kernel streams the logits: every (node row, vocab chunk)
// pair is one workgroup whose threads issue all of their 16-byte loads
// before reducing, so a launch keeps the whole live logits tensor in flight.
// Chunks are 8 KB (two loads per thread) when the grid would otherwise be
// small, and 24 KB (three loads) for large batches, where fewer and larger
// workgroups dispatch faster.  (Measured at a 151,936-entry bf16 vocabulary:
// three loads fill a row's 25 chunks to 99% and run 5% faster than eight,
// whose 10 chunks fill it to 93%; two, four and five loads were slower.)
// A chunk reduces to one packed 64-bit key whose high half is an
// order-preserving image of the value (-0 folded onto +0) and whose low half
// is the complemented index, so an unsigned max picks the largest value and,
// among equal values, the lowest index.
//
// accept_path_kernel (one workgroup per sequence) folds the chunk keys of
// every row with LDS atomics, marks the nodes whose token equals their
// parent's argmax with wave ballots, keeps the nodes whose whole ancestor
// mask is matched, and emits the deepest one's path.
//
// Method: "Draft Less, Retrieve More" (aitrends.kr summary), architecture
// paragraph (lossless verification with retrieval nodes as proposals), read
// for greedy decoding.
#include <hip/hip_bf16.h>

#include "graft_internal.h"

namespace graft {
namespace {

constexpr int kThreads = 256;
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
constexpr int kSmallLoads = 2;      // 16-byte loads per thread, small grids
constexpr int kLargeLoads = 3;      // ... large grids
constexpr int kLargeGrid = 8192;    // workgroups above which chunks grow
// vocab entries per argmax workgroup: L * 2048 bf16 or L * 1024 f32
template <bool BF16, int L>
constexpr int chunk_len() { return L * kThreads * (BF16 ? 8 : 4); }
constexpr int kPathThreads = 256; // >= GRAFT_MAX_NODES
constexpr int kKeyBatch = 16;     // chunk keys per thread loaded at once

// Workgroup barrier that waits for LDS operations only: global loads issued
// before it stay in flight (a full __syncthreads also drains them).
__device__ __forceinline__ void lds_only_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" : : : "memory");
}

__device__ inline uint32_t ord_bf16(uint32_t u) {
  if (u == 0x8000u) u = 0;  // -0 == +0
  return (u & 0x8000u) ? (~u & 0xffffu) : (u | 0x8000u);
}
__device__ inline uint32_t ord_f32(uint32_t u) {
  if (u == 0x80000000u) u = 0;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ inline unsigned long long pack(uint32_t ord, int idx) {
  return ((unsigned long long)ord << 32) | (uint32_t)(~(uint32_t)idx);
}
__device__ inline unsigned long long umax64(unsigned long long a, unsigned long long b) {
  return a > b ? a : b;
}
__device__ inline int wave_max_i32(int v) {
  for (int off = 32; off > 0; off >>= 1) v = max(v, __shfl_xor(v, off));
  return v;
}
__device__ inline int wave_min_i32(int v) {
  for (int off = 32; off > 0; off >>= 1) v = min(v, __shfl_xor(v, off));
  return v;
}
__device__ inline unsigned long long wave_max64(unsigned long long v) {
  for (int off = 32; off > 0; off >>= 1) v = umax64(v, __shfl_xor(v, off));
  return v;
}

template <bool BF16, bool VEC, int kLoads>
__global__ __launch_bounds__(kThreads) void argmax_chunks_kernel(AcceptParams p) {
  const int c = blockIdx.x;
  const int row = blockIdx.y;  // b * n_max + i
  const int b = row / p.n_max;
  const int i = row % p.n_max;
  if (i >= p.n_nodes[b]) return;  // rows past the tree are not read
  constexpr int kChunk = chunk_len<BF16, kLoads>();
  const int lo = c * kChunk;
  const int hi = min(p.vocab, lo + kChunk);
  unsigned long long best = 0ull;
  if (VEC) {
    // 16-byte loads; lo and hi are multiples of the vector width here
    constexpr int kPer = BF16 ? 8 : 4;  // values per load
    const uint4 *x = reinterpret_cast<const uint4 *>(
        static_cast<const char *>(p.logits) + (size_t)row * p.vocab * (BF16 ? 2 : 4));
    uint4 v[kLoads];
#pragma unroll
    for (int k = 0; k < kLoads; ++k) {
      const int e = lo + (k * kThreads + threadIdx.x) * kPer;
      // read once: non-temporal loads stream past the caches
      if (e < hi) {
        const u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(x) + e / kPer);
        v[k] = make_uint4(t.x, t.y, t.z, t.w);
      } else {
        v[k] = make_uint4(0u, 0u, 0u, 0u);
      }
    }
    if (BF16) {
      // The chunk's largest key by packed 16-bit maxima (two values per
      // op), then the lowest index holding it, searched only by the threads
      // whose own maximum it is.
      short2v acc = (short2v){-32768, -32768};
#pragma unroll
      for (int k = 0; k < kLoads; ++k) {
        const int e = lo + (k * kThreads + threadIdx.x) * kPer;
        if (e >= hi) continue;
        const uint32_t w[4] = {v[k].x, v[k].y, v[k].z, v[k].w};
#pragma unroll
        for (int q = 0; q < 4; ++q) acc = __builtin_elementwise_max(acc, okey2(w[q]));
      }
      const int tmax = max((int)acc.x, (int)acc.y);
      __shared__ int s_red[kThreads / 64];
      int m = wave_max_i32(tmax);
      if ((threadIdx.x & 63) == 0) s_red[threadIdx.x >> 6] = m;
      __syncthreads();
      m = s_red[0];
#pragma unroll
      for (int w = 1; w < kThreads / 64; ++w) m = max(m, s_red[w]);
      int idx = 0x7fffffff;
      if (tmax == m) {
#pragma unroll
        for (int k = 0; k < kLoads; ++k) {
          const int e = lo + (k * kThreads + threadIdx.x) * kPer;
          if (e >= hi) continue;
          const uint32_t w[4] = {v[k].x, v[k].y, v[k].z, v[k].w};
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const short2v kq = okey2(w[q]);
            if (kq.x == m) idx = min(idx, e + 2 * q);
            if (kq.y == m) idx = min(idx, e + 2 * q + 1);
          }
        }
      }
      idx = wave_min_i32(idx);
      __syncthreads();  // every wave has read s_red
      if ((threadIdx.x & 63) == 0) s_red[threadIdx.x >> 6] = idx;
      __syncthreads();
      if (threadIdx.x == 0) {
        int i_min = s_red[0];
        for (int w = 1; w < kThreads / 64; ++w) i_min = min(i_min, s_red[w]);
        p.partial[(size_t)row * p.chunks + c] = pack(ord_bf16(key_bf16(m)), i_min);
      }
      return;
    }
#pragma unroll
    for (int k = 0; k < kLoads; ++k) {
      const int e = lo + (k * kThreads + threadIdx.x) * kPer;
      if (e >= hi) continue;
      const uint32_t w[4] = {v[k].x, v[k].y, v[k].z, v[k].w};
#pragma unroll
      for (int q = 0; q < 4; ++q) best = umax64(best, pack(ord_f32(w[q]), e + q));
    }
  } else {
    constexpr int kScalar = kChunk / kThreads;  // scalar loads per thread
    uint32_t v[kScalar];
    if (BF16) {
      const uint16_t *x = static_cast<const uint16_t *>(p.logits) + (size_t)row * p.vocab;
#pragma unroll
      for (int k = 0; k < kScalar; ++k) {
        const int e = lo + k * kThreads + threadIdx.x;
        v[k] = e < hi ? x[e] : 0u;
      }
    } else {
      const uint32_t *x = static_cast<const uint32_t *>(p.logits) + (size_t)row * p.vocab;
#pragma unroll
      for (int k = 0; k < kScalar; ++k) {
        const int e = lo + k * kThreads + threadIdx.x;
        v[k] = e < hi ? x[e] : 0u;
      }
    }
#pragma unroll
    for (int k = 0; k < kScalar; ++k) {
      const int e = lo + k * kThreads + threadIdx.x;
      if (e < hi) best = umax64(best, pack(BF16 ? ord_bf16(v[k]) : ord_f32(v[k]), e));
    }
  }
  __shared__ unsigned long long s_best[kThreads / 64];
  best = wave_max64(best);
  if ((threadIdx.x & 63) == 0) s_best[threadIdx.x >> 6] = best;
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned long long m = s_best[0];
    for (int w = 1; w < kThreads / 64; ++w) m = umax64(m, s_best[w]);
    p.partial[(size_t)row * p.chunks + c] = m;
  }
}

// Path selection, one workgroup per sequence; thread i owns node i.
__global__ __launch_bounds__(kPathThreads) void accept_path_kernel(AcceptParams p) {
  const int b = blockIdx.x;
  const int i = threadIdx.x;
  const int lane = i & 63;
  const int wave = i >> 6;
  __shared__ unsigned long long s_key[GRAFT_MAX_NODES];
  __shared__ int32_t s_am[GRAFT_MAX_NODES];
  __shared__ uint32_t s_mask[GRAFT_MAX_NODES][GRAFT_MAX_NODES / 32];
  __shared__ uint32_t s_match[GRAFT_MAX_NODES / 32];
  __shared__ uint32_t s_best[GRAFT_MAX_NODES / 64];

  // Every load below is independent of the others, so they are all in
  // flight together.
  const int n_nodes = p.n_nodes[b];
  const size_t o = (size_t)b * p.n_max + i;
  const bool in_row = i < p.n_max;
  int par = -1, tok = -1;
  uint32_t mw[4] = {0u, 0u, 0u, 0u};
  if (in_row) {
    par = p.tree_parent[o];
    tok = p.tree_token[o];
    const uint32_t *mrow = p.tree_mask + o * p.words;
#pragma unroll
    for (int w = 0; w < 4; ++w) mw[w] = w < p.words ? mrow[w] : 0u;
  }
  // chunk keys of all rows (rows past the tree are folded too and ignored
  // below): the first kKeyBatch per thread are loaded with the tree arrays,
  // before a barrier that waits only for LDS, so every load of the kernel
  // is in flight at once
  const int total = p.n_max * p.chunks;
  const unsigned long long *part = p.partial + (size_t)b * total;
  unsigned long long kb[kKeyBatch];
#pragma unroll
  for (int j = 0; j < kKeyBatch; ++j) {
    const int k = i + j * kPathThreads;
    kb[j] = k < total ? part[k] : 0ull;
  }
  if (i < GRAFT_MAX_NODES) s_key[i] = 0ull;
  lds_only_barrier();
  for (int k0 = 0; k0 < total; k0 += kKeyBatch * kPathThreads) {
    if (k0 > 0) {
#pragma unroll
      for (int j = 0; j < kKeyBatch; ++j) {
        const int k = k0 + i + j * kPathThreads;
        kb[j] = k < total ? part[k] : 0ull;
      }
    }
#pragma unroll
    for (int j = 0; j < kKeyBatch; ++j) {
      const int k = k0 + i + j * kPathThreads;
      if (k < total) atomicMax(&s_key[k / p.chunks], kb[j]);
    }
  }
  __syncthreads();

  const bool live = in_row && i < n_nodes;
  const int am = live ? (int)(~(uint32_t)(s_key[i] & 0xffffffffull)) : -1;
  if (i < GRAFT_MAX_NODES) {
    s_am[i] = am;
#pragma unroll
    for (int w = 0; w < 4; ++w) s_mask[i][w] = mw[w];
  }
  if (in_row) p.argmax[o] = am;
  __syncthreads();

  // match bit: the root always, else token == argmax of the parent's row
  const bool match = live && ((par < 0) || (par < i && tok == s_am[par]));
  const unsigned long long bal = __ballot(match);
  if (lane == 0 && wave < GRAFT_MAX_NODES / 64) {
    s_match[2 * wave] = (uint32_t)(bal & 0xffffffffull);
    s_match[2 * wave + 1] = (uint32_t)(bal >> 32);
  }
  __syncthreads();

  // fully matched: every ancestor-or-self bit is matched
  uint32_t key = 0u;
  if (live) {
    const bool full = ((mw[0] & s_match[0]) == mw[0]) && ((mw[1] & s_match[1]) == mw[1]) &&
                      ((mw[2] & s_match[2]) == mw[2]) && ((mw[3] & s_match[3]) == mw[3]);
    const int depth = __popc(mw[0]) + __popc(mw[1]) + __popc(mw[2]) + __popc(mw[3]) - 1;
    // deepest first, then the lowest index
    if (full) key = ((uint32_t)(depth + 1) << 8) | (uint32_t)(255 - i);
  }
  uint32_t wk = key;
  for (int off = 32; off > 0; off >>= 1) {
    const uint32_t ok = __shfl_xor(wk, off);
    wk = ok > wk ? ok : wk;
  }
  if (lane == 0 && wave < GRAFT_MAX_NODES / 64) s_best[wave] = wk;
  __syncthreads();
  uint32_t bk = s_best[0];
  for (int w = 1; w < GRAFT_MAX_NODES / 64; ++w) bk = s_best[w] > bk ? s_best[w] : bk;
  // bk == 0 only when no node is live (n_nodes < 1 breaks the precondition):
  // fall back to the root so that every index below stays in bounds.
  const int best = bk ? 255 - (int)(bk & 0xffu) : 0;
  const int L = bk ? (int)(bk >> 8) - 1 : 0;  // accept length = depth of best

  // path = the best node's ancestor-or-self set in index order
  int32_t *pn = p.path_nodes + (size_t)b * p.n_max;
  int32_t *pt = p.path_tokens + (size_t)b * (p.n_max + 1);
  const uint32_t *path = s_mask[best];
  const bool on_path = live && ((path[(i >> 5) & 3] >> (i & 31)) & 1u);
  if (on_path) {
    int pos = 0;
    for (int w = 0; w < (i >> 5); ++w) pos += __popc(path[w]);
    pos += __popc(path[i >> 5] & ((1u << (i & 31)) - 1u));
    if (pos < p.n_max) {
      pn[pos] = i;
      pt[pos] = tok;
    }
  }
  for (int k = i; k < p.n_max + 1; k += kPathThreads) {
    if (k < p.n_max && k > L) pn[k] = -1;
    if (k > L + 1) pt[k] = -1;
  }
  if (i == 0) {
    pt[L + 1] = s_am[best];
    p.accept_len[b] = L;
  }
}

}  // namespace

static int chunk_of(graft_dtype dtype, int loads) {
  return loads * kThreads * (dtype == GRAFT_BF16 ? 8 : 4);
}
static bool vec_ok(graft_dtype dtype, int32_t vocab) {
  return dtype == GRAFT_BF16 ? vocab % 8 == 0 : vocab % 4 == 0;
}
// Loads per thread of a launch: the larger chunks only for 16-byte-aligned
// rows whose small-chunk grid would exceed kLargeGrid workgroups.
static int loads_for(graft_dtype dtype, int32_t rows, int32_t vocab) {
  const long small = (long)rows * ((vocab + chunk_of(dtype, kSmallLoads) - 1) /
                                   chunk_of(dtype, kSmallLoads));
  return vec_ok(dtype, vocab) && small > kLargeGrid ? kLargeLoads : kSmallLoads;
}

int32_t accept_chunks(graft_dtype dtype, int32_t rows, int32_t vocab) {
  const int len = chunk_of(dtype, loads_for(dtype, rows, vocab));
  return (vocab + len - 1) / len;
}
int32_t accept_chunks_max(int32_t vocab) {
  const int len = chunk_of(GRAFT_F32, kSmallLoads);  // the smallest chunk
  return (vocab + len - 1) / len;
}

void launch_accept(graft_dtype dtype, const AcceptParams &p, hipStream_t stream) {
  dim3 g1(p.chunks, p.batch * p.n_max);
  const bool bf = dtype == GRAFT_BF16;
  const bool vec = vec_ok(dtype, p.vocab);
  const bool large = loads_for(dtype, p.batch * p.n_max, p.vocab) == kLargeLoads;
  if (bf) {
    if (large) hipLaunchKernelGGL((argmax_chunks_kernel<true, true, kLargeLoads>), g1, dim3(kThreads), 0, stream, p);
    else if (vec) hipLaunchKernelGGL((argmax_chunks_kernel<true, true, kSmallLoads>), g1, dim3(kThreads), 0, stream, p);
    else hipLaunchKernelGGL((argmax_chunks_kernel<true, false, kSmallLoads>), g1, dim3(kThreads), 0, stream, p);
  } else {
    if (large) hipLaunchKernelGGL((argmax_chunks_kernel<false, true, kLargeLoads>), g1, dim3(kThreads), 0, stream, p);
    else if (vec) hipLaunchKernelGGL((argmax_chunks_kernel<false, true, kSmallLoads>), g1, dim3(kThreads), 0, stream, p);
    else hipLaunchKernelGGL((argmax_chunks_kernel<false, false, kSmallLoads>), g1, dim3(kThreads), 0, stream, p);
  }
  hipLaunchKernelGGL(accept_path_kernel, dim3(p.batch), dim3(kPathThreads), 0, stream, p);
}

}  // namespace graft
