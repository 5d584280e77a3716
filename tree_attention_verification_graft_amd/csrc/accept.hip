// Greedy (lossless) acceptance of the verified hybrid tree.
//
// Stage 1 streams the logits: every (node row, vocab chunk) pair is one
// workgroup that reduces its chunk to a packed 64-bit key whose high half is
// an order-preserving image of the value (-0 folded onto +0) and whose low
// half is the complemented index, so an unsigned max picks the largest value
// and, among equal values, the lowest index.  Stage 2 (one workgroup per
// sequence, one lane per node) finishes each row's argmax, marks the nodes
// whose token equals their parent's argmax with wave ballots, keeps the nodes
// whose whole ancestor mask is matched, and emits the deepest one's path.
//
// Method: "Draft Less, Retrieve More" (aitrends.kr summary), architecture
// paragraph (lossless verification with retrieval nodes as proposals), read
// for greedy decoding.
#include <hip/hip_bf16.h>

#include "graft_internal.h"

namespace graft {
namespace {

constexpr int kThreads = 256;
constexpr int kChunk = 16384;  // vocab entries per stage-1 workgroup

__device__ inline uint32_t ord_bf16(uint16_t u) {
  if (u == 0x8000u) u = 0;  // -0 == +0
  return (u & 0x8000u) ? (uint32_t)(~u & 0xffffu) : (uint32_t)(u | 0x8000u);
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
__device__ inline unsigned long long wave_max64(unsigned long long v) {
  for (int off = 32; off > 0; off >>= 1) {
    const unsigned long long o = __shfl_xor(v, off);
    v = umax64(v, o);
  }
  return v;
}

template <bool BF16, bool VEC>
__global__ __launch_bounds__(kThreads) void argmax_chunks_kernel(AcceptParams p) {
  const int c = blockIdx.x;
  const int row = blockIdx.y;  // b * n_max + i
  const int b = row / p.n_max;
  const int i = row % p.n_max;
  if (i >= p.n_nodes[b]) return;
  const int lo = c * p.chunk_len;
  const int hi = min(p.vocab, lo + p.chunk_len);
  unsigned long long best = 0ull;
  if (BF16) {
    const uint16_t *x = static_cast<const uint16_t *>(p.logits) + (size_t)row * p.vocab;
    if (VEC) {
      // 8 values per 16-byte load; lo and hi are multiples of 8 here
      for (int e = lo + 8 * threadIdx.x; e < hi; e += 8 * kThreads) {
        const uint4 v = *reinterpret_cast<const uint4 *>(x + e);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          best = umax64(best, pack(ord_bf16((uint16_t)(w[q] & 0xffffu)), e + 2 * q));
          best = umax64(best, pack(ord_bf16((uint16_t)(w[q] >> 16)), e + 2 * q + 1));
        }
      }
    } else {
      for (int e = lo + threadIdx.x; e < hi; e += kThreads)
        best = umax64(best, pack(ord_bf16(x[e]), e));
    }
  } else {
    const uint32_t *x = static_cast<const uint32_t *>(p.logits) + (size_t)row * p.vocab;
    if (VEC) {
      for (int e = lo + 4 * threadIdx.x; e < hi; e += 4 * kThreads) {
        const uint4 v = *reinterpret_cast<const uint4 *>(x + e);
        best = umax64(best, pack(ord_f32(v.x), e));
        best = umax64(best, pack(ord_f32(v.y), e + 1));
        best = umax64(best, pack(ord_f32(v.z), e + 2));
        best = umax64(best, pack(ord_f32(v.w), e + 3));
      }
    } else {
      for (int e = lo + threadIdx.x; e < hi; e += kThreads)
        best = umax64(best, pack(ord_f32(x[e]), e));
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

__global__ __launch_bounds__(GRAFT_MAX_NODES) void accept_path_kernel(AcceptParams p) {
  const int b = blockIdx.x;
  const int i = threadIdx.x;
  const int lane = i & 63;
  const int wave = i >> 6;
  const int n_nodes = p.n_nodes[b];
  const bool live = i < n_nodes && i < p.n_max;

  __shared__ int32_t s_am[GRAFT_MAX_NODES];
  __shared__ uint32_t s_match[GRAFT_MAX_NODES / 32];
  __shared__ uint32_t s_best[GRAFT_MAX_NODES / 64];
  __shared__ uint32_t s_bestkey;

  int am = -1;
  if (live) {
    unsigned long long m = 0ull;
    const unsigned long long *part = p.partial + ((size_t)b * p.n_max + i) * p.chunks;
    for (int c = 0; c < p.chunks; ++c) m = umax64(m, part[c]);
    am = (int)(~(uint32_t)(m & 0xffffffffull));
  }
  s_am[i] = am;
  if (i < p.n_max) p.argmax[(size_t)b * p.n_max + i] = am;
  __syncthreads();

  // match bit: the root always, else token == argmax of the parent's row
  const size_t o = (size_t)b * p.n_max + i;
  bool match = false;
  int par = -1;
  if (live) {
    par = p.tree_parent[o];
    match = (par < 0) || (par < i && p.tree_token[o] == s_am[par]);
  }
  const unsigned long long bal = __ballot(match);
  if (lane == 0) {
    s_match[2 * wave] = (uint32_t)(bal & 0xffffffffull);
    s_match[2 * wave + 1] = (uint32_t)(bal >> 32);
  }
  __syncthreads();

  // fully matched: every ancestor-or-self bit is matched
  uint32_t key = 0u;
  uint32_t mw[4] = {0u, 0u, 0u, 0u};
  if (live) {
    const uint32_t *mrow = p.tree_mask + o * p.words;
    mw[0] = p.words > 0 ? mrow[0] : 0u;
    mw[1] = p.words > 1 ? mrow[1] : 0u;
    mw[2] = p.words > 2 ? mrow[2] : 0u;
    mw[3] = p.words > 3 ? mrow[3] : 0u;
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
  if (lane == 0) s_best[wave] = wk;
  __syncthreads();
  if (i == 0) {
    uint32_t m = s_best[0];
    for (int w = 1; w < GRAFT_MAX_NODES / 64; ++w) m = s_best[w] > m ? s_best[w] : m;
    s_bestkey = m;
  }
  __syncthreads();
  const uint32_t bk = s_bestkey;
  // bk == 0 only when no node is live (n_nodes < 1 breaks the precondition):
  // fall back to the root so that every index below stays in bounds.
  const int best = bk ? 255 - (int)(bk & 0xffu) : 0;
  const int L = bk ? (int)(bk >> 8) - 1 : 0;  // accept length = depth of best

  // path = the best node's ancestor-or-self set in index order
  __shared__ uint32_t s_path[4];
  if (i == 0) {
    const uint32_t *mrow = p.tree_mask + ((size_t)b * p.n_max + best) * p.words;
    for (int w = 0; w < 4; ++w) s_path[w] = w < p.words ? mrow[w] : 0u;
  }
  __syncthreads();
  int32_t *pn = p.path_nodes + (size_t)b * p.n_max;
  int32_t *pt = p.path_tokens + (size_t)b * (p.n_max + 1);
  if (live && ((s_path[i >> 5] >> (i & 31)) & 1u)) {
    int pos = 0;
    for (int w = 0; w < (i >> 5); ++w) pos += __popc(s_path[w]);
    pos += __popc(s_path[i >> 5] & ((1u << (i & 31)) - 1u));
    if (pos < p.n_max) {
      pn[pos] = i;
      pt[pos] = p.tree_token[o];
    }
  }
  for (int k = i; k < p.n_max + 1; k += blockDim.x) {
    if (k < p.n_max && k > L) pn[k] = -1;
    if (k > L + 1) pt[k] = -1;
  }
  if (i == 0) {
    pt[L + 1] = s_am[best];
    p.accept_len[b] = L;
  }
}

}  // namespace

int32_t accept_chunks(int32_t vocab) { return (vocab + kChunk - 1) / kChunk; }

void launch_accept(graft_dtype dtype, const AcceptParams &p, hipStream_t stream) {
  dim3 g1(p.chunks, p.batch * p.n_max);
  const bool bf = dtype == GRAFT_BF16;
  const bool vec = bf ? (p.vocab % 8 == 0) : (p.vocab % 4 == 0);
  if (bf) {
    if (vec) hipLaunchKernelGGL((argmax_chunks_kernel<true, true>), g1, dim3(kThreads), 0, stream, p);
    else hipLaunchKernelGGL((argmax_chunks_kernel<true, false>), g1, dim3(kThreads), 0, stream, p);
  } else {
    if (vec) hipLaunchKernelGGL((argmax_chunks_kernel<false, true>), g1, dim3(kThreads), 0, stream, p);
    else hipLaunchKernelGGL((argmax_chunks_kernel<false, false>), g1, dim3(kThreads), 0, stream, p);
  }
  hipLaunchKernelGGL(accept_path_kernel, dim3(p.batch), dim3(GRAFT_MAX_NODES), 0, stream, p);
}

}  // namespace graft
