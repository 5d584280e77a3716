// Commit of the accepted path to the paged KV cache.
//
// After verification, decoding continues from the accepted tokens: the root
// and the accepted nodes path_nodes[b][0 .. accept_len[b]] (their K/V were
// computed in the verification pass at positions prefix_len + depth) become
// cache tokens prefix_len[b] + j.  One workgroup per (sequence, KV head)
// copies those rows: K into token-major pages (each row contiguous), V into
// dim-major pages (one element per dim row of the page).
//
// With a rotary table the tree keys arrive unrotated, and the key committed
// to cache token t is rotated at position t (rotate-half pairing of dim i
// with dim i + D/2, in fp32, rounded once to the cache type).
//
// Method: "Draft Less, Retrieve More" (aitrends.kr summary), architecture
// paragraph (one target forward verifies the hybrid tree; decoding continues
// from the accepted tokens).
#include "graft_internal.h"

namespace graft {
namespace {

constexpr int kThreads = 256;

__device__ inline float to_f32(uint16_t x) { return __uint_as_float((uint32_t)x << 16); }
__device__ inline float to_f32(uint32_t x) { return __uint_as_float(x); }
__device__ inline void from_f32(float f, uint16_t &out) {
  // round to nearest even (finite inputs)
  const uint32_t u = __float_as_uint(f);
  out = (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}
__device__ inline void from_f32(float f, uint32_t &out) { out = __float_as_uint(f); }

template <typename T, bool ROPE>
__global__ __launch_bounds__(kThreads) void append_kv_kernel(AppendParams p) {
  const int b = blockIdx.x / p.hkv;
  const int h = blockIdx.x % p.hkv;
  const int P = p.prefix_len[b];
  const int L = min(p.accept_len[b], p.n_max - 1);
  if (h == 0 && threadIdx.x == 0) p.new_prefix_len[b] = L < 0 ? P : P + L + 1;
  if (L < 0 || P < 0) return;
  const T *k_tree = static_cast<const T *>(p.k_tree);
  const T *v_tree = static_cast<const T *>(p.v_tree);
  T *k_cache = static_cast<T *>(p.k_cache);
  T *v_cache = static_cast<T *>(p.v_cache);
  const long cap = (long)p.max_blocks * p.block_size;
  const int D = p.head_dim;
  for (int e = threadIdx.x; e < (L + 1) * D; e += kThreads) {
    const int j = e / D, d = e % D;
    const long t = (long)P + j;
    const int node = p.path_nodes[(size_t)b * p.n_max + j];
    if (t >= cap || node < 0 || node >= p.n_max) continue;
    const int page = p.block_table[(size_t)b * p.max_blocks + t / p.block_size];
    if (page < 0 || page >= p.num_blocks) continue;  // never write outside the cache
    const int slot = (int)(t % p.block_size);
    const size_t src = (((size_t)b * p.n_max + node) * p.hkv + h) * D + d;
    const size_t ph = (size_t)page * p.hkv + h;
    if (ROPE) {
      // pair (i, i + D/2) at cache position t
      const int half = D / 2;
      const int i = d < half ? d : d - half;
      const float *row = p.rope + (size_t)min((long)p.rope_positions - 1, t) * D;
      const float c = row[i], sn = row[half + i];
      const float x = to_f32(k_tree[src]);
      const float y = to_f32(k_tree[src - d + (d < half ? d + half : d - half)]);
      T out;
      from_f32(d < half ? x * c - y * sn : x * c + y * sn, out);
      k_cache[(ph * p.block_size + slot) * D + d] = out;
    } else {
      k_cache[(ph * p.block_size + slot) * D + d] = k_tree[src];
    }
    v_cache[(ph * D + d) * p.block_size + slot] = v_tree[src];
  }
}

}  // namespace

void launch_append_kv(graft_dtype dtype, const AppendParams &p, hipStream_t stream) {
  const dim3 grid((unsigned)(p.batch * p.hkv));
  if (dtype == GRAFT_BF16) {
    if (p.rope) hipLaunchKernelGGL((append_kv_kernel<uint16_t, true>), grid, dim3(kThreads), 0, stream, p);
    else hipLaunchKernelGGL((append_kv_kernel<uint16_t, false>), grid, dim3(kThreads), 0, stream, p);
  } else {
    if (p.rope) hipLaunchKernelGGL((append_kv_kernel<uint32_t, true>), grid, dim3(kThreads), 0, stream, p);
    else hipLaunchKernelGGL((append_kv_kernel<uint32_t, false>), grid, dim3(kThreads), 0, stream, p);
  }
}

}  // namespace graft
