// Tree-masked verification attention over a paged KV cache.
//
// Every tree node attends to the whole cached prefix of its sequence and to
// its own ancestors-or-self in the hybrid tree, in one pass (the
// tree-attention path of the architecture paragraph of the "Draft Less,
// Retrieve More" summary).
//
// Matrix-core path (bf16, head_dim 128): one workgroup of 4 waves owns a
// (sequence, KV head, row group, prefix split).  The query rows of a KV head
// are its tree nodes times the query heads of the group.  K and V tiles of 64
// keys are staged from the paged cache into LDS once and shared by all waves;
// each wave owns up to NB blocks of 16 query rows.  Scores are computed
// transposed, S^T = K Q^T, with v_mfma_f32_16x16x32_bf16: each lane then holds
// one query column and 16 keys of the tile, so the softmax reductions are
// in-lane plus two cross-lane steps, and the score accumulators convert
// directly into the P^T operand of O^T = V^T P^T without any shuffle (keys are
// placed in LDS in the order that makes this so).  V pages are dim-major in
// the cache, so V^T tiles are contiguous copies.  Prefix splits write fp32
// partial (O, max, sum) and a combine kernel merges them; a single split
// writes the output directly.
//
// Wavefront path (fp32, or fewer than 16 query rows): one wave per query
// row, keys spread over lanes for q.k, head dims over lanes for P V.
#include <hip/hip_bf16.h>

#include "graft_internal.h"

namespace graft {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kD = 128;           // head dim of the matrix-core path
constexpr int kTile = 64;         // keys per LDS tile
constexpr int kBlock = 16;        // tokens per KV page
constexpr int kKStride = kD + 8;  // LDS row stride of the K tile (elements)
constexpr int kVStride = kTile + 8;  // LDS row stride of the V^T tile (elements)
constexpr float kNegBig = -1.0e30f;  // running-max start: finite, below any score
constexpr int kThreads = 256;      // wavefront path
constexpr int kMfmaWaves = 8;      // matrix-core path: 2 waves per SIMD
constexpr int kMfmaThreads = 64 * kMfmaWaves;
constexpr int kMaxNB = 3;          // 16-row blocks per wave

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// LDS row of the K tile that holds key `k` (0..63) of the tile.  Rows are in
// the order the transposed score blocks use: score block kb = 2*kp + half,
// row 4*g + i holds key 32*kp + 8*g + 4*half + i.
__device__ inline int k_row_of_key(int k) {
  const int kp = k >> 5, w = k & 31, g = w >> 3, half = (w >> 2) & 1, i = w & 3;
  return 16 * (2 * kp + half) + 4 * g + i;
}

__device__ inline uint4 zero4() { return make_uint4(0u, 0u, 0u, 0u); }

// Word `idx` (0..3) of a 4-word ancestor mask held in registers, by select so
// that the array is never indexed dynamically.
__device__ inline uint32_t mask_word(const uint32_t (&mw)[4], int idx) {
  return idx == 0 ? mw[0] : idx == 1 ? mw[1] : idx == 2 ? mw[2] : mw[3];
}

// Load up to 4 mask words into registers without dynamic indexing.
__device__ inline void load_mask4(uint32_t (&mw)[4], const uint32_t *src, int words) {
  mw[0] = words > 0 ? src[0] : 0u;
  mw[1] = words > 1 ? src[1] : 0u;
  mw[2] = words > 2 ? src[2] : 0u;
  mw[3] = words > 3 ? src[3] : 0u;
}

// Zero the bf16 lanes of a 16-byte chunk whose key index is >= limit; the
// chunk covers keys first .. first+7.
__device__ inline uint4 mask_v_chunk(uint4 v, int first, int limit) {
  uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int k0 = first + 2 * e;
    if (k0 >= limit) w[e] &= 0x00000000u;
    else if (k0 + 1 >= limit) w[e] &= 0x0000ffffu;
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

template <int NB>
__global__ __launch_bounds__(kMfmaThreads) void attn_mfma_kernel(AttnParams p) {
  __shared__ __attribute__((aligned(16))) __bf16 sK[kTile * kKStride];
  __shared__ __attribute__((aligned(16))) __bf16 sV[kD * kVStride];

  const int split = blockIdx.x;
  const int rg = blockIdx.y % p.n_row_groups;
  const int h = blockIdx.y / p.n_row_groups;
  const int b = blockIdx.z;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int n16 = lane & 15;
  const int g4 = lane >> 4;

  // Clamp caller-supplied counts to the buffer bounds (documented
  // preconditions; the clamp only keeps reads in bounds if they are broken).
  const int n_nodes = min(max(p.n_nodes[b], 0), p.n_max);
  const int P = min(max(p.prefix_len[b], 0), p.max_blocks * kBlock);
  const int G = p.group;
  const int rows_b = n_nodes * G;
  const int row0 = rg * p.rows_per_group;
  if (row0 >= rows_b) return;  // group past this sequence's rows

  const int nt_prefix = (P + kTile - 1) / kTile;
  const int t_begin = split * p.tiles_per_split;
  const int t_end = min(t_begin + p.tiles_per_split, nt_prefix);
  const int n_pref = max(0, t_end - t_begin);
  const int n_tree = split == 0 ? (n_nodes + kTile - 1) / kTile : 0;
  if (n_pref == 0 && n_tree == 0) return;  // empty split

  const __bf16 *q = static_cast<const __bf16 *>(p.q);
  const __bf16 *k_cache = static_cast<const __bf16 *>(p.k_cache);
  const __bf16 *v_cache = static_cast<const __bf16 *>(p.v_cache);
  const int32_t *table = p.block_table + (size_t)b * p.max_blocks;

  // ---- per-wave query blocks: block k of this wave covers rows
  // row0 + 16*(wave + 8k) .. +15 of the (node, query head) row space.
  bf16x8 qf[NB][4];
  f32x4 o[NB][8];
  float m_run[NB], l_run[NB];
  int my_row[NB];
  bool blk_on[NB];
#pragma unroll
  for (int k = 0; k < NB; ++k) {
    const int rl = 16 * (wave + kMfmaWaves * k);
    blk_on[k] = rl < p.rows_per_group && row0 + rl < rows_b;
    const int r = row0 + rl + n16;
    my_row[k] = r;
    const bool rv = blk_on[k] && r < rows_b && rl + n16 < p.rows_per_group;
    const int node = rv ? r / G : 0;
    const int hq = h * G + (rv ? r % G : 0);
    const __bf16 *qrow = q + (((size_t)b * p.n_max + node) * p.hq + hq) * kD;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      uint4 v = rv ? *reinterpret_cast<const uint4 *>(qrow + 32 * kk + 8 * g4) : zero4();
      qf[k][kk] = *reinterpret_cast<bf16x8 *>(&v);
    }
#pragma unroll
    for (int d = 0; d < 8; ++d) o[k][d] = f32x4{0.f, 0.f, 0.f, 0.f};
    m_run[k] = kNegBig;
    l_run[k] = 0.f;
  }

  // ---- tile loaders (global -> registers -> LDS)
  uint4 kreg[2], vreg[2];
  auto load_prefix = [&](int tile) {
    const int key0 = tile * kTile;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int c = tid + kMfmaThreads * r;
      const int kl = c >> 4, dc = c & 15;
      const int key = key0 + kl;
      if (key < P) {
        const int blk = table[key >> 4];
        kreg[r] = *reinterpret_cast<const uint4 *>(
            k_cache + (((size_t)blk * p.hkv + h) * kBlock + (key & 15)) * kD + dc * 8);
      } else {
        kreg[r] = zero4();
      }
      const int pg = c >> 8, w = c & 255, d = w >> 1, half = w & 1;
      const int first = key0 + 16 * pg + 8 * half;
      if (key0 + 16 * pg < P) {
        const int blk = table[(key0 >> 4) + pg];
        uint4 v = *reinterpret_cast<const uint4 *>(
            v_cache + (((size_t)blk * p.hkv + h) * kD + d) * kBlock + 8 * half);
        vreg[r] = (first + 8 <= P) ? v : mask_v_chunk(v, first, P);
      } else {
        vreg[r] = zero4();
      }
    }
  };
  auto store_prefix = [&]() {
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int c = tid + kMfmaThreads * r;
      const int kl = c >> 4, dc = c & 15;
      *reinterpret_cast<uint4 *>(&sK[k_row_of_key(kl) * kKStride + dc * 8]) = kreg[r];
      const int pg = c >> 8, w = c & 255, d = w >> 1, half = w & 1;
      *reinterpret_cast<uint4 *>(&sV[d * kVStride + 16 * pg + 8 * half]) = vreg[r];
    }
  };

  // ---- one tile: two halves of 32 keys, each scores -> softmax -> P V.
  // Half kp covers score blocks 2kp (keys 32kp + 8g + i) and 2kp+1
  // (keys 32kp + 8g + 4 + i) of lane group g, which are exactly the eight
  // key slots lane group g feeds to the P V matrix op.
  auto compute = [&](int key0, bool tree) {
    const int limit = tree ? n_nodes : P;
    uint32_t mw[NB][4];
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      mw[k][0] = mw[k][1] = mw[k][2] = mw[k][3] = 0u;
      if (tree && blk_on[k]) {
        const int r = my_row[k];
        const int node = r < rows_b ? r / G : 0;
        load_mask4(mw[k], p.tree_mask + ((size_t)b * p.n_max + node) * p.words, p.words);
      }
    }
#pragma unroll
    for (int kp = 0; kp < 2; ++kp) {
      f32x4 s[NB][2];
#pragma unroll
      for (int k = 0; k < NB; ++k) s[k][0] = s[k][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const bf16x8 a = *reinterpret_cast<const bf16x8 *>(
              &sK[(16 * (2 * kp + hh) + n16) * kKStride + 32 * kk + 8 * g4]);
#pragma unroll
          for (int k = 0; k < NB; ++k)
            if (blk_on[k])
              s[k][hh] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[k][kk], s[k][hh], 0, 0, 0);
        }
      }
      bf16x8 pb[NB];
#pragma unroll
      for (int k = 0; k < NB; ++k) {
        if (!blk_on[k]) continue;
        float mx = kNegBig;
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int key = key0 + 32 * kp + 8 * g4 + 4 * hh + i;
            bool vis = key < limit;
            if (tree) vis = vis && ((mask_word(mw[k], key >> 5) >> (key & 31)) & 1u);
            const float x = vis ? s[k][hh][i] * p.scale_log2 : -INFINITY;
            s[k][hh][i] = x;
            mx = fmaxf(mx, x);
          }
        }
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m_run[k], mx);
        const float alpha = fast_exp2(m_run[k] - m_new);
        m_run[k] = m_new;
        float rs = 0.f;
        bf16x8 v;
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float e = fast_exp2(s[k][hh][i] - m_new);
            rs += e;
            v[4 * hh + i] = (__bf16)e;
          }
        pb[k] = v;
        l_run[k] = l_run[k] * alpha + rs;
        // rescale the accumulator only when some query's maximum moved
        if (__ballot(alpha < 1.f)) {
#pragma unroll
          for (int d = 0; d < 8; ++d) o[k][d] *= alpha;
        }
      }
#pragma unroll
      for (int d = 0; d < 8; ++d) {
        const bf16x8 a = *reinterpret_cast<const bf16x8 *>(
            &sV[(16 * d + n16) * kVStride + 32 * kp + 8 * g4]);
#pragma unroll
        for (int k = 0; k < NB; ++k)
          if (blk_on[k])
            o[k][d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pb[k], o[k][d], 0, 0, 0);
      }
    }
  };

  // ---- prefix tiles, software-pipelined: the next tile's global loads are
  // in flight while the current tile is computed.
  if (n_pref > 0) load_prefix(t_begin);
  for (int it = 0; it < n_pref; ++it) {
    __syncthreads();
    store_prefix();
    __syncthreads();
    if (it + 1 < n_pref) load_prefix(t_begin + it + 1);
    compute((t_begin + it) * kTile, false);
  }

  // ---- tree tiles (split 0 only): keys are the tree nodes themselves.
  const __bf16 *k_tree = static_cast<const __bf16 *>(p.k_tree);
  const __bf16 *v_tree = static_cast<const __bf16 *>(p.v_tree);
  for (int tt = 0; tt < n_tree; ++tt) {
    const int key0 = tt * kTile;
    __syncthreads();
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int c = tid + kMfmaThreads * r;
      const int kl = c >> 4, dc = c & 15;
      const int j = key0 + kl;
      uint4 kv = zero4(), vv = zero4();
      if (j < n_nodes) {
        const size_t base = (((size_t)b * p.n_max + j) * p.hkv + h) * kD + dc * 8;
        kv = *reinterpret_cast<const uint4 *>(k_tree + base);
        vv = *reinterpret_cast<const uint4 *>(v_tree + base);
      }
      *reinterpret_cast<uint4 *>(&sK[k_row_of_key(kl) * kKStride + dc * 8]) = kv;
      const __bf16 *ve = reinterpret_cast<const __bf16 *>(&vv);
#pragma unroll
      for (int e = 0; e < 8; ++e) sV[(dc * 8 + e) * kVStride + kl] = ve[e];
    }
    __syncthreads();
    compute(key0, true);
  }

  // ---- epilogue: finish the row sums across the four lane groups and
  // write either the output or this split's partials.
#pragma unroll
  for (int k = 0; k < NB; ++k) {
    if (!blk_on[k]) continue;
    float l = l_run[k];
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    const int r = my_row[k];
    const int rl = r - row0;
    if (r >= rows_b || rl >= p.rows_per_group) continue;
    if (p.n_splits == 1) {
      const float inv = 1.f / l;
      const int node = r / G;
      const int hq = h * G + r % G;
      __hip_bfloat16 *out = static_cast<__hip_bfloat16 *>(p.out) +
                            (((size_t)b * p.n_max + node) * p.hq + hq) * kD;
#pragma unroll
      for (int d = 0; d < 8; ++d) {
        ushort4 w;
        w.x = __bfloat16_as_ushort(__float2bfloat16(o[k][d][0] * inv));
        w.y = __bfloat16_as_ushort(__float2bfloat16(o[k][d][1] * inv));
        w.z = __bfloat16_as_ushort(__float2bfloat16(o[k][d][2] * inv));
        w.w = __bfloat16_as_ushort(__float2bfloat16(o[k][d][3] * inv));
        *reinterpret_cast<ushort4 *>(out + 16 * d + 4 * g4) = w;
      }
    } else {
      const size_t prow =
          ((((size_t)b * p.hkv + h) * p.n_row_groups + rg) * p.n_splits + split) *
              p.rows_per_group + rl;
      float *po = p.part_o + prow * kD;
#pragma unroll
      for (int d = 0; d < 8; ++d)
        *reinterpret_cast<f32x4 *>(po + 16 * d + 4 * g4) = o[k][d];
      if (g4 == 0) {
        p.part_ml[prow * 2 + 0] = m_run[k];
        p.part_ml[prow * 2 + 1] = l;
      }
    }
  }
}

// ------------------------------------------------------------------------
// Wavefront path: one wave per query row (sequence, node, query head).
// Each lane scores one key of a 64-key chunk (a full dot product over the
// head dim), then the lanes own head dims for the P V accumulation.  Dim-major
// V pages make the per-dim key runs contiguous.
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void attn_wave_kernel(AttnParams p) {
  constexpr int DPL = D / 64;  // head dims per lane
  __shared__ float s_q[4][D];
  __shared__ float s_p[4][64];

  const int split = blockIdx.x;
  const int rows_pad = p.rows_per_group;  // one group in this path
  const int chunks = rows_pad / 4;
  const int h = blockIdx.y / chunks;
  const int rc = blockIdx.y % chunks;
  const int b = blockIdx.z;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int G = p.group;
  const int n_nodes = min(max(p.n_nodes[b], 0), p.n_max);
  const int P = min(max(p.prefix_len[b], 0), p.max_blocks * kBlock);
  const int r = rc * 4 + wave;
  const bool row_ok = r < n_nodes * G;
  const int node = row_ok ? r / G : 0;
  const int hq = h * G + (row_ok ? r % G : 0);

  const int nt_prefix = (P + 63) / 64;
  const int t_begin = split * p.tiles_per_split;
  const int t_end = min(t_begin + p.tiles_per_split, nt_prefix);
  const int n_tree = split == 0 ? (n_nodes + 63) / 64 : 0;
  if (t_end <= t_begin && n_tree == 0) return;  // empty split (uniform)

  const T *q = static_cast<const T *>(p.q);
  const T *k_cache = static_cast<const T *>(p.k_cache);
  const T *v_cache = static_cast<const T *>(p.v_cache);
  const T *k_tree = static_cast<const T *>(p.k_tree);
  const T *v_tree = static_cast<const T *>(p.v_tree);
  const int32_t *table = p.block_table + (size_t)b * p.max_blocks;

  const T *qrow = q + (((size_t)b * p.n_max + node) * p.hq + hq) * D;
  for (int d = lane; d < D; d += 64) s_q[wave][d] = row_ok ? (float)qrow[d] : 0.f;
  uint32_t mw[GRAFT_MAX_NODES / 32] = {0u, 0u, 0u, 0u};
  if (row_ok) load_mask4(mw, p.tree_mask + ((size_t)b * p.n_max + node) * p.words, p.words);
  __syncthreads();

  float m_run = kNegBig, l_run = 0.f;
  float acc[DPL];
#pragma unroll
  for (int e = 0; e < DPL; ++e) acc[e] = 0.f;

  auto chunk = [&](int key0, bool tree) {
    // score of key key0 + lane
    const int key = key0 + lane;
    bool vis;
    const T *krow;
    if (tree) {
      vis = key < n_nodes && ((mask_word(mw, key >> 5) >> (key & 31)) & 1u);
      krow = k_tree + (((size_t)b * p.n_max + (vis ? key : 0)) * p.hkv + h) * D;
    } else {
      vis = key < P;
      const int blk = vis ? table[key >> 4] : 0;
      krow = k_cache + (((size_t)blk * p.hkv + h) * kBlock + (key & 15)) * D;
    }
    float sc = -INFINITY;
    if (vis && row_ok) {
      float dot = 0.f;
      for (int d = 0; d < D; ++d) dot += s_q[wave][d] * (float)krow[d];
      sc = dot * p.scale_log2;
    }
    float mx = sc;
    for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
    const float m_new = fmaxf(m_run, mx);
    const float alpha = fast_exp2(m_run - m_new);
    const float e = fast_exp2(sc - m_new);
    float rs = e;
    for (int off = 32; off > 0; off >>= 1) rs += __shfl_xor(rs, off);
    l_run = l_run * alpha + rs;
    m_run = m_new;
    s_p[wave][lane] = e;
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int ei = 0; ei < DPL; ++ei) {
      const int d = lane + 64 * ei;
      float a = acc[ei] * alpha;
      const int nk = min(64, (tree ? n_nodes : P) - key0);
      for (int kk = 0; kk < nk; ++kk) {
        const float pk = s_p[wave][kk];
        if (pk == 0.f) continue;
        const int kkey = key0 + kk;
        float v;
        if (tree) {
          v = (float)v_tree[(((size_t)b * p.n_max + kkey) * p.hkv + h) * D + d];
        } else {
          const int blk = table[kkey >> 4];
          v = (float)v_cache[(((size_t)blk * p.hkv + h) * D + d) * kBlock + (kkey & 15)];
        }
        a += pk * v;
      }
      acc[ei] = a;
    }
    __builtin_amdgcn_wave_barrier();
  };

  for (int t = t_begin; t < t_end; ++t) chunk(t * 64, false);
  for (int t = 0; t < n_tree; ++t) chunk(t * 64, true);

  if (!row_ok) return;
  if (p.n_splits == 1) {
    const float inv = 1.f / l_run;
    T *out = static_cast<T *>(p.out) + (((size_t)b * p.n_max + node) * p.hq + hq) * D;
#pragma unroll
    for (int ei = 0; ei < DPL; ++ei) out[lane + 64 * ei] = (T)(acc[ei] * inv);
  } else {
    const size_t prow = (((size_t)b * p.hkv + h) * p.n_splits + split) * p.rows_per_group + r;
    float *po = p.part_o + prow * D;
#pragma unroll
    for (int ei = 0; ei < DPL; ++ei) po[lane + 64 * ei] = acc[ei];
    if (lane == 0) {
      p.part_ml[prow * 2 + 0] = m_run;
      p.part_ml[prow * 2 + 1] = l_run;
    }
  }
}

// ------------------------------------------------------------------------
// Combine: merge the prefix splits of one output row (log-sum-exp in base 2).
template <typename T>
__global__ __launch_bounds__(128) void attn_combine_kernel(AttnParams p) {
  const int hq = blockIdx.x;
  const int node = blockIdx.y;
  const int b = blockIdx.z;
  if (node >= min(p.n_nodes[b], p.n_max)) return;
  const int G = p.group;
  const int h = hq / G;
  const int r = node * G + hq % G;
  const int rg = r / p.rows_per_group;
  const int rl = r % p.rows_per_group;
  const int P = min(max(p.prefix_len[b], 0), p.max_blocks * kBlock);
  const int nt_prefix = (P + kTile - 1) / kTile;
  const int active =
      min(p.n_splits, max(1, (nt_prefix + p.tiles_per_split - 1) / p.tiles_per_split));
  const size_t base = (((size_t)b * p.hkv + h) * p.n_row_groups + rg) * p.n_splits;

  float M = kNegBig;
  for (int s = 0; s < active; ++s)
    M = fmaxf(M, p.part_ml[((base + s) * p.rows_per_group + rl) * 2]);
  float L = 0.f;
  for (int s = 0; s < active; ++s) {
    const size_t pr = (base + s) * p.rows_per_group + rl;
    L += p.part_ml[pr * 2 + 1] * fast_exp2(p.part_ml[pr * 2] - M);
  }
  const float inv = 1.f / L;
  T *out = static_cast<T *>(p.out) + (((size_t)b * p.n_max + node) * p.hq + hq) * p.head_dim;
  for (int d = threadIdx.x; d < p.head_dim; d += blockDim.x) {
    float acc = 0.f;
    for (int s = 0; s < active; ++s) {
      const size_t pr = (base + s) * p.rows_per_group + rl;
      acc += p.part_o[pr * p.head_dim + d] * fast_exp2(p.part_ml[pr * 2] - M);
    }
    out[d] = (T)(acc * inv);
  }
}

}  // namespace

// ------------------------------------------------------------------------
// Launch planning.  Query rows per KV head are n_max * group; the matrix-core
// path tiles them in blocks of 16, at most kMaxNB blocks per wave and
// kMfmaWaves waves (384 rows per workgroup).  Prefix splits are sized so the grid holds about two
// workgroups per compute unit.
AttnPlan plan_attention(graft_dtype dtype, int32_t batch, int32_t n_max, int32_t hq,
                        int32_t hkv, int32_t head_dim, int32_t max_prefix) {
  AttnPlan pl{};
  const int group = hq / hkv;
  const int rows = n_max * group;
  pl.mfma = dtype == GRAFT_BF16 && head_dim == kD && rows >= 16;
  const int tiles = max(1, (max_prefix + kTile - 1) / kTile);
  int per_seq_groups;
  if (pl.mfma) {
    const int blocks = (rows + 15) / 16;
    const int per_group = kMfmaWaves * kMaxNB;
    const int groups = (blocks + per_group - 1) / per_group;
    const int blocks_per_group = (blocks + groups - 1) / groups;
    pl.n_row_groups = groups;
    pl.rows_per_group = 16 * blocks_per_group;
    per_seq_groups = groups;
  } else {
    pl.n_row_groups = 1;
    pl.rows_per_group = (rows + 3) / 4 * 4;
    per_seq_groups = pl.rows_per_group / 4;
  }
  const long target = 512;  // workgroups to aim for (256 CUs x 2)
  const long base = (long)batch * hkv * per_seq_groups;
  int splits = (int)max(1L, min((long)tiles, (target + base - 1) / max(1L, base)));
  // keep splits at least 4 tiles long so partial traffic stays small
  splits = min(splits, max(1, tiles / 4));
  pl.tiles_per_split = (tiles + splits - 1) / splits;
  pl.n_splits = (tiles + pl.tiles_per_split - 1) / pl.tiles_per_split;
  const size_t prows = (size_t)batch * hkv * pl.n_row_groups * pl.n_splits * pl.rows_per_group;
  pl.part_o_bytes = pl.n_splits > 1 ? prows * head_dim * sizeof(float) : 0;
  pl.part_ml_bytes = pl.n_splits > 1 ? prows * 2 * sizeof(float) : 0;
  return pl;
}

void launch_attention_bf16_mfma(const AttnParams &p, hipStream_t stream) {
  dim3 grid(p.n_splits, p.hkv * p.n_row_groups, p.batch);
  const int nb = (p.rows_per_group / 16 + kMfmaWaves - 1) / kMfmaWaves;
  switch (nb) {
    case 1: hipLaunchKernelGGL(attn_mfma_kernel<1>, grid, dim3(kMfmaThreads), 0, stream, p); break;
    case 2: hipLaunchKernelGGL(attn_mfma_kernel<2>, grid, dim3(kMfmaThreads), 0, stream, p); break;
    default: hipLaunchKernelGGL(attn_mfma_kernel<3>, grid, dim3(kMfmaThreads), 0, stream, p); break;
  }
}

void launch_attention_wave(graft_dtype dtype, const AttnParams &p, hipStream_t stream) {
  dim3 grid(p.n_splits, p.hkv * (p.rows_per_group / 4), p.batch);
  if (dtype == GRAFT_F32) {
    if (p.head_dim == 64)
      hipLaunchKernelGGL((attn_wave_kernel<float, 64>), grid, dim3(kThreads), 0, stream, p);
    else
      hipLaunchKernelGGL((attn_wave_kernel<float, 128>), grid, dim3(kThreads), 0, stream, p);
  } else {
    if (p.head_dim == 64)
      hipLaunchKernelGGL((attn_wave_kernel<__hip_bfloat16, 64>), grid, dim3(kThreads), 0, stream, p);
    else
      hipLaunchKernelGGL((attn_wave_kernel<__hip_bfloat16, 128>), grid, dim3(kThreads), 0, stream, p);
  }
}

void launch_attention_combine(graft_dtype dtype, const AttnParams &p, hipStream_t stream) {
  dim3 grid(p.hq, p.n_max, p.batch);
  if (dtype == GRAFT_F32)
    hipLaunchKernelGGL(attn_combine_kernel<float>, grid, dim3(128), 0, stream, p);
  else
    hipLaunchKernelGGL(attn_combine_kernel<__hip_bfloat16>, grid, dim3(128), 0, stream, p);
}

}  // namespace graft
