// Tree-masked verification attention over a paged KV cache.
//
// Every tree node attends to the whole cached prefix of its sequence and to
// its own ancestors-or-self in the hybrid tree, in one pass (the
// tree-attention path of the architecture paragraph of the "Draft Less,
// Retrieve More" summary).
//
// Matrix-core path (bf16, head_dim 128): one workgroup of 8 waves (two per
// SIMD) owns a (sequence, KV head, row group, prefix split).  The query rows of a KV head
// are its tree nodes times the query heads of the group.  K and V tiles of 64
// keys are staged from the paged cache into LDS once and shared by all waves;
// each wave owns up to NB blocks of 16 query rows (with at most 4 blocks per
// group, waves w and w + 4 share blocks and split each tile's keys).  Scores are computed
// transposed, S^T = K Q^T, with v_mfma_f32_16x16x32_bf16: each lane then holds
// one query column and 16 keys of the tile, so the softmax reductions are
// in-lane plus two cross-lane steps, and the score accumulators convert
// directly into the P^T operand of O^T = V^T P^T without any shuffle (keys are
// placed in LDS in the order that makes this so).  V pages are dim-major in
// the cache, so V^T tiles are contiguous copies.  Prefix splits write fp32
// partial (O, max, sum) and a combine kernel merges them; a sequence with a
// single active split writes its output directly.
//
// Wavefront path (fp32, or fewer than 16 query rows): one wave per query
// row, keys spread over lanes for q.k, head dims over lanes for P V.
//
// Both paths optionally rotate the queries and the tree keys by their tree
// positions on load (rotary embedding, rotate-half pairing of dim i with
// dim i + D/2, cosines and sines from a caller table), so that unrotated
// projections need no separate pass; the cached prefix keys were rotated
// when they were written.
#include <hip/hip_bf16.h>

#include <algorithm>

#include "graft_internal.h"

namespace graft {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kD = 128;           // head dim of the matrix-core path
constexpr int kTile = 64;         // keys per LDS tile
constexpr int kBlock = 16;        // tokens per KV page
constexpr float kNegBig = -1.0e30f;  // running-max start: finite, below any score
constexpr int kThreads = 256;      // wavefront path
constexpr int kMfmaWaves = 8;      // matrix-core path: 2 waves per SIMD
constexpr int kMfmaThreads = 64 * kMfmaWaves;
constexpr int kMaxNB = 3;          // 16-row blocks per wave

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Cosines and sines of dims i0 .. i0 + 7 at table row `pos` (a row holds
// D/2 cosines, then D/2 sines).
struct Rot8 {
  float c[8], s[8];
};
__device__ inline Rot8 load_rot8(const float *rope, int D, int pos, int i0) {
  const float *row = rope + (size_t)pos * D;
  const float4 c0 = *reinterpret_cast<const float4 *>(row + i0);
  const float4 c1 = *reinterpret_cast<const float4 *>(row + i0 + 4);
  const float4 s0 = *reinterpret_cast<const float4 *>(row + D / 2 + i0);
  const float4 s1 = *reinterpret_cast<const float4 *>(row + D / 2 + i0 + 4);
  Rot8 r;
  r.c[0] = c0.x; r.c[1] = c0.y; r.c[2] = c0.z; r.c[3] = c0.w;
  r.c[4] = c1.x; r.c[5] = c1.y; r.c[6] = c1.z; r.c[7] = c1.w;
  r.s[0] = s0.x; r.s[1] = s0.y; r.s[2] = s0.z; r.s[3] = s0.w;
  r.s[4] = s1.x; r.s[5] = s1.y; r.s[6] = s1.z; r.s[7] = s1.w;
  return r;
}
// Table row of a tree position (clamped into the table: positions outside
// it are a caller error, and the clamp only keeps reads in bounds).
__device__ inline int rope_row(const AttnParams &p, int b, int node) {
  return min(max(p.tree_pos[(size_t)b * p.n_max + node], 0), p.rope_positions - 1);
}

// Maximum of two finite-or-(-inf) floats as one v_med3_f32 (median of a, b
// and +inf); unlike fmaxf it needs no NaN canonicalisation of its inputs.
// The +inf operand goes through an empty asm statement so that the compiler
// cannot turn the median back into maxnum.
__device__ inline float pos_inf() {
  float x = INFINITY;
  asm volatile("" : "+s"(x));
  return x;
}
__device__ inline float fmax2(float a, float b, float inf) {
  return __builtin_amdgcn_fmed3f(a, b, inf);
}
// Maximum of eight scores (finite or -inf): the IEEE maximum operation,
// which gfx950 evaluates three inputs at a time (v_maximum3_f32), four
// instructions where a chain of two-input maxima takes seven.
__device__ inline float max8(const f32x4 &a, const f32x4 &b, float) {
  float m = __builtin_elementwise_maximum(a[0], a[1]);
  m = __builtin_elementwise_maximum(m, a[2]);
  m = __builtin_elementwise_maximum(m, a[3]);
  m = __builtin_elementwise_maximum(m, b[0]);
  m = __builtin_elementwise_maximum(m, b[1]);
  m = __builtin_elementwise_maximum(m, b[2]);
  return __builtin_elementwise_maximum(m, b[3]);
}

// Reductions over the four 16-lane groups of a wave (lanes l, l^16, l^32,
// l^48) with the gfx950 row-swap permutes, which stay in the vector ALU.
__device__ inline float group4_max(float x, float inf) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  const float m1 = fmax2(__uint_as_float(a[0]), __uint_as_float(a[1]), inf);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(m1), __float_as_uint(m1), false,
                                                  false);
  return fmax2(__uint_as_float(b[0]), __uint_as_float(b[1]), inf);
}
__device__ inline float group4_sum(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  const float s1 = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(s1), __float_as_uint(s1), false,
                                                  false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// The running maximum used as the exponent offset is only moved when a new
// score exceeds it by more than 2^kRescaleLog2; until then probabilities up
// to 2^8 are accumulated as they are (exact softmax either way, since the
// accumulator and the row sum share the offset), which saves most rescales.
constexpr float kRescaleLog2 = 8.f;

// Prefix splits holding work for a sequence of nt_prefix prefix tiles (split
// 0 always, for its tree tiles).  A sequence with one has its output written
// by the attention kernel itself, and the combine skips its rows.
__device__ inline int active_splits(const AttnParams &p, int nt_prefix) {
  return min(p.n_splits,
             max(1, (nt_prefix + p.tree_shift + p.tiles_per_split - 1) / p.tiles_per_split));
}

// First query row of row group rg, and the row group holding query row r
// (matrix-core path: the first group_blocks_rem groups hold one 16-row block
// more than the others, so that no two groups differ by more than a block).
__device__ inline int group_row0(const AttnParams &p, int rg) {
  return 16 * (rg * p.group_blocks_lo + min(rg, p.group_blocks_rem));
}
__device__ inline int group_of_row(const AttnParams &p, int r) {
  if (p.n_row_groups == 1) return 0;
  const int blk = r >> 4, big = p.group_blocks_rem * (p.group_blocks_lo + 1);
  return blk < big ? blk / (p.group_blocks_lo + 1)
                   : p.group_blocks_rem + (blk - big) / p.group_blocks_lo;
}

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


// ---------------------------------------------------------------------------
// Matrix-core path.
//
// LDS holds kStages tile buffers (K 16 KB + V 16 KB each) filled by
// asynchronous global->LDS loads (global_load_lds_dwordx4: each lane's 16
// bytes land at M0 + 16 * lane), so up to kStages - 1 tiles are in flight
// while one is computed, without staging registers.  The loads are issued
// from inline assembly so that the compiler does not serialise every LDS
// read behind them; the kernel waits on vmcnt itself.  Every load
// instruction reads one KV page (base address in SGPRs, 32-bit lane
// offsets).  The K tile is unpadded and XOR-swizzled: row R (in the order
// the transposed score blocks use) holds its 16-byte chunk c at position
// c ^ (R & 15).  The V tile keeps the cache's dim-major pages as they are
// (page p at 4 KB * p, dim row d at 32 bytes * d) except that the two
// 8-key halves of a row swap places when bits 2 and 3 of d differ.  Both
// make the 16 lanes of a matrix-operand read hit 16 distinct 16-byte bank
// groups.  Each wave
// issues exactly kDmaPerStage loads per stage (a page past the prefix is
// redirected to the tile's first page and later masked), so vmcnt counts
// stay exact.  Without rotary embedding the tree tiles follow the prefix
// tiles through the same ring: K rows as for the prefix, V rows key-major,
// transposed in LDS when the tile comes up (node ids past the tree are
// clamped to the last node, whose keys get masked and values zeroed).
constexpr int kStages = 4;
constexpr int kKBytes = kTile * kD * 2;  // 16 KB
constexpr int kVBytes = kD * kTile * 2;  // 16 KB
constexpr int kStageBytes = kKBytes + kVBytes;
constexpr int kDmaPerStage = 4;          // per wave: four 1 KB blocks of one page (K or V)
// Behind the ring: a sequence's ancestor masks (n_max * words <= 128 * 4
// words), one 64-word block per wave.
constexpr int kMaskBytes = kMfmaWaves * 64 * 4;
static_assert(GRAFT_MAX_NODES * ((GRAFT_MAX_NODES + 31) / 32) <= kMfmaWaves * 64,
              "a sequence's ancestor masks fill at most one dword per lane");

// Issue one asynchronous 16-byte-per-lane global->LDS load from
// base + voffset (base wave-uniform, in SGPRs).  lds_base is the
// wave-uniform LDS byte address of the 1 KB destination block.  The
// non-temporal form is for tiles no other workgroup reads again.
// The LDS address goes in as an M0 operand, so the compiler writes M0 itself
// ahead of the instruction (it knows M0 is read here and clobbers nothing).
// The compiler's hazard checks do not look inside inline assembly, so the
// asm provides the wait states itself: the page base reaches its SGPR pair
// through v_readfirstlane, and a vector-ALU write of an SGPR needs five wait
// states before a vector-memory instruction reads it (an M0 write needs one
// before an LDS-DMA load).  Without them the load can use the pair's stale
// value as its address.
__device__ __forceinline__ void dma16(const void *base, uint32_t voffset, uint32_t lds_base) {
  asm volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voffset), "s"(base), "{m0}"(lds_base)
               : "memory");
}
__device__ __forceinline__ void dma16_nt(const void *base, uint32_t voffset, uint32_t lds_base) {
  asm volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %0, %1 nt"
               :
               : "v"(voffset), "s"(base), "{m0}"(lds_base)
               : "memory");
}
// The 4-byte form (lane bytes at M0 + 4 * lane), for the ancestor masks.
__device__ __forceinline__ void dma4(const void *base, uint32_t voffset, uint32_t lds_base) {
  asm volatile("s_nop 4\n\tglobal_load_lds_dword %0, %1"
               :
               : "v"(voffset), "s"(base), "{m0}"(lds_base)
               : "memory");
}
// Wait until at most N of this wave's vector-memory operations are pending.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}
// Workgroup barrier that also orders LDS traffic for the compiler.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" : : : "memory");
}

// Key (0..63) of the tile held in K-tile row R: the inverse of k_row_of_key.
__device__ inline int key_of_krow(int R) {
  const int kb = R >> 4, m = R & 15;
  return 32 * (kb >> 1) + 8 * (m >> 2) + 4 * (kb & 1) + (m & 3);
}

// Byte offset of element (dim d, key) in a V tile.
__device__ inline int v_lds_offset(int d, int key) {
  return (key >> 4) * 4096 + d * 32 + ((((key >> 3) & 1) ^ (((d >> 2) ^ (d >> 3)) & 1)) << 4) +
         2 * (key & 7);
}

// Per-workgroup context of the matrix-core kernel (wave-uniform values).
struct MfmaCtx {
  int b, h, rg, split, tid, lane, n16, g4, wave;
  int n_nodes, P, G, rows_b, row0, n_pages_b, t_begin, n_pref, n_tree;
  // Row blocks of the wave: rows row0 + 16 * (wslot + wstride * k).  With
  // key pairs, waves w and w + 4 own the same blocks (wslot = w & 3,
  // wstride 4) and each takes one 32-key half (khalf) of every tile.
  int wslot, wstride, khalf;
  bool direct;  // this sequence has one active split: write the output itself
  uint32_t lds0;  // LDS byte address of stage 0
  // The wave's page-table entries for the split's first three tiles and the
  // sequence's first page, loaded before the prefix length is known (indices
  // clamped to the table row; entries past the prefix are replaced later).
  int pre_page[3];
  int first_page;
  // rotary embedding: tree positions of the wave's query rows and of node
  // `tid` (loaded with the first round of scalar loads)
  int qpos[kMaxNB];
  int tpos;
};

// One wave's share, specialised on the number NA of 16-row query blocks it
// owns (wave-uniform), so that no matrix instruction sits behind a per-block
// branch.  Every wave runs the same loads and barriers whatever NA is.
template <int NA, bool ROPE, bool PAIR, bool NT>
__device__ __forceinline__ void mfma_wave_body(const AttnParams &p, const MfmaCtx &c,
                                               uint8_t *smem, int32_t *s_tpos) {
  constexpr int NQ = NA > 0 ? NA : 1;
  const __bf16 *q = static_cast<const __bf16 *>(p.q);
  const __bf16 *k_cache = static_cast<const __bf16 *>(p.k_cache);
  const __bf16 *v_cache = static_cast<const __bf16 *>(p.v_cache);
  const int tid = c.tid, lane = c.lane, n16 = c.n16, g4 = c.g4, wave = c.wave;

  // ---- query blocks: block k covers rows row0 + 16*(wave + 8k) .. +15
  bf16x8 qf[NQ][4];
  f32x4 o[NQ][8];
  // Row sums come from the same bf16 probabilities the P V op consumes, via
  // one more matrix op against a ones operand, so every element of l_acc
  // holds the sum over all keys of the lane's query.
  f32x4 l_acc[NQ];
  float m_run[NQ];
  // raw score above which a block must move its exponent offset:
  // (m_run + kRescaleLog2) / (scale * log2 e)
  float thr_raw[NQ];
  const float inv_scale_log2 = 1.f / p.scale_log2;
  const float pinf = pos_inf();
  auto row_of = [&](int k) { return c.row0 + 16 * (c.wslot + c.wstride * k) + n16; };
#pragma unroll
  for (int k = 0; k < NA; ++k) {
    const int r = row_of(k);
    const bool rv = r < c.rows_b;
    const int node = rv ? r / c.G : 0;
    const int hq = c.h * c.G + (rv ? r % c.G : 0);
    const __bf16 *qrow = q + (((size_t)c.b * p.n_max + node) * p.hq + hq) * kD;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      uint4 v = rv ? *reinterpret_cast<const uint4 *>(qrow + 32 * kk + 8 * g4) : zero4();
      qf[k][kk] = *reinterpret_cast<bf16x8 *>(&v);
    }

#pragma unroll
    for (int d = 0; d < 8; ++d) o[k][d] = f32x4{0.f, 0.f, 0.f, 0.f};
    m_run[k] = kNegBig;
    thr_raw[k] = kNegBig;  // the first scores always set the offset
    l_acc[k] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  // rotary embedding of the queries: the table rows are loaded with the
  // queries and the rotation waits until the prologue's own wait below;
  // with three blocks per wave the registers do not allow holding them, so
  // they are loaded after that wait instead
  constexpr bool kEarlyRot = NA <= 2;
  Rot8 rq[ROPE && kEarlyRot ? NQ : 1][2];
  if (ROPE && kEarlyRot) {
#pragma unroll
    for (int k = 0; k < NA; ++k) {
      const int pos = min(max(c.qpos[k], 0), p.rope_positions - 1);
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) rq[k][kk] = load_rot8(p.rope, kD, pos, 32 * kk + 8 * g4);
    }
  }

  // ---- asynchronous loads of the prefix tiles.  Every wave loads one page
  // of each tile: waves 0..3 the K rows of page (wave & 3), waves 4..7 the V
  // dim rows of that page, as four 1 KB blocks, so a wave needs one page id
  // and one base address per tile.  The page table is read-only for the
  // whole kernel: reading it through the constant address space lets
  // uniform indices become scalar loads.
  typedef const __attribute__((address_space(4))) int32_t const_i32;
  const_i32 *table = (const_i32 *)(p.block_table + (size_t)c.b * p.max_blocks);
  const int my_page = wave & 3;
  const bool my_v = wave >= 4;
  const char *kv_base = reinterpret_cast<const char *>(my_v ? v_cache : k_cache) +
                        (size_t)c.h * (kBlock * kD * 2);
  const uint32_t page_stride = (uint32_t)p.hkv * (kBlock * kD * 2);
  // LDS destination of block q within a stage (wave-uniform)
  auto dma_dst = [&](int q) {
    return my_v ? (uint32_t)(kKBytes + (4 * my_page + q) * 1024)
                : (uint32_t)((8 * (my_page >> 1) + 2 * (my_page & 1) + (q & 1) + 4 * (q >> 1)) *
                             1024);
  };
  uint32_t dma_off[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    if (!my_v) {
      // K blocks of page j: inst = 8 (j >> 1) + 2 (j & 1) + {0, 1, 4, 5};
      // block inst holds tile rows 4 inst .. + 3 (lane -> row 4 inst +
      // lane / 16, chunk position lane % 16)
      const int inst = 8 * (my_page >> 1) + 2 * (my_page & 1) + (q & 1) + 4 * (q >> 1);
      const int R = 4 * inst + (lane >> 4);
      const int kl = key_of_krow(R);
      dma_off[q] = (uint32_t)((kl & 15) * 256 + (((lane & 15) ^ (R & 15)) << 4));
    } else {
      // V blocks of page j: dim rows 32 q .. + 31 (lane -> dim row 32 q +
      // lane / 2, half position lane % 2)
      const int d = 32 * q + (lane >> 1);
      dma_off[q] = (uint32_t)(d * 32 + (((lane & 1) ^ (((d >> 2) ^ (d >> 3)) & 1)) << 4));
    }
  }
  // The first three tiles' page ids were loaded before the prefix length
  // was known, at indices clamped to the table row: a page past the prefix
  // becomes the sequence's first page, whose keys there get masked (and its
  // values zeroed).
  auto fix_page = [&](int r, int it) {
    return (c.t_begin + it) * 4 + my_page < c.n_pages_b ? r : c.first_page;
  };
  // In the loop the prefix length is known, so the index is clamped to the
  // sequence's last page instead: the loaded id is used as it is, a tile
  // later, and the scalar load never stalls the tile that issues it.
  const int last_page = max(c.n_pages_b - 1, 0);
  auto tile_page = [&](int it) {
    return table[(uint32_t)min((c.t_begin + it) * 4 + my_page, last_page)];
  };
  // NT (plans with one row group): no other workgroup reads a tile again,
  // so the tiles stream past the caches; several row groups re-read each
  // other's tiles through L2.  A template parameter rather than a runtime
  // test, which would split the tile loop's basic blocks.
  auto issue_prefix = [&](int st, int blk) {
    // the page base is wave-uniform; read it from lane 0 so that it stays in
    // SGPRs for the asm operand whatever the register pressure around it
    const uint64_t ba = (uint64_t)(uintptr_t)(kv_base + (uint64_t)(uint32_t)blk * page_stride);
    // (readfirstlane returns int: each half goes through uint32_t so that
    // the low half is zero-extended, never sign-extended into the high one)
    const uint32_t ba_hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(ba >> 32));
    const uint32_t ba_lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)ba);
    const char *base =
        reinterpret_cast<const char *>(((uint64_t)ba_hi << 32) | (uint64_t)ba_lo);
    const uint32_t sbase = c.lds0 + st * kStageBytes;
    if constexpr (NT) {
#pragma unroll
      for (int q = 0; q < 4; ++q) dma16_nt(base, dma_off[q], sbase + dma_dst(q));
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) dma16(base, dma_off[q], sbase + dma_dst(q));
    }
  };

  // ancestor masks of the wave's rows (read before the tree tiles)
  uint32_t tmask[NQ][4];
#pragma unroll
  for (int k = 0; k < NQ; ++k) tmask[k][0] = tmask[k][1] = tmask[k][2] = tmask[k][3] = 0u;

  // ---- one half tile (32 keys) in two pieces: scores, then softmax and
  // P V.  Half kp covers score blocks 2kp (keys 32kp + 8g + i) and 2kp+1
  // (keys 32kp + 8g + 4 + i) of lane group g, which are exactly the eight
  // key slots lane group g feeds to the P V matrix op.
  // Per-lane LDS offsets: K chunk kk of score-block row n16, and the V row
  // of dim 16 d + n16 (its half-swap bit does not depend on d).
  uint32_t k_off[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) k_off[kk] = n16 * 256 + (((4 * kk + g4) ^ n16) << 4);
  const uint32_t v_off = (g4 >> 1) * 4096 + n16 * 32 +
                         ((((g4 & 1) ^ (((n16 >> 2) ^ (n16 >> 3)) & 1))) << 4);
  auto qk_half = [&](int st, int kp, f32x4 (&sc)[NQ][2]) {
    const uint8_t *sK = smem + st * kStageBytes + kp * 8192;
    // K operands are read two chunks (four operands) at a time ahead of
    // their matrix ops (all eight at once for single-block waves)
    constexpr int kKB = NA >= 2 ? 2 : 4;
#pragma unroll
    for (int k = 0; k < NA; ++k) sc[k][0] = sc[k][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < 4; kb += kKB) {
      bf16x8 ka[kKB][2];
#pragma unroll
      for (int kk = 0; kk < kKB; ++kk)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
          ka[kk][hh] = *reinterpret_cast<const bf16x8 *>(sK + hh * 4096 + k_off[kb + kk]);
#pragma unroll
      for (int kk = 0; kk < kKB; ++kk)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
          for (int k = 0; k < NA; ++k)
            sc[k][hh] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[kk][hh], qf[k][kb + kk],
                                                                sc[k][hh], 0, 0, 0);
    }
  };
  // Softmax of one half in three pieces, so that a half's vector work can
  // sit beside the other half's matrix ops in one basic block:
  //  - prep_half masks the scores where needed and returns, as a
  //    wave-uniform bit set, the blocks whose exponent offset must move
  //    (their lane maxima are left in mx);
  //  - rescale_half moves those offsets (the rare branch);
  //  - exp_half turns the scores into bf16 probabilities.
  auto prep_half = [&](int kp, int key0, bool tree, f32x4 (&sc)[NQ][2], float (&mx)[NQ]) {
    const int limit = tree ? c.n_nodes : c.P;
    const bool masked = tree || key0 + kTile > c.P;  // wave-uniform
    uint32_t rs = 0;
#pragma unroll
    for (int k = 0; k < NA; ++k) {
      f32x4(&s)[2] = sc[k];
      if (masked) {
        const uint32_t(&mw)[4] = tmask[k];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int key = key0 + 32 * kp + 8 * g4 + 4 * hh + i;
            bool vis = key < limit;
            if (tree) vis = vis && ((mask_word(mw, key >> 5) >> (key & 31)) & 1u);
            s[hh][i] = vis ? s[hh][i] : -INFINITY;
          }
      }
      // the lane's maximum of its 8 raw scores against the raw-score
      // threshold of the lazy rescale; the maximum over the half (across
      // the four lane groups) is only needed when some score crosses it
      mx[k] = max8(s[0], s[1], pinf);
      if (__ballot(mx[k] > thr_raw[k]) != 0ull) rs |= 1u << k;
    }
    return rs;
  };
  auto rescale_half = [&](const float (&mx)[NQ], uint32_t rs) {
#pragma unroll
    for (int k = 0; k < NA; ++k) {
      if (rs & (1u << k)) {
        // new offset: the half's maximum (in log2 units) if it is larger
        const float m_new = fmaxf(m_run[k], group4_max(mx[k], pinf) * p.scale_log2);
        const float alpha = fast_exp2(m_run[k] - m_new);
        m_run[k] = m_new;
        thr_raw[k] = (m_new + kRescaleLog2) * inv_scale_log2;
        l_acc[k] *= alpha;
#pragma unroll
        for (int d = 0; d < 8; ++d) o[k][d] *= alpha;
      }
    }
  };
  auto exp_half = [&](const f32x4 (&sc)[NQ][2], bf16x8 (&pb)[NQ]) {
#pragma unroll
    for (int k = 0; k < NA; ++k) {
      const float neg_m = -m_run[k];
      bf16x8 v;
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          v[4 * hh + i] = (__bf16)fast_exp2(fmaf(sc[k][hh][i], p.scale_log2, neg_m));
      pb[k] = v;
    }
  };
  // P V ops of half kp (and the row-sum op against a ones operand).
  auto pv_half = [&](int st, int kp, const bf16x8 (&pb)[NQ]) {
    const uint8_t *sV = smem + st * kStageBytes + kKBytes + kp * 8192 + v_off;
    bf16x8 ones;
#pragma unroll
    for (int e = 0; e < 8; ++e) ones[e] = (__bf16)1.f;
    // all eight V operands are read before the first P V op, so that their
    // LDS latency is paid once per half instead of once per dim block
    bf16x8 av[8];
#pragma unroll
    for (int d = 0; d < 8; ++d) av[d] = *reinterpret_cast<const bf16x8 *>(sV + d * 512);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int k = 0; k < NA; ++k)
      l_acc[k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pb[k], l_acc[k], 0, 0, 0);
#pragma unroll
    for (int d = 0; d < 8; ++d) {
#pragma unroll
      for (int k = 0; k < NA; ++k)
        o[k][d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[d], pb[k], o[k][d], 0, 0, 0);
    }
  };
  // One 64-key tile.  Up to two blocks per wave it is software-pipelined
  // over its two halves: the first half's exponentials share a basic block
  // with the second half's score ops, and the first half's P V ops with the
  // second half's masking and maxima, so that each wave keeps its matrix
  // cores busy through much of its own softmax.  Three blocks do not leave
  // the registers for two halves of scores, so there the halves run one
  // after the other.
  // (K from stage st, V from stage vst)
  auto compute = [&](int st, int key0, bool tree, int vst) {
    if constexpr (PAIR) {
      f32x4 sc[NQ][2];
      float mx[NQ];
      bf16x8 pb[NQ];
      qk_half(st, c.khalf, sc);
      rescale_half(mx, prep_half(c.khalf, key0, tree, sc, mx));
      exp_half(sc, pb);
      pv_half(vst, c.khalf, pb);
    } else if constexpr (NA <= 2) {
      f32x4 sa[NQ][2], sb[NQ][2];
      float ma[NQ], mb[NQ];
      bf16x8 pa[NQ], pz[NQ];
      qk_half(st, 0, sa);
      rescale_half(ma, prep_half(0, key0, tree, sa, ma));
      exp_half(sa, pa);
      qk_half(st, 1, sb);
      pv_half(vst, 0, pa);
      const uint32_t rb = prep_half(1, key0, tree, sb, mb);
      rescale_half(mb, rb);
      exp_half(sb, pz);
      pv_half(vst, 1, pz);
    } else {
#pragma unroll 1
      for (int kp = 0; kp < 2; ++kp) {
        f32x4 sc[NQ][2];
        float mx[NQ];
        bf16x8 pb[NQ];
        qk_half(st, kp, sc);
        rescale_half(mx, prep_half(kp, key0, tree, sc, mx));
        exp_half(sc, pb);
        pv_half(vst, kp, pb);
      }
    }
  };

  // ---- the tiles through the stage ring: the prefix tiles, then (without
  // rotary embedding) the tree tiles.  Prologue: the first two stages are
  // issued behind the query loads and the wait for both is made visible to
  // the compiler (otherwise it would drain every load in flight before the
  // first matrix op of each tile); later stages are issued three tiles
  // ahead of use, prefix page ids fetched by scalar loads a tile earlier.
  constexpr bool kTreeRing = !ROPE;
  const int n_ring = c.n_pref + (kTreeRing ? c.n_tree : 0);
  const __bf16 *k_tree = static_cast<const __bf16 *>(p.k_tree);
  const __bf16 *v_tree = static_cast<const __bf16 *>(p.v_tree);
  // Tree tile tt: each wave loads the 16 nodes tt * 64 + 16 * my_page ..
  // + 15 (ids clamped to the last node), waves 0..3 their K rows into the
  // swizzled rows of the K tile (chunk and row from the prefix offsets),
  // waves 4..7 their V rows key-major (key at 256 bytes * key) into the V
  // tile, to be transposed when the tile comes up.
  auto issue_tree = [&](int st, int tt) {
    // the arguments through an opaque copy of their address, so that they
    // are loaded here, where a prefix iteration issues a tree tile, instead
    // of being hoisted to stay live (and spill) through the prefix loop
    typedef const __attribute__((address_space(4))) AttnParams const_params;
    const_params *ka = (const_params *)__builtin_amdgcn_kernarg_segment_ptr();
    asm volatile("" : "+s"(ka));
    const int last = max(c.n_nodes - 1, 0);
    const int key_base = tt * kTile + 16 * my_page;
    const uint32_t node_stride = (uint32_t)ka->hkv * (kD * 2);
    const uint64_t ba = (uint64_t)(uintptr_t)(
        reinterpret_cast<const char *>(my_v ? ka->v_tree : ka->k_tree) +
        ((size_t)c.b * ka->n_max * ka->hkv + c.h) * (kD * 2));
    const uint32_t ba_hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(ba >> 32));
    const uint32_t ba_lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)ba);
    const char *base =
        reinterpret_cast<const char *>(((uint64_t)ba_hi << 32) | (uint64_t)ba_lo);
    const uint32_t sbase = c.lds0 + st * kStageBytes;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      // K: dma_off holds (key within the page) * 256 + the swizzled chunk's
      // offset; V: key 4 q + lane / 16 of the wave's 16, chunk lane % 16
      const int kq = my_v ? 4 * q + (lane >> 4) : (int)(dma_off[q] >> 8);
      const uint32_t chunk = my_v ? (uint32_t)(lane & 15) << 4 : (dma_off[q] & 255u);
      const uint32_t off = (uint32_t)min(key_base + kq, last) * node_stride + chunk;
      dma16(base, off, sbase + dma_dst(q));
    }
  };
  auto issue_tile = [&](int v, int page) {
    if (kTreeRing && v >= c.n_pref) issue_tree(v % kStages, v - c.n_pref);
    else issue_prefix(v % kStages, page);
  };
  int page_next = 0;
  if (n_ring > 0) issue_tile(0, fix_page(c.pre_page[0], 0));
  if (n_ring > 1) issue_tile(1, fix_page(c.pre_page[1], 1));
  if (c.n_pref > 2) page_next = fix_page(c.pre_page[2], 2);
  // The sequence's ancestor masks go to LDS with the queries: wave w copies
  // words 64 w .. + 63 of its mask rows (indices clamped to the rows), one
  // dword per lane, landed by the wait below.
  uint32_t *s_mask = reinterpret_cast<uint32_t *>(smem + kStages * kStageBytes);
  if (c.n_tree > 0) {
    const uint32_t n_words = (uint32_t)(p.n_max * p.words);  // <= 512 (host check)
    const uint64_t ma =
        (uint64_t)(uintptr_t)(p.tree_mask + (size_t)c.b * p.n_max * p.words);
    const uint32_t ma_hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(ma >> 32));
    const uint32_t ma_lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)ma);
    const char *mbase =
        reinterpret_cast<const char *>(((uint64_t)ma_hi << 32) | (uint64_t)ma_lo);
    const uint32_t widx = min((uint32_t)(64 * wave + lane), n_words - 1u);
    dma4(mbase, widx * 4u, c.lds0 + kStages * kStageBytes + 256u * wave);
  }
  auto load_masks = [&]() {
#pragma unroll
    for (int k = 0; k < NA; ++k) {
      const int r = row_of(k);
      const int node = r < c.rows_b ? r / c.G : 0;
      load_mask4(tmask[k], s_mask + node * p.words, p.words);
    }
  };
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): queries, masks and stages 0, 1
  if (ROPE) {
    // the lane holds dims 32 kk + 8 g4 + j; kk and kk + 2 are the pairs
    // (i, i + 64), rotated in fp32 and rounded once to bf16
#pragma unroll
    for (int k = 0; k < NA; ++k) {
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const Rot8 r = kEarlyRot ? rq[kEarlyRot ? k : 0][kk]
                                 : load_rot8(p.rope, kD,
                                             min(max(c.qpos[k], 0), p.rope_positions - 1),
                                             32 * kk + 8 * g4);
        bf16x8 a = qf[k][kk], e = qf[k][kk + 2];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float x1 = (float)a[j], x2 = (float)e[j];
          a[j] = (__bf16)(x1 * r.c[j] - x2 * r.s[j]);
          e[j] = (__bf16)(x2 * r.c[j] + x1 * r.s[j]);
        }
        qf[k][kk] = a;
        qf[k][kk + 2] = e;
      }
    }
    // tree positions for the tree tiles (published by the loop's first
    // barrier)
    if (tid < p.n_max) s_tpos[tid] = c.tpos;
  }
  if (n_ring > 2) issue_tile(2, page_next);
  if (c.n_pref > 3) page_next = tile_page(3);
  // stage `it` has landed once at most the loads issued after it remain
  auto wait_stage = [&](int it) {
    const int after = min(n_ring - 1 - it, kStages - 2);
    if (after >= 2) wait_vmcnt<2 * kDmaPerStage>();
    else if (after == 1) wait_vmcnt<kDmaPerStage>();
    else wait_vmcnt<0>();
    lds_barrier();  // every wave's loads for stage `it` are in LDS; stage it-1 is free
  };
  auto prefix_tile = [&](int it) {
    const int st = it % kStages;
    const int key0 = (c.t_begin + it) * kTile;
    if (key0 + kTile > c.P) {
      // values past the prefix may be anything: zero them so P = 0 times V
      // stays 0 (keys are masked out of the scores separately)
      uint8_t *sV = smem + st * kStageBytes + kKBytes;
      const int valid = c.P - key0;
      for (int e = tid; e < kD * kTile; e += kMfmaThreads) {
        const int d = e >> 6, key = e & 63;
        if (key >= valid) *reinterpret_cast<__bf16 *>(sV + v_lds_offset(d, key)) = (__bf16)0.f;
      }
      lds_barrier();
    }
    if (NA > 0) compute(st, key0, false, st);
  };
  // Two loops over the prefix tiles, so that the main one, whose
  // iterations each issue the prefix tile three ahead, carries no test
  // for the tree tiles (a taken branch per tile costs more than the code
  // it would save); the last three prefix tiles issue the tree tiles.
  const int n_main = max(c.n_pref - (kStages - 1), 0);
  for (int it = 0; it < n_main; ++it) {
    wait_vmcnt<2 * kDmaPerStage>();  // two tiles are issued after this one
    lds_barrier();  // every wave's loads for stage `it` are in LDS; stage it-1 is free
    issue_prefix((it + kStages - 1) % kStages, page_next);
    if (it + kStages < c.n_pref) page_next = tile_page(it + kStages);
    prefix_tile(it);
  }
  for (int it = n_main; it < c.n_pref; ++it) {
    wait_stage(it);
    if (kTreeRing && it + kStages - 1 < n_ring)
      issue_tree((it + kStages - 1) % kStages, it + kStages - 1 - c.n_pref);
    prefix_tile(it);
  }

  // ---- tree tiles from the ring (split 0 only): the keys are the tree
  // nodes themselves.  A loop of its own, so that the masks and the
  // transposition's registers are live here only.
  if (kTreeRing && c.n_tree > 0) load_masks();
  // (a tree has at most two tiles, and the ring runs three ahead, so every
  // tree tile has been issued by the time the first one comes up)
  static_assert((GRAFT_MAX_NODES + kTile - 1) / kTile <= kStages - 1,
                "the tree tiles are issued from the prefix loop and the prologue");
  for (int it = c.n_pref; it < n_ring; ++it) {
    wait_stage(it);
    const int st = it % kStages;
    const int key0 = (it - c.n_pref) * kTile;
    // V key-major -> dim rows in the V part of stage it + 2, which no tile
    // uses any more (the ring holds at most the next tree tile): thread
    // t < 128 reads the 8 x 8 block of keys 8 kc .. + 7 and dims 8 dc .. + 7
    // (keys past the tree as zeros) and writes it transposed as eight
    // 16-byte dim rows
    const int vst = (it + 2) % kStages;
    if (wave < 2) {
      const uint8_t *sR = smem + st * kStageBytes + kKBytes;
      uint8_t *sV = smem + vst * kStageBytes + kKBytes;
      const int dc = tid & 15, kc = (tid >> 4) & 7;
      uint32_t w[8][4];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int kl = 8 * kc + i;
        const uint4 vv = key0 + kl < c.n_nodes
                             ? *reinterpret_cast<const uint4 *>(sR + kl * 256 + dc * 16)
                             : zero4();
        w[i][0] = vv.x;
        w[i][1] = vv.y;
        w[i][2] = vv.z;
        w[i][3] = vv.w;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int q = e >> 1;
        uint32_t o4[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const uint32_t a = w[2 * m][q], b2 = w[2 * m + 1][q];
          o4[m] = (e & 1) ? ((a >> 16) | (b2 & 0xffff0000u)) : ((a & 0xffffu) | (b2 << 16));
        }
        const int d = dc * 8 + e;
        *reinterpret_cast<uint4 *>(sV + (kc >> 1) * 4096 + d * 32 +
                                   (((kc & 1) ^ (((d >> 2) ^ (d >> 3)) & 1)) << 4)) =
            make_uint4(o4[0], o4[1], o4[2], o4[3]);
      }
    }
    lds_barrier();
    if (NA > 0) compute(st, key0, true, vst);
  }

  // ---- tree tiles with rotary embedding (split 0 only): the keys are
  // rotated by their tree positions on the way into LDS.
  if (!kTreeRing && c.n_tree > 0) load_masks();
  for (int tt = 0; tt < (kTreeRing ? 0 : c.n_tree); ++tt) {
    const int key0 = tt * kTile;
    uint8_t *sK = smem;  // stage 0 (all prefix loads have completed)
    uint8_t *sV = smem + kKBytes;
    wait_vmcnt<0>();
    lds_barrier();
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int ch = tid + kMfmaThreads * r;
      const int kl = ch >> 4, dc = ch & 15;
      const int j = key0 + kl;
      Rot8 rk;
      if (ROPE) {
        // the table row first, so that it loads alongside the key chunk
        const int pos = j < c.n_nodes ? min(max(s_tpos[j], 0), p.rope_positions - 1) : 0;
        rk = load_rot8(p.rope, kD, pos, 8 * (dc & 7));
      }
      uint4 kv = zero4();
      if (j < c.n_nodes)
        kv = *reinterpret_cast<const uint4 *>(
            k_tree + (((size_t)c.b * p.n_max + j) * p.hkv + c.h) * kD + dc * 8);
      if (ROPE) {
        // dims 8 dc .. + 7 pair with dims 8 (dc ^ 8) .. + 7, held by lane ^ 8
        // (same key): x' = x c - y s in the first half, x c + y s in the second
        uint4 pv;
        pv.x = __shfl_xor((int)kv.x, 8);
        pv.y = __shfl_xor((int)kv.y, 8);
        pv.z = __shfl_xor((int)kv.z, 8);
        pv.w = __shfl_xor((int)kv.w, 8);
        const float sg = dc < 8 ? -1.f : 1.f;
        const bf16x8 x = *reinterpret_cast<const bf16x8 *>(&kv);
        const bf16x8 y = *reinterpret_cast<const bf16x8 *>(&pv);
        bf16x8 o8;
#pragma unroll
        for (int e = 0; e < 8; ++e)
          o8[e] = (__bf16)((float)x[e] * rk.c[e] + sg * ((float)y[e] * rk.s[e]));
        kv = *reinterpret_cast<const uint4 *>(&o8);
      }
      const int R = k_row_of_key(kl);
      *reinterpret_cast<uint4 *>(sK + R * 256 + ((dc ^ (R & 15)) << 4)) = kv;
    }
    // V: thread t < 128 takes the 8 x 8 block of keys 8 * kc .. + 7 and
    // dims 8 * dc .. + 7, transposes it in registers and writes eight
    // 16-byte dim rows.
    if (tid < 128) {
      const int dc = tid & 15, kc = tid >> 4;
      uint32_t w[8][4];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int j = key0 + 8 * kc + i;
        uint4 vv = zero4();
        if (j < c.n_nodes)
          vv = *reinterpret_cast<const uint4 *>(
              v_tree + (((size_t)c.b * p.n_max + j) * p.hkv + c.h) * kD + dc * 8);
        w[i][0] = vv.x;
        w[i][1] = vv.y;
        w[i][2] = vv.z;
        w[i][3] = vv.w;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int q = e >> 1;
        uint32_t o4[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const uint32_t a = w[2 * m][q], b2 = w[2 * m + 1][q];
          o4[m] = (e & 1) ? ((a >> 16) | (b2 & 0xffff0000u)) : ((a & 0xffffu) | (b2 << 16));
        }
        const int d = dc * 8 + e;
        *reinterpret_cast<uint4 *>(sV + (kc >> 1) * 4096 + d * 32 +
                                   (((kc & 1) ^ (((d >> 2) ^ (d >> 3)) & 1)) << 4)) =
            make_uint4(o4[0], o4[1], o4[2], o4[3]);
      }
    }
    lds_barrier();
    if (NA > 0) compute(0, key0, true, 0);
  }

  // ---- key pairs: the wave of the second half hands its (O, max, sum)
  // to its partner through LDS (the stage ring is free once every wave is
  // past its last tile), and the partner merges them by log-sum-exp.
  if constexpr (PAIR) {
    lds_barrier();
    f32x4 *xo = reinterpret_cast<f32x4 *>(smem);  // [slot][k][d][lane]
    float *xml = reinterpret_cast<float *>(smem + 4 * NQ * 8 * 64 * 16);  // [slot][k][lane][2]
    if (c.khalf == 1) {
#pragma unroll
      for (int k = 0; k < NA; ++k) {
#pragma unroll
        for (int d = 0; d < 8; ++d) xo[((c.wslot * NQ + k) * 8 + d) * 64 + lane] = o[k][d];
        xml[((c.wslot * NQ + k) * 64 + lane) * 2 + 0] = m_run[k];
        xml[((c.wslot * NQ + k) * 64 + lane) * 2 + 1] = l_acc[k][0];
      }
    }
    lds_barrier();
    if (c.khalf == 1) return;
#pragma unroll
    for (int k = 0; k < NA; ++k) {
      const float mb = xml[((c.wslot * NQ + k) * 64 + lane) * 2 + 0];
      const float lb = xml[((c.wslot * NQ + k) * 64 + lane) * 2 + 1];
      const float mm = fmaxf(m_run[k], mb);
      const float fa = fast_exp2(m_run[k] - mm), fb = fast_exp2(mb - mm);
      m_run[k] = mm;
      l_acc[k][0] = l_acc[k][0] * fa + lb * fb;
#pragma unroll
      for (int d = 0; d < 8; ++d)
        o[k][d] = o[k][d] * fa + xo[((c.wslot * NQ + k) * 8 + d) * 64 + lane] * fb;
    }
  }

  // ---- epilogue: finish the row sums across the four lane groups and
  // write either the output or this split's partials.
#pragma unroll
  for (int k = 0; k < NA; ++k) {
    const float l = l_acc[k][0];
    const int r = row_of(k);
    if (r >= c.rows_b) continue;
    const int rl = r - c.row0;
    if (c.direct) {
      const float inv = 1.f / l;
      const int node = r / c.G;
      const int hq = c.h * c.G + r % c.G;
      __hip_bfloat16 *out = static_cast<__hip_bfloat16 *>(p.out) +
                            (((size_t)c.b * p.n_max + node) * p.hq + hq) * kD;
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
          ((((size_t)c.b * p.hkv + c.h) * p.n_row_groups + c.rg) * p.n_splits + c.split) *
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

// One work item of the matrix-core kernel: the (sequence, KV head, row
// group, prefix split) that item `id` decodes to.  Items are laid out for
// the XCDs: id = xcd + 8 * slot, and the row groups of one KV stream
// (sequence, head, split) take consecutive slots on one XCD and share its
// L2.
template <int NB, bool ROPE, bool LPT, bool NT>
__device__ __forceinline__ void attn_mfma_item(const AttnParams &p, int id, uint8_t *smem,
                                               int32_t *s_tpos) {
  // the thread index, through an opaque copy: every value derived from it
  // is computed in the item that uses it, not hoisted out of the item loop
  // to stay live (and spill) through every item
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  MfmaCtx c;
  {
    const int xcd = id & 7, slot = id >> 3;
    c.rg = slot % p.n_row_groups;
    const int cluster = (slot / p.n_row_groups) * 8 + xcd;
    const int n_clusters = p.batch * p.hkv * p.n_splits;
    if (cluster >= n_clusters) return;
    if (LPT) {
      // Longest first: (sequence, split) pairs ranked by their tile count
      // (the tree tiles counted in split 0), descending, ties by pair index;
      // cluster k takes the pair of rank k / hkv and KV head k % hkv, so the
      // dispatcher starts the longest work first whatever the prefix lengths.
      __shared__ int32_t s_w[kMfmaThreads];
      __shared__ int32_t s_pair;
      const int t = tid, S = p.n_splits;
      const int n_pairs = p.batch * S;  // <= kMfmaThreads (host check)
      int w = -1;
      if (t < n_pairs) {
        const int b = t / S, sp = t % S;
        const int P = min(max(p.prefix_len[b], 0), p.max_blocks * kBlock);
        const int tiles = (P + kTile - 1) / kTile;
        const int tb = max(0, sp * p.tiles_per_split - p.tree_shift);
        w = max(0, min((sp + 1) * p.tiles_per_split - p.tree_shift, tiles) - tb);
        if (sp == 0) w += (min(max(p.n_nodes[b], 0), p.n_max) + kTile - 1) / kTile;
        s_w[t] = w;
      }
      __syncthreads();
      const int q = cluster / p.hkv;
      if (t < n_pairs) {
        int rank = 0;
        for (int u = 0; u < n_pairs; ++u) {
          const int wu = s_w[u];
          rank += (wu > w || (wu == w && u < t)) ? 1 : 0;
        }
        if (rank == q) s_pair = t;
      }
      __syncthreads();
      const int pair = s_pair;
      c.split = pair % S;
      c.b = pair / S;
      c.h = cluster % p.hkv;
    } else {
      c.split = cluster % p.n_splits;
      c.h = (cluster / p.n_splits) % p.hkv;
      c.b = cluster / (p.n_splits * p.hkv);
    }
  }
  c.tid = tid;
  c.lane = c.tid & 63;
  c.wave = __builtin_amdgcn_readfirstlane(c.tid >> 6);
  const bool pair = NB == 1 && p.key_pairs;
  c.wslot = pair ? (c.wave & 3) : c.wave;
  c.wstride = pair ? 4 : kMfmaWaves;
  c.khalf = pair ? (c.wave >> 2) : 0;
  if (ROPE) {
    // before the node count is known: indices clamped to the row
    const int32_t *tp = p.tree_pos + (size_t)c.b * p.n_max;
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      const int r = group_row0(p, c.rg) + 16 * (c.wslot + c.wstride * k) + (c.lane & 15);
      c.qpos[k] = tp[min(r / p.group, p.n_max - 1)];
    }
    c.tpos = c.tid < p.n_max ? tp[c.tid] : 0;
  }
  {
    typedef const __attribute__((address_space(4))) int32_t const_i32;
    const_i32 *trow = (const_i32 *)(p.block_table + (size_t)c.b * p.max_blocks);
    const int last = p.max_blocks - 1;
    // split s covers prefix tiles [s * tps - shift, (s + 1) * tps - shift):
    // the first `shift` tiles of split 0 are its tree tiles
    const int pg0 = max(0, c.split * p.tiles_per_split - p.tree_shift) * 4 + (c.wave & 3);
    c.first_page = trow[0];
#pragma unroll
    for (int i = 0; i < 3; ++i) c.pre_page[i] = trow[(uint32_t)min(pg0 + 4 * i, last)];
  }
  c.n16 = c.lane & 15;
  c.g4 = c.lane >> 4;
  c.lds0 = (uint32_t)(uintptr_t)smem;

  // Clamp caller-supplied counts to the buffer bounds (documented
  // preconditions; the clamp only keeps reads in bounds if they are broken).
  c.n_nodes = min(max(p.n_nodes[c.b], 0), p.n_max);
  c.P = min(max(p.prefix_len[c.b], 0), p.max_blocks * kBlock);
  c.G = p.group;
  c.rows_b = c.n_nodes * c.G;
  c.row0 = group_row0(p, c.rg);
  const int group_rows = 16 * (p.group_blocks_lo + (c.rg < p.group_blocks_rem ? 1 : 0));
  if (c.row0 >= c.rows_b) return;  // group past this sequence's rows

  const int nt_prefix = (c.P + kTile - 1) / kTile;
  c.n_pages_b = (c.P + kBlock - 1) / kBlock;
  c.t_begin = max(0, c.split * p.tiles_per_split - p.tree_shift);
  const int t_end = min((c.split + 1) * p.tiles_per_split - p.tree_shift, nt_prefix);
  c.n_pref = max(0, t_end - c.t_begin);
  c.n_tree = c.split == 0 ? (c.n_nodes + kTile - 1) / kTile : 0;
  c.direct = active_splits(p, nt_prefix) == 1;
  if (c.n_pref == 0 && c.n_tree == 0) return;  // empty split


  // the wave's active 16-row blocks are k = 0 .. na-1
  int na = 0;
#pragma unroll
  for (int k = 0; k < NB; ++k) {
    const int rl = 16 * (c.wslot + c.wstride * k);
    if (rl < group_rows && c.row0 + rl < c.rows_b) na = k + 1;
  }
  if (NB >= 3 && na == 3) mfma_wave_body<3, ROPE, false, NT>(p, c, smem, s_tpos);
  else if (NB >= 2 && na == 2) mfma_wave_body<(NB >= 2 ? 2 : 1), ROPE, false, NT>(p, c, smem, s_tpos);
  else if (na == 1) {
    if (pair) mfma_wave_body<1, ROPE, true, NT>(p, c, smem, s_tpos);
    else mfma_wave_body<1, ROPE, false, NT>(p, c, smem, s_tpos);
  } else if (pair) {
    mfma_wave_body<0, ROPE, true, NT>(p, c, smem, s_tpos);
  } else {
    mfma_wave_body<0, ROPE, false, NT>(p, c, smem, s_tpos);
  }
}

// Persistent over the items.  With more items than compute units a
// uniform plan's grid holds one workgroup per compute unit (the LDS ring
// fills a unit) and each runs its items back to back, so no workgroup
// waits on the dispatcher between them: measured per-workgroup timestamps
// showed each XCD starting its second wave of workgroups only once its
// whole first wave had ended.  (Ragged plans launch one workgroup per
// item: there the dispatcher's longest-first order packs better.)
// Workgroup s of an XCD (of W there) takes item slot s first, then slot
// 2W - 1 - s, then 2W + s, and so on, alternating direction: the four row
// groups of a stream move together (their L2 sharing holds) and a
// workgroup that had a long item next takes a short one (longest-first
// ranks, and the 17-block row groups).
template <int NB, bool ROPE, bool LPT, bool NT>
__global__ __launch_bounds__(kMfmaThreads) void attn_mfma_kernel(AttnParams p) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kStages * kStageBytes + kMaskBytes];
  __shared__ int32_t s_tpos[ROPE ? GRAFT_MAX_NODES : 1];  // tree positions (rotary path)
  const int xcd = blockIdx.x & 7;
  const int per_xcd = gridDim.x >> 3;  // workgroups per XCD (the grid is a multiple of 8)
  const int s_local = blockIdx.x >> 3;
  const long clusters = (long)p.batch * p.hkv * p.n_splits;
  const int n_slots = (int)(p.n_row_groups * ((clusters + 7) / 8));  // item slots per XCD
  for (int r = 0;; ++r) {
    const int slot = r * per_xcd + ((r & 1) ? per_xcd - 1 - s_local : s_local);
    if (slot >= n_slots) break;
    if (r > 0) __syncthreads();  // every wave is done with the last item's LDS
    // The item reads the arguments at their uses.  Taken through a pointer
    // the compiler cannot see to be the same each round, they are loaded
    // in the round that uses them; otherwise they are hoisted out of the
    // loop, overflow the scalar registers and spill.
    typedef const __attribute__((address_space(4))) AttnParams const_params;
    const_params *kp = (const_params *)__builtin_amdgcn_kernarg_segment_ptr();
    asm volatile("" : "+s"(kp));
    attn_mfma_item<NB, ROPE, LPT, NT>(*(const AttnParams *)kp, xcd + 8 * slot, smem, s_tpos);
  }
}

// ------------------------------------------------------------------------
// Wavefront path: one wave per query row (sequence, node, query head).
// Each lane scores one key of a 64-key chunk (a full dot product over the
// head dim), then the lanes own head dims for the P V accumulation.  Dim-major
// V pages make the per-dim key runs contiguous.
template <typename T, int D, bool ROPE>
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
  if (ROPE) {
    // each lane rotates its own pairs (i, i + D/2) in place, kept in fp32
    __builtin_amdgcn_wave_barrier();
    const float *rrow = p.rope + (size_t)rope_row(p, b, node) * D;
    for (int i = lane; i < D / 2; i += 64) {
      const float c = rrow[i], sn = rrow[D / 2 + i];
      const float x1 = s_q[wave][i], x2 = s_q[wave][i + D / 2];
      s_q[wave][i] = x1 * c - x2 * sn;
      s_q[wave][i + D / 2] = x2 * c + x1 * sn;
    }
  }
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
      if (ROPE && tree) {
        // the tree key rotated at its own position, pair by pair
        const float *rrow = p.rope + (size_t)rope_row(p, b, key) * D;
        for (int i = 0; i < D / 2; ++i) {
          const float k1 = (float)krow[i], k2 = (float)krow[i + D / 2];
          const float c = rrow[i], sn = rrow[D / 2 + i];
          dot += s_q[wave][i] * (k1 * c - k2 * sn) + s_q[wave][i + D / 2] * (k2 * c + k1 * sn);
        }
      } else {
        for (int d = 0; d < D; ++d) dot += s_q[wave][d] * (float)krow[d];
      }
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
  if (active_splits(p, nt_prefix) == 1) {
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
// Two forms.  Launches with few output rows (and often many splits) take one
// wave per row: lane s reads split s's (max, sum), the wave reduces them, and
// each lane accumulates two head dims over the splits, taking split j's
// weight from lane j with a scalar read-lane.  Launches with many output
// rows and few splits take sixteen lanes per row, each owning head_dim / 16
// dims and folding the splits' (max, sum) pairs itself (the same addresses
// for the row's lanes), so that no cross-lane reduction is needed and each
// split's partial row is one contiguous read.
constexpr int kMaxSplits = 256;
constexpr int kCombineManyRows = 8192;  // output rows from which the 16-lane form pays

__device__ inline float wave_max(float x) {
  for (int off = 32; off > 0; off >>= 1) x = fmaxf(x, __shfl_xor(x, off));
  return x;
}
__device__ inline float wave_sum(float x) {
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
  return x;
}

template <typename T>
__global__ __launch_bounds__(256) void attn_combine_wave_kernel(AttnParams p) {
  const int lane = threadIdx.x & 63;
  const long row = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int hq = (int)(row % p.hq);
  const int node = (int)((row / p.hq) % p.n_max);
  const int b = (int)(row / ((long)p.hq * p.n_max));
  if (b >= p.batch || node >= min(p.n_nodes[b], p.n_max)) return;  // whole wave
  const int G = p.group;
  const int h = hq / G;
  const int r = node * G + hq % G;
  const int rg = group_of_row(p, r);
  const int rl = p.n_row_groups == 1 ? r : r - group_row0(p, rg);
  const int P = min(max(p.prefix_len[b], 0), p.max_blocks * kBlock);
  const int nt_prefix = (P + kTile - 1) / kTile;
  const int active = active_splits(p, nt_prefix);
  if (active == 1) return;  // written by the attention kernel
  const size_t base = (((size_t)b * p.hkv + h) * p.n_row_groups + rg) * p.n_splits;
  const size_t stride = (size_t)p.rows_per_group;  // partial rows between splits
  const float *ml = p.part_ml + (base * stride + rl) * 2;
  const float *po = p.part_o + (base * stride + rl) * p.head_dim;
  const int dpl = p.head_dim / 64;  // 1 or 2 dims per lane

  const size_t sstride = stride * p.head_dim;  // floats between splits
  auto load_o = [&](int j) {
    const float *src = po + (size_t)j * sstride + dpl * lane;
    return dpl == 2 ? *reinterpret_cast<const float2 *>(src) : make_float2(src[0], 0.f);
  };
  float L = 0.f, acc0 = 0.f, acc1 = 0.f;
  if (active <= 64) {
    // Every load is issued before the reductions: the first eight splits'
    // values, and lane s's (max, sum) of split s.
    float2 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = u < active ? load_o(u) : make_float2(0.f, 0.f);
    float m_s = kNegBig, l_s = 0.f;
    if (lane < active) {
      m_s = ml[(size_t)lane * stride * 2];
      l_s = ml[(size_t)lane * stride * 2 + 1];
    }
    const float M = wave_max(m_s);
    const float w = lane < active ? fast_exp2(m_s - M) : 0.f;
    L = w * l_s;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const float wj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), u));
      acc0 += wj * v[u].x;
      acc1 += wj * v[u].y;
    }
    for (int j0 = 8; j0 < active; j0 += 8) {
      float2 x[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) x[u] = j0 + u < active ? load_o(j0 + u) : make_float2(0.f, 0.f);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const float wj =
            __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), min(j0 + u, 63)));
        acc0 += wj * x[u].x;
        acc1 += wj * x[u].y;
      }
    }
  } else {
    float M = kNegBig;
    for (int s0 = 0; s0 < active; s0 += 64)
      if (s0 + lane < active) M = fmaxf(M, ml[(size_t)(s0 + lane) * stride * 2]);
    M = wave_max(M);
    for (int s0 = 0; s0 < active; s0 += 64) {
      float w = 0.f;
      if (s0 + lane < active) {
        const float *e = ml + (size_t)(s0 + lane) * stride * 2;
        w = fast_exp2(e[0] - M);
        L += w * e[1];
      }
      const int n = min(64, active - s0);
      for (int j = 0; j < n; ++j) {
        const float wj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), j));
        const float2 x = load_o(s0 + j);
        acc0 += wj * x.x;
        acc1 += wj * x.y;
      }
    }
  }
  const float inv = 1.f / wave_sum(L);
  T *out = static_cast<T *>(p.out) + (((size_t)b * p.n_max + node) * p.hq + hq) * p.head_dim;
  if (dpl == 2) {
    out[2 * lane] = (T)(acc0 * inv);
    out[2 * lane + 1] = (T)(acc1 * inv);
  } else {
    out[lane] = (T)(acc0 * inv);
  }
}


template <typename T, int D>
__global__ __launch_bounds__(256) void attn_combine_rows_kernel(AttnParams p) {
  constexpr int DPL = D / 16;  // dims per lane: 8 or 4
  const int ln = threadIdx.x & 15;
  const long row = (long)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int hq = (int)(row % p.hq);
  const int node = (int)((row / p.hq) % p.n_max);
  const int b = (int)(row / ((long)p.hq * p.n_max));
  if (b >= p.batch || node >= min(p.n_nodes[b], p.n_max)) return;  // a row's lanes together
  const int G = p.group;
  const int h = hq / G;
  const int r = node * G + hq % G;
  const int rg = group_of_row(p, r);
  const int rl = p.n_row_groups == 1 ? r : r - group_row0(p, rg);
  const int P = min(max(p.prefix_len[b], 0), p.max_blocks * kBlock);
  const int nt_prefix = (P + kTile - 1) / kTile;
  const int active = active_splits(p, nt_prefix);
  if (active == 1) return;  // written by the attention kernel
  const size_t base = (((size_t)b * p.hkv + h) * p.n_row_groups + rg) * p.n_splits;
  const size_t stride = (size_t)p.rows_per_group;  // partial rows between splits
  const float *ml = p.part_ml + (base * stride + rl) * 2;
  const float *po = p.part_o + (base * stride + rl) * D + DPL * ln;
  float M = kNegBig;
  for (int j = 0; j < active; ++j) M = fmaxf(M, ml[(size_t)j * stride * 2]);
  float L = 0.f, acc[DPL];
#pragma unroll
  for (int e = 0; e < DPL; ++e) acc[e] = 0.f;
  const size_t sstride = stride * D;  // floats between splits
  auto load = [&](float (&x)[DPL], const float *src) {
#pragma unroll
    for (int q = 0; q < DPL / 4; ++q) {
      const float4 v = *reinterpret_cast<const float4 *>(src + 4 * q);
      x[4 * q] = v.x; x[4 * q + 1] = v.y; x[4 * q + 2] = v.z; x[4 * q + 3] = v.w;
    }
  };
  int j = 0;
  for (; j + 4 <= active; j += 4) {
    float x[4][DPL], mj[4], lj[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      load(x[u], po + (size_t)(j + u) * sstride);
      mj[u] = ml[(size_t)(j + u) * stride * 2];
      lj[u] = ml[(size_t)(j + u) * stride * 2 + 1];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float w = fast_exp2(mj[u] - M);
      L += w * lj[u];
#pragma unroll
      for (int e = 0; e < DPL; ++e) acc[e] += w * x[u][e];
    }
  }
  for (; j < active; ++j) {
    float x[DPL];
    load(x, po + (size_t)j * sstride);
    const float w = fast_exp2(ml[(size_t)j * stride * 2] - M);
    L += w * ml[(size_t)j * stride * 2 + 1];
#pragma unroll
    for (int e = 0; e < DPL; ++e) acc[e] += w * x[e];
  }
  const float inv = 1.f / L;
  T *out = static_cast<T *>(p.out) + (((size_t)b * p.n_max + node) * p.hq + hq) * D + DPL * ln;
#pragma unroll
  for (int e = 0; e < DPL; ++e) out[e] = (T)(acc[e] * inv);
}

}  // namespace

// ------------------------------------------------------------------------
// Launch planning.  Query rows per KV head are n_max * group, in blocks of
// 16.  The matrix-core path holds one workgroup per compute unit (its LDS
// ring and registers fill one), so the plan picks the number of row groups
// and prefix splits that minimise an estimate of the kernel's time:
//   rounds * tiles per workgroup * (a per-tile cost + a cost per 16-row
//   block on the busiest SIMD + a cost per block of the workgroup)
// bounded below by the HBM and L2 streams, plus a fixed cost per round
// (dispatch, prologue, epilogue) and, when the prefix is split, the combine
// launch and the split partials' traffic.  The constants are measured on
// MI355X.  The wavefront path splits the prefix so the grid holds about two
// workgroups per compute unit.
namespace {
constexpr int kComputeUnits = 256;
constexpr double kTileFixedUs = 0.4;          // per 64-key tile, any block count
constexpr double kTileBlockUs = 0.15;         // per 16-row block on the busiest SIMD
constexpr double kTileGroupBlockUs = 0.07;    // per 16-row block of the workgroup
constexpr double kRoundUs = 6.0;              // dispatch + prologue + epilogue
constexpr double kCombineUs = 4.0;            // combine launch
constexpr double kPartialBytesPerUs = 5.0e6;  // partials written, then read back
constexpr double kL2BytesPerUs = 16.0e6;      // KV re-reads by extra row groups (L2)
constexpr double kHbmBytesPerUs = 5.0e6;      // streaming reads from HBM

int busiest_simd_blocks(int blocks_per_group) {
  int best = 0;
  for (int j = 0; j < 4; ++j) {  // SIMD j runs waves j and j + 4
    const int a = max(0, (blocks_per_group - j + kMfmaWaves - 1) / kMfmaWaves);
    const int b = max(0, (blocks_per_group - j - 4 + kMfmaWaves - 1) / kMfmaWaves);
    best = max(best, a + b);
  }
  return best;
}
}  // namespace

AttnPlan plan_attention(graft_dtype dtype, int32_t batch, int32_t n_max, int32_t hq,
                        int32_t hkv, int32_t head_dim, int32_t max_prefix, int64_t sum_prefix) {
  AttnPlan pl{};
  const int group = hq / hkv;
  const int rows = n_max * group;
  pl.mfma = dtype == GRAFT_BF16 && head_dim == kD && rows >= 16;
  const int tiles = max(1, (max_prefix + kTile - 1) / kTile);
  if (pl.mfma) {
    const int blocks = (rows + 15) / 16;
    const int per_group = kMfmaWaves * kMaxNB;
    const int g_min = (blocks + per_group - 1) / per_group;
    // Modelled prefix lengths: every sequence at max_prefix, unless the
    // caller's sum says the batch is ragged; then M representative lengths
    // spread evenly around the mean up to the maximum (each standing for
    // batch / M sequences).
    // (the device ranks batch x splits pairs in one workgroup pass, so a
    // ragged plan needs batch <= kMfmaThreads)
    const bool ragged = batch > 1 && batch <= kMfmaThreads && sum_prefix > 0 &&
                        sum_prefix < (int64_t)batch * max_prefix;
    const int M = ragged ? min(batch, 64) : 1;
    const double mult = (double)batch / M;
    double len[64];
    {
      const double mean = ragged ? (double)sum_prefix / batch : (double)max_prefix;
      const double hi = ragged ? std::min((double)max_prefix, 2.0 * mean) : (double)max_prefix;
      const double lo = ragged ? std::max(0.0, 2.0 * mean - hi) : hi;
      for (int i = 0; i < M; ++i) len[i] = lo + (hi - lo) * (i + 0.5) / M;
    }
    pl.lpt = ragged;
    const int tree_tiles = (n_max + kTile - 1) / kTile;
    double best = 1e30;
    for (int groups = g_min; groups <= min(blocks, 4 * g_min); ++groups) {
      const int bpg = (blocks + groups - 1) / groups;
      // up to 4 blocks: key pairs, each SIMD's two waves on half the keys
      const bool pairs = bpg <= 4;
      const double simd = pairs ? 0.5 : busiest_simd_blocks(bpg);
      const double tile_us = kTileFixedUs + simd * kTileBlockUs + bpg * kTileGroupBlockUs;
      for (int splits = 1; splits <= min(tiles, kMaxSplits); ++splits) {
        const int tps = (tiles + splits - 1) / splits;
        const int eff_splits = (tiles + tps - 1) / tps;
        if (eff_splits != splits) continue;
        if (ragged && (long)batch * splits > kMfmaThreads) continue;  // device ranking
        // workgroups per modelled sequence, their total time and the longest
        double n_wg = 0, total_us = 0, longest_us = 0, kv_bytes = 0, active = 0;
        for (int i = 0; i < M; ++i) {
          const int t_i = (int)((len[i] + kTile - 1) / kTile);
          const int s_i = max(1, (t_i + tps - 1) / tps);
          const double wgs_i = mult * hkv * groups * s_i;
          n_wg += wgs_i;
          total_us += mult * hkv * groups * ((t_i + tree_tiles) * tile_us + s_i * kRoundUs);
          longest_us = std::max(longest_us, (std::min(tps, t_i) + tree_tiles) * tile_us + kRoundUs);
          kv_bytes += mult * hkv * (double)t_i * kTile * kD * 2 * 2;
          active += mult * s_i;
        }
        // one workgroup per compute unit at a time: with every workgroup
        // equal this is rounds x (tps tiles + overhead); ragged batches run
        // longest first, which packs to about total / CUs, never below the
        // longest workgroup
        const double t_l2 = groups * kv_bytes / kL2BytesPerUs;
        const double t_hbm = kv_bytes / kHbmBytesPerUs;
        double t;
        if (!ragged) {
          const long rounds = (long)((n_wg + kComputeUnits - 1) / kComputeUnits);
          t = std::max(rounds * tps * tile_us, std::max(t_l2, t_hbm)) + rounds * kRoundUs;
        } else {
          const double t_tiles =
              std::max(longest_us, total_us / kComputeUnits + 0.5 * total_us / n_wg);
          t = std::max(t_tiles, std::max(t_l2, t_hbm));
        }
        if (splits > 1)
          t += kCombineUs + active * n_max * hq * (head_dim + 2) * 4.0 * 2.0 / kPartialBytesPerUs;
        if (t < best) {
          best = t;
          pl.n_row_groups = groups;
          pl.rows_per_group = 16 * bpg;
          pl.group_blocks_lo = blocks / groups;
          pl.group_blocks_rem = blocks % groups;
          pl.tiles_per_split = tps;
          pl.n_splits = splits;
          pl.key_pairs = pairs;
        }
      }
    }
    // Split 0 also runs the tree tiles, so with equal prefix shares it ends
    // last.  The tree tiles count as the first tiles of split 0 instead,
    // when that keeps the split count and leaves split 0 at least one prefix
    // tile (so that the splits with prefix work stay the first ones, as the
    // combine assumes).
    if (pl.n_splits > 1) {
      const int tps = (tiles + tree_tiles + pl.n_splits - 1) / pl.n_splits;
      if (tps >= tree_tiles + 1 && (tiles + tree_tiles + tps - 1) / tps == pl.n_splits) {
        pl.tiles_per_split = tps;
        pl.tree_shift = tree_tiles;
      }
    }
  } else {
    pl.n_row_groups = 1;
    pl.rows_per_group = (rows + 3) / 4 * 4;
    pl.group_blocks_lo = pl.group_blocks_rem = 0;
    const long base = (long)batch * hkv * (pl.rows_per_group / 4);
    int splits = (int)max(1L, min((long)tiles, (512 + base - 1) / max(1L, base)));
    splits = min(min(splits, max(1, tiles / 4)), kMaxSplits);
    pl.tiles_per_split = (tiles + splits - 1) / splits;
    pl.n_splits = (tiles + pl.tiles_per_split - 1) / pl.tiles_per_split;
  }
  const size_t prows = (size_t)batch * hkv * pl.n_row_groups * pl.n_splits * pl.rows_per_group;
  pl.part_o_bytes = pl.n_splits > 1 ? prows * head_dim * sizeof(float) : 0;
  pl.part_ml_bytes = pl.n_splits > 1 ? prows * 2 * sizeof(float) : 0;
  return pl;
}

namespace {
template <int NB>
void launch_mfma(const AttnParams &p, dim3 grid, hipStream_t stream) {
  // non-temporal tile loads when no other row group re-reads the tiles
  const bool nt = p.n_row_groups == 1;
  const int kind = (p.rope ? 1 : 0) + (p.lpt ? 2 : 0) + (nt ? 4 : 0);
  const dim3 block(kMfmaThreads);
  switch (kind) {
    case 0: hipLaunchKernelGGL((attn_mfma_kernel<NB, false, false, false>), grid, block, 0, stream, p); break;
    case 1: hipLaunchKernelGGL((attn_mfma_kernel<NB, true, false, false>), grid, block, 0, stream, p); break;
    case 2: hipLaunchKernelGGL((attn_mfma_kernel<NB, false, true, false>), grid, block, 0, stream, p); break;
    case 3: hipLaunchKernelGGL((attn_mfma_kernel<NB, true, true, false>), grid, block, 0, stream, p); break;
    case 4: hipLaunchKernelGGL((attn_mfma_kernel<NB, false, false, true>), grid, block, 0, stream, p); break;
    case 5: hipLaunchKernelGGL((attn_mfma_kernel<NB, true, false, true>), grid, block, 0, stream, p); break;
    case 6: hipLaunchKernelGGL((attn_mfma_kernel<NB, false, true, true>), grid, block, 0, stream, p); break;
    default: hipLaunchKernelGGL((attn_mfma_kernel<NB, true, true, true>), grid, block, 0, stream, p); break;
  }
}
}  // namespace

long attention_workgroups(const AttnPlan &pl, int32_t batch, int32_t hkv) {
  if (pl.mfma) {
    const long clusters = (long)batch * hkv * pl.n_splits;
    const long items = 8L * pl.n_row_groups * ((clusters + 7) / 8);
    return pl.lpt ? items : std::min<long>(items, kComputeUnits);
  }
  return (long)pl.n_splits * hkv * (pl.rows_per_group / 4) * batch;
}

void launch_attention_bf16_mfma(const AttnParams &p, hipStream_t stream) {
  const long clusters = (long)p.batch * p.hkv * p.n_splits;
  const long items = 8L * p.n_row_groups * ((clusters + 7) / 8);
  // ragged batches keep one workgroup per item: the dispatcher's longest-
  // first order packs their unequal items better than a fixed assignment
  dim3 grid((unsigned)(p.lpt ? items : std::min<long>(items, kComputeUnits)));
  const int nb = (p.rows_per_group / 16 + kMfmaWaves - 1) / kMfmaWaves;
  switch (nb) {
    case 1: launch_mfma<1>(p, grid, stream); break;
    case 2: launch_mfma<2>(p, grid, stream); break;
    default: launch_mfma<3>(p, grid, stream); break;
  }
}

namespace {
template <typename T, int D>
void launch_wave(const AttnParams &p, dim3 grid, hipStream_t stream) {
  if (p.rope)
    hipLaunchKernelGGL((attn_wave_kernel<T, D, true>), grid, dim3(kThreads), 0, stream, p);
  else
    hipLaunchKernelGGL((attn_wave_kernel<T, D, false>), grid, dim3(kThreads), 0, stream, p);
}
}  // namespace

void launch_attention_wave(graft_dtype dtype, const AttnParams &p, hipStream_t stream) {
  dim3 grid(p.n_splits, p.hkv * (p.rows_per_group / 4), p.batch);
  if (dtype == GRAFT_F32) {
    if (p.head_dim == 64) launch_wave<float, 64>(p, grid, stream);
    else launch_wave<float, 128>(p, grid, stream);
  } else {
    if (p.head_dim == 64) launch_wave<__hip_bfloat16, 64>(p, grid, stream);
    else launch_wave<__hip_bfloat16, 128>(p, grid, stream);
  }
}

namespace {
template <typename T>
void launch_combine(const AttnParams &p, long rows, hipStream_t stream) {
  if (rows >= kCombineManyRows) {
    dim3 grid((unsigned)((rows + 15) / 16));
    if (p.head_dim == 128)
      hipLaunchKernelGGL((attn_combine_rows_kernel<T, 128>), grid, dim3(256), 0, stream, p);
    else
      hipLaunchKernelGGL((attn_combine_rows_kernel<T, 64>), grid, dim3(256), 0, stream, p);
  } else {
    dim3 grid((unsigned)((rows + 3) / 4));
    hipLaunchKernelGGL(attn_combine_wave_kernel<T>, grid, dim3(256), 0, stream, p);
  }
}
}  // namespace

void launch_attention_combine(graft_dtype dtype, const AttnParams &p, hipStream_t stream) {
  const long rows = (long)p.batch * p.n_max * p.hq;
  if (dtype == GRAFT_F32) launch_combine<float>(p, rows, stream);
  else launch_combine<__hip_bfloat16>(p, rows, stream);
}

}  // namespace graft
