// Lossless sampling acceptance (temperature T > 0) of the verified hybrid
// tree, by recursive rejection sampling.
//
// Every child of a node proposes its token deterministically; the children
// are tried in index order against the node's target distribution
// p = softmax(logits / T).  With residual r (initially p) a proposal of
// token x is accepted iff u < r(x) = p(x) / (1 - removed mass); on rejection
// x's mass leaves r, so a repeated token is always rejected.  When no child
// is accepted the bonus token is drawn from r by inverse CDF over increasing
// token ids.  The random numbers are inputs (one per child for its test, one
// per node for its bonus draw).
//
// Two modes, by the size of the tree's logits.
//
// Staged mode (at most 384 MiB of logits), three launches whose cost does
// not depend on how deep the walks go:
//  * chunk_stats_kernel, one workgroup per (node row, vocabulary chunk):
//    every row's chunk max and float32-exponential sum.
//  * sample_staged_kernel, one workgroup per (vocabulary chunk, sequence):
//    every workgroup of a sequence stages the chunk statistics of all node
//    rows in LDS, folds them to per-row (max, sum), computes each node's
//    proposal probability and walks the tree on one wave (all of them
//    identically).  Then each sums the float64 masses of its own chunk of
//    the stop node's row, rejected tokens left out.
//  * sample_pick_kernel, one workgroup per sequence, the bonus draw.
//
// Lazy mode (larger trees, or vocabularies whose chunk records exceed the
// staging area) reads only the rows a walk reaches:
//  * sample_root_kernel, one workgroup per (vocabulary chunk, sequence):
//    the root row's chunk max and float64 mass sums over all entries and
//    over those that are not a root child's token.
//  * sample_walk_kernel, one workgroup of 1024 threads per sequence: from
//    the root, the current node's row statistics (max m and sum of
//    2^((l - m) log2(e) / T)), then its children tried in index order on
//    one wave.  At the root the statistics fold the root's records; below
//    it the workgroup reads the row once, one float32 exponential per
//    entry, summed pairwise in float32 within a 16-byte load and in float64
//    across loads (relative error near 1e-6).  A stop at the root rejected
//    every root child, whose tokens the records' residual sums already
//    leave out, so the walk draws the bonus token itself; a stop below it
//    is handed on, with its row max and rejected tokens, to
//  * sample_residual_kernel, one workgroup per (vocabulary chunk,
//    sequence): the float64 masses of its chunk of the stop node's row,
//    rejected tokens left out, and
//  * sample_pick_kernel, the bonus draw.
//
// The bonus draw: a block scan over the chunk masses finds the chunk that
// holds rand_sample * total, a block scan over that chunk's float64 masses
// finds the token.
//
// The bonus token is located among intervals of width p(y), often below
// 1e-5 of the total for large vocabularies, so its masses are float64 end
// to end; the acceptance tests compare a random number with one
// probability, for which the statistics' precision suffices.
//
// Method: "Draft Less, Retrieve More" (aitrends.kr summary), architecture
// paragraph (retrieval nodes are proposals like drafts and verification
// keeps the target distribution) and the paper's abstract (lossless).
#include <hip/hip_bf16.h>

#include <climits>

#include "graft_internal.h"

namespace graft {
namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kLoads = 2;  // 16-byte loads per thread per chunk
constexpr int kStageLoads = kSampleStage / kThreads;
constexpr int kWalkThreads = 1024;  // the lazy walk's workgroup
constexpr int kWalkWaves = kWalkThreads / 64;
constexpr int kRowLoads = 16;  // 16-byte loads per thread per round of a lazy row pass
template <bool BF16>
constexpr int per_load() { return BF16 ? 8 : 4; }
template <bool BF16>
constexpr int vals() { return kLoads * per_load<BF16>(); }
template <bool BF16>
constexpr int chunk_len() { return kThreads * vals<BF16>(); }

// Thread t's values of the L-load chunk starting at lo: element
// lo + (k * kThreads + t) * per_load + j is v[k * per_load + j], so each
// load instruction of a wave reads one contiguous kilobyte; entries at or
// past the vocabulary read as -inf.
template <bool BF16, bool VEC, int L>
__device__ inline void load_strided(const void *logits, size_t row, int vocab, int lo,
                                    float (&v)[L * per_load<BF16>()]) {
  constexpr int kPer = per_load<BF16>();
  const int hi = min(vocab, lo + kThreads * L * kPer);
  if (VEC) {
    // lo and vocab are multiples of the vector width here
    const uint4 *x = reinterpret_cast<const uint4 *>(
        static_cast<const char *>(logits) + row * vocab * (BF16 ? 2 : 4));
    uint4 raw[L];
#pragma unroll
    for (int k = 0; k < L; ++k) {
      const int e = lo + (k * kThreads + (int)threadIdx.x) * kPer;
      // every row is read once here: non-temporal loads stream past the
      // caches (3% off the call at a 316 MB tree of logits)
      if (e < hi) {
        const u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(x) + e / kPer);
        raw[k] = make_uint4(t.x, t.y, t.z, t.w);
      } else {
        raw[k] = make_uint4(0u, 0u, 0u, 0u);
      }
    }
#pragma unroll
    for (int k = 0; k < L; ++k) {
      const bool in = lo + (k * kThreads + (int)threadIdx.x) * kPer < hi;
      const uint32_t w[4] = {raw[k].x, raw[k].y, raw[k].z, raw[k].w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (BF16) {
          v[k * 8 + 2 * q] = in ? __uint_as_float(w[q] << 16) : -INFINITY;
          v[k * 8 + 2 * q + 1] = in ? __uint_as_float(w[q] & 0xffff0000u) : -INFINITY;
        } else {
          v[k * 4 + q] = in ? __uint_as_float(w[q]) : -INFINITY;
        }
      }
    }
  } else {
#pragma unroll
    for (int k = 0; k < L; ++k) {
#pragma unroll
      for (int j = 0; j < kPer; ++j) {
        const int e = lo + (k * kThreads + (int)threadIdx.x) * kPer + j;
        float x = -INFINITY;
        if (e < hi) {
          if (BF16)
            x = __uint_as_float((uint32_t)static_cast<const uint16_t *>(logits)[row * vocab + e]
                                << 16);
          else
            x = static_cast<const float *>(logits)[row * vocab + e];
        }
        v[k * kPer + j] = x;
      }
    }
  }
}

// Thread t's values of the chunk starting at lo, contiguous: element
// lo + t * vals + j is v[j] (two 16-byte loads per thread); entries at or
// past the vocabulary read as -inf.
template <bool BF16, bool VEC>
__device__ inline void load_chunk_contig(const void *logits, size_t row, int vocab, int lo,
                                         float (&v)[vals<BF16>()]) {
  constexpr int kPer = per_load<BF16>();
  constexpr int kV = vals<BF16>();
  const int hi = min(vocab, lo + chunk_len<BF16>());
  const int e0 = lo + (int)threadIdx.x * kV;
  if (VEC) {
    const uint4 *x = reinterpret_cast<const uint4 *>(
        static_cast<const char *>(logits) + row * vocab * (BF16 ? 2 : 4));
    uint4 raw[kLoads];
#pragma unroll
    for (int k = 0; k < kLoads; ++k) {
      const int e = e0 + k * kPer;
      raw[k] = e < hi ? x[e / kPer] : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int k = 0; k < kLoads; ++k) {
      const bool in = e0 + k * kPer < hi;
      const uint32_t w[4] = {raw[k].x, raw[k].y, raw[k].z, raw[k].w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (BF16) {
          v[k * 8 + 2 * q] = in ? __uint_as_float(w[q] << 16) : -INFINITY;
          v[k * 8 + 2 * q + 1] = in ? __uint_as_float(w[q] & 0xffff0000u) : -INFINITY;
        } else {
          v[k * 4 + q] = in ? __uint_as_float(w[q]) : -INFINITY;
        }
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < kV; ++j) {
      const int e = e0 + j;
      float x = -INFINITY;
      if (e < hi) {
        if (BF16)
          x = __uint_as_float((uint32_t)static_cast<const uint16_t *>(logits)[row * vocab + e]
                              << 16);
        else
          x = static_cast<const float *>(logits)[row * vocab + e];
      }
      v[j] = x;
    }
  }
}

// 2^x in float64 for x <= 0, without branches: x = n + f with n = rint(x)
// and |f| <= 1/2, 2^f = e^(f ln 2) by its Taylor series to degree 13
// (truncation below 5e-18 relative), then scaled by 2^n.  Arguments below
// -1100 (and -inf) give 0.
struct Exp2Coeffs {
  double c[14];
  constexpr Exp2Coeffs() : c() {
    const double ln2 = 0.69314718055994530942;
    double t = 1.0;
    for (int i = 0; i < 14; ++i) {
      c[i] = t;
      t = t * ln2 / (i + 1);
    }
  }
};
constexpr Exp2Coeffs kExp2{};
__device__ inline double exp2_nonpos(double x) {
  x = fmax(x, -1100.0);
  const double n = __builtin_rint(x);
  const double f = x - n;
  double p = kExp2.c[13];
#pragma unroll
  for (int i = 12; i >= 0; --i) p = fma(p, f, kExp2.c[i]);
  return __builtin_ldexp(p, (int)n);
}

// Bit j: this thread's contiguous value j of the chunk starting at lo is
// one of the n tokens in gone[].
template <bool BF16>
__device__ inline uint32_t gone_bits_contig(const int32_t *gone, int n, int lo) {
  constexpr int kV = vals<BF16>();
  uint32_t bits = 0;
  for (int g = 0; g < n; ++g) {
    const int off = gone[g] - lo;
    if (off >= 0 && off < chunk_len<BF16>() && off / kV == (int)threadIdx.x)
      bits |= 1u << (off % kV);
  }
  return bits;
}

__device__ inline float logit_at(const void *logits, bool bf16, size_t idx) {
  if (bf16) return __uint_as_float((uint32_t)static_cast<const uint16_t *>(logits)[idx] << 16);
  return static_cast<const float *>(logits)[idx];
}

__device__ inline float wave_max_f(float x) {
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}
__device__ inline double wave_sum_d(double x) {
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

// Block-wide sum in a fixed order; every thread gets the total.
__device__ inline double block_sum_d(double x, double *red) {
  x = wave_sum_d(x);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  double t = 0.0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) t += red[w];
  __syncthreads();
  return t;
}

// Block-wide scan in thread order.  Returns the inclusive prefix; *excl gets
// the exclusive one and *total the block total.  Thread t's exclusive prefix
// is bit-identical to thread t-1's inclusive one and the last thread's
// inclusive prefix to the total, so the intervals [excl, incl) tile
// [0, total) without gaps or overlaps.
template <int W = kWaves>
__device__ inline double block_scan_d(double x, double *red, double *excl, double *total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int o = 1; o < 64; o <<= 1) {
    const double y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  double prev = __shfl_up(x, 1);
  if (lane == 0) prev = 0.0;
  if (lane == 63) red[wave] = x;
  __syncthreads();
  double before = 0.0, t = 0.0;
#pragma unroll
  for (int w = 0; w < W; ++w) {
    if (w < wave) before += red[w];
    t += red[w];
  }
  __syncthreads();
  *total = t;
  *excl = lane == 0 ? before : before + prev;
  return before + x;
}

// float64 mass of a logit of a row whose max is row_max (0 for -inf).
__device__ inline double mass64(float l, float row_max, double k) {
  return exp2_nonpos(((double)l - (double)row_max) * k);
}

// float32 2^(d k) for d <= 0 (-inf included) with the exponent's product
// rounding corrected to first order (k = k_hi + k_lo); relative error near
// 1.2e-7.  Exponents below -160 give 0 (the select also discards the
// non-finite corrections of huge products).
__device__ inline float exp2_split(float d, float k_hi, float k_lo) {
  constexpr float kLn2f = 0.69314718055994531f;
  const float xh = d * k_hi;
  const float xl = fmaf(d, k_hi, -xh) + d * k_lo;
  const float e = __builtin_amdgcn_exp2f(xh);
  const float r = fmaf(e, xl * kLn2f, e);
  return xh > -160.f ? r : 0.f;
}

// ------------------------------------------------------------ the bonus draw
struct PickShared {
  double red[kWalkWaves];
  double tin;
  int cstar, clast, bonus, elast;
};

// The bonus token of sequence b, drawn from the residual of stop node s:
// a block scan over the chunk masses chunk_w[b][*] (w0: thread t's mass of
// chunk t) finds the chunk that holds u * total, a block scan over that
// chunk's float64 masses finds the token, written after the len path
// tokens.  NT threads take part; the first kThreads hold the chunk's
// entries.
template <bool BF16, bool VEC, int NT>
__device__ void bonus_pick(const SampleParams &p, int b, int s, int len, float row_max, float u,
                           const int32_t *s_gone, int ng, double w0, PickShared &sh) {
  constexpr int W = NT / 64;
  constexpr int kVals = vals<BF16>();
  constexpr int kChunk = chunk_len<BF16>();
  const int tid = threadIdx.x;
  const int chunks = p.wchunks;
  const double *w_row = p.chunk_w + (size_t)b * chunks;
  if (tid == 0) {
    sh.cstar = -1;
    sh.clast = -1;
    sh.bonus = -1;
    sh.elast = -1;
  }
  // total residual mass, then the chunk holding the target.  With at most
  // one chunk per thread a single scan gives both; otherwise the same scan
  // runs twice, so that the final carry equals the total bit for bit.  (The
  // scans' barriers order the initialisation above before its uses.)
  double total = 0.0, incl0 = 0.0, ex0 = 0.0;
  for (int c0 = 0; c0 < chunks; c0 += NT) {
    const int c = c0 + tid;
    const double w = c0 == 0 ? w0 : (c < chunks ? w_row[c] : 0.0);
    double ex, gt;
    const double incl = block_scan_d<W>(w, sh.red, &ex, &gt);
    if (c0 == 0) {
      incl0 = incl;
      ex0 = ex;
    }
    total += gt;
  }
  const double target = (double)u * total;
  double carry = 0.0;
  for (int c0 = 0; c0 < chunks; c0 += NT) {
    const int c = c0 + tid;
    const double w = c0 == 0 ? w0 : (c < chunks ? w_row[c] : 0.0);
    double ex = ex0, incl = incl0, gt = total;
    if (chunks > NT) incl = block_scan_d<W>(w, sh.red, &ex, &gt);
    const double lo = carry + ex, hi = carry + incl;
    if (w > 0.0) {
      atomicMax(&sh.clast, c);
      if (target >= lo && target < hi) {
        sh.cstar = c;
        sh.tin = target - lo;
      }
    }
    carry += gt;
  }
  __syncthreads();
  int cstar = sh.cstar;
  double tin = sh.tin;
  if (cstar < 0) {
    // total 0 (every token rejected), or rounding put the target at the top
    cstar = sh.clast;
    tin = cstar >= 0 ? w_row[cstar] : 0.0;
  }
  if (cstar >= 0) {
    // the chunk's float64 masses, each of the first kThreads threads a
    // contiguous run of entries (the loads of the others fall past the
    // chunk and read as -inf)
    const size_t srow = (size_t)b * p.n_max + s;
    const int lo_e = cstar * kChunk;
    float v[kVals];
    load_chunk_contig<BF16, VEC>(p.logits, srow, p.vocab, lo_e, v);
    const uint32_t bits = gone_bits_contig<BF16>(s_gone, ng, lo_e);
    // a row of -inf logits has no mass: compare against -inf as a max of 0
    const float mref = row_max > -INFINITY ? row_max : 0.f;
    double mass[kVals];
    double gs = 0.0;
    int jlast = -1;
#pragma unroll
    for (int k = 0; k < kVals; ++k)
      mass[k] = mass64(v[k], mref, p.k_log2) * (double)(1u - ((bits >> k) & 1u));
#pragma unroll
    for (int k = 0; k < kVals; ++k) {
      gs += mass[k];
      if (mass[k] > 0.0) jlast = k;
    }
    const int e0 = lo_e + tid * kVals;
    if (jlast >= 0) atomicMax(&sh.elast, e0 + jlast);
    double ex, gt;
    const double incl = block_scan_d<W>(gs, sh.red, &ex, &gt);
    if (gs > 0.0 && tin >= ex && tin < incl) {
      double acc = ex;
      int pick = jlast;
#pragma unroll
      for (int k = 0; k < kVals; ++k) {
        acc += mass[k];
        if (acc > tin && mass[k] > 0.0) {
          pick = k;
          break;
        }
      }
      sh.bonus = e0 + pick;
    }
  }
  __syncthreads();
  if (tid == 0) {
    int y = sh.bonus;
    if (y < 0) y = sh.elast >= 0 ? sh.elast : p.vocab - 1;
    p.path_tokens[(size_t)b * (p.n_max + 1) + len] = y;
  }
}

// One workgroup per sequence: the bonus draw from the chunk masses of the
// staged walk, or of the residual launch after a lazy walk that stopped
// below the root.
template <bool BF16, bool VEC>
__global__ __launch_bounds__(kThreads) void sample_pick_kernel(SampleParams p) {
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  __shared__ int32_t s_gone[GRAFT_MAX_NODES];
  __shared__ PickShared sh;
  const SampleRec *rec = p.rec + b;
  const int s = rec->stop;
  if (p.lazy && s == 0) return;  // the lazy walk drew it
  const int len = rec->len, ng = rec->ngone;
  const double w0 = tid < p.wchunks ? p.chunk_w[(size_t)b * p.wchunks + tid] : 0.0;
  if (tid < ng) s_gone[tid] = rec->gone[tid];
  bonus_pick<BF16, VEC, kThreads>(p, b, s, len, rec->row_max, rec->u, s_gone, ng, w0, sh);
}

// ===================================================== staged mode (small trees)
// ------------------------------------------------------------ row statistics
// One workgroup per (vocabulary chunk, node row): the chunk's max and its
// sum of float32 2^((l - m) log2(e) / T), summed pairwise in float32 within
// a load and in float64 across loads.
template <bool BF16, bool VEC, int L>
__global__ __launch_bounds__(kThreads) void chunk_stats_kernel(SampleParams p) {
  constexpr int kPer = per_load<BF16>();
  constexpr int kV = L * kPer;
  const int c = blockIdx.x;
  const int row = blockIdx.y;
  const int b = row / p.n_max, i = row % p.n_max;
  if (i >= max(p.n_nodes[b], 1)) return;  // rows past the tree are not read
  float v[kV];
  __shared__ float red[kWaves];
  __shared__ int ired[kWaves];
  __shared__ double zred[kWaves];
  float m = -INFINITY;
  if constexpr (BF16 && VEC) {
    // bf16 words as loaded: the maximum by packed 16-bit order keys (two
    // values per op, -0 folded onto +0), then the values unpacked for the
    // exponentials; loads past the vocabulary hold -inf pairs
    const int lo = c * kThreads * kV, hi = min(p.vocab, lo + kThreads * kV);
    const u32x4 *x = reinterpret_cast<const u32x4 *>(static_cast<const char *>(p.logits) +
                                                     (size_t)row * p.vocab * 2);
    u32x4 raw[L];
#pragma unroll
    for (int k = 0; k < L; ++k) {
      const int e = lo + (k * kThreads + (int)threadIdx.x) * kPer;
      raw[k] = e < hi ? __builtin_nontemporal_load(x + e / kPer)
                      : (u32x4){0xFF80FF80u, 0xFF80FF80u, 0xFF80FF80u, 0xFF80FF80u};
    }
    short2v acc = (short2v){-32768, -32768};
#pragma unroll
    for (int k = 0; k < L; ++k)
#pragma unroll
      for (int q = 0; q < 4; ++q) acc = __builtin_elementwise_max(acc, okey2(raw[k][q]));
    int km = max((int)acc.x, (int)acc.y);
    for (int o = 32; o > 0; o >>= 1) km = max(km, __shfl_xor(km, o));
    if ((threadIdx.x & 63) == 0) ired[threadIdx.x >> 6] = km;
#pragma unroll
    for (int k = 0; k < L; ++k)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        v[k * 8 + 2 * q] = __uint_as_float(raw[k][q] << 16);
        v[k * 8 + 2 * q + 1] = __uint_as_float(raw[k][q] & 0xffff0000u);
      }
    __syncthreads();
    km = max(max(ired[0], ired[1]), max(ired[2], ired[3]));
    m = __uint_as_float(key_bf16(km) << 16);
  } else {
    load_strided<BF16, VEC, L>(p.logits, (size_t)row, p.vocab, c * kThreads * kV, v);
#pragma unroll
    for (int k = 0; k < kV; ++k) m = fmaxf(m, v[k]);
    m = wave_max_f(m);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  }
  // each load's values summed pairwise in float32 (three roundings at
  // most), the loads' sums in float64
  double z = 0.0;
#pragma unroll
  for (int k = 0; k < L; ++k) {
    float e[kPer];
#pragma unroll
    for (int j = 0; j < kPer; ++j) e[j] = __builtin_amdgcn_exp2f((v[k * kPer + j] - m) * p.k_hi);
#pragma unroll
    for (int w = kPer / 2; w > 0; w >>= 1)
#pragma unroll
      for (int j = 0; j < w; ++j) e[j] += e[j + w];
    z += (double)e[0];
  }
  z = wave_sum_d(z);
  if ((threadIdx.x & 63) == 0) zred[threadIdx.x >> 6] = z;
  __syncthreads();
  if (threadIdx.x == 0) {
    ChunkStat st;
    st.m = m;
    st.pad = 0.f;
    st.z = m > -INFINITY ? ((zred[0] + zred[1]) + zred[2]) + zred[3] : 0.0;
    p.stats[(size_t)row * p.chunks + c] = st;
  }
}

// ------------------------------------------------------- the staged walk
// One workgroup per (vocabulary chunk, sequence).  Every workgroup of a
// sequence stages the chunk statistics of all node rows in LDS, folds them
// to per-row (max, sum), computes each node's proposal probability
// p_parent(token) and walks the tree on one wave (all of them
// identically).  Then each sums the float64 masses of its own chunk of the
// stop node's row, rejected tokens left out; the first writes the accepted
// path and the hand-over record of the pick launch.
template <bool BF16, bool VEC>
__global__ __launch_bounds__(kThreads) void sample_staged_kernel(SampleParams p) {
  constexpr int kVals = vals<BF16>();
  constexpr int kChunk = chunk_len<BF16>();
  const int c_own = blockIdx.x;  // this workgroup's chunk of the stop row
  const int b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  __shared__ ChunkStat s_stage[kSampleStage];
  __shared__ float s_m[GRAFT_MAX_NODES];      // row max
  __shared__ double s_z[GRAFT_MAX_NODES];     // row sum of 2^((l - max) k)
  __shared__ int32_t s_parent[GRAFT_MAX_NODES];
  __shared__ int32_t s_token[GRAFT_MAX_NODES];
  __shared__ double s_prob[GRAFT_MAX_NODES];  // p_parent(token) of each node
  __shared__ float s_u[GRAFT_MAX_NODES];
  __shared__ int32_t s_path[GRAFT_MAX_NODES];
  __shared__ int32_t s_gone[GRAFT_MAX_NODES];  // tokens rejected at the stop node
  __shared__ double s_red[kWaves];
  __shared__ int s_len, s_ngone, s_stop;

  const size_t base_row = (size_t)b * p.n_max;
  // ---- tree arrays, random numbers and node count (one round of loads)
  const int nn = p.n_nodes[b];
  int par = -1, tok = -1;
  float u = 0.f;
  if (tid < p.n_max) {
    par = p.tree_parent[base_row + tid];
    tok = p.tree_token[base_row + tid];
    u = p.rand_accept[base_row + tid];
  }
  const int n = min(max(nn, 1), p.n_max);
  if (tid >= n) par = tok = -1;
  if (par >= tid) par = -1;
  if (tid < p.n_max) {
    s_parent[tid] = par;
    s_token[tid] = tok;
    s_u[tid] = u;
    s_prob[tid] = 0.0;
  }
  // ---- the proposal's logit under its parent's row (issued before the
  // statistics are staged)
  const bool has_logit = tid > 0 && par >= 0 && tok >= 0 && tok < p.vocab;
  const float l_prop =
      has_logit ? logit_at(p.logits, BF16, (base_row + par) * p.vocab + tok) : 0.f;

  // ---- fold the chunk statistics of every row: stage a group of rows in
  // LDS with all loads issued at once, then Q threads per row
  const int chunks = p.chunks;
  const int rows_per_group = max(1, kSampleStage / chunks);
  for (int r0 = 0; r0 < n; r0 += rows_per_group) {
    const int R = min(rows_per_group, n - r0);
    const int ents = R * chunks;
    const uint4 *src = reinterpret_cast<const uint4 *>(p.stats + (base_row + r0) * chunks);
    uint4 tmp[kStageLoads];
#pragma unroll
    for (int k = 0; k < kStageLoads; ++k) {
      const int e = k * kThreads + tid;
      tmp[k] = e < ents ? src[e] : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int k = 0; k < kStageLoads; ++k) {
      const int e = k * kThreads + tid;
      if (e < ents) reinterpret_cast<uint4 *>(s_stage)[e] = tmp[k];
    }
    __syncthreads();
    int Q = 1;
    while (Q < 64 && Q * 2 * R <= kThreads) Q *= 2;
    const int ri = tid / Q, q = tid % Q;
    float m = -INFINITY;
    if (ri < R)
      for (int c = q; c < chunks; c += Q) {
        const ChunkStat st = s_stage[ri * chunks + c];
        if (st.z > 0.0) m = fmaxf(m, st.m);
      }
    for (int o = 1; o < Q; o <<= 1) m = fmaxf(m, __shfl_xor(m, o));
    double z = 0.0;
    if (ri < R && m > -INFINITY)
      for (int c = q; c < chunks; c += Q) {
        const ChunkStat st = s_stage[ri * chunks + c];
        z = fma(st.z, (double)exp2_split(st.m - m, p.k_hi, p.k_lo), z);
      }
    for (int o = 1; o < Q; o <<= 1) z += __shfl_xor(z, o);
    if (ri < R && q == 0) {
      s_m[r0 + ri] = m;
      s_z[r0 + ri] = z;
    }
    __syncthreads();  // the next group overwrites the staging area
  }
  // ---- proposal probability of every node under its parent's distribution
  if (has_logit && s_z[par] > 0.0) s_prob[tid] = mass64(l_prop, s_m[par], p.k_log2) / s_z[par];
  __syncthreads();

  // ---- the walk (wave 0): children of the current node in index order
  if (wave == 0) {
    int node = 0, len = 1, ngone = 0;
    int gone_lo = INT_MIN, gone_hi = INT_MIN;  // lane g holds rejected token g / g + 64
    while (true) {
      double removed = 0.0;
      ngone = 0;
      gone_lo = gone_hi = INT_MIN;
      int next = -1;
      for (int base = node + 1; base < n && next < 0; base += 64) {
        const int c = base + lane;
        unsigned long long bal = __ballot(c < n && s_parent[c] == node);
        while (bal) {
          const int cc = base + __builtin_ctzll(bal);  // uniform
          bal &= bal - 1;
          const int x = s_token[cc];
          if (__ballot(gone_lo == x || gone_hi == x)) continue;  // mass already gone
          // u < p(x) / (1 - removed), without the division
          if ((double)s_u[cc] * (1.0 - removed) < s_prob[cc]) {
            next = cc;
            break;
          }
          if (ngone < 64) {
            if (lane == ngone) gone_lo = x;
          } else if (lane == ngone - 64) {
            gone_hi = x;
          }
          ++ngone;
          removed += s_prob[cc];
        }
      }
      if (next < 0) break;
      node = next;
      if (lane == 0) s_path[len] = node;
      ++len;
    }
    if (lane == 0) {
      s_path[0] = 0;
      s_len = len;
      s_ngone = ngone;
      s_stop = node;
    }
    if (lane < ngone) s_gone[lane] = gone_lo;
    if (lane + 64 < ngone) s_gone[lane + 64] = gone_hi;
  }
  __syncthreads();

  // ---- this workgroup's chunk of the stop row: float64 residual mass
  const int s = s_stop, ng = s_ngone, len = s_len;
  const size_t srow = base_row + s;
  const float row_max = s_m[s];
  {
    float v[kVals];
    load_chunk_contig<BF16, VEC>(p.logits, srow, p.vocab, c_own * kChunk, v);
    const uint32_t bits = gone_bits_contig<BF16>(s_gone, ng, c_own * kChunk);
    const float mref = row_max > -INFINITY ? row_max : 0.f;  // -inf row: no mass
    double mk[kVals];
#pragma unroll
    for (int k = 0; k < kVals; ++k)
      mk[k] = mass64(v[k], mref, p.k_log2) * (double)(1u - ((bits >> k) & 1u));
    double part = 0.0;
#pragma unroll
    for (int k = 0; k < kVals; ++k) part += mk[k];
    const double tot = block_sum_d(part, s_red);
    if (tid == 0) p.chunk_w[(size_t)b * p.wchunks + c_own] = tot;
  }
  if (c_own != 0) return;

  // ---- the accepted path (the bonus token is written by the pick kernel)
  int32_t *pn = p.path_nodes + base_row;
  int32_t *pt = p.path_tokens + (size_t)b * (p.n_max + 1);
  for (int k = tid; k < p.n_max + 1; k += kThreads) {
    if (k < p.n_max) pn[k] = k < len ? s_path[k] : -1;
    if (k != len) pt[k] = k < len ? s_token[s_path[k]] : -1;
  }
  SampleRec *rec = p.rec + b;
  if (tid < ng) rec->gone[tid] = s_gone[tid];
  if (tid == 0) {
    p.accept_len[b] = len - 1;
    rec->stop = s;
    rec->len = len;
    rec->ngone = ng;
    rec->row_max = row_max;
    rec->u = p.rand_sample[srow];
  }
}

// ====================================================== lazy mode (large trees)
// Lane l's double (l wave-uniform).
__device__ inline double readlane_d(double v, int l) {
  const unsigned long long u = (unsigned long long)__double_as_longlong(v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, l);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), l);
  return __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
}

template <int W>
__device__ inline float block_max_f(float x, float *red) {
  x = wave_max_f(x);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  float t = red[0];
#pragma unroll
  for (int w = 1; w < W; ++w) t = fmaxf(t, red[w]);
  __syncthreads();
  return t;
}
template <int W>
__device__ inline double block_sum_w(double x, double *red) {
  x = wave_sum_d(x);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  double t = 0.0;
#pragma unroll
  for (int w = 0; w < W; ++w) t += red[w];
  __syncthreads();
  return t;
}

// ------------------------------------------------------------ the root row
// One workgroup per (vocabulary chunk, sequence): the chunk's max and
// float64 mass sums of the root's row relative to that max, over all
// entries (for the root's acceptance tests) and over the entries that are
// not a token of the root's children.  A walk that stops at the root has
// tried and rejected every child, so the second sum is its residual mass
// there, and no later launch reads the root row in full again.
template <bool BF16, bool VEC>
__global__ __launch_bounds__(kThreads) void sample_root_kernel(SampleParams p) {
  constexpr int kVals = vals<BF16>();
  constexpr int kChunk = chunk_len<BF16>();
  constexpr int node = 0;
  const int c_own = blockIdx.x;
  const int b = blockIdx.y;
  const int tid = threadIdx.x;
  __shared__ int32_t s_gone[GRAFT_MAX_NODES];
  __shared__ int s_ng;
  __shared__ float s_redf[kWaves];
  __shared__ double s_redz[kWaves], s_redr[kWaves];
  const size_t base_row = (size_t)b * p.n_max;
  const int n = min(max(p.n_nodes[b], 1), p.n_max);
  // the root's children: later nodes whose parent it is
  int tok = 0;
  const bool child = tid > node && tid < n && p.tree_parent[base_row + tid] == node;
  if (child) tok = p.tree_token[base_row + tid];
  float v[kVals];
  load_chunk_contig<BF16, VEC>(p.logits, base_row + node, p.vocab, c_own * kChunk, v);
  if (tid == 0) s_ng = 0;
  __syncthreads();
  if (child) s_gone[atomicAdd(&s_ng, 1)] = tok;
  float mt = -INFINITY;
#pragma unroll
  for (int k = 0; k < kVals; ++k) mt = fmaxf(mt, v[k]);
  const float mc = block_max_f<kWaves>(mt, s_redf);  // its barriers publish s_gone
  const uint32_t bits = gone_bits_contig<BF16>(s_gone, s_ng, c_own * kChunk);
  const float mref = mc > -INFINITY ? mc : 0.f;  // -inf chunk: no mass
  double zt = 0.0, rt = 0.0;
#pragma unroll
  for (int k = 0; k < kVals; ++k) {
    const double mk = mass64(v[k], mref, p.k_log2);
    zt += mk;
    rt += mk * (double)(1u - ((bits >> k) & 1u));
  }
  zt = wave_sum_d(zt);
  rt = wave_sum_d(rt);
  if ((tid & 63) == 0) {
    s_redz[tid >> 6] = zt;
    s_redr[tid >> 6] = rt;
  }
  __syncthreads();
  if (tid == 0) {
    double z = 0.0, r = 0.0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      z += s_redz[w];
      r += s_redr[w];
    }
    RootChunk out;
    out.z = z;
    out.r = r;
    out.m = mc;
    out.pad[0] = out.pad[1] = out.pad[2] = 0;
    p.root[(size_t)b * p.wchunks + c_own] = out;
  }
}

// ------------------------------------------------------------------ the walk

// The values of one 16-byte load (8 bf16 or 4 float32).
template <bool BF16>
__device__ inline void unpack(const uint4 &r, float (&v)[per_load<BF16>()]) {
  const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    if (BF16) {
      v[2 * q] = __uint_as_float(w[q] << 16);
      v[2 * q + 1] = __uint_as_float(w[q] & 0xffff0000u);
    } else {
      v[q] = __uint_as_float(w[q]);
    }
  }
}
// Sum of 2^((l - m) k) over one load's values: float32 exponentials summed
// pairwise in float32.
template <bool BF16>
__device__ inline float load_sum(const float (&v)[per_load<BF16>()], float m, float k_hi) {
  constexpr int kPer = per_load<BF16>();
  float e[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) e[j] = __builtin_amdgcn_exp2f((v[j] - m) * k_hi);
#pragma unroll
  for (int w = kPer / 2; w > 0; w >>= 1)
#pragma unroll
    for (int j = 0; j < w; ++j) e[j] += e[j + w];
  return e[0];
}

// Statistics of one node row by the whole workgroup: its max m and
// z = sum of 2^((l - m) log2(e) / T), with one read of the row.  Each thread
// keeps a running max and a sum relative to it over its rounds of loads:
// float32 exponentials summed pairwise in float32 within a 16-byte load and
// in float64 across loads, the sum moved to a new max by a float32 power of
// two with its product rounding corrected (exp2_split).  The workgroup then
// folds the threads' sums onto the row max the same way (relative error of
// z near 1e-6).
template <bool BF16, bool VEC>
__device__ void row_stats(const SampleParams &p, size_t row, float *redf, double *redd,
                          float &m_out, double &z_out) {
  constexpr int kPer = per_load<BF16>();
  const int tid = threadIdx.x;
  const int V = p.vocab;
  float m = -INFINITY;
  double z = 0.0;
  // fold a round's max into the running one, rescaling the sum
  auto raise = [&](float mr) {
    if (mr > m) {
      if (m > -INFINITY) z *= (double)exp2_split(m - mr, p.k_hi, p.k_lo);
      m = mr;
    }
  };
  if (VEC) {
    const uint4 *x = reinterpret_cast<const uint4 *>(static_cast<const char *>(p.logits) +
                                                     row * V * (BF16 ? 2 : 4));
    const int nvec = V / kPer;
    for (int r0 = 0; r0 < nvec; r0 += kWalkThreads * kRowLoads) {
      uint4 raw[kRowLoads];
#pragma unroll
      for (int k = 0; k < kRowLoads; ++k) {
        const int e = r0 + k * kWalkThreads + tid;
        raw[k] = e < nvec ? x[e] : make_uint4(0u, 0u, 0u, 0u);
      }
      float mr = -INFINITY;
#pragma unroll
      for (int k = 0; k < kRowLoads; ++k) {
        if (r0 + k * kWalkThreads + tid < nvec) {
          float v[kPer];
          unpack<BF16>(raw[k], v);
#pragma unroll
          for (int j = 0; j < kPer; ++j) mr = fmaxf(mr, v[j]);
        }
      }
      raise(mr);
      if (m > -INFINITY) {
#pragma unroll
        for (int k = 0; k < kRowLoads; ++k) {
          if (r0 + k * kWalkThreads + tid < nvec) {
            float v[kPer];
            unpack<BF16>(raw[k], v);
            z += (double)load_sum<BF16>(v, m, p.k_hi);
          }
        }
      }
    }
  } else {
    // rows whose length is not a multiple of the vector width: one entry
    // at a time, each its own round
    const size_t base = row * V;
    for (int e = tid; e < V; e += kWalkThreads) {
      const float l = logit_at(p.logits, BF16, base + e);
      raise(l);
      if (m > -INFINITY) z += (double)__builtin_amdgcn_exp2f((l - m) * p.k_hi);
    }
  }
  const float M = block_max_f<kWalkWaves>(m, redf);
  const double zt = m > -INFINITY ? z * (double)exp2_split(m - M, p.k_hi, p.k_lo) : 0.0;
  z_out = block_sum_w<kWalkWaves>(zt, redd);
  m_out = M;
}

// One workgroup per sequence walks its tree from the root.  Up front it
// loads the tree, each node's logit of its own token in its parent's row
// and the root's chunk records, which wave 0 folds into the root row's max
// and sum.  At each node it takes the node's row statistics (folded at the
// root, else one read of the row: only the rows the walk reaches are read)
// and tries the node's children in index order on wave 0; an accepted
// child becomes the current node.  At a root stop it also draws the bonus
// token; below the root it hands the stop node, its row max and rejected
// tokens to the residual and pick launches.
template <bool BF16, bool VEC>
__global__ __launch_bounds__(kWalkThreads) void sample_walk_kernel(SampleParams p) {
  const int b = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  __shared__ int32_t s_parent[GRAFT_MAX_NODES];
  __shared__ int32_t s_token[GRAFT_MAX_NODES];
  __shared__ float s_u[GRAFT_MAX_NODES];
  __shared__ float s_lc[GRAFT_MAX_NODES];  // node c's token's logit in its parent's row
  __shared__ int32_t s_path[GRAFT_MAX_NODES];
  __shared__ int32_t s_gone[GRAFT_MAX_NODES];  // tokens rejected at the stop node
  __shared__ float s_redf[kWalkWaves];
  __shared__ PickShared sh;
  __shared__ int s_next, s_ngone;
  __shared__ float s_root_m;
  __shared__ double s_root_z;

  const size_t base_row = (size_t)b * p.n_max;
  const int W = p.wchunks;
  const RootChunk *rc = p.root + (size_t)b * W;
  // ---- tree arrays and random numbers (one round of loads)
  const int n = min(max(p.n_nodes[b], 1), p.n_max);
  if (tid < p.n_max) {
    int par = p.tree_parent[base_row + tid];
    int tok = p.tree_token[base_row + tid];
    if (tid >= n) par = tok = -1;
    if (par >= tid) par = -1;
    s_parent[tid] = par;
    s_token[tid] = tok;
    s_u[tid] = p.rand_accept[base_row + tid];
  }
  __syncthreads();
  // ---- the candidates' logits and the root's statistics (one round)
  if (tid < n) {
    const int par = s_parent[tid], x = s_token[tid];
    s_lc[tid] = par >= 0 && x >= 0 && x < p.vocab
                    ? logit_at(p.logits, BF16, (base_row + par) * p.vocab + x)
                    : -INFINITY;  // no mass: never accepted
  }
  if (wave == 0) {
    // the row max, then the chunk sums moved onto it by float64 powers of two
    RootChunk r0;
    r0.m = -INFINITY;
    r0.z = 0.0;
    if (lane < W) r0 = rc[lane];
    float mt = r0.m;
    for (int c = lane + 64; c < W; c += 64) mt = fmaxf(mt, rc[c].m);
    const float M = wave_max_f(mt);
    double zt = r0.m > -INFINITY ? r0.z * mass64(r0.m, M, p.k_log2) : 0.0;
    for (int c = lane + 64; c < W; c += 64) {
      const RootChunk rk = rc[c];
      if (rk.m > -INFINITY) zt += rk.z * mass64(rk.m, M, p.k_log2);
    }
    zt = wave_sum_d(zt);
    if (lane == 0) {
      s_root_m = M;
      s_root_z = zt;
    }
  }
  __syncthreads();

  int node = 0, len = 1;
  float m = -INFINITY;
  while (true) {
    double z;
    if (node == 0) {
      m = s_root_m;
      z = s_root_z;
    } else {
      row_stats<BF16, VEC>(p, base_row + node, s_redf, sh.red, m, z);
    }
    if (wave == 0) {
      // children of the node in index order: each lane holds the
      // probability of the child in its slot of a 64-node block
      double removed = 0.0;
      int ngone = 0, next = -1;
      int gone_lo = INT_MIN, gone_hi = INT_MIN;  // lane g holds rejected token g / g + 64
      for (int base = node + 1; base < n && next < 0; base += 64) {
        const int c = base + lane;
        const bool child = c < n && s_parent[c] == node;
        const double prob = child && z > 0.0 ? mass64(s_lc[c], m, p.k_log2) / z : 0.0;
        unsigned long long bal = __ballot(child);
        while (bal) {
          const int slot = __builtin_ctzll(bal);  // uniform
          const int cc = base + slot;
          bal &= bal - 1;
          const int x = s_token[cc];
          if (__ballot(gone_lo == x || gone_hi == x)) continue;  // mass already gone
          const double pc = readlane_d(prob, slot);
          // u < p(x) / (1 - removed), without the division
          if ((double)s_u[cc] * (1.0 - removed) < pc) {
            next = cc;
            break;
          }
          if (ngone < 64) {
            if (lane == ngone) gone_lo = x;
          } else if (lane == ngone - 64) {
            gone_hi = x;
          }
          ++ngone;
          removed += pc;
        }
      }
      if (lane == 0) {
        s_next = next;
        s_ngone = ngone;
      }
      if (next < 0) {
        if (lane < ngone) s_gone[lane] = gone_lo;
        if (lane + 64 < ngone) s_gone[lane + 64] = gone_hi;
      }
    }
    __syncthreads();
    const int next = s_next;
    if (next < 0) break;
    if (tid == 0) s_path[len] = next;
    node = next;
    ++len;
    __syncthreads();  // s_next is read before the next node overwrites it
  }

  // ---- the accepted path (the bonus token is written by the bonus draw)
  if (tid == 0) s_path[0] = 0;
  __syncthreads();
  const int ng = s_ngone;
  int32_t *pn = p.path_nodes + base_row;
  int32_t *pt = p.path_tokens + (size_t)b * (p.n_max + 1);
  for (int k = tid; k < p.n_max + 1; k += kWalkThreads) {
    if (k < p.n_max) pn[k] = k < len ? s_path[k] : -1;
    if (k != len) pt[k] = k < len ? s_token[s_path[k]] : -1;
  }
  SampleRec *rec = p.rec + b;
  const float u = p.rand_sample[base_row + node];
  if (tid == 0) {
    p.accept_len[b] = len - 1;
    rec->stop = node;
  }
  if (node == 0) {
    // every root child was rejected, so the records' residual sums are the
    // residual's chunk masses, to be moved onto the row max
    double *cw = p.chunk_w + (size_t)b * W;
    double w0 = 0.0;
    for (int c = tid; c < W; c += kWalkThreads) {
      const RootChunk rk = rc[c];
      const double w = rk.m > -INFINITY ? rk.r * mass64(rk.m, m, p.k_log2) : 0.0;
      cw[c] = w;
      if (c == tid) w0 = w;
    }
    __syncthreads();  // chunk_w is read back by other threads
    bonus_pick<BF16, VEC, kWalkThreads>(p, b, node, len, m, u, s_gone, ng, w0, sh);
  } else {
    if (tid < ng) rec->gone[tid] = s_gone[tid];
    if (tid == 0) {
      rec->len = len;
      rec->ngone = ng;
      rec->row_max = m;
      rec->u = u;
    }
  }
}

// ------------------------------------------- the stop row's residual masses
// One workgroup per (vocabulary chunk, sequence): the chunk's float64
// residual mass of the stop node's row, rejected tokens left out, after a
// lazy walk that stopped below the root.
template <bool BF16, bool VEC>
__global__ __launch_bounds__(kThreads) void sample_residual_kernel(SampleParams p) {
  constexpr int kVals = vals<BF16>();
  constexpr int kChunk = chunk_len<BF16>();
  const int c_own = blockIdx.x;
  const int b = blockIdx.y;
  const int tid = threadIdx.x;
  __shared__ int32_t s_gone[GRAFT_MAX_NODES];
  __shared__ double s_red[kWaves];
  const SampleRec *rec = p.rec + b;
  const int s = rec->stop, ng = rec->ngone;
  if (s == 0) return;  // the root: the walk drew the bonus token
  const float row_max = rec->row_max;
  if (tid < ng) s_gone[tid] = rec->gone[tid];
  const size_t srow = (size_t)b * p.n_max + s;
  float v[kVals];
  load_chunk_contig<BF16, VEC>(p.logits, srow, p.vocab, c_own * kChunk, v);
  __syncthreads();
  const uint32_t bits = gone_bits_contig<BF16>(s_gone, ng, c_own * kChunk);
  const float mref = row_max > -INFINITY ? row_max : 0.f;  // -inf row: no mass
  double mk[kVals];
#pragma unroll
  for (int k = 0; k < kVals; ++k)
    mk[k] = mass64(v[k], mref, p.k_log2) * (double)(1u - ((bits >> k) & 1u));
  double part = 0.0;
#pragma unroll
  for (int k = 0; k < kVals; ++k) part += mk[k];
  const double tot = block_sum_d(part, s_red);
  if (tid == 0) p.chunk_w[(size_t)b * p.wchunks + c_own] = tot;
}

// 16-byte loads per thread of a staged-mode statistics chunk: 2 (4096 bf16
// / 2048 f32 entries) while the grid is small, 8 once it would exceed 8192
// workgroups, where fewer and larger workgroups stream faster.
constexpr int kStatSmall = 2, kStatLarge = 8, kStatLargeGrid = 8192;
int stat_loads(graft_dtype dtype, int32_t rows, int32_t vocab) {
  const long long small = (vocab + (long long)kThreads * kStatSmall * (dtype == GRAFT_BF16 ? 8 : 4) - 1) /
                          ((long long)kThreads * kStatSmall * (dtype == GRAFT_BF16 ? 8 : 4));
  return (long long)rows * small > kStatLargeGrid ? kStatLarge : kStatSmall;
}

template <bool BF16, bool VEC>
void launch(const SampleParams &p, hipStream_t stream) {
  if (!p.lazy) {
    if (p.stat_loads == kStatLarge)
      hipLaunchKernelGGL((chunk_stats_kernel<BF16, VEC, kStatLarge>),
                         dim3(p.chunks, p.batch * p.n_max), dim3(kThreads), 0, stream, p);
    else
      hipLaunchKernelGGL((chunk_stats_kernel<BF16, VEC, kStatSmall>),
                         dim3(p.chunks, p.batch * p.n_max), dim3(kThreads), 0, stream, p);
    hipLaunchKernelGGL((sample_staged_kernel<BF16, VEC>), dim3(p.wchunks, p.batch),
                       dim3(kThreads), 0, stream, p);
    hipLaunchKernelGGL((sample_pick_kernel<BF16, VEC>), dim3(p.batch), dim3(kThreads), 0,
                       stream, p);
    return;
  }
  hipLaunchKernelGGL((sample_root_kernel<BF16, VEC>), dim3(p.wchunks, p.batch), dim3(kThreads),
                     0, stream, p);
  hipLaunchKernelGGL((sample_walk_kernel<BF16, VEC>), dim3(p.batch), dim3(kWalkThreads), 0, stream,
                     p);
  if (p.n_max > 1) {
    // stops below the root
    hipLaunchKernelGGL((sample_residual_kernel<BF16, VEC>), dim3(p.wchunks, p.batch),
                       dim3(kThreads), 0, stream, p);
    hipLaunchKernelGGL((sample_pick_kernel<BF16, VEC>), dim3(p.batch), dim3(kThreads), 0,
                       stream, p);
  }
}

}  // namespace

int32_t sample_stat_loads(graft_dtype dtype, int32_t rows, int32_t vocab) {
  return stat_loads(dtype, rows, vocab);
}

int32_t sample_stat_chunks(graft_dtype dtype, int32_t loads, int32_t vocab) {
  const long long len = (long long)kThreads * loads * (dtype == GRAFT_BF16 ? 8 : 4);
  return (int32_t)((vocab + len - 1) / len);
}

// Staged mode reads every row of the tree once, wide, so its cost follows
// the tree's logits and not the walk's depth.  Lazy mode reads the root row
// wide and each deeper row a walk reaches on one compute unit (about 8 us
// for 150K entries, arithmetic-bound), so its cost follows the deepest walk
// of the batch.  Staged while the tree's logits take at most 384 MiB (about
// 70 us of reading: the deepest walk would have to stop within seven or
// eight levels for lazy mode to win) and a row's chunk records fit one
// workgroup's staging area; lazy beyond either.
constexpr size_t kStagedBytes = size_t{384} << 20;

bool sample_lazy(graft_dtype dtype, int32_t batch, int32_t n_max, int32_t vocab) {
  const size_t e = dtype == GRAFT_BF16 ? 2 : 4;
  const size_t bytes = (size_t)batch * n_max * vocab * e;
  return bytes > kStagedBytes || sample_stat_chunks(dtype, kStatSmall, vocab) > kSampleStage;
}

int32_t sample_walk_chunks(graft_dtype dtype, int32_t vocab) {
  const int len = dtype == GRAFT_BF16 ? chunk_len<true>() : chunk_len<false>();
  return (vocab + len - 1) / len;
}

void launch_accept_sample(graft_dtype dtype, const SampleParams &p, hipStream_t stream) {
  if (dtype == GRAFT_BF16) {
    if (p.vocab % 8 == 0) launch<true, true>(p, stream);
    else launch<true, false>(p, stream);
  } else {
    if (p.vocab % 4 == 0) launch<false, true>(p, stream);
    else launch<false, false>(p, stream);
  }
}

}  // namespace graft
