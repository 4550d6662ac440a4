// KVQuant-style non-uniform quantization (NUQ) with dense-and-sparse outliers
// and attention-sink tokens.
//
// ["veloxquant_mlx.cache.kvquant_cache module", module docstring: quantization
//  axes, level lifecycle, performance, byte accounting, attention-sink
//  quantization; KVQuantKVCache property docs] keys get one level table per
// channel (samples = tokens), values one per token (samples = channels); key
// levels and |key| thresholds are fit at prefill and frozen, value levels are
// fit on every call; the first n_sink tokens of a sequence stay exact and are
// excluded from every fit; a nominal fraction of |x|-largest samples per
// vector is kept exact in a side channel; levels are fit by Lloyd-Max
// iterations (unweighted 1-D k-means).
//
// Readings fixed here (the pages leave them open): k = floor(frac*n)
// outliers at most, threshold tau = (k+1)-th largest |x|, outlier iff
// |x| > tau; quantile initialisation at probabilities (j+1/2)/L with linear
// interpolation; nearest level with ties to the lower index; empty cells keep
// their level; levels are binary32 roundings of exact cell means; the table
// is kept in ascending order after every update (an ordered signpost table).
//
// GPU formulation. A vector of n samples is split over CPC lanes, 128
// samples per lane. Each lane sorts its chunk in registers (a bitonic network
// on packed 16-bit order keys, all compare-exchanges ascending) and keeps it
// in LDS. Everything the fit needs then comes from binary searches in those
// sorted chunks plus sums over CPC lanes:
//   - tau: binary search on |x| for the largest c with #{|x| >= c} >= k+1;
//   - the inliers of a chunk are a contiguous index range [lo, hi);
//   - quantile order statistics: binary search over fp16 order keys;
//   - a Lloyd iteration: the nearest-level cells are contiguous index ranges
//     cut at exact fp16 thresholds T_j (largest fp16 t with 2t <= l_j +
//     l_{j+1}); cell sums are kept as prefix sums P_j at the cut points and
//     updated by walking the cut from its old to its new position. Sums are
//     doubles, exact while |sum| < 2^29 (fp16 values are multiples of 2^-24),
//     so each level is the exact mean rounded once to binary32.
// Codes are then #{j : x > T_j}, which equals the first index of the nearest
// level. The side channel (flat index, fp16 value) is emitted in ascending
// flat order: each block reserves a staging range with one atomic, an
// ordered scan of the block counts places the blocks, a copy kernel moves the
// entries (no inter-block waiting).
#include "common.h"
#include "kernels.h"

namespace kvq {
namespace {

constexpr int CH = 128;             // samples per lane chunk

typedef short s16x2 __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2v __attribute__((ext_vector_type(2)));

// ----------------------------------------------------------------- keys
__device__ __forceinline__ uint32_t key16(uint32_t h) {  // order-preserving key of an fp16 pattern
  return (h & 0x8000u) ? (~h & 0xffffu) : (h | 0x8000u);
}
__device__ __forceinline__ uint32_t unkey16(uint32_t k) {
  return (k & 0x8000u) ? (k & 0x7fffu) : (~k & 0xffffu);
}
// both halves of a packed pair of fp16 patterns -> keys
__device__ __forceinline__ uint32_t key_pair(uint32_t w) {
  const s16x2 s = __builtin_bit_cast(s16x2, w) >> (short)15;  // 0xffff where negative
  return w ^ 0x80008000u ^ (__builtin_bit_cast(uint32_t, s) & 0x7fff7fffu);
}
__device__ __forceinline__ double kval(uint32_t k) { return (double)h2f((uint16_t)unkey16(k)); }

// ----------------------------------------------------------------- sorting
__device__ __forceinline__ void ce(uint32_t &a, uint32_t &b) {
  const u16x2v x = __builtin_bit_cast(u16x2v, a), y = __builtin_bit_cast(u16x2v, b);
  a = __builtin_bit_cast(uint32_t, __builtin_elementwise_min(x, y));
  b = __builtin_bit_cast(uint32_t, __builtin_elementwise_max(x, y));
}
// element i of the chunk lives in register i % 64, half i / 64
template <int K>
__device__ __forceinline__ void flip(uint32_t *v) {
#pragma unroll
  for (int r = 0; r < 64; ++r) {
    const int p = r ^ (K - 1);
    if (p > r) ce(v[r], v[p]);
  }
}
template <int J>
__device__ __forceinline__ void disperse(uint32_t *v) {
#pragma unroll
  for (int r = 0; r < 64; ++r) {
    const int p = r ^ J;
    if (p > r) ce(v[r], v[p]);
  }
}
template <int K>
__device__ __forceinline__ void merge(uint32_t *v) {
  flip<K>(v);
  if constexpr (K / 4 >= 32) disperse<32>(v);
  if constexpr (K / 4 >= 16) disperse<16>(v);
  if constexpr (K / 4 >= 8) disperse<8>(v);
  if constexpr (K / 4 >= 4) disperse<4>(v);
  if constexpr (K / 4 >= 2) disperse<2>(v);
  if constexpr (K / 4 >= 1) disperse<1>(v);
}
// the K = 128 flip pairs element r with 127 - r: low half of register r with
// the high half of register 63 - r, and vice versa
__device__ __forceinline__ void flip128(uint32_t *v) {
#pragma unroll
  for (int r = 0; r < 32; ++r) {
    const int p = 63 - r;
    const u16x2v a = __builtin_bit_cast(u16x2v, v[r]);
    const u16x2v b = __builtin_bit_cast(u16x2v, v[p]);
    const u16x2v bs = {b.y, b.x};
    const u16x2v mn = __builtin_elementwise_min(a, bs), mx = __builtin_elementwise_max(a, bs);
    v[r] = (uint32_t)mn.x | ((uint32_t)mx.y << 16);
    v[p] = (uint32_t)mn.y | ((uint32_t)mx.x << 16);
  }
}
__device__ __forceinline__ void sort128(uint32_t *v) {
  merge<2>(v);
  merge<4>(v);
  merge<8>(v);
  merge<16>(v);
  merge<32>(v);
  merge<64>(v);
  flip128(v);
  disperse<32>(v);
  disperse<16>(v);
  disperse<8>(v);
  disperse<4>(v);
  disperse<2>(v);
  disperse<1>(v);
}

// ----------------------------------------------------------------- sorted chunk in LDS
// 64 words per lane; word r holds keys of elements r and 64 + r; the word
// index is XOR-swizzled with the lane so equal indices hit different banks.
struct Chunk {
  const uint32_t *w;  // this lane's 64 words
  int sw;
  __device__ __forceinline__ uint32_t at(int i) const {
    const uint32_t x = w[(i & 63) ^ sw];
    return (i & 64) ? (x >> 16) : (x & 0xffffu);
  }
  // #elements with key <= k (keys of padding are above every finite key)
  __device__ __forceinline__ int upper(uint32_t k) const {
    int pos = 0;
#pragma unroll
    for (int s = 64; s >= 1; s >>= 1)
      if (at(pos + s - 1) <= k) pos += s;
    if (pos < CH && at(pos) <= k) ++pos;
    return pos;
  }
  // #elements with key < k
  __device__ __forceinline__ int lower(uint32_t k) const {
    int pos = 0;
#pragma unroll
    for (int s = 64; s >= 1; s >>= 1)
      if (at(pos + s - 1) < k) pos += s;
    if (pos < CH && at(pos) < k) ++pos;
    return pos;
  }
};

// sums over groups of G consecutive lanes
template <int G>
__device__ __forceinline__ int gsum(int v) {
#pragma unroll
  for (int m = 1; m < G; m <<= 1) v += __shfl_xor(v, m);
  return v;
}
template <int G>
__device__ __forceinline__ double gsum(double v) {
#pragma unroll
  for (int m = 1; m < G; m <<= 1) v += __shfl_xor(v, m);
  return v;
}
template <int G>
__device__ __forceinline__ uint32_t gmin(uint32_t v) {
#pragma unroll
  for (int m = 1; m < G; m <<= 1) v = min(v, (uint32_t)__shfl_xor((int)v, m));
  return v;
}

// ----------------------------------------------------------------- exact thresholds
__device__ __forceinline__ uint16_t next16(uint16_t h) {
  if ((h & 0x7fffu) == 0) return 0x0001u;
  if (h & 0x8000u) {
    const uint16_t r = (uint16_t)(h - 1);
    return r == 0x8000u ? (uint16_t)0 : r;
  }
  return h == 0x7bffu ? h : (uint16_t)(h + 1);
}
__device__ __forceinline__ uint16_t prev16(uint16_t h) {
  if ((h & 0x7fffu) == 0) return 0x8001u;
  if (h & 0x8000u) return h == 0xfbffu ? h : (uint16_t)(h + 1);
  return (uint16_t)(h - 1);
}
// exact test 2u > a + b. TwoSum gives s + e == a + b exactly. If 2u and s
// are within a factor of two (same sign), d = 2u - s is exact (Sterbenz) and
// the sign of 2u - s - e is that of d - e; otherwise |d| >= |s|/2 > |e|, so
// the sign is that of d. In both cases "d > e" decides exactly.
__device__ __forceinline__ bool upper_of(double u, double a, double b) {
  const double s = a + b;
  const double bb = s - a;
  const double e = (a - (s - bb)) + (b - bb);
  const double d = 2.0 * u - s;
  return d > e;
}
// largest finite fp16 t with 2t <= a + b, for levels a < b
__device__ uint16_t thr16(float a, float b) {
  const double da = a, db = b;
  const double s = da + db;
  const double bb = s - da;
  const double e = (da - (s - bb)) + (db - bb);
  const double m = s * 0.5;
  uint16_t c = f2h((float)m);
  if ((c & 0x7fffu) > 0x7bffu) c = (uint16_t)((c & 0x8000u) | 0x7bffu);
  if (e == 0.0) {
    // the midpoint is exact: c is within one fp16 step of it, on either side
    if ((double)h2f(c) > m) c = prev16(c);
  } else {
    for (int i = 0; i < 4 && upper_of((double)h2f(c), da, db); ++i) c = prev16(c);
    for (int i = 0; i < 4; ++i) {
      const uint16_t n = next16(c);
      if (n == c || upper_of((double)h2f(n), da, db)) break;
      c = n;
    }
  }
  return c == 0x8000u ? (uint16_t)0 : c;
}
// cut keys for sorted levels: cell j is (T[j-1], T[j]] on the key line;
// duplicates of a level get an empty cell (the first copy wins ties)
template <int L>
__device__ __forceinline__ void cut_keys(const float *lev, uint32_t *T) {
  uint32_t nt = 0xffffu;  // above every finite key
#pragma unroll
  for (int j = L - 2; j >= 0; --j) {
    if (lev[j] < lev[j + 1]) nt = key16(thr16(lev[j], lev[j + 1]));
    T[j] = nt;
  }
}

// ascending order of the level table after an update (odd-even transposition)
template <int L>
__device__ __forceinline__ void sort_levels(float *lev) {
#pragma unroll
  for (int p = 0; p < L; ++p) {
#pragma unroll
    for (int i = p & 1; i + 1 < L; i += 2) {
      const float x = lev[i], y = lev[i + 1];
      lev[i] = fminf(x, y);
      lev[i + 1] = fmaxf(x, y);
    }
  }
}

// ----------------------------------------------------------------- the fit
struct FitOut {
  uint32_t tau_key;  // key of tau (non-negative fp16)
  uint16_t tau;
};

// Fit one vector split over CPC lanes (this lane holds `nq` valid samples in
// its sorted chunk `c`). Returns levels (identical in all CPC lanes).
template <int CPC, int L>
__device__ void fit_vector(const Chunk &c, int nq, float frac, int iters, float *lev, FitOut &fo) {
  const int n = gsum<CPC>(nq);
  fo.tau = 0;
  fo.tau_key = key16(0);
#pragma unroll
  for (int j = 0; j < L; ++j) lev[j] = 0.0f;
  if (n == 0) return;
  const long long k = (long long)floor((double)frac * (double)n);
  // ---- tau: largest non-negative fp16 c with #{|x| >= c} >= k + 1
  uint32_t tau;
  if (CPC == 1) {
    // (k+1)-th largest |x| by walking in from both ends of the sorted chunk
    int i = 0, j = nq - 1;
    uint32_t last = 0;
    for (long long t = 0; t <= k; ++t) {
      const uint32_t a = unkey16(c.at(i)) & 0x7fffu, b = unkey16(c.at(j)) & 0x7fffu;
      if (a >= b) { last = a; ++i; } else { last = b; --j; }
    }
    tau = last;
  } else {
    int pos = 0;  // count of c values in [0, 0x7bff] satisfying the predicate
#pragma unroll 1
    for (int s = 16384; s >= 1; s >>= 1) {
      const int cand = pos + s - 1;
      if (cand > 0x7bff) continue;
      int cnt;
      if (cand == 0) {
        cnt = nq;
      } else {
        cnt = (nq - c.lower(key16((uint32_t)cand))) + c.upper(key16((uint32_t)cand | 0x8000u));
      }
      if ((long long)gsum<CPC>(cnt) >= k + 1) pos += s;
    }
    tau = (uint32_t)(pos - 1);
  }
  fo.tau = (uint16_t)tau;
  fo.tau_key = key16(tau);
  // inliers: keys in [key(-tau), key(tau)]; with tau == 0 both zeros count
  const uint32_t klo = tau == 0 ? key16(0x8000u) : key16(tau | 0x8000u);
  const int lo = c.lower(klo);
  const int hi = c.upper(key16(tau));
  const int m = gsum<CPC>(hi - lo);
  // ---- quantile initialisation (positions exact in integers)
  auto select = [&](int r) -> uint32_t {  // key of the r-th smallest inlier (0-based)
    if (CPC == 1) return c.at(lo + r);
    int pos = 0;
#pragma unroll 1
    for (int s = 32768; s >= 1; s >>= 1) {
      const int cand = pos + s - 1;  // key
      bool adv;
      if (cand > 0xfbff) {
        adv = false;
      } else {
        const int cnt = min(max(c.upper((uint32_t)cand), lo), hi) - lo;
        adv = gsum<CPC>(cnt) <= r;
      }
      if (adv) pos += s;
    }
    return (uint32_t)pos;
  };
  auto successor = [&](int r, uint32_t kr) -> uint32_t {  // key of the (r+1)-th smallest inlier
    if (CPC == 1) return c.at(lo + r + 1);
    const int le = min(max(c.upper(kr), lo), hi) - lo;
    if (gsum<CPC>(le) > r + 1) return kr;
    const int idx = min(max(c.upper(kr), lo), hi);
    return gmin<CPC>(idx < hi ? c.at(idx) : 0xffffu);
  };
#pragma unroll
  for (int j = 0; j < L; ++j) {
    const long long num = (long long)(2 * j + 1) * (long long)(m - 1);
    const int r = (int)(num / (2 * L));
    const long long rem = num % (2 * L);
    const uint32_t kr = select(r);
    double v = kval(kr);
    if (rem != 0) {
      const double u1 = kval(successor(r, kr));
      v = v + ((double)rem / (double)(2 * L)) * (u1 - v);
    }
    lev[j] = (float)v + 0.0f;
  }
  // ---- Lloyd iterations on the sorted inlier ranges
  int cut[L];      // per lane: cut positions (exclusive ends of cells), cut[L-1] = hi
  double P[L];     // prefix sums of this lane's inliers up to each cut
  uint32_t T[L];
  for (int it = 0; it < iters; ++it) {
    cut_keys<L>(lev, T);
    if (it == 0) {
      // one pass over the inliers, cell by cell, recording the running sum at every cut
      double acc = 0.0;
      int prev = lo;
#pragma unroll
      for (int q = 0; q < L; ++q) {
        const int nc = q < L - 1 ? min(max(c.upper(T[q]), lo), hi) : hi;
        for (int i = prev; i < nc; ++i) acc += kval(c.at(i));
        P[q] = acc;
        cut[q] = nc;
        prev = max(prev, nc);
      }
    } else {
#pragma unroll
      for (int q = 0; q < L - 1; ++q) {
        const int nc = min(max(c.upper(T[q]), lo), hi);
        double p = P[q];
        for (int i = cut[q]; i < nc; ++i) p += kval(c.at(i));
        for (int i = nc; i < cut[q]; ++i) p -= kval(c.at(i));
        P[q] = p;
        cut[q] = nc;
      }
    }
    int prev_cut = lo;
    double prev_p = 0.0;
#pragma unroll
    for (int q = 0; q < L; ++q) {
      const int cnt = gsum<CPC>(cut[q] - prev_cut);
      const double sum = gsum<CPC>(P[q] - prev_p);
      if (cnt > 0) lev[q] = (float)(sum / (double)cnt);
      prev_cut = cut[q];
      prev_p = P[q];
    }
    // an empty duplicate keeps its level while its twin moves: keep the table
    // ordered so the cells stay contiguous ranges
    sort_levels<L>(lev);
  }
}

// load the 128-sample chunk from a register array of fp16 pairs (element i
// in word i/2) into the sort layout (element i in register i%64, half i/64)
__device__ __forceinline__ void to_sort_layout(const uint32_t *raw, uint32_t *v) {
#pragma unroll
  for (int r = 0; r < 64; ++r) {
    const uint32_t lo = (raw[r / 2] >> (16 * (r & 1))) & 0xffffu;
    const uint32_t hi = (raw[32 + r / 2] >> (16 * (r & 1))) & 0xffffu;
    v[r] = lo | (hi << 16);
  }
#pragma unroll
  for (int r = 0; r < 64; ++r) v[r] = key_pair(v[r]);
}

__device__ __forceinline__ void store_chunk(uint32_t *w, int sw, const uint32_t *v) {
#pragma unroll
  for (int r = 0; r < 64; ++r) w[r ^ sw] = v[r];
}

// exclusive prefix over the 64 lanes of a wave
__device__ __forceinline__ int wave_excl(int v, int &total) {
  int x = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(x, d);
    if ((int)(threadIdx.x & 63) >= d) x += y;
  }
  total = __shfl(x, 63);
  return x - v;
}

}  // namespace

// ================================================================== kernels
__global__ void nuq_zero(uint32_t *ctr) {
  if (threadIdx.x < 4) ctr[threadIdx.x] = 0;
}

// Key fit: lanes (channel g, chunk q) with CPC chunks per channel; a
// workgroup of 256 lanes covers 256/CPC channels of one (b,h).
template <int CPC, int L>
__global__ __launch_bounds__(256) void nuq_key_fit(NuqArgs a) {
  extern __shared__ uint32_t lds[];
  const int lane = threadIdx.x;
  const int chans = 256 / CPC;
  const int bh = blockIdx.y;
  const int g = lane / CPC, q = lane % CPC;
  const int d = blockIdx.x * chans + g;
  const bool active = d < a.D;
  const int t0 = a.n_sink_eff + q * CH;
  uint32_t raw[64];
#pragma unroll
  for (int i = 0; i < 64; ++i) raw[i] = 0x7c007c00u;  // fp16 +inf padding sorts last
  int nq = 0;
  if (active) {
    const uint16_t *col = a.keys + (size_t)bh * a.S * a.D + d;
    nq = max(0, min(CH, a.S - t0));
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      if (i < nq) {
        const uint32_t x = col[(size_t)(t0 + i) * a.D];
        raw[i / 2] = (raw[i / 2] & (0xffffu << (16 * (1 - (i & 1))))) | (x << (16 * (i & 1)));
      }
    }
  }
  uint32_t v[64];
  to_sort_layout(raw, v);
  sort128(v);
  const int sw = lane & 63;
  uint32_t *w = lds + lane * 64;
  store_chunk(w, sw, v);
  __syncthreads();
  Chunk c{w, sw};
  float lev[L];
  FitOut fo;
  fit_vector<CPC, L>(c, nq, a.frac, a.iters, lev, fo);
  if (active && q == 0) {
    float *kl = a.key_levels + ((size_t)bh * a.D + d) * L;
#pragma unroll
    for (int j = 0; j < L; ++j) kl[j] = lev[j];
    a.key_thresh[(size_t)bh * a.D + d] = fo.tau;
  }
}

// Frozen-level cut keys per key channel (every call; also after a fit).
template <int L>
__global__ __launch_bounds__(256) void nuq_key_cuts(NuqArgs a) {
  const int64_t id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (id >= (int64_t)a.BH * a.D) return;
  float lev[L];
#pragma unroll
  for (int j = 0; j < L; ++j) lev[j] = a.key_levels[id * L + j];
  uint32_t T[L];
  cut_keys<L>(lev, T);
  uint16_t *dst = a.ws_kcut + id * 16;
#pragma unroll
  for (int j = 0; j < L - 1; ++j) dst[j] = (uint16_t)T[j];
}

// Key quantize: flat order. A wave handles 64 / (D/8) token rows per step,
// lane = 8 consecutive channels; 4 lanes pack their codes into one
// dword-aligned store. Outliers are compacted in flat order per block.
template <int BITS>
__global__ __launch_bounds__(256) void nuq_key_quant(NuqArgs a) {
  constexpr int L = 1 << BITS;
  __shared__ int wave_cnt[4];
  __shared__ uint32_t blk_base;
  const int D = a.D;
  const int CL = D / 8;               // lanes per token row
  const int RPW = 64 / CL;            // rows per wave
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int bh = blockIdx.y;
  const int row = (blockIdx.x * 4 + wv) * RPW + lane / CL;  // token within bh
  const int ck = lane % CL;
  const bool valid = row < a.S;
  uint32_t codes = 0;
  uint16_t x[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  uint16_t rec[8];
  bool out[8];
  int nout = 0;
  if (valid) {
    const uint4 in = *reinterpret_cast<const uint4 *>(a.keys + ((size_t)bh * a.S + row) * D + ck * 8);
    const uint32_t wds[4] = {in.x, in.y, in.z, in.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = (uint16_t)(wds[i / 2] >> (16 * (i & 1)));
    const bool sink = row < a.n_sink_eff;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int d = ck * 8 + i;
      const size_t ch = (size_t)bh * D + d;
      const uint16_t tau = a.key_thresh[ch];
      const bool o = !sink && h2f((uint16_t)(x[i] & 0x7fffu)) > h2f(tau);
      out[i] = o;
      nout += o;
      uint32_t code = 0;
      if (!sink && !o) {
        const uint32_t kx = key16(x[i]);
        const uint16_t *cuts = a.ws_kcut + ch * 16;
#pragma unroll
        for (int j = 0; j < L - 1; ++j) code += kx > cuts[j];
      }
      codes |= code << (BITS * i);
      rec[i] = (sink || o) ? x[i] : f2h(a.key_levels[ch * L + code]);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) { out[i] = false; rec[i] = 0; }
  }
  // pack: 4 consecutive lanes hold 32 codes = 4*BITS bytes
  const uint32_t c1 = __shfl_down(codes, 1), c2 = __shfl_down(codes, 2), c3 = __shfl_down(codes, 3);
  if (valid && (ck & 3) == 0) {
    const uint64_t lo = (uint64_t)codes | ((uint64_t)c1 << (8 * BITS));
    const uint64_t hi = (uint64_t)c2 | ((uint64_t)c3 << (8 * BITS));
    uint32_t *dst = reinterpret_cast<uint32_t *>(a.k_codes + ((size_t)bh * a.S + row) * (D * BITS / 8) +
                                                 (ck / 4) * 4 * BITS);
    // 16*BITS bits per half: write BITS dwords
    uint32_t wd[4];
    if constexpr (BITS == 1) { wd[0] = (uint32_t)(lo | (hi << 16)); }
    if constexpr (BITS == 2) { wd[0] = (uint32_t)lo; wd[1] = (uint32_t)hi; }
    if constexpr (BITS == 3) {  // lo and hi hold 48 bits each
      wd[0] = (uint32_t)lo; wd[1] = (uint32_t)(lo >> 32) | (uint32_t)(hi << 16); wd[2] = (uint32_t)(hi >> 16);
    }
    if constexpr (BITS == 4) {
      wd[0] = (uint32_t)lo; wd[1] = (uint32_t)(lo >> 32); wd[2] = (uint32_t)hi; wd[3] = (uint32_t)(hi >> 32);
    }
#pragma unroll
    for (int j = 0; j < BITS; ++j) dst[j] = wd[j];
  }
  if (valid && a.k_recon) {
    *reinterpret_cast<uint4 *>(a.k_recon + ((size_t)bh * a.S + row) * D + ck * 8) =
        make_uint4(rec[0] | (rec[1] << 16), rec[2] | ((uint32_t)rec[3] << 16),
                   rec[4] | ((uint32_t)rec[5] << 16), rec[6] | ((uint32_t)rec[7] << 16));
  }
  // ordered compaction of outliers (lane order = flat order inside the block)
  int wtot;
  const int wpre = wave_excl(nout, wtot);
  if (lane == 0) wave_cnt[wv] = wtot;
  __syncthreads();
  int before = 0, btot = 0;
  for (int i = 0; i < 4; ++i) {
    if (i < wv) before += wave_cnt[i];
    btot += wave_cnt[i];
  }
  const int64_t blk = (int64_t)blockIdx.y * gridDim.x + blockIdx.x;
  if (threadIdx.x == 0) {
    const uint32_t base = btot ? atomicAdd(&a.ws_ctr[0], (uint32_t)btot) : 0u;
    blk_base = base;
    a.ws_kblk[blk * 2] = base;
    a.ws_kblk[blk * 2 + 1] = (uint32_t)btot;
  }
  __syncthreads();
  int slot = blk_base + before + wpre;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    if (out[i]) {
      a.ws_kpos[slot] = (int32_t)(((size_t)bh * a.S + row) * D + ck * 8 + i);
      a.ws_kval[slot] = x[i];
      ++slot;
    }
  }
}

// Value fit + quantize: one token per lane group of CPC lanes (128 channels
// per lane); a wave holds 64/CPC tokens. Sink tokens are passed through.
template <int CPC, int BITS>
__global__ __launch_bounds__(64) void nuq_value(NuqArgs a) {
  constexpr int L = 1 << BITS;
  __shared__ uint32_t lds[64 * 64];
  const int lane = threadIdx.x;
  const int q = lane % CPC;
  const int64_t tok = (int64_t)blockIdx.x * (64 / CPC) + lane / CPC;  // flat token id bh*S + s
  const int64_t ntok = (int64_t)a.BH * a.S;
  const bool valid = tok < ntok;
  const int s = valid ? (int)(tok % a.S) : 0;
  const bool sink = valid && s < a.n_sink_eff;
  const int D = a.D;
  const int c0 = q * CH;                          // first channel of this lane
  const int nch = max(0, min(CH, D - c0));        // channels held by this lane
  const uint16_t *row = a.values + (size_t)(valid ? tok : 0) * D;
  uint32_t raw[64];
#pragma unroll
  for (int i = 0; i < 64; ++i) raw[i] = 0x7c007c00u;
  if (valid && !sink) {
#pragma unroll
    for (int i = 0; i < CH / 8; ++i)
      if (i * 8 < nch) {
        const uint4 w = *reinterpret_cast<const uint4 *>(row + c0 + i * 8);
        raw[4 * i] = w.x; raw[4 * i + 1] = w.y; raw[4 * i + 2] = w.z; raw[4 * i + 3] = w.w;
      }
  }
  const int nq = (valid && !sink) ? nch : 0;
  uint32_t v[64];
  to_sort_layout(raw, v);
  sort128(v);
  const int sw = lane & 63;
  uint32_t *w = lds + lane * 64;
  store_chunk(w, sw, v);
  __syncthreads();
  Chunk c{w, sw};
  float lev[L];
  FitOut fo;
  fit_vector<CPC, L>(c, nq, a.frac, a.iters, lev, fo);
  uint32_t T[L];
  cut_keys<L>(lev, T);
  if (valid && q == 0) {
    float *vl = a.value_levels + (size_t)tok * L;
#pragma unroll
    for (int j = 0; j < L; ++j) vl[j] = sink ? 0.0f : lev[j];
  }
  // quantize this lane's channels: codes packed LSB-first along D
  int nout = 0;
  constexpr int OBW = CH * BITS / 32;  // dwords of packed codes for 128 channels
  uint32_t ob[OBW + 1];
#pragma unroll
  for (int i = 0; i <= OBW; ++i) ob[i] = 0;
  if (valid) {
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      if (i < nch) {
        const uint16_t x = row[c0 + i];
        uint32_t code = 0;
        bool o = false;
        if (!sink) {
          o = h2f((uint16_t)(x & 0x7fffu)) > h2f(fo.tau);
          if (!o) {
            const uint32_t kx = key16(x);
#pragma unroll
            for (int j = 0; j < L - 1; ++j) code += kx > T[j];
          }
        }
        nout += o;
        const int bit = i * BITS;
        ob[bit / 32] |= code << (bit % 32);
        if (bit % 32 + BITS > 32) ob[bit / 32 + 1] |= code >> (32 - bit % 32);
        if (a.v_recon) {
          float lv = lev[0];
#pragma unroll
          for (int j = 1; j < L; ++j) lv = code == (uint32_t)j ? lev[j] : lv;
          a.v_recon[(size_t)tok * D + c0 + i] = (sink || o) ? x : f2h(lv);
        }
      }
    }
    // the lane's code bytes start on a dword boundary (D >= 32, 128-channel chunks)
    uint32_t *crow = reinterpret_cast<uint32_t *>(a.v_codes + (size_t)tok * (D * BITS / 8) +
                                                  (size_t)c0 * BITS / 8);
    const int ndw = nch * BITS / 32;
#pragma unroll
    for (int j = 0; j < OBW; ++j)
      if (j < ndw) crow[j] = ob[j];
  }
  // ordered compaction (lanes are in flat order)
  int tot;
  const int pre = wave_excl(nout, tot);
  __shared__ uint32_t base_s;
  if (lane == 0) {
    const uint32_t base = tot ? atomicAdd(&a.ws_ctr[1], (uint32_t)tot) : 0u;
    base_s = base;
    a.ws_vblk[blockIdx.x * 2] = base;
    a.ws_vblk[blockIdx.x * 2 + 1] = (uint32_t)tot;
  }
  __syncthreads();
  if (valid && !sink && nout) {
    int slot = base_s + pre;
    for (int i = 0; i < nch; ++i) {
      const uint16_t x = row[c0 + i];
      if (h2f((uint16_t)(x & 0x7fffu)) > h2f(fo.tau)) {
        a.ws_vpos[slot] = (int32_t)((size_t)tok * D + c0 + i);
        a.ws_vval[slot] = x;
        ++slot;
      }
    }
  }
}

// exclusive scan of block counts in block order (one workgroup), then the
// totals; info[2b] = staging base, info[2b+1] = count -> final offset in [2b+1]
__global__ __launch_bounds__(1024) void nuq_scan(uint32_t *info, int64_t nblk, int64_t *total) {
  __shared__ uint32_t part[1024];
  uint32_t carry = 0;
  for (int64_t b0 = 0; b0 < nblk; b0 += 1024) {
    const int64_t b = b0 + threadIdx.x;
    const uint32_t cnt = b < nblk ? info[b * 2 + 1] : 0u;
    part[threadIdx.x] = cnt;
    __syncthreads();
    for (int d = 1; d < 1024; d <<= 1) {
      const uint32_t y = threadIdx.x >= (unsigned)d ? part[threadIdx.x - d] : 0u;
      __syncthreads();
      part[threadIdx.x] += y;
      __syncthreads();
    }
    const uint32_t incl = part[threadIdx.x];
    if (b < nblk) {
      info[b * 2 + 1] = carry + incl - cnt;  // final offset
      // keep the count recoverable: next offset - this offset
    }
    const uint32_t last = part[1023];
    __syncthreads();
    carry += last;
  }
  if (threadIdx.x == 0) *total = carry;
}

// move each block's staged entries to their final place; counts are the
// differences of consecutive final offsets
__global__ __launch_bounds__(256) void nuq_copy(const uint32_t *info, int64_t nblk, const int64_t *total,
                                                const int32_t *spos, const uint16_t *sval, int32_t *opos,
                                                uint16_t *oval) {
  const int64_t b = blockIdx.x;
  if (b >= nblk) return;
  const uint32_t off = info[b * 2 + 1];
  const uint32_t end = b + 1 < nblk ? info[b * 2 + 3] : (uint32_t)*total;
  const uint32_t base = info[b * 2];
  for (uint32_t i = threadIdx.x; i < end - off; i += blockDim.x) {
    opos[off + i] = spos[base + i];
    oval[off + i] = sval[base + i];
  }
}

// ================================================================== launch
namespace {
template <int CPC, int L>
hipError_t launch_key_fit_cpc(const NuqArgs &a, hipStream_t st) {
  const int chans = 256 / CPC;
  dim3 grid((a.D + chans - 1) / chans, a.BH);
  hipLaunchKernelGGL((nuq_key_fit<CPC, L>), grid, dim3(256), 256 * 64 * 4, st, a);
  return hipGetLastError();
}
template <int L>
hipError_t launch_key_fit(const NuqArgs &a, int cpc, hipStream_t st) {
  switch (cpc) {
    case 1: return launch_key_fit_cpc<1, L>(a, st);
    case 2: return launch_key_fit_cpc<2, L>(a, st);
    case 4: return launch_key_fit_cpc<4, L>(a, st);
    case 8: return launch_key_fit_cpc<8, L>(a, st);
    case 16: return launch_key_fit_cpc<16, L>(a, st);
    case 32: return launch_key_fit_cpc<32, L>(a, st);
    default: return launch_key_fit_cpc<64, L>(a, st);
  }
}
template <int BITS>
hipError_t launch_bits(const NuqArgs &a, int key_cpc, int val_cpc, hipStream_t st) {
  constexpr int L = 1 << BITS;
  hipError_t e;
  hipLaunchKernelGGL(nuq_zero, dim3(1), dim3(64), 0, st, a.ws_ctr);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (a.fit_keys && (e = launch_key_fit<L>(a, key_cpc, st)) != hipSuccess) return e;
  const int64_t nch = (int64_t)a.BH * a.D;
  hipLaunchKernelGGL((nuq_key_cuts<L>), dim3((unsigned)((nch + 255) / 256)), dim3(256), 0, st, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL((nuq_key_quant<BITS>), dim3((unsigned)a.k_blk_x, a.BH), dim3(256), 0, st, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (val_cpc == 1)
    hipLaunchKernelGGL((nuq_value<1, BITS>), dim3((unsigned)a.v_nblk), dim3(64), 0, st, a);
  else
    hipLaunchKernelGGL((nuq_value<2, BITS>), dim3((unsigned)a.v_nblk), dim3(64), 0, st, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int64_t k_nblk = a.k_blk_x * (int64_t)a.BH;
  hipLaunchKernelGGL(nuq_scan, dim3(1), dim3(1024), 0, st, a.ws_kblk, k_nblk, a.out_counts);
  hipLaunchKernelGGL(nuq_scan, dim3(1), dim3(1024), 0, st, a.ws_vblk, a.v_nblk, a.out_counts + 1);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(nuq_copy, dim3((unsigned)k_nblk), dim3(256), 0, st, a.ws_kblk, k_nblk, a.out_counts,
                     a.ws_kpos, a.ws_kval, a.k_opos, a.k_oval);
  hipLaunchKernelGGL(nuq_copy, dim3((unsigned)a.v_nblk), dim3(256), 0, st, a.ws_vblk, a.v_nblk,
                     a.out_counts + 1, a.ws_vpos, a.ws_vval, a.v_opos, a.v_oval);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_nuq(const NuqArgs &a, int key_cpc, int val_cpc, hipStream_t st) {
  switch (a.bits) {
    case 1: return launch_bits<1>(a, key_cpc, val_cpc, st);
    case 2: return launch_bits<2>(a, key_cpc, val_cpc, st);
    case 3: return launch_bits<3>(a, key_cpc, val_cpc, st);
    default: return launch_bits<4>(a, key_cpc, val_cpc, st);
  }
}

}  // namespace kvq
