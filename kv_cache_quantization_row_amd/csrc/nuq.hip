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
// GPU formulation.
// Values (and short vectors): a vector of n samples is split over CPC lanes,
// 128 samples per lane. Each lane sorts its chunk in registers (a bitonic
// network on packed 16-bit order keys, all compare-exchanges ascending) and
// keeps it in LDS. Everything the fit needs then comes from binary searches in
// those sorted chunks plus sums over CPC lanes:
//   - tau: the (k+1)-th largest |x|, walked in from both ends of the chunk;
//   - the inliers of a chunk are a contiguous index range [lo, hi);
//   - quantile order statistics: direct reads (one lane) or a bitwise search
//     over fp16 order keys;
//   - a Lloyd iteration: the nearest-level cells are contiguous index ranges
//     cut at exact fp16 thresholds T_j (largest fp16 t with 2t <= l_j +
//     l_{j+1}); cell sums are kept as prefix sums P_j at the cut points and
//     updated by walking the cut from its old to its new position. Sums are
//     doubles, exact while |sum| < 2^29 (fp16 values are multiples of 2^-24),
//     so each level is the exact mean rounded once to binary32.
// Keys at prefill: a counting sort of each channel's samples by the high byte
// of their order key, then every query of the fit is a table read plus one
// bucket scan (the "bucketed key fit" section below); sums there are int64.
// The Lloyd iterations of up to 8 levels run two channels per wave, 32 lanes
// each ("Lloyd by rows").
// Up to 4,096 vectors the value fit runs one token per wave instead
// (value_wave_body: keys sorted across the wave, sorted keys and exact
// prefix sums in the wave's LDS, one level per lane); beyond that at D = 128
// a quad of lanes shares a token (nuq_value_quad: the same LDS tables per
// token, two levels per lane at 3 bits).
// Codes are #{j : x > T_j}, which equals the first index of the nearest
// level (a binary search over the sorted cut keys, two samples per packed
// step). The side channel (flat index, fp16 value) is emitted in ascending
// flat order: each producer workgroup records its count of outliers and
// either stages its entries (value workgroups at fixed ranges, k_val slots
// per token; key workgroups of a small call at the flat index of their first
// element) or, for keys otherwise, marks them in a bitmap with one bit per
// key element; the placement kernel puts every workgroup's entries at the
// sum of the counts before it (per-64-workgroup sums; no inter-workgroup
// waiting), a bitmap block's as its set bits in order with the values read
// back from the keys.
#include <algorithm>
#include <mutex>


#include "common.h"
#include "kernels.h"

namespace kvq {
namespace {

constexpr int CH = 128;             // samples per lane chunk

typedef short s16x2 __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2v __attribute__((ext_vector_type(2)));

// DPP lane move for patterns whose every source lane lies in its own row
// (quad permutes, row mirrors): no lane keeps an old value, so none is
// materialised (the generic helper writes a 0 first, one extra move each)
template <int CTRL>
__device__ __forceinline__ uint32_t dppm(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xf, 0xf, true);
}

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

// ----------------------------------------------------------------- packed codes
// Per 16-bit half: 1 where a > b (unsigned), else 0. A saturating subtract
// then a minimum with 1, both packed (two VALU instructions for two
// samples); written out because the compiler rewrites the pattern into
// per-half compares through the scalar condition registers.
__device__ __forceinline__ uint32_t pk_gt01(uint32_t a, uint32_t b) {
  uint32_t r;
  const uint32_t one = 0x00010001u;
  asm("v_pk_sub_u16 %0, %1, %2 clamp\n\tv_pk_min_u16 %0, %0, %3" : "=&v"(r) : "v"(a), "v"(b), "v"(one));
  return r;
}
// 0xffff in each half that holds 1 (halves hold 0 or 1: a 24-bit product)
__device__ __forceinline__ uint32_t pk_mask01(uint32_t g) { return __umul24(g, 0xffffu); }
// select per half: (m & a) | (~m & b)
__device__ __forceinline__ uint32_t bsel(uint32_t m, uint32_t a, uint32_t b) { return (m & a) | (~m & b); }
// codes #{j : key > T_j} of two keys (packed halves) for ascending thresholds
// T2[j] (each repeated in both halves): a binary search, one code bit per
// step from the top; the threshold a step tests is picked by the bits above
// it (bit-select on the masks of the steps before)
template <int BITS>
__device__ __forceinline__ uint32_t code_pair(uint32_t kx, const uint32_t *T2) {
  uint32_t code = 0, msk[BITS];
#pragma unroll
  for (int s = BITS - 1; s >= 0; --s) {
    constexpr int MAXC = 1 << (BITS - 1);
    uint32_t cand[MAXC];
    const int nc = 1 << (BITS - 1 - s);  // candidates: one per value of the bits above s
#pragma unroll
    for (int p = 0; p < MAXC; ++p)
      if (p < nc) cand[p] = T2[(p << (s + 1)) + (1 << s) - 1];
#pragma unroll
    for (int r = 0; r < BITS - 1 - s; ++r) {  // fold by code bit s + 1 + r
#pragma unroll
      for (int p = 0; p < MAXC / 2; ++p)
        if (p < (nc >> (r + 1))) cand[p] = bsel(msk[s + 1 + r], cand[2 * p + 1], cand[2 * p]);
    }
    const uint32_t g = pk_gt01(kx, cand[0]);
    code |= g << s;
    msk[s] = pk_mask01(g);
  }
  return code;
}
// fp16 reconstructions of two codes (packed halves) from the level table as
// fp16 pairs LH[i] = lev[2i] | lev[2i+1] << 16: byte permutes over pairs of
// table words, then a bit-select per higher code bit
template <int L>
__device__ __forceinline__ uint32_t pick_lev16(const uint32_t *LH, uint32_t code) {
  const uint32_t sel = (code & 0x00030003u) * 0x0202u + 0x01000100u;  // bytes 2c, 2c+1 of each half
  if constexpr (L == 2) {
    return __builtin_amdgcn_perm(LH[0], LH[0], sel);
  } else if constexpr (L == 4) {
    return __builtin_amdgcn_perm(LH[1], LH[0], sel);
  } else {
    uint32_t w[L / 4];
#pragma unroll
    for (int i = 0; i < L / 4; ++i) w[i] = __builtin_amdgcn_perm(LH[2 * i + 1], LH[2 * i], sel);
    const uint32_t m2 = pk_mask01((code >> 2) & 0x00010001u);
    if constexpr (L == 8) {
      return bsel(m2, w[1], w[0]);
    } else {
      const uint32_t m3 = pk_mask01((code >> 3) & 0x00010001u);
      return bsel(m3, bsel(m2, w[3], w[2]), bsel(m2, w[1], w[0]));
    }
  }
}

// #{keys <= t} among 8 keys (16 bytes), t repeated in both halves of t2
__device__ __forceinline__ int count_le8(const uint4 &w, uint32_t t2) {
  const uint32_t g = pk_gt01(w.x, t2) + pk_gt01(w.y, t2) + pk_gt01(w.z, t2) + pk_gt01(w.w, t2);
  return 8 - (int)((g & 0xffffu) + (g >> 16));
}
// #{i < N : key[i] <= t} over the wave's N ascending keys: a count over the
// last keys of the runs of 8 gives the number of runs wholly <= t, a count
// inside the next run finishes (two rounds of 16-byte LDS reads)
// the same, with the run ends already in registers (N/16 words, two keys each)
template <int N>
__device__ __forceinline__ int lds_upper_r(const uint32_t *l8, const uint16_t *key, uint32_t t) {
  const uint32_t t2 = t * 0x10001u;
  int r = 0;
#pragma unroll
  for (int q = 0; q < N / 64; ++q) r += count_le8(make_uint4(l8[4 * q], l8[4 * q + 1], l8[4 * q + 2], l8[4 * q + 3]), t2);
  if (r == N / 8) return N;
  return 8 * r + count_le8(*reinterpret_cast<const uint4 *>(key + 8 * r), t2);
}
template <int N>
__device__ __forceinline__ int lds_upper(const uint16_t *key, const uint16_t *last8, uint32_t t) {
  const uint32_t t2 = t * 0x10001u;
  int r = 0;
#pragma unroll
  for (int q = 0; q < N / 64; ++q) r += count_le8(*reinterpret_cast<const uint4 *>(last8 + 8 * q), t2);
  if (r == N / 8) return N;
  return 8 * r + count_le8(*reinterpret_cast<const uint4 *>(key + 8 * r), t2);
}

// ----------------------------------------------------------------- sorting
__device__ __forceinline__ void ce(uint32_t &a, uint32_t &b) {
  const u16x2v x = __builtin_bit_cast(u16x2v, a), y = __builtin_bit_cast(u16x2v, b);
  a = __builtin_bit_cast(uint32_t, __builtin_elementwise_min(x, y));
  b = __builtin_bit_cast(uint32_t, __builtin_elementwise_max(x, y));
}
// A lane's NR packed registers hold 2*NR keys: element i in register i % NR,
// half i / NR. Bitonic sort with mirrored ("flip") stages, all ascending.
template <int NR, int K>
__device__ __forceinline__ void flip_r(uint32_t *v) {  // i <-> i ^ (K-1) inside one half (K <= NR)
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    const int p = r ^ (K - 1);
    if (p > r) ce(v[r], v[p]);
  }
}
template <int NR, int J>
__device__ __forceinline__ void disp_r(uint32_t *v) {  // i <-> i ^ J inside one half (J < NR)
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    const int p = r ^ J;
    if (p > r) ce(v[r], v[p]);
  }
}
template <int NR, int J>
__device__ __forceinline__ void disp_down(uint32_t *v) {  // distances J, J/2, ..., 1
  if constexpr (J >= 1) {
    disp_r<NR, J>(v);
    disp_down<NR, J / 2>(v);
  }
}
template <int NR, int K>
__device__ __forceinline__ void merge_r(uint32_t *v) {
  flip_r<NR, K>(v);
  disp_down<NR, K / 4>(v);
}
// the flip across the halves: element r of half 0 with element 2NR-1-r,
// the high half of register NR-1-r (and vice versa)
template <int NR>
__device__ __forceinline__ void flip_halves(uint32_t *v) {
#pragma unroll
  for (int r = 0; r < NR / 2; ++r) {
    const int p = NR - 1 - r;
    const u16x2v a = __builtin_bit_cast(u16x2v, v[r]);
    const u16x2v b = __builtin_bit_cast(u16x2v, v[p]);
    const u16x2v bs = {b.y, b.x};
    const u16x2v mn = __builtin_elementwise_min(a, bs), mx = __builtin_elementwise_max(a, bs);
    v[r] = (uint32_t)mn.x | ((uint32_t)mx.y << 16);
    v[p] = (uint32_t)mn.y | ((uint32_t)mx.x << 16);
  }
}
template <int NR, int K>
__device__ __forceinline__ void merges_up(uint32_t *v) {  // merge levels K, 2K, ..., NR
  if constexpr (K <= NR) {
    merge_r<NR, K>(v);
    merges_up<NR, 2 * K>(v);
  }
}
template <int NR>
__device__ __forceinline__ void sort_regs(uint32_t *v) {  // all 2*NR keys ascending
  merges_up<NR, 2>(v);
  flip_halves<NR>(v);
  disp_down<NR, NR / 2>(v);
}
__device__ __forceinline__ void sort128(uint32_t *v) { sort_regs<64>(v); }

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

// reductions over groups of G consecutive lanes (G a power of two <= 64):
// DPP inside a 16-lane row (pairs, quads, half-row mirror, row mirror), then
// a lane swizzle across rows; every lane of the group receives the result
template <int G, typename Op>
__device__ __forceinline__ uint32_t gred_u32(uint32_t v, Op op) {
  if constexpr (G >= 2) v = op(v, dppm<DPP_XOR1>(v));
  if constexpr (G >= 4) v = op(v, dppm<DPP_XOR2>(v));
  if constexpr (G >= 8) v = op(v, dppm<DPP_HALF_MIRROR>(v));
  if constexpr (G >= 16) v = op(v, dppm<DPP_MIRROR>(v));
  if constexpr (G >= 32) v = op(v, (uint32_t)__shfl_xor((int)v, 16));
  if constexpr (G >= 64) v = op(v, (uint32_t)__shfl_xor((int)v, 32));
  return v;
}
template <int G>
__device__ __forceinline__ int gsum(int v) {
  return (int)gred_u32<G>((uint32_t)v, [](uint32_t x, uint32_t y) { return x + y; });
}
template <int G>
__device__ __forceinline__ uint32_t gmin(uint32_t v) {
  return gred_u32<G>(v, [](uint32_t x, uint32_t y) { return min(x, y); });
}
template <int CTRL>
__device__ __forceinline__ double dppd(double v) {
  const uint64_t b = __builtin_bit_cast(uint64_t, v);
  const uint64_t lo = dppm<CTRL>((uint32_t)b), hi = dppm<CTRL>((uint32_t)(b >> 32));
  return __builtin_bit_cast(double, lo | (hi << 32));
}
// (the partial sums are exact, so the reduction order does not matter)
template <int G>
__device__ __forceinline__ double gsum(double v) {
  if constexpr (G >= 2) v += dppd<DPP_XOR1>(v);
  if constexpr (G >= 4) v += dppd<DPP_XOR2>(v);
  if constexpr (G >= 8) v += dppd<DPP_HALF_MIRROR>(v);
  if constexpr (G >= 16) v += dppd<DPP_MIRROR>(v);
  if constexpr (G >= 32) v += __shfl_xor(v, 16);
  if constexpr (G >= 64) v += __shfl_xor(v, 32);
  return v;
}

// ----------------------------------------------------------------- exact thresholds
// the next fp16 value below a finite h (-inf below -65504)
__device__ __forceinline__ uint16_t prev16(uint16_t h) {
  if ((h & 0x7fffu) == 0) return 0x8001u;
  if (h & 0x8000u) return (uint16_t)(h + 1);
  return (uint16_t)(h - 1);
}
// largest fp16 t with 2t <= a + b, for levels a < b: finite, or -inf when
// a + b < -131008 (every finite input then lies above the cut). TwoSum in
// binary32 gives s + e == a + b exactly, |e| <= ulp(s)/2. c = fp16(s/2),
// clamped to the finite range, is the largest fp16 <= a + b or the next one
// up (fp16 values are 13 bits coarser than binary32 rounding, and a halving
// that underflows keeps the sign); 2c is exact, and two different floats are
// at least one ulp of s apart, so 2c > a + b exactly when 2c > s, or 2c == s
// and e < 0. That case steps c down once.
__device__ __forceinline__ uint16_t thr16(float a, float b) {
  const float s = a + b;
  const float bb = s - a;
  const float e = (a - (s - bb)) + (b - bb);
  uint16_t c = f2h(s * 0.5f);
  if ((c & 0x7fffu) > 0x7bffu) c = (uint16_t)((c & 0x8000u) | 0x7bffu);
  const float c2 = 2.0f * h2f(c);
  if (c2 > s || (c2 == s && e < 0.0f)) c = prev16(c);
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

// min / max of two levels by compare and select: level tables hold no NaN
// and no -0 (a mean is +0 when its sum is 0, sentinels are +-inf), where
// these equal fminf / fmaxf without the NaN-quieting instructions
__device__ __forceinline__ float lmin(float x, float y) { return y < x ? y : x; }
__device__ __forceinline__ float lmax(float x, float y) { return y > x ? y : x; }

// ascending order of the level table after an update (odd-even transposition)
template <int L>
__device__ __forceinline__ void sort_levels(float *lev) {
#pragma unroll
  for (int p = 0; p < L; ++p) {
#pragma unroll
    for (int i = p & 1; i + 1 < L; i += 2) {
      const float x = lev[i], y = lev[i + 1];
      lev[i] = lmin(x, y);
      lev[i + 1] = lmax(x, y);
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
__device__ void fit_vector(const Chunk &c, int nq, int kout, int iters, float *lev, FitOut &fo) {
  const int n = gsum<CPC>(nq);
  fo.tau = 0;
  fo.tau_key = key16(0);
#pragma unroll
  for (int j = 0; j < L; ++j) lev[j] = 0.0f;
  if (n == 0) return;
  const long long k = kout;  // floor(frac * n), computed on the host
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
  // ---- quantile initialisation (positions exact in integers): level j
  // interpolates between the r_j-th and (r_j+1)-th smallest inliers with
  // r_j + f_j = (j + 1/2)(m - 1)/L
  int rk[L];
  int rem[L];
#pragma unroll
  for (int j = 0; j < L; ++j) {
    const long long num = (long long)(2 * j + 1) * (long long)(m - 1);
    rk[j] = (int)(num / (2 * L));
    rem[j] = (int)(num % (2 * L));
  }
  uint32_t kr[L], ks[L];  // keys of the r_j-th and (r_j+1)-th smallest inliers
  if (CPC == 1) {
#pragma unroll
    for (int j = 0; j < L; ++j) {
      kr[j] = c.at(lo + rk[j]);
      ks[j] = rem[j] ? c.at(lo + rk[j] + 1) : kr[j];
    }
  } else {
    // all L ranks in one bitwise search over the 16-bit key line: after the
    // step for bit s, pos[j] is the largest prefix with #{inliers with key <
    // pos[j]} <= r_j. Each lane keeps, per rank, the window [wa, wb] of its
    // chunk that holds the count of any remaining candidate (wa = count of
    // inliers <= pos - 1, wb = count <= pos + s - 1), so each step searches
    // only inside the window, which shrinks with the key range.
    int pos[L], wa[L], wb[L];
#pragma unroll
    for (int j = 0; j < L; ++j) { pos[j] = 0; wa[j] = lo; wb[j] = hi; }
#pragma unroll 1
    for (int sbit = 32768; sbit >= 1; sbit >>= 1) {
      int sa[L], sb[L];
      uint32_t cd[L];
#pragma unroll
      for (int j = 0; j < L; ++j) {
        cd[j] = (uint32_t)(pos[j] + sbit - 1);
        sa[j] = wa[j];
        sb[j] = cd[j] > 0xfbffu ? wa[j] : wb[j];  // beyond the finite keys: no advance, nothing to search
      }
      for (;;) {  // binary searches inside the windows (no cross-lane operations)
        bool act = false;
#pragma unroll
        for (int j = 0; j < L; ++j) act |= sa[j] < sb[j];
        if (!act) break;
#pragma unroll
        for (int j = 0; j < L; ++j) {
          const int m = (sa[j] + sb[j]) >> 1;
          const bool le = c.at(m) <= cd[j];
          const bool on = sa[j] < sb[j];
          sa[j] = on && le ? m + 1 : sa[j];
          sb[j] = on && !le ? m : sb[j];
        }
      }
#pragma unroll
      for (int j = 0; j < L; ++j) {
        const int tot = gsum<CPC>(sa[j] - lo);
        if (cd[j] <= 0xfbffu && tot <= rk[j]) {
          pos[j] += sbit;
          wa[j] = sa[j];
        } else {
          wb[j] = cd[j] > 0xfbffu ? wb[j] : sa[j];
        }
      }
    }
#pragma unroll
    for (int j = 0; j < L; ++j) {
      kr[j] = (uint32_t)pos[j];
      // successor: the same key while more than r_j + 1 inliers are <= it,
      // else the smallest inlier key above it; wb[j] is now the count of
      // this lane's inliers <= kr[j]
      const int idx = wb[j];
      const int le = gsum<CPC>(idx - lo);
      const uint32_t nx = gmin<CPC>(idx < hi ? c.at(idx) : 0xffffu);
      ks[j] = le > rk[j] + 1 ? kr[j] : nx;
    }
  }
#pragma unroll
  for (int j = 0; j < L; ++j) {
    double v = kval(kr[j]);
    if (rem[j] != 0) {
      const double u1 = kval(ks[j]);
      v = v + ((double)rem[j] / (double)(2 * L)) * (u1 - v);
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
      // the cut positions clamp(#{keys <= T_q}, lo, hi): the L-1 binary
      // searches run side by side (independent reads)
      int pos[L - 1];
#pragma unroll
      for (int q = 0; q < L - 1; ++q) pos[q] = 0;
#pragma unroll
      for (int sb = 64; sb >= 1; sb >>= 1) {
#pragma unroll
        for (int q = 0; q < L - 1; ++q)
          if (c.at(pos[q] + sb - 1) <= T[q]) pos[q] += sb;
      }
#pragma unroll
      for (int q = 0; q < L - 1; ++q) {
        if (pos[q] < CH && c.at(pos[q]) <= T[q]) ++pos[q];
        cut[q] = min(max(pos[q], lo), hi);
      }
      cut[L - 1] = hi;
      // one pass over the inliers, cell by cell, recording the running sum at
      // every cut (four independent partial sums; every partial sum is exact,
      // so the order of the additions does not matter)
      double acc = 0.0;
      int prev = lo;
#pragma unroll
      for (int q = 0; q < L; ++q) {
        const int nc = cut[q];
        double a0 = 0.0, a1 = 0.0, a2 = 0.0, a3 = 0.0;
        int i = prev;
        for (; i + 4 <= nc; i += 4) {
          a0 += kval(c.at(i));
          a1 += kval(c.at(i + 1));
          a2 += kval(c.at(i + 2));
          a3 += kval(c.at(i + 3));
        }
        for (; i < nc; ++i) a0 += kval(c.at(i));
        acc += (a0 + a1) + (a2 + a3);
        P[q] = acc;
        prev = max(prev, nc);
      }
    } else {
      // cuts move little between iterations: walk each from its old position
      // (the same result as a fresh search clamped to [lo, hi]), updating
      // its prefix sum with the elements it passes
#pragma unroll
      for (int q = 0; q < L - 1; ++q) {
        int pc = cut[q];
        double ps = P[q];
        const uint32_t t = T[q];
        while (pc < hi && c.at(pc) <= t) { ps += kval(c.at(pc)); ++pc; }
        while (pc > lo && c.at(pc - 1) > t) { --pc; ps -= kval(c.at(pc)); }
        P[q] = ps;
        cut[q] = pc;
      }
    }
    int prev_cut = lo;
    double prev_p = 0.0;
    bool empty = false;
#pragma unroll
    for (int q = 0; q < L; ++q) {
      const int cnt = gsum<CPC>(cut[q] - prev_cut);
      const double sum = gsum<CPC>(P[q] - prev_p);
      if (cnt > 0) lev[q] = (float)(sum / (double)cnt);
      empty |= cnt <= 0;
      prev_cut = cut[q];
      prev_p = P[q];
    }
    // an empty cell keeps its level while its neighbours move: keep the table
    // ordered so the cells stay contiguous ranges (without an empty cell the
    // new means are already ascending; the wave skips the sort then)
    if (__any(empty)) sort_levels<L>(lev);
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

// ================================================================== bucketed key fit
// Prefill key fit without a sort. Each channel's non-sink samples are
// counting-sorted by the high byte of their 16-bit order key (sign, exponent,
// two significand bits): a workgroup of KB_CH waves covers KB_CH consecutive
// channels of one (b, h); its threads read token rows of those channels (one
// 16-byte load per row) and, per sample, add one to its bucket's count and the
// sample's integer significand to the bucket's significand sum (one 64-bit LDS
// atomic); after the exclusive prefix of the counts they store each key's low
// byte at its bucket's cursor (unordered inside a bucket). The members of a
// bucket share sign and binade, so the bucket's exact sum in 2^-24 units is
// its significand sum shifted by the exponent; exclusive prefixes of counts and
// sums over the buckets then give the exact count and sum below every bucket.
// Each fit query is a table read plus a scan of one bucket by the channel's
// wave (one wave per channel):
//  - count and exact sum of the samples with key <= T: the prefixes at T's
//    bucket plus that bucket's members whose low byte is <= T's;
//  - the r-th smallest key: the bucket whose range holds rank r (ballot over
//    the bucket ends), then a 256-bin histogram of that bucket's low bytes;
//  - tau: the |x| bin (the two buckets of opposite sign with the same
//    magnitude byte) holding the (k+1)-th largest |x|, then a histogram of the
//    two buckets' |x| low bytes.
// Sums are int64 in 2^-24 units: fp16 magnitudes are below 2^40 units and a
// fit covers at most NUQ_KFIT_MAX_N (2^20) samples, so every sum is exact, and a level is
// the binary32 rounding of the exact mean. A Lloyd iteration that leaves the
// ordered table unchanged is a fixed point (every later iteration would
// repeat it), so the loop stops there with the same result.
constexpr int KB_CH = 8;                // channels per workgroup (one 16-byte row load)
constexpr int KB_T = 64 * KB_CH;        // threads: one wave per channel in the fit
constexpr int KB_LDS_MAX_N = NUQ_KFIT_LDS_N;  // bucketed samples per channel kept in LDS (beyond: in the workspace)

// sign, exponent shift and significand base of the members of bucket b
__device__ __forceinline__ void kb_bucket(int b, bool &neg, int &sh, uint32_t &mbase) {
  const int hh = b >= 0x80 ? b - 0x80 : 0x7f - b;  // bits 8..14 of the fp16 pattern
  const int e = hh >> 2;
  neg = b < 0x80;
  sh = e > 0 ? e - 1 : 0;                          // units per significand step: 2^(e-1), subnormals 1
  mbase = (e > 0 ? 0x400u : 0u) + ((uint32_t)(hh & 3) << 8);
}

// fp16 pattern of channel ch (0..7, may differ per lane) of a 16-byte row:
// byte permutes pick half ch & 3 of (x, y) and of (z, w), without an
// indexed access
__device__ __forceinline__ uint32_t kb_pick(const uint4 &q, int ch) {
  const uint32_t h = (uint32_t)(ch & 3);
  const uint32_t sel = (2 * h) | ((2 * h + 1) << 8) | 0x0c0c0000u;  // bytes 2h, 2h+1, then zeros
  const uint32_t lo = __builtin_amdgcn_perm(q.y, q.x, sel);
  const uint32_t hi = __builtin_amdgcn_perm(q.w, q.z, sel);
  return (ch & 4) ? hi : lo;
}

// binary32 rounding of (s / c) * 2^-24 for an exact int64 sum s in 2^-24
// units and a count c (round to nearest even, as the exact quotient would)
__device__ __forceinline__ float kb_mean(int64_t s, uint32_t c) {
  const uint64_t a = s < 0 ? (uint64_t)(-s) : (uint64_t)s;
  float f;
  if (a < (1ull << 53)) {
    f = (float)((double)a / (double)c);  // a exact; 53 >= 2*24 + 2: the double rounding is innocuous
  } else {
    const uint64_t q = a / c, r = a % c;
    if (q < (1ull << 24)) {
      // q + r/c below 2^24: the double sum errs by < 2^-29, and a tie point
      // of the 24-bit grid is at least 2^-24/c... away unless hit exactly
      f = (float)((double)q + (double)r / (double)c);
    } else {
      const int sh = 64 - __builtin_clzll(q) - 24;
      uint64_t qh = q >> sh;
      const uint64_t rb = q & ((1ull << sh) - 1), half = 1ull << (sh - 1);
      const uint64_t lhs = rb * c + r, rhs = half * c;
      if (lhs > rhs || (lhs == rhs && (qh & 1))) ++qh;
      f = __builtin_ldexpf((float)qh, sh);
    }
  }
  f *= 0x1p-24f;
  return s < 0 ? -f : f;
}

// exclusive prefix over the 64 lanes of a wave, of a count and an int64 sum
// (once per channel, in the table set-up)
__device__ __forceinline__ void kb_excl(uint32_t c, int64_t u, uint32_t &ce, int64_t &ue) {
  const int lane = threadIdx.x & 63;
  uint32_t xc = c;
  int64_t xu = u;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t yc = (uint32_t)__shfl_up((int)xc, d);
    const int64_t yu = __shfl_up(xu, d);
    if (lane >= d) {
      xc += yc;
      xu += yu;
    }
  }
  ce = xc - c;
  ue = xu - u;
}

// DPP move with a fill value for lanes without a source (row shifts,
// broadcasts; rows outside ROWMASK keep the fill)
template <int CTRL, int ROWMASK = 0xf>
__device__ __forceinline__ uint32_t kb_dpp(uint32_t v, uint32_t fill) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)fill, (int)v, CTRL, ROWMASK, 0xf, false);
}
constexpr int DPP_ROW_SHL1 = 0x101, DPP_ROW_SHR1 = 0x111, DPP_ROW_SHR2 = 0x112, DPP_ROW_SHR4 = 0x114,
              DPP_ROW_SHR8 = 0x118, DPP_ROW_BCAST15 = 0x142, DPP_ROW_BCAST31 = 0x143;

// inclusive prefix sum over the wave (Hillis-Steele inside each 16-lane row,
// then the row totals carried by row broadcasts): no LDS round trips
__device__ __forceinline__ uint32_t kb_wscan(uint32_t x) {
  x += kb_dpp<DPP_ROW_SHR1>(x, 0);
  x += kb_dpp<DPP_ROW_SHR2>(x, 0);
  x += kb_dpp<DPP_ROW_SHR4>(x, 0);
  x += kb_dpp<DPP_ROW_SHR8>(x, 0);
  x += kb_dpp<DPP_ROW_BCAST15, 0xa>(x, 0);
  x += kb_dpp<DPP_ROW_BCAST31, 0xc>(x, 0);
  return x;
}

// wave-uniform sum: DPP inside the rows, the row totals carried by row
// broadcasts into lane 63, one readlane
__device__ __forceinline__ uint32_t kb_wsum(uint32_t v) {
  v += dppm<DPP_XOR1>(v);
  v += dppm<DPP_XOR2>(v);
  v += dppm<DPP_HALF_MIRROR>(v);
  v += dppm<DPP_MIRROR>(v);
  v += kb_dpp<DPP_ROW_BCAST15, 0xa>(v, 0);
  v += kb_dpp<DPP_ROW_BCAST31, 0xc>(v, 0);
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

__device__ __forceinline__ uint32_t kb_rl(uint32_t v, int lane) { return (uint32_t)__builtin_amdgcn_readlane((int)v, lane); }
__device__ __forceinline__ double rl_d(double v, int lane) {
  const uint64_t b = __builtin_bit_cast(uint64_t, v);
  return __builtin_bit_cast(double, (uint64_t)kb_rl((uint32_t)b, lane) | ((uint64_t)kb_rl((uint32_t)(b >> 32), lane) << 32));
}
// a DPP move of a double (0.0 in lanes without a source)
template <int CTRL, int ROWMASK = 0xf>
__device__ __forceinline__ double kb_dppd0(double v) {
  const uint64_t b = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = kb_dpp<CTRL, ROWMASK>((uint32_t)b, 0u), hi = kb_dpp<CTRL, ROWMASK>((uint32_t)(b >> 32), 0u);
  return __builtin_bit_cast(double, (uint64_t)lo | ((uint64_t)hi << 32));
}
// inclusive prefix sum of doubles over the wave, the pattern of kb_wscan
__device__ __forceinline__ double wscan_d(double x) {
  x += kb_dppd0<DPP_ROW_SHR1>(x);
  x += kb_dppd0<DPP_ROW_SHR2>(x);
  x += kb_dppd0<DPP_ROW_SHR4>(x);
  x += kb_dppd0<DPP_ROW_SHR8>(x);
  x += kb_dppd0<DPP_ROW_BCAST15, 0xa>(x);
  x += kb_dppd0<DPP_ROW_BCAST31, 0xc>(x);
  return x;
}

// H16: the wave's 256-bin histogram as 16-bit counts, two per word (every
// count is at most n < 65536), so that it takes 512 bytes of LDS instead of
// 1 KiB; else 32-bit counts
template <typename DatPtr, bool H16>
struct KbView {
  const uint64_t *pre;  // [257] exclusive prefix sums (2^-24 units, int64 bits); [256] = total
  const uint32_t *end;  // [256] bucket ends (exclusive prefix of the counts, shifted by one bucket)
  DatPtr dat;           // bucketed key low bytes: bucket b at [start(b), end(b))
  uint32_t *hist;       // wave scratch: [128] (H16) or [256] words
  __device__ __forceinline__ uint32_t start(int b) const { return b == 0 ? 0u : end[b - 1]; }
  __device__ __forceinline__ void hist_zero(int lane) const {
    if constexpr (H16) *reinterpret_cast<uint2 *>(hist + 2 * lane) = make_uint2(0, 0);
    else *reinterpret_cast<uint4 *>(hist + 4 * lane) = make_uint4(0, 0, 0, 0);
  }
  __device__ __forceinline__ void hist_add(uint32_t bin) const {
    if constexpr (H16) atomicAdd(&hist[bin >> 1], 1u << (16 * (bin & 1u)));
    else atomicAdd(&hist[bin], 1u);
  }
  __device__ __forceinline__ uint4 hist_read(int lane) const {  // bins 4*lane .. 4*lane+3
    if constexpr (H16) {
      const uint2 w = *reinterpret_cast<const uint2 *>(hist + 2 * lane);
      return make_uint4(w.x & 0xffffu, w.x >> 16, w.y & 0xffffu, w.y >> 16);
    } else {
      return *reinterpret_cast<const uint4 *>(hist + 4 * lane);
    }
  }
};

// count and exact sum of the samples with key <= T[j], for every cut j whose
// bit is set in `need` (T[j] wave-uniform): one interleaved pass over all the
// cuts' buckets, four key bytes per read (a byte-wise compare in packed 16-bit
// arithmetic, a byte mask for the bucket's ends, then v_dot4 for the count
// and the sum of the selected bytes), then one wave sum per count and per
// low-byte sum
__device__ __forceinline__ uint32_t kb_le_bytes(uint32_t w, uint32_t t2) {  // 1 in each byte <= t
  const uint32_t ge = pk_gt01(w & 0x00ff00ffu, t2), go = pk_gt01((w >> 8) & 0x00ff00ffu, t2);
  return (ge ^ 0x00010001u) | ((go ^ 0x00010001u) << 8);
}
template <typename P>
__device__ __forceinline__ uint32_t kb_word(P dat, uint32_t pos) {  // 4 key bytes at a multiple of 4
  return *reinterpret_cast<const uint32_t *>(&dat[pos]);
}
template <int NC, typename V>
__device__ __forceinline__ void kb_le_many(const V &v, const uint32_t *T, uint32_t need, uint32_t *cnt,
                                           int64_t *sum) {
  const int lane = threadIdx.x & 63;
  uint32_t s0[NC], e0[NC], c[NC], sl[NC], t2[NC];
  uint32_t maxw = 0;
#pragma unroll
  for (int j = 0; j < NC; ++j) {
    c[j] = sl[j] = 0;
    s0[j] = e0[j] = 0;
    t2[j] = (T[j] & 0xffu) * 0x10001u;
    if ((need >> j) & 1u) {
      const int b = (int)(T[j] >> 8);
      s0[j] = v.start(b);
      e0[j] = v.end[b];
      if (e0[j] > s0[j]) maxw = max(maxw, ((e0[j] + 3u) >> 2) - (s0[j] >> 2));
    }
  }
  // the bucket's words: from the one holding its first byte to the one
  // holding its last; bytes outside [s0, e0) are masked off
  for (uint32_t i = lane; i < maxw; i += 64) {
#pragma unroll
    for (int j = 0; j < NC; ++j) {
      const uint32_t p0 = ((s0[j] >> 2) + i) << 2;
      if (p0 < e0[j]) {
        const uint32_t w = kb_word(v.dat, p0);
        const uint32_t nb = min(e0[j] - p0, 4u);                      // bytes before the end
        const uint32_t sk = s0[j] > p0 ? s0[j] - p0 : 0u;             // bytes before the start
        const uint32_t m = ((nb == 4u ? 0x01010101u : (0x01010101u & ((1u << (8 * nb)) - 1u))) >> (8 * sk)) << (8 * sk);
        const uint32_t le = kb_le_bytes(w, t2[j]) & m;
        c[j] = __builtin_amdgcn_udot4(le, 0x01010101u, c[j], false);
        sl[j] = __builtin_amdgcn_udot4(w, le, sl[j], false);
      }
    }
  }
#pragma unroll
  for (int j = 0; j < NC; ++j) {
    if (!((need >> j) & 1u)) continue;
    const uint32_t cc = kb_wsum(c[j]), ss = kb_wsum(sl[j]);
    const int b = (int)(T[j] >> 8);
    bool neg;
    int sh;
    uint32_t mbase;
    kb_bucket(b, neg, sh, mbase);
    const uint64_t hl = neg ? (uint64_t)cc * 255u - ss : (uint64_t)ss;  // sum of the fp16 low bytes
    const int64_t u = (int64_t)(((uint64_t)cc * mbase + hl) << sh);
    cnt[j] = s0[j] + cc;
    sum[j] = (int64_t)v.pre[b] + (neg ? -u : u);
  }
}

template <typename V>
__device__ __forceinline__ void kb_le(const V &v, uint32_t T, uint32_t &cnt, int64_t &sum) {
  kb_le_many<1>(v, &T, 1u, &cnt, &sum);
}

// the smallest e with (hist[0] + ... + hist[e]) > q, every lane holding
// entries 4*lane .. 4*lane+3 and the count below them
__device__ __forceinline__ uint32_t kb_hist_rank(const uint32_t *h4, uint32_t excl, uint32_t q) {
  const int lane = threadIdx.x & 63;
  const uint32_t c0 = excl + h4[0], c1 = c0 + h4[1], c2 = c1 + h4[2], c3 = c2 + h4[3];
  const int i = c0 > q ? 0 : c1 > q ? 1 : c2 > q ? 2 : 3;
  const uint64_t bal = __ballot(c3 > q);
  return kb_rl((uint32_t)(4 * lane + i), __ffsll((unsigned long long)bal) - 1);
}

// the bucket holding rank r (the first b with end(b) > r) and the histogram
// of its key low bytes (the wave's scratch); returns b
template <typename V>
__device__ __forceinline__ int kb_bucket_hist(const V &v, uint32_t r, uint32_t *h4, uint32_t &excl) {
  const int lane = threadIdx.x & 63;
  const uint4 e4 = *reinterpret_cast<const uint4 *>(v.end + 4 * lane);
  const int i = e4.x > r ? 0 : e4.y > r ? 1 : e4.z > r ? 2 : 3;
  const uint64_t bal = __ballot(e4.w > r);
  const int b = (int)kb_rl((uint32_t)(4 * lane + i), __ffsll((unsigned long long)bal) - 1);
  const uint32_t s0 = v.start(b), e0 = v.end[b];
  v.hist_zero(lane);
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
  for (uint32_t j = s0 + lane; j < e0; j += 64) v.hist_add(v.dat[j]);
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
  const uint4 hv = v.hist_read(lane);
  h4[0] = hv.x; h4[1] = hv.y; h4[2] = hv.z; h4[3] = hv.w;
  const uint32_t t = h4[0] + h4[1] + h4[2] + h4[3];
  excl = kb_wscan(t) - t;
  return b;
}

// keys of the r-th and (want_next) the (r+1)-th smallest samples (0-based;
// r + want_next < n)
template <typename V>
__device__ __forceinline__ void kb_kth2(const V &v, uint32_t r, bool want_next, uint32_t &k1, uint32_t &k2) {
  uint32_t h4[4], excl;
  const int b = kb_bucket_hist(v, r, h4, excl);
  const uint32_t s0 = v.start(b);
  k1 = ((uint32_t)b << 8) | kb_hist_rank(h4, excl, r - s0);
  k2 = k1;
  if (want_next) {
    if (r + 1 < v.end[b]) {
      k2 = ((uint32_t)b << 8) | kb_hist_rank(h4, excl, r + 1 - s0);
    } else {  // rank r + 1 opens the next non-empty bucket
      const int b2 = kb_bucket_hist(v, r + 1, h4, excl);
      k2 = ((uint32_t)b2 << 8) | kb_hist_rank(h4, excl, r + 1 - v.start(b2));
    }
  }
}

// (k+1)-th largest |x| (as a non-negative fp16 pattern) among the samples
template <typename V>
__device__ __forceinline__ uint32_t kb_tau(const V &v, uint32_t kp1) {
  const int lane = threadIdx.x & 63;
  // |x| bins a = 2*lane, 2*lane+1: buckets 0x80+a (x >= 0) and 0x7f-a (x < 0)
  uint32_t A[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int a = 2 * lane + j;
    const int bp = 0x80 + a, bn = 0x7f - a;
    A[j] = (v.end[bp] - v.start(bp)) + (v.end[bn] - v.start(bn));
  }
  const uint32_t incl = kb_wscan(A[0] + A[1]);
  const uint32_t total = kb_rl(incl, 63);
  const uint32_t above1 = total - incl;  // samples in bins > 2*lane+1
  const uint32_t above0 = above1 + A[1];
  // the bin a* with above(a*) < kp1 <= above(a*) + A(a*)
  const bool f1 = above1 < kp1 && above1 + A[1] >= kp1;
  const bool f0 = above0 < kp1 && above0 + A[0] >= kp1;
  const uint64_t bal = __ballot(f0 || f1);
  const int src = __ffsll((unsigned long long)bal) - 1;
  const int astar = (int)kb_rl((uint32_t)(f1 ? 2 * lane + 1 : 2 * lane), src);
  const uint32_t q = kp1 - kb_rl(f1 ? above1 : above0, src);  // 1-based, from the top
  // histogram of the |x| low bytes of the bin's two buckets
  v.hist_zero(lane);
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
  {
    const int bp = 0x80 + astar, bn = 0x7f - astar;
    for (uint32_t j = v.start(bp) + lane; j < v.end[bp]; j += 64) v.hist_add(v.dat[j]);
    for (uint32_t j = v.start(bn) + lane; j < v.end[bn]; j += 64) v.hist_add(255u - v.dat[j]);
  }
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
  const uint4 hv = v.hist_read(lane);
  // largest low byte w with #{|x| low >= w} >= q
  const uint32_t t4 = hv.x + hv.y + hv.z + hv.w;
  const uint32_t inc2 = kb_wscan(t4);
  const uint32_t ge0 = kb_rl(inc2, 63) - (inc2 - t4);  // #{>= 4*lane}
  const uint32_t ge1 = ge0 - hv.x, ge2 = ge1 - hv.y, ge3 = ge2 - hv.z;
  const int last = ge3 >= q ? 3 : ge2 >= q ? 2 : ge1 >= q ? 1 : 0;
  const uint64_t b2 = __ballot(ge0 >= q);
  const uint32_t w = kb_rl((uint32_t)(4 * lane + last), 63 - __clzll((long long)b2));
  return ((uint32_t)astar << 8) | w;
}

// a channel's inlier range: keys [klo, khi]; lo samples have keys below klo
// and hi samples keys at most khi, with exact sums s_lo and s_hi
struct KbInl {
  uint32_t klo, khi, lo, hi;
  int64_t s_lo, s_hi;
};

// the start of one channel's fit by one wave: tau, the inlier range and the
// quantile initialisation (lane j < L: level j)
template <int L, typename V>
__device__ void kb_init(const V &v, uint32_t n, int kout, float &lev_me, uint16_t &tau_out, KbInl &r) {
  const int lane = threadIdx.x & 63;
  lev_me = 0.0f;
  tau_out = 0;
  r = KbInl{0, 0, 0, 0, 0, 0};
  if (n == 0) return;
  const uint32_t tau = kb_tau(v, (uint32_t)kout + 1u);
  tau_out = (uint16_t)tau;
  // inliers: keys in [klo, khi] (with tau == 0 both zeros count)
  const uint32_t klo = tau == 0 ? key16(0x8000u) : key16(tau | 0x8000u);
  const uint32_t khi = key16(tau);
  uint32_t lohi[2];
  int64_t slohi[2];
  {
    const uint32_t T2[2] = {klo - 1, khi};
    kb_le_many<2>(v, T2, 3u, lohi, slohi);
  }
  const uint32_t lo = lohi[0], hi = lohi[1];
  const int64_t s_lo = slohi[0], s_hi = slohi[1];
  const uint32_t m = hi - lo;
  // quantile initialisation: level j interpolates between the r_j-th and
  // (r_j+1)-th smallest inliers with r_j + f_j = (j + 1/2)(m - 1)/L
#pragma unroll 1
  for (int j = 0; j < L; ++j) {
    const long long num = (long long)(2 * j + 1) * (long long)(m - 1);
    const uint32_t rk = (uint32_t)(num / (2 * L));
    const int rem = (int)(num % (2 * L));
    uint32_t k1, k2;
    kb_kth2(v, lo + rk, rem != 0, k1, k2);
    double x = kval(k1);
    if (rem != 0) {
      const double u1 = kval(k2);
      x = x + ((double)rem / (double)(2 * L)) * (u1 - x);
    }
    if (lane == j) lev_me = (float)x + 0.0f;
  }
  r = KbInl{klo, khi, lo, hi, s_lo, s_hi};
}

// Lloyd iterations of one channel by one wave. Lane j < L holds level j and
// lane j < L-1 cut j (its key and the count and exact sum at it).
template <int L, typename V>
__device__ void kb_lloyd_wave(const V &v, const KbInl &r, int iters, float &lev_me) {
  const int lane = threadIdx.x & 63;
  const uint32_t klo = r.klo, khi = r.khi, lo = r.lo, hi = r.hi;
  const int64_t s_lo = r.s_lo, s_hi = r.s_hi;
  // Lloyd iterations: cells are key ranges cut at exact fp16 thresholds.
  // The cuts' keys and the count and exact sum at each are wave-uniform
  // (scalar registers); lane j picks its cell's upper bound by lane-indexed
  // selects and the lower one from the lane below (DPP).
  uint32_t Tp[L - 1], Cu[L - 1];  // previous cut keys (none yet), counts at the cuts
  int64_t Su[L - 1];              // exact sums at the cuts
#pragma unroll
  for (int j = 0; j < L - 1; ++j) {
    Tp[j] = 0xffffffffu;
    Cu[j] = hi;
    Su[j] = s_hi;
  }
  const float inf = __builtin_inff();
  if (lane >= L) lev_me = inf;  // lanes above the table sort last
#pragma unroll 1
  for (int it = 0; it < iters; ++it) {
    // thresholds between neighbouring levels (0 marks equal levels, whose
    // cut is the one above: the first copy wins ties)
    const float lnext = __uint_as_float(kb_dpp<DPP_ROW_SHL1>(__float_as_uint(lev_me), __float_as_uint(inf)));
    uint32_t tmine = 0;
    if (lane < L - 1 && lev_me < lnext) tmine = key16(thr16(lev_me, lnext));
    // the cuts from the top, clamped to the inliers; a cut where it was last
    // iteration, or where the cut above it is, keeps that result
    uint32_t T[L - 1];
    uint32_t need = 0, nt = 0xffffu;
#pragma unroll
    for (int j = L - 2; j >= 0; --j) {
      const uint32_t t = kb_rl(tmine, j);
      if (t) nt = t;
      T[j] = min(max(nt, klo - 1), khi);
      const bool same_up = j < L - 2 && T[j] == T[j + 1];
      if (T[j] != Tp[j] && !same_up) need |= 1u << j;
    }
    uint32_t qc[L - 1];
    int64_t qs[L - 1];
    kb_le_many<L - 1>(v, T, need, qc, qs);
    uint32_t c_up = hi;
    int64_t s_up = s_hi;
#pragma unroll
    for (int j = L - 2; j >= 0; --j) {
      if ((need >> j) & 1u) {
        Cu[j] = qc[j];
        Su[j] = qs[j];
      } else if (T[j] != Tp[j]) {  // the same key as the cut above
        Cu[j] = c_up;
        Su[j] = s_up;
      }
      Tp[j] = T[j];
      c_up = Cu[j];
      s_up = Su[j];
    }
    // lane j < L updates level j from its cell (cut j-1, cut j]: lane j of
    // c_top / s_top holds cut j (lane L-1: hi), the lane below it cut j-1
    uint32_t c_top = hi, st_l = (uint32_t)s_hi, st_h = (uint32_t)((uint64_t)s_hi >> 32);
#pragma unroll
    for (int j = 0; j < L - 1; ++j) {
      const bool mine = lane == j;
      c_top = mine ? Cu[j] : c_top;
      st_l = mine ? (uint32_t)Su[j] : st_l;
      st_h = mine ? (uint32_t)((uint64_t)Su[j] >> 32) : st_h;
    }
    const int64_t s_top = (int64_t)(((uint64_t)st_h << 32) | st_l);
    uint32_t c_lo = kb_dpp<DPP_ROW_SHR1>(c_top, lo);
    const uint32_t slo_l = kb_dpp<DPP_ROW_SHR1>(st_l, (uint32_t)s_lo);
    const uint32_t slo_h = kb_dpp<DPP_ROW_SHR1>(st_h, (uint32_t)((uint64_t)s_lo >> 32));
    int64_t s_below = (int64_t)(((uint64_t)slo_h << 32) | slo_l);
    if (lane == 0) {
      c_lo = lo;
      s_below = s_lo;
    }
    float nl = lev_me;
    if (lane < L && c_top > c_lo) nl = kb_mean(s_top - s_below, c_top - c_lo);
    // an empty cell keeps its level while its neighbours move: keep the table
    // ordered so the cells stay contiguous ranges (odd-even transposition
    // sort over lanes 0..L-1 with DPP moves; lanes above hold +inf). Without
    // an empty cell the new means are already ascending: skipped.
    const bool any_empty = __any(lane < L && c_top <= c_lo);
#pragma unroll
    for (int p = 0; p < L && any_empty; ++p) {
      const uint32_t x = __float_as_uint(nl);
      if ((p & 1) == 0) {  // pairs (0,1), (2,3), ...
        const float o = __uint_as_float(dppm<DPP_XOR1>(x));
        nl = (lane & 1) ? lmax(nl, o) : lmin(nl, o);
      } else {             // pairs (1,2), (3,4), ...; lane 0 and lane 15 of the row sit out
        const float up = __uint_as_float(kb_dpp<DPP_ROW_SHL1>(x, __float_as_uint(inf)));
        const float dn = __uint_as_float(kb_dpp<DPP_ROW_SHR1>(x, __float_as_uint(-inf)));
        nl = (lane & 1) ? lmin(nl, up) : lmax(nl, dn);
      }
    }
    const bool changed = lane < L && __float_as_uint(nl) != __float_as_uint(lev_me);
    lev_me = lane < L ? nl : inf;
    if (__ballot(changed) == 0) break;  // a fixed point: every remaining iteration would repeat it
  }
  if (lane >= L) lev_me = 0.0f;
}

// ------------------------------------------------------------------ Lloyd by rows
// The Lloyd iterations of 64/G channels per wave, G lanes each (up to
// KB_ROW_MAX_L levels). Every lane of a group holds the channel's whole level
// table and every cut; the bucket scans stride over the group's G lanes, and
// a group sum takes four DPP adds inside each 16-lane row (plus one
// cross-row shuffle at G = 32; no readlane). Each lane j < L of the group
// computes the mean of cell j, and the group reads the new table back from
// its LDS slot. The arithmetic is that of kb_lloyd_wave: the same cut keys,
// exact int64 cell sums, binary32 means and ordering rule. G = 32 (two
// channels per wave, four waves of a workgroup) against G = 16 (four
// channels per wave, two waves): 75 against 81 us for the key fit alone,
// the second wave per SIMD hiding the iteration's latency.
constexpr int KB_ROW_MAX_L = 8;

constexpr int KB_G = 32;  // lanes per channel in the Lloyd loop (16 or 32)

// sum over the lane's group of G lanes (one or two 16-lane rows), in every
// lane of the group
template <int G>
__device__ __forceinline__ uint32_t row_sum(uint32_t v) {
  v += dppm<DPP_XOR1>(v);
  v += dppm<DPP_XOR2>(v);
  v += dppm<DPP_HALF_MIRROR>(v);
  v += dppm<DPP_MIRROR>(v);
  if constexpr (G == 32) v += (uint32_t)__shfl_xor((int)v, 16);
  return v;
}

// kb_le_many for the group's channel (tables pre / end, bucketed low bytes
// dat): count and exact sum at every cut whose bit is set in need
template <int NC, int G>
__device__ __forceinline__ void kb_le_rows(const uint64_t *pre, const uint32_t *end, const uint8_t *dat,
                                           const uint32_t *T, uint32_t need, uint32_t *cnt, int64_t *sum) {
  const uint32_t gl = threadIdx.x & (G - 1);
  uint32_t s0[NC], e0[NC], c[NC], sl[NC], t2[NC];
  uint32_t maxw = 0;
#pragma unroll
  for (int j = 0; j < NC; ++j) {
    c[j] = sl[j] = 0;
    t2[j] = (T[j] & 0xffu) * 0x10001u;
    const int b = (int)(T[j] >> 8);
    const bool nd = (need >> j) & 1u;
    s0[j] = nd && b > 0 ? end[b - 1] : 0u;
    e0[j] = nd ? end[b] : 0u;
    if (e0[j] > s0[j]) maxw = max(maxw, ((e0[j] + 3u) >> 2) - (s0[j] >> 2));
  }
  for (uint32_t i = gl; i < maxw; i += G) {
#pragma unroll
    for (int j = 0; j < NC; ++j) {
      const uint32_t p0 = ((s0[j] >> 2) + i) << 2;
      if (p0 < e0[j]) {
        const uint32_t w = kb_word(dat, p0);
        const uint32_t nb = min(e0[j] - p0, 4u);
        const uint32_t sk = s0[j] > p0 ? s0[j] - p0 : 0u;
        const uint32_t m = ((nb == 4u ? 0x01010101u : (0x01010101u & ((1u << (8 * nb)) - 1u))) >> (8 * sk)) << (8 * sk);
        const uint32_t le = kb_le_bytes(w, t2[j]) & m;
        c[j] = __builtin_amdgcn_udot4(le, 0x01010101u, c[j], false);
        sl[j] = __builtin_amdgcn_udot4(w, le, sl[j], false);
      }
    }
  }
#pragma unroll
  for (int j = 0; j < NC; ++j) {
    cnt[j] = 0;
    sum[j] = 0;
    if (!__any((need >> j) & 1u)) continue;
    const uint32_t cc = row_sum<G>(c[j]), ss = row_sum<G>(sl[j]);
    const int b = (int)(T[j] >> 8);
    bool neg;
    int sh;
    uint32_t mbase;
    kb_bucket(b, neg, sh, mbase);
    const uint64_t hl = neg ? (uint64_t)cc * 255u - ss : (uint64_t)ss;
    const int64_t u = (int64_t)(((uint64_t)cc * mbase + hl) << sh);
    cnt[j] = s0[j] + cc;
    sum[j] = (int64_t)pre[b] + (neg ? -u : u);
  }
}

// lev: the group's level table (ascending, in every lane); xch: the group's
// LDS slot of L floats
template <int L, int G>
__device__ void kb_lloyd_rows(const uint64_t *pre, const uint32_t *end, const uint8_t *dat, float *xch,
                              const KbInl &r, int iters, float (&lev)[L]) {
  const uint32_t gl = threadIdx.x & (G - 1);
  uint32_t Tp[L - 1], Cu[L - 1];  // previous cut keys (none yet), counts at the cuts
  int64_t Su[L - 1];              // exact sums at the cuts
#pragma unroll
  for (int j = 0; j < L - 1; ++j) {
    Tp[j] = 0xffffffffu;
    Cu[j] = r.hi;
    Su[j] = r.s_hi;
  }
#pragma unroll 1
  for (int it = 0; it < iters; ++it) {
    // cut keys from the top (equal levels take the cut above), clamped to
    // the inliers; a cut where it was last iteration, or where the cut
    // above it is, keeps that result
    uint32_t T[L - 1];
    uint32_t need = 0, nt = 0xffffu;
#pragma unroll
    for (int j = L - 2; j >= 0; --j) {
      if (lev[j] < lev[j + 1]) nt = key16(thr16(lev[j], lev[j + 1]));
      T[j] = min(max(nt, r.klo - 1), r.khi);
      const bool same_up = j < L - 2 && T[j] == T[j + 1];
      if (T[j] != Tp[j] && !same_up) need |= 1u << j;
    }
    uint32_t qc[L - 1];
    int64_t qs[L - 1];
    kb_le_rows<L - 1, G>(pre, end, dat, T, need, qc, qs);
    uint32_t c_up = r.hi;
    int64_t s_up = r.s_hi;
#pragma unroll
    for (int j = L - 2; j >= 0; --j) {
      if ((need >> j) & 1u) {
        Cu[j] = qc[j];
        Su[j] = qs[j];
      } else if (T[j] != Tp[j]) {  // the same key as the cut above
        Cu[j] = c_up;
        Su[j] = s_up;
      }
      Tp[j] = T[j];
      c_up = Cu[j];
      s_up = Su[j];
    }
    // lane gl < L: level gl from its cell (cut gl-1, cut gl] (cut -1: lo,
    // cut L-1: hi); an empty cell keeps its level
    uint32_t c_top = r.hi, c_bot = r.lo;
    int64_t s_top = r.s_hi, s_bot = r.s_lo;
    float nl = 0.0f;
#pragma unroll
    for (int j = 0; j < L; ++j) nl = gl == (uint32_t)j ? lev[j] : nl;
#pragma unroll
    for (int j = 0; j < L - 1; ++j) {
      c_top = gl == (uint32_t)j ? Cu[j] : c_top;
      s_top = gl == (uint32_t)j ? Su[j] : s_top;
      c_bot = gl == (uint32_t)j + 1 ? Cu[j] : c_bot;
      s_bot = gl == (uint32_t)j + 1 ? Su[j] : s_bot;
    }
    const bool mine = gl < (uint32_t)L;
    if (mine && c_top > c_bot) nl = kb_mean(s_top - s_bot, c_top - c_bot);
    const bool any_empty = __any(mine && c_top <= c_bot);
    if (mine) xch[gl] = nl;
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
    float nw[L];
#pragma unroll
    for (int j = 0; j < L; ++j) nw[j] = xch[j];
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
    // with an empty cell, keep the table ordered (the odd-even transposition
    // network of kb_lloyd_wave); without one the means are already ascending
    if (any_empty) {
#pragma unroll
      for (int p = 0; p < L; ++p) {
#pragma unroll
        for (int j = p & 1; j + 1 < L; j += 2) {
          const float x = nw[j], y = nw[j + 1];
          nw[j] = lmin(x, y);
          nw[j + 1] = lmax(x, y);
        }
      }
    }
    bool changed = false;
#pragma unroll
    for (int j = 0; j < L; ++j) {
      changed |= __float_as_uint(nw[j]) != __float_as_uint(lev[j]);
      lev[j] = nw[j];
    }
    if (__ballot(changed) == 0) break;  // every row at a fixed point
  }
}

}  // namespace

// ================================================================== kernels
// the per-64-workgroup count sums start at zero
__global__ __launch_bounds__(256) void nuq_zero(NuqArgs a) {
  const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x, nthr = (int64_t)gridDim.x * 256;
  const int64_t ks = (a.k_blk_x * a.BH + 63) >> 6, vs = (a.v_nblk + 63) >> 6;
  for (int64_t i = g; i < ks; i += nthr) a.ws_ksup[i] = 0;
  for (int64_t i = g; i < vs; i += nthr) a.ws_vsup[i] = 0;
}

// Key quantize against the (frozen or just fitted) per-channel tables. A
// workgroup covers KQ_NIT * 4 * 64 / (D/8) consecutive token rows of one
// (b,h): each of its 4 waves a contiguous run of KQ_NIT row steps, each step
// 64 / (D/8) rows with D/8 lanes per row and 8 consecutive channels per lane
// (one 16-byte load). The workgroup first turns the D level tables into cut
// keys in LDS; each lane then keeps the cut keys and |x| thresholds of its 8
// channels in registers, packed in channel pairs, and classifies two samples
// per packed 16-bit operation. Outliers are recorded as per-step bit masks:
// in a small call written in flat order at the flat index of the workgroup's
// first element, otherwise stored as the bitmap bytes of its rows (one byte
// per row and lane) with the workgroup's count.
constexpr int KQ_NIT = 8;
template <int BITS>
__device__ __forceinline__ void key_quant_body(const NuqArgs &a, int bx, int bh, int64_t blk) {
  constexpr int L = 1 << BITS;
  __shared__ uint16_t cut_s[256 * 16];  // [channel][j]: cut key between levels j and j+1
  __shared__ uint16_t tau_s[256];
  __shared__ float lev_s[256 * L];      // level tables of this (b,h)
  __shared__ int wave_cnt[4];
  __shared__ uint32_t blk_base;
  const int D = a.D;
  const int CL = D / 8;                 // lanes per token row
  const int RPW = 64 / CL;              // rows per wave step
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int ck = lane % CL;
  const bool want_rec = a.k_recon != nullptr;
  const int row_w = (bx * 4 + wv) * (RPW * KQ_NIT) + lane / CL;  // first row of this lane
  const uint16_t *kin = a.keys + (size_t)bh * a.S * D + ck * 8;
  // ---- cut keys of this (b,h): T[j] = key of thr16(l_j, l_{j+1}) for distinct
  // neighbours; a duplicate level takes the cut above it (empty cell); the
  // last cut is above every finite key
  const float *kl = a.key_levels + (size_t)bh * D * L;
  uint4 inr[KQ_NIT];
  {
    float lv[(256 * L) / 256];  // all level loads in flight at once
#pragma unroll
    for (int i = 0; i < L; ++i)
      if (threadIdx.x + 256 * i < D * L) lv[i] = kl[threadIdx.x + 256 * i];
    const uint32_t tau = threadIdx.x < D ? a.key_thresh[(size_t)bh * D + threadIdx.x] : 0u;
    // every row step's load is issued after the tables' and before the
    // set-up, so the wave waits for one load latency, not one per step, and
    // the set-up waits only for the tables; rows past the end read the last
    // row (S >= 1) and are not stored
#pragma unroll
    for (int it = 0; it < KQ_NIT; ++it)
      inr[it] = *reinterpret_cast<const uint4 *>(kin + (size_t)min(row_w + it * RPW, a.S - 1) * D);
#pragma unroll
    for (int i = 0; i < L; ++i)
      if (threadIdx.x + 256 * i < D * L) lev_s[threadIdx.x + 256 * i] = lv[i];
    if (threadIdx.x < D) tau_s[threadIdx.x] = (uint16_t)tau;
  }
  __syncthreads();
  for (int t = threadIdx.x; t < D * (L - 1); t += 256) {
    const int c = t / (L - 1), j = t - c * (L - 1);
    const float l0 = lev_s[c * L + j], l1 = lev_s[c * L + j + 1];
    cut_s[c * 16 + j] = l0 < l1 ? (uint16_t)key16(thr16(l0, l1)) : (uint16_t)0;  // key 0 is a NaN: marks "none"
  }
  __syncthreads();
  if (threadIdx.x < D) {
    uint32_t nt = 0xffffu;
    for (int j = L - 2; j >= 0; --j) {
      const uint32_t r = cut_s[threadIdx.x * 16 + j];
      if (r) nt = r;
      cut_s[threadIdx.x * 16 + j] = (uint16_t)nt;
    }
  }
  __syncthreads();
  // ---- this lane's 8 channels: cut keys and thresholds as channel pairs
  uint32_t cutp[4][L - 1], taup[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int c = ck * 8 + 2 * p;
#pragma unroll
    for (int j = 0; j < L - 1; ++j) cutp[p][j] = (uint32_t)cut_s[c * 16 + j] | ((uint32_t)cut_s[(c + 1) * 16 + j] << 16);
    taup[p] = (uint32_t)tau_s[c] | ((uint32_t)tau_s[c + 1] << 16);
  }
  uint8_t *kout = a.k_codes + (size_t)bh * a.S * (D * BITS / 8);
  uint32_t omask[KQ_NIT];  // bit e: channel ck*8+e of step it is an outlier
#pragma unroll
  for (int it = 0; it < KQ_NIT; ++it) omask[it] = 0;
  const int wrow0 = (bx * 4 + wv) * (RPW * KQ_NIT);  // the wave's first row
#pragma unroll
  for (int it = 0; it < KQ_NIT; ++it) {
    if (wrow0 + it * RPW >= a.S) break;  // this step's rows and all later ones lie past the end
    const int row = row_w + it * RPW;
    const bool valid = row < a.S;
    const bool sink = row < a.n_sink_eff;
    const uint4 in = inr[it];
    const uint32_t wd[4] = {in.x, in.y, in.z, in.w};
    const uint32_t live = sink ? 0u : 0xffffffffu;  // sinks: code 0, no outliers
    uint32_t codes = 0, om = 0;
    uint32_t rec[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      // two channels at a time in packed 16-bit arithmetic. Outlier: |x| >
      // tau (non-negative fp16 patterns order as integers); outliers get code 0
      const uint32_t isout = pk_gt01(wd[p] & 0x7fff7fffu, taup[p]) & live;
      const uint32_t code = code_pair<BITS>(key_pair(wd[p]), cutp[p]) & ~pk_mask01(isout) & live;
      const uint32_t c0 = code & 0xffffu, c1 = code >> 16, o0 = isout & 1u, o1 = isout >> 16;
      codes |= (c0 | (c1 << BITS)) << (2 * p * BITS);
      om |= (o0 | (o1 << 1)) << (2 * p);
      if (want_rec) {
        const int c = ck * 8 + 2 * p;
        const uint32_t x0 = wd[p] & 0xffffu, x1 = wd[p] >> 16;
        const uint32_t r0 = (sink || o0) ? x0 : (uint32_t)f2h(lev_s[c * L + c0]);
        const uint32_t r1 = (sink || o1) ? x1 : (uint32_t)f2h(lev_s[(c + 1) * L + c1]);
        rec[p] = r0 | (r1 << 16);
      }
    }
    omask[it] = valid ? om : 0u;
    // pack: the 4 lanes of a quad hold 32 consecutive codes = 4*BITS bytes
    const uint32_t n1 = dppm<0x39>(codes), n2 = dppm<0x4e>(codes), n3 = dppm<0x93>(codes);  // lanes +1, +2, +3
    if (valid && (ck & 3) == 0) {
      const uint64_t lo = (uint64_t)codes | ((uint64_t)n1 << (8 * BITS));
      const uint64_t hi = (uint64_t)n2 | ((uint64_t)n3 << (8 * BITS));
      uint32_t *dst = reinterpret_cast<uint32_t *>(kout + (size_t)row * (D * BITS / 8) + (ck / 4) * 4 * BITS);
      uint32_t wo[4];
      if constexpr (BITS == 1) { wo[0] = (uint32_t)(lo | (hi << 16)); }
      if constexpr (BITS == 2) { wo[0] = (uint32_t)lo; wo[1] = (uint32_t)hi; }
      if constexpr (BITS == 3) {  // lo and hi hold 48 bits each
        wo[0] = (uint32_t)lo; wo[1] = (uint32_t)(lo >> 32) | (uint32_t)(hi << 16); wo[2] = (uint32_t)(hi >> 16);
      }
      if constexpr (BITS == 4) {
        wo[0] = (uint32_t)lo; wo[1] = (uint32_t)(lo >> 32); wo[2] = (uint32_t)hi; wo[3] = (uint32_t)(hi >> 32);
      }
#pragma unroll
      for (int j = 0; j < BITS; ++j) dst[j] = wo[j];
    }
    if (valid && want_rec)
      *reinterpret_cast<uint4 *>(a.k_recon + ((size_t)bh * a.S + row) * D + ck * 8) =
          make_uint4(rec[0], rec[1], rec[2], rec[3]);
  }
  if (!a.small) {
    // ---- the outlier bitmap (byte ck of each row: this lane's 8 channels)
    // and the block's count; the placement emits the entries in flat order
    uint8_t *kbits = a.ws_kbits + (size_t)bh * a.S * (D / 8) + ck;
    int n = 0;
#pragma unroll
    for (int it = 0; it < KQ_NIT; ++it) {
      const int row = row_w + it * RPW;
      if (row < a.S) kbits[(size_t)row * (D / 8)] = (uint8_t)omask[it];
      n += __builtin_popcount(omask[it]);
    }
    int tot;
    (void)wave_excl(n, tot);
    if (lane == 0) wave_cnt[wv] = tot;
    __syncthreads();
    if (threadIdx.x == 0) {
      const uint32_t btot = (uint32_t)(wave_cnt[0] + wave_cnt[1] + wave_cnt[2] + wave_cnt[3]);
      a.ws_kblk[blk * 2 + 1] = btot;  // the block's only producer
      if (btot) atomicAdd(&a.ws_ksup[blk >> 6], btot);
    }
    return;
  }
  // ---- ordered compaction (a small call): flat order is (wave, step, lane,
  // channel). Step counts (<= 8 per lane, <= 512 per wave) are scanned three
  // at a time in 10-bit fields of one word.
  int pre[KQ_NIT], stot[KQ_NIT];
#pragma unroll
  for (int g = 0; g < KQ_NIT; g += 3) {
    uint32_t packed = 0;
#pragma unroll
    for (int t = 0; t < 3; ++t)
      if (g + t < KQ_NIT) packed |= (uint32_t)__builtin_popcount(omask[g + t]) << (10 * t);
    int tot;
    const uint32_t ex = (uint32_t)wave_excl((int)packed, tot);
#pragma unroll
    for (int t = 0; t < 3; ++t)
      if (g + t < KQ_NIT) {
        pre[g + t] = (int)((ex >> (10 * t)) & 1023u);
        stot[g + t] = (int)(((uint32_t)tot >> (10 * t)) & 1023u);
      }
  }
  int wsum = 0;
#pragma unroll
  for (int it = 0; it < KQ_NIT; ++it) {
    const int s_ = stot[it];
    stot[it] = wsum;  // now: offset of step it inside the wave
    wsum += s_;
  }
  if (lane == 0) wave_cnt[wv] = wsum;
  __syncthreads();
  int before = 0, btot = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (i < wv) before += wave_cnt[i];
    btot += wave_cnt[i];
  }
  if (threadIdx.x == 0) {
    // a small call stages at the flat index of the workgroup's first element
    // (its entries never exceed its rows times D)
    const uint32_t base = (uint32_t)(((int64_t)bh * a.S + (int64_t)bx * (4 * RPW * KQ_NIT)) * D);
    blk_base = base;
    a.ws_kblk[blk * 2] = base;
    a.ws_kblk[blk * 2 + 1] = (uint32_t)btot;
  }
  __syncthreads();
  const int wbase = (int)blk_base + before;
#pragma unroll
  for (int it = 0; it < KQ_NIT; ++it) {
    uint32_t m = omask[it];
    if (m) {
      const int row = row_w + it * RPW;
      const uint4 in = *reinterpret_cast<const uint4 *>(kin + (size_t)row * D);
      const uint32_t wd[4] = {in.x, in.y, in.z, in.w};
      int slot = wbase + stot[it] + pre[it];
      const int32_t fpos = (int32_t)(((size_t)bh * a.S + row) * D + ck * 8);
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (m & (1u << e)) {
          if (slot < a.k_scap) {  // holds by the outlier bound; never written past otherwise
            a.ws_kpos[slot] = fpos + e;
            a.ws_kval[slot] = (uint16_t)(wd[e / 2] >> (16 * (e & 1)));
          }
          ++slot;
        }
    }
  }
}

template <int BITS>
__global__ __launch_bounds__(256) void nuq_key_quant(NuqArgs a) {
  key_quant_body<BITS>(a, blockIdx.x, blockIdx.y, (int64_t)blockIdx.y * gridDim.x + blockIdx.x);
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
  // the lane's channels as fp16 pairs (element i in word i/2); channels past
  // nch are +inf padding, which sorts last
  uint32_t raw[64];
#pragma unroll
  for (int i = 0; i < 64; ++i) raw[i] = 0x7c007c00u;
  if (valid) {
#pragma unroll
    for (int i = 0; i < CH / 8; ++i)
      if (i * 8 < nch) {
        const uint4 w = *reinterpret_cast<const uint4 *>(row + c0 + i * 8);
        raw[4 * i] = w.x; raw[4 * i + 1] = w.y; raw[4 * i + 2] = w.z; raw[4 * i + 3] = w.w;
      }
  }
  const int nq = (valid && !sink) ? nch : 0;
  {
    uint32_t v[64];
    to_sort_layout(raw, v);  // a sink's fit reads nothing, so its chunk content is irrelevant
    sort128(v);
    store_chunk(lds + lane * 64, lane & 63, v);
  }
  __syncthreads();
  Chunk c{lds + lane * 64, lane & 63};
  float lev[L];
  FitOut fo;
  fit_vector<CPC, L>(c, nq, a.k_val, a.iters, lev, fo);
  uint32_t T[L];
  cut_keys<L>(lev, T);
  if (valid && q == 0) {
    float *vl = a.value_levels + (size_t)tok * L;
#pragma unroll
    for (int j = 0; j < L; ++j) vl[j] = sink ? 0.0f : lev[j];
  }
  // ---- quantize this lane's channels. The row is read again with all its
  // 16-byte loads in flight at once and kept in registers. Two samples (one
  // word) at a time in packed 16-bit arithmetic: outlier flags, codes by a
  // binary search over the cut keys, reconstructions by byte permutes of the
  // fp16 level table. Sinks get all-ones cut keys and an unreachable tau
  // (code 0, no outliers) and keep their input as reconstruction.
  uint4 rw[CH / 8];
#pragma unroll
  for (int g = 0; g < CH / 8; ++g)
    rw[g] = (valid && g * 8 < nch) ? *reinterpret_cast<const uint4 *>(row + c0 + g * 8) : make_uint4(0, 0, 0, 0);
  uint32_t T2[L - 1];
#pragma unroll
  for (int j = 0; j < L - 1; ++j) T2[j] = sink ? 0xffffffffu : T[j] * 0x10001u;
  const uint32_t tau2 = (sink ? 0x7fffu : (uint32_t)fo.tau) * 0x10001u;
  const uint32_t keep_in = sink ? 0xffffffffu : 0u;
  uint32_t LH[L / 2];
#pragma unroll
  for (int i = 0; i < L / 2; ++i) LH[i] = (uint32_t)f2h(lev[2 * i]) | ((uint32_t)f2h(lev[2 * i + 1]) << 16);
  const bool want_rec = valid && a.v_recon != nullptr;
  constexpr int OBW = CH * BITS / 32;  // dwords of packed codes for 128 channels
  uint32_t ob[OBW + 1], om[CH / 32];   // codes LSB-first along D; outlier bit per channel
#pragma unroll
  for (int i = 0; i <= OBW; ++i) ob[i] = 0;
#pragma unroll
  for (int i = 0; i < CH / 32; ++i) om[i] = 0;
  uint32_t onum = 0;  // outlier counts per half
#pragma unroll
  for (int g = 0; g < CH / 8; ++g) {
    const uint32_t wd[4] = {rw[g].x, rw[g].y, rw[g].z, rw[g].w};
    uint32_t rec[4];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int e = g * 8 + 2 * w;  // channel (within the lane) of the low half
      const uint32_t x = wd[w];
      // |x| > tau on non-negative fp16 patterns is an integer comparison
      const uint32_t o = pk_gt01(x & 0x7fff7fffu, tau2);
      onum += o;
      om[e / 32] |= ((o & 1u) | (o >> 15)) << (e % 32);
      const uint32_t omask = pk_mask01(o);
      const uint32_t code = code_pair<BITS>(key_pair(x), T2) & ~omask;
      const uint32_t pc = (code & 0xffffu) | (code >> (16 - BITS));  // codes of channels e, e + 1
      const int bit = e * BITS;
      ob[bit / 32] |= pc << (bit % 32);
      if (bit % 32 + 2 * BITS > 32) ob[bit / 32 + 1] |= pc >> (32 - bit % 32);
      rec[w] = bsel(omask | keep_in, x, pick_lev16<L>(LH, code));
    }
    if (want_rec && g * 8 < nch)
      *reinterpret_cast<uint4 *>(a.v_recon + (size_t)tok * D + c0 + g * 8) = make_uint4(rec[0], rec[1], rec[2], rec[3]);
  }
  if (valid) {
    // the lane's code bytes start on a dword boundary (D >= 32, 128-channel chunks)
    uint32_t *crow = reinterpret_cast<uint32_t *>(a.v_codes + (size_t)tok * (D * BITS / 8) +
                                                  (size_t)c0 * BITS / 8);
    const int ndw = nch * BITS / 32;
#pragma unroll
    for (int j = 0; j < OBW; ++j)
      if (j < ndw) crow[j] = ob[j];
  }
  // ---- side channel in flat order (lanes are in flat order). A token has at
  // most k_val outliers, so the workgroup's entries go to its own fixed
  // staging range (k_val slots per token it covers) at the exclusive prefix of
  // the lane counts; the placement kernel reads the range and the count.
  const int nout = (int)((onum & 0xffffu) + (onum >> 16));
  int tot;
  const int pre = wave_excl(nout, tot);
  const int64_t base = (int64_t)blockIdx.x * (64 / CPC) * a.k_val;
  if (lane == 0) {
    if (tot) atomicAdd(&a.ws_vsup[blockIdx.x >> 6], (uint32_t)tot);
    a.ws_vblk[blockIdx.x * 2] = (uint32_t)base;
    a.ws_vblk[blockIdx.x * 2 + 1] = (uint32_t)tot;
  }
  if (nout) {
    int64_t slot = base + pre;
#pragma unroll
    for (int d = 0; d < CH / 32; ++d) {
      uint32_t m = om[d];
      while (m) {
        const int b = __builtin_ctz(m);
        m &= m - 1;
        const int ch = c0 + d * 32 + b;
        if (slot < a.v_scap) {
          a.ws_vpos[slot] = (int32_t)((size_t)tok * D + ch);
          a.ws_vval[slot] = row[ch];
        }
        ++slot;
      }
    }
  }
}

// ================================================================== one token per quad (D = 128)
// Many-token value fit at D = 128: four lanes per token (a DPP quad), 32
// channels per lane, 16 tokens per wave, 64 per workgroup. The quad sorts
// the token's 128 keys (each lane its 32 in registers, then two cross-lane
// bitonic merge levels with quad permutes) and keeps, per token in LDS, the
// sorted keys, the last key of every run of 8 and the exact prefix sums at
// every 4th position. Every query of the fit is then a fixed-cost LDS
// lookup, with no per-lane walks: a cut's position is two rounds of 16-byte
// reads (run ends, then one run), the exact sum below it one table entry
// plus at most 3 samples. Lane q holds levels LPL*q .. LPL*q + LPL-1 and the
// cuts above them; neighbours come by quad permutes. The arithmetic is the
// same as in nuq_value.
constexpr int QPERM_REV = 0x1b;    // quad_perm [3,2,1,0]
constexpr int QPERM_NEXT = 0xf9;   // [1,2,3,3]: lane q reads q+1 (lane 3 itself)
constexpr int QPERM_PREV = 0x90;   // [0,0,1,2]: lane q reads q-1 (lane 0 itself)

struct alignas(16) QuadLds {
  uint16_t key[128];   // the token's order keys, ascending
  uint16_t last8[16];  // last8[r] = key[8r + 7]
  double pre4[33];     // pre4[i]: exact sum of the 4i smallest samples
};

template <int CTRL>
__device__ __forceinline__ double dppd_q(double v) {  // a quad permute of a double
  const uint64_t b = __builtin_bit_cast(uint64_t, v);
  return __builtin_bit_cast(double, (uint64_t)dppm<CTRL>((uint32_t)b) | ((uint64_t)dppm<CTRL>((uint32_t)(b >> 32)) << 32));
}
__device__ __forceinline__ uint32_t qbcast(uint32_t v, int src) {  // value of quad lane src (uniform src)
  switch (src) {
    case 0: return dppm<0x00>(v);
    case 1: return dppm<0x55>(v);
    case 2: return dppm<0xaa>(v);
    default: return dppm<0xff>(v);
  }
}
// cross-lane bitonic flip: element p of this lane against element 31-p of
// the partner (register 15-r, halves swapped); the lower lane keeps minima
template <int CTRL>
__device__ __forceinline__ void qflip(uint32_t *v, bool lower) {
  uint32_t o[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const uint32_t x = dppm<CTRL>(v[15 - r]);
    o[r] = __builtin_amdgcn_alignbit(x, x, 16);
  }
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const u16x2v a = __builtin_bit_cast(u16x2v, v[r]), b = __builtin_bit_cast(u16x2v, o[r]);
    v[r] = lower ? __builtin_bit_cast(uint32_t, __builtin_elementwise_min(a, b))
                 : __builtin_bit_cast(uint32_t, __builtin_elementwise_max(a, b));
  }
}
// cross-lane disperse: the same element of the partner lane
template <int CTRL>
__device__ __forceinline__ void qdisp(uint32_t *v, bool lower) {
  uint32_t o[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) o[r] = dppm<CTRL>(v[r]);
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const u16x2v a = __builtin_bit_cast(u16x2v, v[r]), b = __builtin_bit_cast(u16x2v, o[r]);
    v[r] = lower ? __builtin_bit_cast(uint32_t, __builtin_elementwise_min(a, b))
                 : __builtin_bit_cast(uint32_t, __builtin_elementwise_max(a, b));
  }
}
// element p <-> p + 16: the two halves of each register
__device__ __forceinline__ void half_ce16(uint32_t *v) {
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const uint32_t lo = v[r] & 0xffffu, hi = v[r] >> 16;
    v[r] = min(lo, hi) | (max(lo, hi) << 16);
  }
}
// exact sum of the c smallest samples of the token
__device__ __forceinline__ double quad_pref(const QuadLds &ql, int c) {
  double s_ = ql.pre4[c >> 2];
  const int n = c & 3;
  const uint2 w = *reinterpret_cast<const uint2 *>(ql.key + min(c & ~3, 124));
  const double a0 = kval(w.x & 0xffffu), a1 = kval(w.x >> 16), a2 = kval(w.y & 0xffffu);
  s_ = n > 0 ? s_ + a0 : s_;
  s_ = n > 1 ? s_ + a1 : s_;
  s_ = n > 2 ? s_ + a2 : s_;
  return s_;
}

// lane q's cut keys from its levels (slots s: level LPL*q + s): cut j lies
// between levels j and j+1; equal neighbours take the cut above (the first
// copy wins ties); the last cut and slots past it hold 0xffff
template <int L, int LPL>
__device__ __forceinline__ void quad_cut_keys(const float *lev, int q, uint32_t *t) {
  const float inf = __builtin_inff();
  const float nx0 = __uint_as_float(dppm<QPERM_NEXT>(__float_as_uint(lev[0])));
#pragma unroll
  for (int s_ = 0; s_ < LPL; ++s_) {
    const int j = LPL * q + s_;
    const float up = s_ + 1 < LPL ? lev[s_ + 1] : (q < 3 ? nx0 : inf);
    t[s_] = j < L - 1 ? (lev[s_] < up ? key16(thr16(lev[s_], up)) : 0u) : 0xffffu;
  }
  // a 0 takes the first nonzero cut above it: inside the lane, then across
  // lanes (each move runs in every lane before the select). Equal neighbours
  // are rare: the wave skips the fill when none of its tokens has any.
  bool zero = false;
#pragma unroll
  for (int s_ = 0; s_ < LPL; ++s_) zero |= t[s_] == 0;
  if (!__any(zero)) return;
#pragma unroll
  for (int s_ = LPL - 2; s_ >= 0; --s_) t[s_] = t[s_] ? t[s_] : t[s_ + 1];
#pragma unroll
  for (int step = 0; step < 3; ++step) {
    uint32_t nx = dppm<QPERM_NEXT>(t[0]);
    nx = q < 3 ? nx : 0xffffu;
    t[LPL - 1] = t[LPL - 1] ? t[LPL - 1] : nx;
#pragma unroll
    for (int s_ = LPL - 2; s_ >= 0; --s_) t[s_] = t[s_] ? t[s_] : t[s_ + 1];
  }
}

// odd-even transposition over the L levels held LPL per lane (slots past
// L hold +inf); the same network as sort_levels
template <int L, int LPL>
__device__ __forceinline__ void quad_sort_levels(float *lev, int q) {
  const float inf = __builtin_inff();
#pragma unroll
  for (int ph = 0; ph < L; ++ph) {
    if constexpr (LPL == 1) {
      if ((ph & 1) == 0) {  // pairs (0,1), (2,3): lane q with q ^ 1
        const float o = __uint_as_float(dppm<DPP_XOR1>(__float_as_uint(lev[0])));
        lev[0] = (q & 1) ? lmax(lev[0], o) : lmin(lev[0], o);
      } else {              // pair (1,2): lanes 1 and 2
        const float up = __uint_as_float(dppm<QPERM_NEXT>(__float_as_uint(lev[0])));
        const float dn = __uint_as_float(dppm<QPERM_PREV>(__float_as_uint(lev[0])));
        if (q == 1) lev[0] = lmin(lev[0], up);
        if (q == 2) lev[0] = lmax(lev[0], dn);
      }
    } else {
      if ((ph & 1) == 0) {  // pairs inside the lane: (0,1), (2,3), ...
#pragma unroll
        for (int s_ = 0; s_ + 1 < LPL; s_ += 2) {
          const float x = lev[s_], y = lev[s_ + 1];
          lev[s_] = lmin(x, y);
          lev[s_ + 1] = lmax(x, y);
        }
      } else {              // (1,2), ... inside the lane; (LPL-1, LPL) across lanes
        const float up = __uint_as_float(dppm<QPERM_NEXT>(__float_as_uint(lev[0])));
        const float dn = __uint_as_float(dppm<QPERM_PREV>(__float_as_uint(lev[LPL - 1])));
#pragma unroll
        for (int s_ = 1; s_ + 1 < LPL; s_ += 2) {
          const float x = lev[s_], y = lev[s_ + 1];
          lev[s_] = lmin(x, y);
          lev[s_ + 1] = lmax(x, y);
        }
        if (q < 3) lev[LPL - 1] = lmin(lev[LPL - 1], up);
        if (q > 0) lev[0] = lmax(lev[0], dn);
        (void)inf;
      }
    }
  }
}

template <int BITS>
__global__ __launch_bounds__(256) void nuq_value_quad(NuqArgs a) {
  constexpr int L = 1 << BITS;
  constexpr int LPL = L >= 4 ? L / 4 : 1;  // levels per lane
  constexpr int D = 128;
  __shared__ QuadLds qls[64];
  __shared__ uint32_t wtot[4];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int q = lane & 3, tq = threadIdx.x >> 2;  // quarter; token within the workgroup
  QuadLds &ql = qls[tq];
  const int64_t tok = (int64_t)blockIdx.x * 64 + tq;
  const int64_t ntok = (int64_t)a.BH * a.S;
  const bool valid = tok < ntok;
  const int s_pos = valid ? (int)(tok % a.S) : 0;
  const bool live = valid && s_pos >= a.n_sink_eff;  // sinks: exact, no fit
  const uint16_t *row = a.values + (size_t)(valid ? tok : 0) * D + 32 * q;
  // ---- this lane's 32 channels (element i in word i / 2)
  uint32_t raw[16];
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const uint4 w = valid ? *reinterpret_cast<const uint4 *>(row + 8 * g) : make_uint4(0, 0, 0, 0);
    raw[4 * g] = w.x; raw[4 * g + 1] = w.y; raw[4 * g + 2] = w.z; raw[4 * g + 3] = w.w;
  }
  // ---- sort the token's 128 keys: element p of the lane in register p % 16, half p / 16
  uint32_t v[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const uint32_t lo = (raw[r / 2] >> (16 * (r & 1))) & 0xffffu;
    const uint32_t hi = (raw[8 + r / 2] >> (16 * (r & 1))) & 0xffffu;
    v[r] = key_pair(lo | (hi << 16));
  }
  sort_regs<16>(v);
  qflip<DPP_XOR1>(v, (q & 1) == 0);  // pairs of lanes: 64 keys
  half_ce16(v);
  disp_down<16, 8>(v);
  qflip<QPERM_REV>(v, q < 2);        // the quad: 128 keys
  qdisp<DPP_XOR1>(v, (q & 1) == 0);
  half_ce16(v);
  disp_down<16, 8>(v);
  // lane q now holds sorted elements 32q .. 32q+31
  {
    uint32_t w[16];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      w[i] = __builtin_amdgcn_perm(v[2 * i + 1], v[2 * i], 0x05040100u);      // positions 2i, 2i+1
      w[8 + i] = __builtin_amdgcn_perm(v[2 * i + 1], v[2 * i], 0x07060302u);  // positions 16+2i, 17+2i
    }
    uint4 *kd = reinterpret_cast<uint4 *>(ql.key + 32 * q);
#pragma unroll
    for (int i = 0; i < 4; ++i) kd[i] = make_uint4(w[4 * i], w[4 * i + 1], w[4 * i + 2], w[4 * i + 3]);
    *reinterpret_cast<uint2 *>(ql.last8 + 4 * q) =
        make_uint2(__builtin_amdgcn_perm(v[15], v[7], 0x05040100u), __builtin_amdgcn_perm(v[15], v[7], 0x07060302u));
  }
  // exact prefix sums every 4th position: group sums of 4, their running
  // sum in the lane, the lanes below added by quad broadcasts
  {
    double g4[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int r0 = (4 * j) & 15, h = (4 * j) >> 4;
      double x[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) x[i] = kval((v[r0 + i] >> (16 * h)) & 0xffffu);
      g4[j] = (x[0] + x[1]) + (x[2] + x[3]);
    }
    double loc[8];
    loc[0] = 0.0;
#pragma unroll
    for (int j = 1; j < 8; ++j) loc[j] = loc[j - 1] + g4[j - 1];
    const double tot = loc[7] + g4[7];
    const double t0 = dppd_q<0x00>(tot), t1 = dppd_q<0x55>(tot), t2 = dppd_q<0xaa>(tot);
    double base = 0.0;
    base = q > 0 ? base + t0 : base;
    base = q > 1 ? base + t1 : base;
    base = q > 2 ? base + t2 : base;
    double *pd = ql.pre4 + 8 * q;
#pragma unroll
    for (int j = 0; j < 8; j += 2) *reinterpret_cast<double2 *>(pd + j) = make_double2(base + loc[j], base + loc[j + 1]);
    if (q == 3) ql.pre4[32] = base + tot;
  }
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
  // ---- tau: the (k+1)-th largest |x| (k = floor(frac * D), computed on the host):
  // the largest min(front_a, back_(k+1-a)) over the splits of the sorted ends
  uint32_t nneg2 = 0;
#pragma unroll
  for (int r = 0; r < 16; ++r) nneg2 += pk_gt01(0x80008000u, v[r]);  // keys below 0x8000: x < 0 or x = -0
  uint32_t nneg = (nneg2 & 0xffffu) + (nneg2 >> 16);
  nneg += dppm<DPP_XOR1>(nneg);
  nneg += dppm<DPP_XOR2>(nneg);
  const int kp1 = a.k_val + 1;
  uint32_t best = 0;
  for (int a0 = 0; a0 <= kp1; a0 += 4) {
    const int fa = a0 + q, fb = kp1 - fa;
    if (fa <= kp1 && fa <= (int)nneg && fb <= D - (int)nneg) {
      const uint32_t af = fa > 0 ? unkey16(ql.key[fa - 1]) & 0x7fffu : 0x8000u;
      const uint32_t ab = fb > 0 ? unkey16(ql.key[D - fb]) & 0x7fffu : 0x8000u;
      best = max(best, min(af, ab));
    }
  }
  best = max(best, dppm<DPP_XOR1>(best));
  best = max(best, dppm<DPP_XOR2>(best));
  const uint32_t tau = min(best, 0x7bffu);
  const uint32_t klo = tau == 0 ? key16(0x8000u) : key16(tau | 0x8000u);
  const int lo = lds_upper<D>(ql.key, ql.last8, klo - 1), hi = lds_upper<D>(ql.key, ql.last8, key16(tau));
  const int m = hi - lo;
  // ---- quantile initialisation: level j interpolates between the r-th and
  // (r+1)-th smallest inliers, r + f = (j + 1/2)(m - 1)/L
  const float inf = __builtin_inff();
  float lev[LPL];
#pragma unroll
  for (int s_ = 0; s_ < LPL; ++s_) {
    const int j = LPL * q + s_;
    lev[s_] = inf;
    if (j < L) {
      const long long num = (long long)(2 * j + 1) * (long long)(m - 1);
      const int r = (int)(num / (2 * L));
      const int rem = (int)(num % (2 * L));
      double val = kval(ql.key[lo + r]);
      if (rem != 0) val = val + ((double)rem / (double)(2 * L)) * (kval(ql.key[lo + r + 1]) - val);
      lev[s_] = (float)val + 0.0f;
    }
  }
  const double p_lo = quad_pref(ql, lo), p_hi = quad_pref(ql, hi);
  // ---- Lloyd iterations
  uint32_t t[LPL];
  for (int it = 0; it < a.iters; ++it) {
    quad_cut_keys<L, LPL>(lev, q, t);
    int cut[LPL];
    double pc[LPL];
#pragma unroll
    for (int s_ = 0; s_ < LPL; ++s_) {
      const int j = LPL * q + s_;
      cut[s_] = hi;
      pc[s_] = p_hi;
      if (j < L - 1) {
        cut[s_] = min(max(lds_upper<D>(ql.key, ql.last8, t[s_]), lo), hi);
        pc[s_] = quad_pref(ql, cut[s_]);
      }
    }
    // the cell of slot 0 starts at the previous lane's last cut (lane 0: lo)
    int cb = (int)dppm<QPERM_PREV>((uint32_t)cut[LPL - 1]);
    double pb = dppd_q<QPERM_PREV>(pc[LPL - 1]);
    cb = q > 0 ? cb : lo;
    pb = q > 0 ? pb : p_lo;
    bool empty = false;
#pragma unroll
    for (int s_ = 0; s_ < LPL; ++s_) {
      const int j = LPL * q + s_;
      const int cnt = cut[s_] - cb;
      if (j < L && cnt > 0) lev[s_] = (float)((pc[s_] - pb) / (double)cnt);
      empty |= j < L && cnt <= 0;
      cb = cut[s_];
      pb = pc[s_];
    }
    // an empty cell keeps its level while its neighbours move: keep the table
    // ordered. Without an empty cell the new table is already ascending (the
    // cells are ascending ranges of the sorted samples, so are their means),
    // and the sort would leave it as it is: the wave skips it then.
    if (__any(empty)) quad_sort_levels<L, LPL>(lev, q);
  }
  // ---- codes, reconstruction, level row
  quad_cut_keys<L, LPL>(lev, q, t);
  uint32_t T2[L - 1];
#pragma unroll
  for (int j = 0; j < L - 1; ++j) T2[j] = live ? qbcast(t[j % LPL], j / LPL) * 0x10001u : 0xffffffffu;
  uint32_t LH[L / 2];
#pragma unroll
  for (int i = 0; i < L / 2; ++i) {
    const float l0 = __uint_as_float(qbcast(__float_as_uint(lev[(2 * i) % LPL]), (2 * i) / LPL));
    const float l1 = __uint_as_float(qbcast(__float_as_uint(lev[(2 * i + 1) % LPL]), (2 * i + 1) / LPL));
    LH[i] = (uint32_t)f2h(l0) | ((uint32_t)f2h(l1) << 16);
  }
  if (valid) {
#pragma unroll
    for (int s_ = 0; s_ < LPL; ++s_) {
      const int j = LPL * q + s_;
      if (j < L) a.value_levels[(size_t)tok * L + j] = live ? lev[s_] : 0.0f;
    }
  }
  const uint32_t tau2 = (live ? tau : 0x7fffu) * 0x10001u;
  const uint32_t keep_in = live ? 0u : 0xffffffffu;
  const bool want_rec = valid && a.v_recon != nullptr;
  uint32_t ob[BITS + 1], om = 0, onum = 0;
#pragma unroll
  for (int i = 0; i <= BITS; ++i) ob[i] = 0;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    uint32_t rec[4];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int e = g * 8 + 2 * w;  // channel (within the lane) of the low half
      const uint32_t x = raw[4 * g + w];
      const uint32_t o = pk_gt01(x & 0x7fff7fffu, tau2);
      onum += o;
      om |= ((o & 1u) | (o >> 15)) << e;
      const uint32_t omask = pk_mask01(o);
      const uint32_t code = code_pair<BITS>(key_pair(x), T2) & ~omask;
      const uint32_t pcw = (code & 0xffffu) | (code >> (16 - BITS));
      const int bit = e * BITS;
      ob[bit / 32] |= pcw << (bit % 32);
      if (bit % 32 + 2 * BITS > 32) ob[bit / 32 + 1] |= pcw >> (32 - bit % 32);
      rec[w] = bsel(omask | keep_in, x, pick_lev16<L>(LH, code));
    }
    if (want_rec)
      *reinterpret_cast<uint4 *>(a.v_recon + (size_t)tok * D + 32 * q + 8 * g) = make_uint4(rec[0], rec[1], rec[2], rec[3]);
  }
  if (valid) {
    uint32_t *crow = reinterpret_cast<uint32_t *>(a.v_codes + (size_t)tok * (D * BITS / 8)) + q * BITS;
#pragma unroll
    for (int j = 0; j < BITS; ++j) crow[j] = ob[j];
  }
  // ---- side channel in flat order (lanes are in flat order): the
  // workgroup's fixed staging range holds k_val slots per token
  const int nout = (int)((onum & 0xffffu) + (onum >> 16));
  const uint32_t incl = kb_wscan((uint32_t)nout);
  if (lane == 63) wtot[wv] = incl;
  __syncthreads();
  uint32_t before = 0, btot = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    before += i < wv ? wtot[i] : 0u;
    btot += wtot[i];
  }
  const int64_t base = (int64_t)blockIdx.x * 64 * a.k_val;
  if (threadIdx.x == 0) {
    if (btot) atomicAdd(&a.ws_vsup[blockIdx.x >> 6], btot);
    a.ws_vblk[blockIdx.x * 2] = (uint32_t)base;
    a.ws_vblk[blockIdx.x * 2 + 1] = btot;
  }
  if (nout) {
    int64_t slot = base + before + incl - (uint32_t)nout;
    uint32_t mm = om;
    while (mm) {
      const int b = __builtin_ctz(mm);
      mm &= mm - 1;
      if (slot < a.v_scap) {
        a.ws_vpos[slot] = (int32_t)((size_t)tok * D + 32 * q + b);
        a.ws_vval[slot] = (uint16_t)(raw[b >> 1] >> (16 * (b & 1)));
      }
      ++slot;
    }
  }
}

// Value fit + quantize for few tokens (decode steps, short chunks): one wave
// per token, channel l*E + e in lane l (E = max(1, D/64)). The token's keys
// are sorted across the wave (bitonic network on packed 16-bit keys, sorted
// element i in lane i % 64, slot i / 64, two slots per register), with exact
// double prefix sums of the sorted values. Then every count is a ballot over
// the wave, tau is a bitwise search with ballot counts, the quantile order
// statistics are reads of the sorted keys, and a Lloyd cell sum is the
// difference of two prefix sums at its cut positions; the per-level work of
// an iteration (one cut threshold, one division) is spread over lanes and
// broadcast. The arithmetic is the same as in nuq_value.
template <int E>
__device__ __forceinline__ int wave_count(const bool (&p)[E]) {
  int c = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) c += __popcll(__ballot(p[e]));
  return c;
}
template <int L>
__device__ __forceinline__ float pick(const float (&v)[L], int i) {  // v[i] for a lane-varying i
  float r = v[0];
#pragma unroll
  for (int j = 1; j < L; ++j) {
    r = i == j ? v[j] : r;
    asm volatile("" : "+v"(r));  // keep the select chain in registers (no indexed scratch table)
  }
  return r;
}
template <int J>
__device__ __forceinline__ uint32_t lane_xor(uint32_t v) {  // value of lane ^ J
  if constexpr (J == 1) return dppm<DPP_XOR1>(v);
  else if constexpr (J == 2) return dppm<DPP_XOR2>(v);
  else if constexpr (J < 32) return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, (J << 10) | 0x1f);
  else return (uint32_t)__shfl_xor((int)v, 32);
}
// one bitonic stage (block K, distance J) over NS = 2R slots of 64 lanes
template <int R, int K, int J>
__device__ __forceinline__ void bstage(uint32_t (&v)[R], int lane) {
  if constexpr (J >= 128) {  // slots s and s ^ 2: registers 0 and 1; K = 256, ascending
    const u16x2v a = __builtin_bit_cast(u16x2v, v[0]), b = __builtin_bit_cast(u16x2v, v[1]);
    v[0] = __builtin_bit_cast(uint32_t, __builtin_elementwise_min(a, b));
    v[1] = __builtin_bit_cast(uint32_t, __builtin_elementwise_max(a, b));
  } else if constexpr (J == 64) {  // slots 2r and 2r+1: the two halves of register r
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const uint32_t lo = v[r] & 0xffffu, hi = v[r] >> 16;
      const bool asc = ((128 * r) & K) == 0;
      const uint32_t mn = min(lo, hi), mx = max(lo, hi);
      v[r] = asc ? (mn | (mx << 16)) : (mx | (mn << 16));
    }
  } else {  // partner lane ^ J, same slot
    const bool lower = (lane & J) == 0;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const uint32_t p = lane_xor<J>(v[r]);
      const u16x2v a = __builtin_bit_cast(u16x2v, v[r]), b = __builtin_bit_cast(u16x2v, p);
      const uint32_t mn = __builtin_bit_cast(uint32_t, __builtin_elementwise_min(a, b));
      const uint32_t mx = __builtin_bit_cast(uint32_t, __builtin_elementwise_max(a, b));
      const bool asc0 = ((lane + 64 * (2 * r)) & K) == 0, asc1 = ((lane + 64 * (2 * r + 1)) & K) == 0;
      const uint32_t sel = ((asc0 == lower) ? 0x0000ffffu : 0u) | ((asc1 == lower) ? 0xffff0000u : 0u);
      v[r] = (mn & sel) | (mx & ~sel);
    }
  }
}
template <int R, int K, int J>
__device__ __forceinline__ void bmerge(uint32_t (&v)[R], int lane) {
  bstage<R, K, J>(v, lane);
  if constexpr (J > 1) bmerge<R, K, J / 2>(v, lane);
}
template <int R, int K>
__device__ __forceinline__ void bsort(uint32_t (&v)[R], int lane) {
  if constexpr (K <= 128 * R) {
    bmerge<R, K, K / 2>(v, lane);
    bsort<R, 2 * K>(v, lane);
  }
}
// per-wave LDS of the one-wave-per-token value fit
struct alignas(16) WaveLds {
  uint16_t key[256];   // the token's order keys, ascending (absent channels 0xffff, last)
  uint16_t last8[32];  // last8[r] = key[8r + 7], the last key of each run of 8
  double pre[257];     // pre[i]: exact sum of the i smallest samples
  uint8_t cb[256];     // one code per channel
};


// lane j < L-1: cut key j between levels j and j+1 of the lane-distributed
// table (lane j holds level j, lanes >= L hold +inf); equal neighbours take
// the cut above them (the first copy wins ties), the last cut is above every
// finite key. Lanes >= L-1 return 0xffff.
template <int L>
__device__ __forceinline__ uint32_t lane_cut_key(float lev_me, int lane) {
  const float inf = __builtin_inff();
  const float lnext = __uint_as_float(kb_dpp<DPP_ROW_SHL1>(__float_as_uint(lev_me), __float_as_uint(inf)));
  uint32_t t = 0xffffu;
  if (lane < L - 1) t = lev_me < lnext ? key16(thr16(lev_me, lnext)) : 0u;
  if (!__any(t == 0u)) return t;  // no equal neighbours in the table (the common case)
  // a 0 takes the first nonzero key above it (lane L-1 holds 0xffff)
  // (row shifts by 1, 2, 4, 8: after the shift by s a lane holds the first
  // nonzero key among its next 2s - 1 neighbours). Each move runs in every
  // lane before the select: a DPP read from a lane that is switched off
  // returns the fill value.
  uint32_t u = kb_dpp<0x101>(t, 0xffffu);
  t = t ? t : u;
  if constexpr (L > 2) { u = kb_dpp<0x102>(t, 0xffffu); t = t ? t : u; }
  if constexpr (L > 4) { u = kb_dpp<0x104>(t, 0xffffu); t = t ? t : u; }
  if constexpr (L > 8) { u = kb_dpp<0x108>(t, 0xffffu); t = t ? t : u; }
  return t;
}

// One token per wave (E channels per lane). The token's keys are sorted
// across the wave (bitonic network on packed 16-bit keys) and kept in the
// wave's LDS with their exact prefix sums (DPP scans), so that every query
// of the fit is a read or a binary search there. Level j lives in lane j:
//  - tau, the (k+1)-th largest |x|: the largest samples by |x| are the two
//    ends of the sorted row (negatives from the front, the rest from the
//    back); taking a from the front and k+1-a from the back, the answer is
//    the largest min(front_a, back_(k+1-a)) over the splits, one split per
//    lane;
//  - the inliers are the sorted range [lo, hi) (ballot counts);
//  - quantile initialisation: lane j reads its two order statistics;
//  - a Lloyd iteration: lane j < L-1 computes cut key j from its neighbour
//    level (DPP), binary-searches it in the sorted keys and reads the prefix
//    sum there; lane q takes cut q-1 from its neighbour (DPP) and divides its
//    cell's exact sum by its count; an odd-even transposition over lanes
//    keeps the table ordered.
// The arithmetic is the same as in nuq_value. Every wave of the workgroup runs
// the body (inactive waves too); wl is the wave's own LDS.
template <int E, int BITS>
__device__ __forceinline__ void value_wave_body(const NuqArgs &a, int64_t tok, bool active, WaveLds &wl) {
  constexpr int L = 1 << BITS;
  constexpr int R = E == 4 ? 2 : 1;  // packed sort registers per lane
  constexpr int N = 64 * E;          // sorted slots
  const int lane = threadIdx.x & 63;
  const bool sink = !active || (int)(tok % a.S) < a.n_sink_eff;
  const int D = a.D;
  const uint16_t *row = a.values + (size_t)tok * D;
  uint32_t x[E];
  bool ok[E];
#pragma unroll
  for (int e = 0; e < E; ++e) ok[e] = active && lane * E + e < D;
#pragma unroll
  for (int e = 0; e < E; ++e) x[e] = 0;
  if (active) {
    if constexpr (E == 1) {
      x[0] = ok[0] ? row[lane] : 0u;
    } else if constexpr (E == 2) {
      const uint32_t w = *reinterpret_cast<const uint32_t *>(row + 2 * lane);
      x[0] = w & 0xffffu; x[1] = w >> 16;
    } else {
      const uint2 w = *reinterpret_cast<const uint2 *>(row + 4 * lane);
      x[0] = w.x & 0xffffu; x[1] = w.x >> 16; x[2] = w.y & 0xffffu; x[3] = w.y >> 16;
    }
  }
  uint32_t ky[E];
#pragma unroll
  for (int e = 0; e < E; ++e) ky[e] = key16(x[e]);
  const float inf = __builtin_inff();
  float lev_me = lane < L ? 0.0f : inf;  // level `lane` (lanes >= L: +inf)
  uint32_t tau = 0x7fffu;                // no outliers in sink tokens
  if (!sink) {
    // ---- sort the keys across the wave (absent channels are 0xffff and sort last)
    uint32_t v[R];
    if constexpr (E == 1) v[0] = (ok[0] ? ky[0] : 0xffffu) | 0xffff0000u;
    else if constexpr (E == 2) v[0] = ky[0] | (ky[1] << 16);
    else { v[0] = ky[0] | (ky[1] << 16); v[1] = ky[2] | (ky[3] << 16); }
    bsort<R, 2>(v, lane);
    // sorted element i sits in lane i % 64, slot i / 64 (slot s: register
    // s / 2, half s % 2); keys and exact prefix sums go to the wave's LDS
    double carry = 0.0;
    if (lane == 0) wl.pre[0] = 0.0;
#pragma unroll
    for (int sl = 0; sl < 2 * R; ++sl) {
      if (sl >= E && E < 2) break;  // E = 1: the high halves are padding
      const uint32_t kk = (sl & 1) ? (v[sl >> 1] >> 16) : (v[sl >> 1] & 0xffffu);
      wl.key[sl * 64 + lane] = (uint16_t)kk;
      if ((lane & 7) == 7) wl.last8[(sl * 64 + lane) >> 3] = (uint16_t)kk;
      const double inc = wscan_d(kk == 0xffffu ? 0.0 : kval(kk)) + carry;
      wl.pre[sl * 64 + lane + 1] = inc;
      carry = rl_d(inc, 63);
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
    // ---- tau: the (k+1)-th largest |x| (k = floor(frac * D) < D, computed on the host)
    const int kp1 = a.k_val + 1;
    bool neg[E];
#pragma unroll
    for (int e = 0; e < E; ++e) neg[e] = ok[e] && ky[e] < 0x8000u;  // x < 0 or x = -0
    const int nneg = wave_count<E>(neg);
    uint32_t best = 0;
    for (int a0 = 0; a0 <= kp1; a0 += 64) {
      const int fa = a0 + lane, fb = kp1 - fa;  // fa from the front, fb from the back
      if (fa <= kp1 && fa <= nneg && fb <= D - nneg) {
        const uint32_t af = fa > 0 ? unkey16(wl.key[fa - 1]) & 0x7fffu : 0x8000u;
        const uint32_t ab = fb > 0 ? unkey16(wl.key[D - fb]) & 0x7fffu : 0x8000u;
        best = max(best, min(af, ab));
      }
    }
    tau = min(gred_u32<64>(best, [](uint32_t p_, uint32_t q_) { return max(p_, q_); }), 0x7bffu);
    const uint32_t klo = tau == 0 ? key16(0x8000u) : key16(tau | 0x8000u);
    bool inl[E], below[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
      inl[e] = ok[e] && (x[e] & 0x7fffu) <= tau;
      below[e] = ok[e] && ky[e] < klo;
    }
    const int m = wave_count<E>(inl);
    const int lo = wave_count<E>(below), hi = lo + m;  // inliers: sorted positions [lo, hi)
    // ---- quantile initialisation: lane j interpolates between the r-th and
    // (r+1)-th smallest inliers, r + f = (j + 1/2)(m - 1)/L
    if (lane < L) {
      const long long num = (long long)(2 * lane + 1) * (long long)(m - 1);
      const int r = (int)(num / (2 * L));
      const int rem = (int)(num % (2 * L));
      double val = kval(wl.key[lo + r]);
      if (rem != 0) val = val + ((double)rem / (double)(2 * L)) * (kval(wl.key[lo + r + 1]) - val);
      lev_me = (float)val + 0.0f;
    }
    const double p_lo = wl.pre[lo], p_hi = wl.pre[hi];
    uint32_t l8[N / 16];  // the run ends, kept in registers for the searches
#pragma unroll
    for (int i = 0; i < N / 16; ++i) l8[i] = reinterpret_cast<const uint32_t *>(wl.last8)[i];
    // ---- Lloyd iterations
    for (int it = 0; it < a.iters; ++it) {
      const uint32_t t = lane_cut_key<L>(lev_me, lane);
      int cut = hi;
      double pc = p_hi;
      if (lane < L - 1) {
        cut = min(max(lds_upper_r<N>(l8, wl.key, t), lo), hi);
        pc = wl.pre[cut];
      }
      // cell q = (cut q-1, cut q]; lane 0 starts at lo
      const int c_lo = (int)kb_dpp<DPP_ROW_SHR1>((uint32_t)cut, (uint32_t)lo);
      const uint64_t pb = __builtin_bit_cast(uint64_t, pc), plb = __builtin_bit_cast(uint64_t, p_lo);
      const uint32_t pl_lo = kb_dpp<DPP_ROW_SHR1>((uint32_t)pb, (uint32_t)plb);
      const uint32_t pl_hi = kb_dpp<DPP_ROW_SHR1>((uint32_t)(pb >> 32), (uint32_t)(plb >> 32));
      const double p_below = __builtin_bit_cast(double, (uint64_t)pl_lo | ((uint64_t)pl_hi << 32));
      const int cnt = cut - c_lo;
      float nl = lev_me;
      if (lane < L && cnt > 0) nl = (float)((pc - p_below) / (double)cnt);
      // an empty cell keeps its level while its neighbours move: keep the
      // table ordered (odd-even transposition over lanes 0..L-1 with DPP
      // moves; lane 0 and lane 15 of the row sit out of the odd phases).
      // Without an empty cell the new means are already ascending: skipped.
      const bool any_empty = __any(lane < L && cnt <= 0);
#pragma unroll
      for (int ph = 0; ph < L && any_empty; ++ph) {
        const uint32_t xb = __float_as_uint(nl);
        if ((ph & 1) == 0) {  // pairs (0,1), (2,3), ...
          const float o = __uint_as_float(dppm<DPP_XOR1>(xb));
          nl = (lane & 1) ? lmax(nl, o) : lmin(nl, o);
        } else {              // pairs (1,2), (3,4), ...
          const float up = __uint_as_float(kb_dpp<DPP_ROW_SHL1>(xb, __float_as_uint(inf)));
          const float dn = __uint_as_float(kb_dpp<DPP_ROW_SHR1>(xb, __float_as_uint(-inf)));
          nl = (lane & 1) ? lmin(nl, up) : lmax(nl, dn);
        }
      }
      lev_me = lane < L ? nl : inf;
    }
  }
  // ---- codes, reconstruction, level row
  const uint32_t t_me = lane_cut_key<L>(lev_me, lane);
  uint32_t T[L - 1];
  float lev[L];
#pragma unroll
  for (int j = 0; j < L - 1; ++j) T[j] = kb_rl(t_me, j);
#pragma unroll
  for (int j = 0; j < L; ++j) lev[j] = __uint_as_float(kb_rl(__float_as_uint(lev_me), j));
  bool out[E];
  uint32_t code[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    out[e] = ok[e] && (x[e] & 0x7fffu) > tau;
    uint32_t c = 0;
#pragma unroll
    for (int j = 0; j < L - 1; ++j) c += ky[e] > T[j];
    code[e] = (sink || out[e]) ? 0u : c;
    if (ok[e]) wl.cb[lane * E + e] = (uint8_t)code[e];
  }
  if (a.v_recon) {
#pragma unroll
    for (int e = 0; e < E; ++e)
      if (ok[e])
        a.v_recon[(size_t)tok * D + lane * E + e] =
            (sink || out[e]) ? (uint16_t)x[e] : f2h(pick<L>(lev, (int)code[e]));
  }
  if (active && lane < L) a.value_levels[(size_t)tok * L + lane] = lev_me;  // 0 for sinks
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
  // codes LSB-first along D: lane w builds dword w of the row from the code
  // bytes c0 .. c1 that overlap it, read four at a time
  if (active && lane < D * BITS / 32) {
    const int bit0 = 32 * lane;
    const int c0 = bit0 / BITS, c1 = (bit0 + 31) / BITS;
    const int w0 = c0 >> 2, nw = (c1 >> 2) - w0 + 1;
    constexpr int MAXW = (32 / BITS + 1) / 4 + 2;  // dwords any lane needs
    const uint32_t *cw = reinterpret_cast<const uint32_t *>(wl.cb);
    uint32_t acc = 0;
#pragma unroll
    for (int i = 0; i < MAXW; ++i) {
      if (i < nw) {
        const uint32_t word = cw[w0 + i];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const int c = 4 * (w0 + i) + b, sh = c * BITS - bit0;
          const uint32_t byte = (word >> (8 * b)) & 0xffu;
          if (c >= c0 && c <= c1) acc |= sh >= 0 ? byte << sh : byte >> -sh;
        }
      }
    }
    reinterpret_cast<uint32_t *>(a.v_codes + (size_t)tok * (D * BITS / 8))[lane] = acc;
  }
  // ---- side channel: flat order is (lane, e)
  // (at most k_val outliers: the token's fixed staging range of k_val slots)
  const int nout = wave_count<E>(out);
  const int64_t base = tok * a.k_val;
  if (active && lane == 0) {
    if (nout && !a.small) atomicAdd(&a.ws_vsup[tok >> 6], (uint32_t)nout);
    a.ws_vblk[tok * 2] = (uint32_t)base;
    a.ws_vblk[tok * 2 + 1] = (uint32_t)nout;
  }
  int nb = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const uint64_t b = __ballot(out[e]);
    nb += (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(b >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)b, 0u));
  }
  int64_t slot = base + nb;
#pragma unroll
  for (int e = 0; e < E; ++e)
    if (out[e]) {
      if (slot < a.v_scap) {
        a.ws_vpos[slot] = (int32_t)((size_t)tok * D + lane * E + e);
        a.ws_vval[slot] = (uint16_t)x[e];
      }
      ++slot;
    }
}

template <int E, int BITS>
__global__ __launch_bounds__(64) void nuq_value_wave(NuqArgs a) {
  __shared__ WaveLds wl;
  value_wave_body<E, BITS>(a, blockIdx.x, true, wl);
}

// Both side-channel lists placed by one workgroup of 256 threads, the two
// lists side by side (threads 0..127 the key producers, 128..255 the value
// producers): exclusive scans of the producer counts in producer order, then
// each thread copies its producer's staged entries.
__device__ void place_all(const NuqArgs &a, int64_t kn, int64_t vn) {
  __shared__ uint32_t wsum[4];
  const int side = (int)(threadIdx.x >> 7), t = (int)(threadIdx.x & 127);
  const int64_t nblk = side ? vn : kn;
  const uint32_t *info = side ? a.ws_vblk : a.ws_kblk;
  const int32_t *spos = side ? a.ws_vpos : a.ws_kpos;
  const uint16_t *sval = side ? a.ws_vval : a.ws_kval;
  int32_t *opos = side ? a.v_opos : a.k_opos;
  uint16_t *oval = side ? a.v_oval : a.k_oval;
  const int64_t cap = side ? a.v_cap : a.k_cap, scap = side ? a.v_scap : a.k_scap;
  const int64_t nmax = kn > vn ? kn : vn;  // the same trip count on both sides (barriers)
  uint32_t running = 0;
  for (int64_t b0 = 0; b0 < nmax; b0 += 128) {
    const int64_t b = b0 + t;
    const uint32_t cnt = b < nblk ? info[2 * b + 1] : 0u;
    const uint32_t inc = kb_wscan(cnt);
    if ((threadIdx.x & 63) == 63) wsum[threadIdx.x >> 6] = inc;
    __syncthreads();
    const uint32_t w0 = wsum[2 * side], w1 = wsum[2 * side + 1];
    if (b < nblk) {
      const uint32_t off = running + ((threadIdx.x & 64) ? w0 : 0u) + inc - cnt, base = info[2 * b];
      for (uint32_t i = 0; i < cnt; ++i) {
        if ((int64_t)off + i >= cap || (int64_t)base + i >= scap) break;
        opos[off + i] = spos[base + i];
        oval[off + i] = sval[base + i];
      }
    }
    running += w0 + w1;
    __syncthreads();
  }
  if (t == 0) a.out_counts[side] = (int64_t)running;
}

// Small calls: key quantization and the value fits (one token per wave, four
// per workgroup) in one launch; workgroups [0, kn) quantize keys, the rest
// fit values. Every producer stages its outliers at a fixed offset, so no
// counter needs clearing; one workgroup of nuq_place_small then places both
// lists.
template <int E, int BITS>
__global__ __launch_bounds__(256) void nuq_small(NuqArgs a, int64_t kn, int64_t ntok) {
  __shared__ WaveLds wls[4];
  const int64_t b = blockIdx.x;
  if (b < kn) {
    key_quant_body<BITS>(a, (int)(b % a.k_blk_x), (int)(b / a.k_blk_x), b);
  } else {
    const int wv = threadIdx.x >> 6;
    const int64_t tok = (b - kn) * 4 + wv;
    value_wave_body<E, BITS>(a, tok < ntok ? tok : 0, tok < ntok, wls[wv]);
  }
}
__global__ __launch_bounds__(256) void nuq_place_small(NuqArgs a, int64_t kn, int64_t ntok) { place_all(a, kn, ntok); }

// Place the side-channel entries in flat order, keys and values in one
// launch: workgroups [0, kn) expand the key blocks' bitmaps, the rest move the
// value workgroups' staged entries. A producer workgroup b left its count in
// info[2b + 1] (a value workgroup also its staging base in info[2b]) and
// added it to sup[b/64]; the output offset of b is the sum of the counts
// before it, read as whole groups of 64 from sup plus single counts inside
// its own group. The last workgroup of each list writes the list length.
__global__ __launch_bounds__(256) void nuq_place(NuqArgs a, int64_t kn) {
  __shared__ uint32_t red[4];
  const bool isv = (int64_t)blockIdx.x >= kn;
  const int64_t b = isv ? (int64_t)blockIdx.x - kn : (int64_t)blockIdx.x;
  const int64_t nblk = isv ? a.v_nblk : kn;
  const uint32_t *info = isv ? a.ws_vblk : a.ws_kblk;
  const uint32_t *sup = isv ? a.ws_vsup : a.ws_ksup;
  const int64_t g0 = b >> 6;
  uint32_t part = 0;
  for (int64_t i = threadIdx.x; i < g0; i += 256) part += sup[i];
  for (int64_t i = (g0 << 6) + threadIdx.x; i < b; i += 256) part += info[2 * i + 1];
  for (int m = 1; m < 64; m <<= 1) part += (uint32_t)__shfl_xor((int)part, m);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = part;
  __syncthreads();
  const uint32_t off = red[0] + red[1] + red[2] + red[3];
  if (!isv) {
    // key block b: 16384/D rows of one (b, h), 2048 bitmap bytes in flat
    // order; thread t holds bytes [8t, 8t + 8) (elements 64t .. 64t + 63),
    // an exclusive prefix of the threads' counts orders the entries, and
    // each value is read back from the keys
    const int64_t bh = b / a.k_blk_x, RB = 16384 / a.D;
    const int64_t r0 = (b - bh * a.k_blk_x) * RB;
    const int64_t nbytes = (min(RB, (int64_t)a.S - r0)) * (a.D / 8);
    const int64_t e0 = ((int64_t)bh * a.S + r0) * a.D;  // flat index of the block's first element
    const uint32_t *bw = reinterpret_cast<const uint32_t *>(a.ws_kbits + e0 / 8);
    uint32_t m0 = 0, m1 = 0;
    if (8 * (int64_t)threadIdx.x < nbytes) {  // the rows' bytes come in whole 4-byte words (D/8 >= 4)
      m0 = bw[2 * threadIdx.x];
      if (8 * (int64_t)threadIdx.x + 4 < nbytes) m1 = bw[2 * threadIdx.x + 1];
    }
    const uint32_t c = (uint32_t)(__builtin_popcount(m0) + __builtin_popcount(m1));
    const uint32_t incl = kb_wscan(c);
    __syncthreads();
    if ((threadIdx.x & 63) == 63) red[threadIdx.x >> 6] = incl;
    __syncthreads();
    uint32_t pre = incl - c;
#pragma unroll
    for (int i = 0; i < 4; ++i) pre += i < (int)(threadIdx.x >> 6) ? red[i] : 0u;
    int64_t slot = (int64_t)off + pre;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      uint32_t m = h ? m1 : m0;
      while (m) {
        const int k = __builtin_ctz(m);
        m &= m - 1;
        const int64_t e = e0 + 64 * (int64_t)threadIdx.x + 32 * h + k;
        if (slot < a.k_cap) {  // holds by the outlier bound; never written past otherwise
          a.k_opos[slot] = (int32_t)e;
          a.k_oval[slot] = a.keys[e];
        }
        ++slot;
      }
    }
    if (b == nblk - 1 && threadIdx.x == 255) a.out_counts[0] = (int64_t)off + pre + c;  // the last thread's end
    return;
  }
  const uint32_t base = info[2 * b], cnt = info[2 * b + 1];
  const int32_t *spos = isv ? a.ws_vpos : a.ws_kpos;
  const uint16_t *sval = isv ? a.ws_vval : a.ws_kval;
  int32_t *opos = isv ? a.v_opos : a.k_opos;
  uint16_t *oval = isv ? a.v_oval : a.k_oval;
  const int64_t cap = isv ? a.v_cap : a.k_cap, scap = isv ? a.v_scap : a.k_scap;
  for (uint32_t i = threadIdx.x; i < cnt; i += 256) {
    if ((int64_t)off + i >= cap || (int64_t)base + i >= scap) break;
    opos[off + i] = spos[base + i];
    oval[off + i] = sval[base + i];
  }
  if (b == nblk - 1 && threadIdx.x == 0) a.out_counts[isv ? 1 : 0] = (int64_t)off + cnt;
}

// Workgroups go to the eight XCDs (each with its own L2) in turn by linear
// id. xcd_tile maps the id to a tile index such that consecutive tiles run
// on one XCD: XCD x = id % 8 takes tiles [x*q + min(x, r), ...) in order,
// q = n / 8, r = n % 8 (a bijection on [0, n)).
__device__ __forceinline__ uint32_t xcd_tile(uint32_t id, uint32_t n) {
  const uint32_t x = id & 7u, q = n >> 3, r = n & 7u;
  return x * q + min(x, r) + (id >> 3);
}

template <int L, bool LDS_DAT>
__global__ __launch_bounds__(KB_T) void nuq_key_fit_bk(NuqArgs a) {
  extern __shared__ uint64_t kb_lds[];
  uint64_t *tab = kb_lds;                                            // [KB_CH][257]
  uint32_t *cur = reinterpret_cast<uint32_t *>(tab + KB_CH * 257);   // [KB_CH][256]
  // per-wave histogram words: 16-bit counts with the samples in LDS (n <= KB_LDS_MAX_N)
  constexpr bool H16 = LDS_DAT;
  constexpr int KB_HW = H16 ? 128 : 256;
  uint32_t *hist = cur + KB_CH * 256;                                // [KB_CH][KB_HW]
  // the channel groups of one (b, h) read the same token rows: keep them on
  // one XCD so that its L2 fetches each row once
  const int ngrp = a.D / KB_CH;
  const int t = (int)xcd_tile(blockIdx.x, gridDim.x);
  const int bh = t / ngrp, d0 = (t - bh * ngrp) * KB_CH;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int t0 = a.n_sink_eff;
  const int n = a.S - t0;
  const int npad = (n + 15) & ~15;
  uint8_t *dat = LDS_DAT ? reinterpret_cast<uint8_t *>(hist + KB_CH * KB_HW)
                         : a.ws_kdat + ((size_t)bh * a.D + d0) * (size_t)npad;
  for (int i = tid; i < KB_CH * 257; i += KB_T) tab[i] = 0;
  __syncthreads();
  const uint16_t *kin = a.keys + ((size_t)bh * a.S + t0) * a.D + d0;
  // ---- bucket counts and significand sums (high word: count, low: sum).
  // KB_R row loads are in flight before their atomics; at step c lane l works
  // on channel (c + l) mod 8 of its row, so one instruction's atomics spread
  // over all eight channels' tables instead of piling onto one. With one
  // batch of rows per thread (n <= KB_T * KB_R) the rows stay in registers
  // for the scatter.
  constexpr int KB_R = 8;
  const int rot = lane & 7;
  const bool one_batch = n <= KB_T * KB_R;
  uint4 w4[KB_R];
  for (int tb = 0; tb < n; tb += KB_T * KB_R) {
#pragma unroll
    for (int r = 0; r < KB_R; ++r) {
      const int t = tb + tid + r * KB_T;
      w4[r] = t < n ? *reinterpret_cast<const uint4 *>(kin + (size_t)t * a.D) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int r = 0; r < KB_R; ++r) {
      if (tb + tid + r * KB_T >= n) continue;
#pragma unroll
      for (int c = 0; c < KB_CH; ++c) {
        const uint32_t h = kb_pick(w4[r], (c + rot) & 7);
        const uint32_t e = (h >> 10) & 31u;
        const uint32_t m = (h & 0x3ffu) | (e ? 0x400u : 0u);
        atomicAdd(&tab[((c + rot) & 7) * 257 + (key16(h) >> 8)], (1ull << 32) | m);
      }
    }
  }
  __syncthreads();
  // ---- per channel (wave w): exclusive prefixes of counts and exact sums
  {
    uint64_t *tb = tab + w * 257;
    uint32_t cnt[4];
    int64_t un[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int b = 4 * lane + i;
      const uint64_t x = tb[b];
      bool neg;
      int sh;
      uint32_t mbase;
      kb_bucket(b, neg, sh, mbase);
      cnt[i] = (uint32_t)(x >> 32);
      const int64_t u = (int64_t)((uint64_t)(uint32_t)x << sh);
      un[i] = neg ? -u : u;
    }
    uint32_t ce;
    int64_t ue;
    kb_excl(cnt[0] + cnt[1] + cnt[2] + cnt[3], (un[0] + un[1]) + (un[2] + un[3]), ce, ue);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int b = 4 * lane + i;
      cur[w * 256 + b] = ce;           // scatter cursor: starts at the bucket's first slot
      tb[b] = (uint64_t)ue;            // exact sum of the buckets below b
      ce += cnt[i];
      ue += un[i];
    }
    if (lane == 63) tb[256] = (uint64_t)ue;
  }
  __syncthreads();
  // ---- scatter the key low bytes (cursors end as bucket ends)
  for (int tb = 0; tb < n; tb += KB_T * KB_R) {
    if (!one_batch) {
#pragma unroll
      for (int r = 0; r < KB_R; ++r) {
        const int t = tb + tid + r * KB_T;
        w4[r] = t < n ? *reinterpret_cast<const uint4 *>(kin + (size_t)t * a.D) : make_uint4(0, 0, 0, 0);
      }
    }
#pragma unroll
    for (int r = 0; r < KB_R; ++r) {
      if (tb + tid + r * KB_T >= n) continue;
#pragma unroll
      for (int c = 0; c < KB_CH; ++c) {
        const int ch = (c + rot) & 7;
        const uint32_t k = key16(kb_pick(w4[r], ch));
        const uint32_t pos = atomicAdd(&cur[ch * 256 + (k >> 8)], 1u);
        dat[(size_t)ch * npad + pos] = (uint8_t)k;
      }
    }
  }
  __syncthreads();
  // ---- the fit of channel d0 + w by wave w: tau, inliers, initial levels
  KbView<const uint8_t *, H16> v{tab + w * 257, cur + w * 256, dat + (size_t)w * npad, hist + w * KB_HW};
  float mine;
  uint16_t tau;
  KbInl inl;
  kb_init<L>(v, (uint32_t)n, a.k_key, mine, tau, inl);
  const size_t ch = (size_t)bh * a.D + d0 + w;
  if (lane == 0) a.key_thresh[ch] = tau;
  if constexpr (L > KB_ROW_MAX_L) {
    if (n > 0) kb_lloyd_wave<L>(v, inl, a.iters, mine);
    if (lane < L) a.key_levels[ch * L + lane] = mine;
  } else {
    // ---- Lloyd iterations by rows: wave w hands its channel over in its
    // histogram words (free now: the level table, then the inlier range), and
    // waves 0 .. KB_CH/CPW - 1 take CPW channels each
    static_assert(KB_CH % 4 == 0 && 16 * 4 + sizeof(KbInl) <= 128 * 4, "row slots");
    float *slot = reinterpret_cast<float *>(hist + w * KB_HW);
    if (lane < L) slot[lane] = mine;
    if (lane == 0) *reinterpret_cast<KbInl *>(slot + 16) = inl;
    __syncthreads();
    constexpr int CPW = 64 / KB_G;  // channels per wave
    if (w >= KB_CH / CPW) return;
    const int c = CPW * w + lane / KB_G, gl = lane & (KB_G - 1);
    float *cs = reinterpret_cast<float *>(hist + c * KB_HW);
    const KbInl r = *reinterpret_cast<const KbInl *>(cs + 16);
    float lev[L];
#pragma unroll
    for (int j = 0; j < L; ++j) lev[j] = cs[j];
    if (n > 0) kb_lloyd_rows<L, KB_G>(tab + c * 257, cur + c * 256, dat + (size_t)c * npad, cs, r, a.iters, lev);
    float out = 0.0f;
#pragma unroll
    for (int j = 0; j < L; ++j) out = gl == j ? lev[j] : out;
    if (gl < L) a.key_levels[((size_t)bh * a.D + d0 + c) * L + gl] = out;
  }
}

// ================================================================== launch
namespace {
template <int L>
hipError_t launch_key_fit(const NuqArgs &a, int /*cpc*/, hipStream_t st) {
  const int n = a.S - a.n_sink_eff;
  const dim3 grid((unsigned)(a.D / KB_CH) * (unsigned)a.BH);
  const size_t tables = (size_t)KB_CH * 257 * 8 + (size_t)KB_CH * 256 * 4 * 2;  // 32-bit histograms
  if (n <= KB_LDS_MAX_N) {  // bucketed samples in LDS, 16-bit histograms (n < 65536)
    static_assert(KB_LDS_MAX_N < 65536, "16-bit histogram counts");
    hipLaunchKernelGGL((nuq_key_fit_bk<L, true>), grid, dim3(KB_T),
                       tables - (size_t)KB_CH * 128 * 4 + (size_t)KB_CH * ((n + 15) & ~15), st, a);
  } else {                  // in the workspace
    hipLaunchKernelGGL((nuq_key_fit_bk<L, false>), grid, dim3(KB_T), tables, st, a);
  }
  return hipGetLastError();
}
// The value fit reads nothing the key kernels write, so for many tokens it
// runs on a second stream of the device, forked from the caller's stream at
// the start of the call and joined before the placement kernel: the two fits
// then share the machine instead of running back to back. The key fit is
// submitted first, right after the fork point: it heads the longer chain (key
// fit, key quantization, placement), and the value workgroups take the LDS
// the key fit leaves free (two key-fit workgroups with 16-bit histograms
// leave room for one value workgroup per CU). Submitted the other way round,
// the value fit filled the CUs first and delayed the key fit (prefill 0.205
// -> 0.185 ms in a kernel trace). The counters are cleared on the second
// stream ahead of the value fit, and the key quantization waits for that
// clear (a third event), so that no launch stands between the fork point and
// the key fit. One stream and three events per device, created on first use
// (default priority); the fork/join section is serialised on the host so
// that concurrent callers never interleave their event records.
struct Fork {
  hipStream_t aux = nullptr;
  hipEvent_t fork = nullptr, join = nullptr, zero = nullptr;
};
std::mutex g_fork_mu;
Fork g_fork[64];
hipError_t fork_for_device(Fork *&f) {  // g_fork_mu held
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  f = &g_fork[dev];
  if (f->aux == nullptr) {
    if ((e = hipEventCreateWithFlags(&f->fork, hipEventDisableTiming)) != hipSuccess) return e;
    if ((e = hipEventCreateWithFlags(&f->join, hipEventDisableTiming)) != hipSuccess) return e;
    if ((e = hipEventCreateWithFlags(&f->zero, hipEventDisableTiming)) != hipSuccess) return e;
    if ((e = hipStreamCreateWithFlags(&f->aux, hipStreamNonBlocking)) != hipSuccess) return e;
  }
  return hipSuccess;
}

template <int BITS>
hipError_t launch_values(const NuqArgs &a, int val_cpc, hipStream_t st) {
  if (val_cpc == 0) {  // one wave per token
    if (a.D <= 64)
      hipLaunchKernelGGL((nuq_value_wave<1, BITS>), dim3((unsigned)a.v_nblk), dim3(64), 0, st, a);
    else if (a.D == 128)
      hipLaunchKernelGGL((nuq_value_wave<2, BITS>), dim3((unsigned)a.v_nblk), dim3(64), 0, st, a);
    else
      hipLaunchKernelGGL((nuq_value_wave<4, BITS>), dim3((unsigned)a.v_nblk), dim3(64), 0, st, a);
  } else if (val_cpc == 1 && a.D == 128) {  // one token per quad of lanes
    hipLaunchKernelGGL((nuq_value_quad<BITS>), dim3((unsigned)a.v_nblk), dim3(256), 0, st, a);
  } else if (val_cpc == 1) {
    hipLaunchKernelGGL((nuq_value<1, BITS>), dim3((unsigned)a.v_nblk), dim3(64), 0, st, a);
  } else {
    hipLaunchKernelGGL((nuq_value<2, BITS>), dim3((unsigned)a.v_nblk), dim3(64), 0, st, a);
  }
  return hipGetLastError();
}

template <int BITS>
hipError_t launch_bits(const NuqArgs &a, int key_cpc, int val_cpc, bool fork, hipStream_t st) {
  constexpr int L = 1 << BITS;
  hipError_t e;
  const int64_t ntok = (int64_t)a.BH * a.S;
  if (a.small) {  // decode-sized: key quant and values in one launch, then the placement
    if (a.fit_keys && (e = launch_key_fit<L>(a, key_cpc, st)) != hipSuccess) return e;
    const int64_t kn = a.k_blk_x * (int64_t)a.BH;
    const dim3 grid((unsigned)(kn + (ntok + 3) / 4));
    if (a.D <= 64)
      hipLaunchKernelGGL((nuq_small<1, BITS>), grid, dim3(256), 0, st, a, kn, ntok);
    else if (a.D == 128)
      hipLaunchKernelGGL((nuq_small<2, BITS>), grid, dim3(256), 0, st, a, kn, ntok);
    else
      hipLaunchKernelGGL((nuq_small<4, BITS>), grid, dim3(256), 0, st, a, kn, ntok);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(nuq_place_small, dim3(1), dim3(256), 0, st, a, kn, ntok);
    return hipGetLastError();
  }
  const dim3 zgrid((unsigned)std::min<int64_t>(
      (std::max<int64_t>(a.k_blk_x * a.BH, a.v_nblk) / 64 + 4095) / 4096 + 1, 256));
  if (val_cpc == 0 || !fork) {  // few tokens (a cross-stream join costs more than it hides), or one stream asked for
    hipLaunchKernelGGL(nuq_zero, zgrid, dim3(256), 0, st, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (a.fit_keys && (e = launch_key_fit<L>(a, key_cpc, st)) != hipSuccess) return e;
    hipLaunchKernelGGL((nuq_key_quant<BITS>), dim3((unsigned)a.k_blk_x, a.BH), dim3(256), 0, st, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if ((e = launch_values<BITS>(a, val_cpc, st)) != hipSuccess) return e;
  } else {
    // the key fit starts first, right after the fork point; the sums are
    // cleared on the second stream ahead of the value fit, and the key
    // quantization (their other user) waits for that
    std::lock_guard<std::mutex> lock(g_fork_mu);
    Fork *f = nullptr;
    if ((e = fork_for_device(f)) != hipSuccess) return e;
    if ((e = hipEventRecord(f->fork, st)) != hipSuccess) return e;
    if (a.fit_keys && (e = launch_key_fit<L>(a, key_cpc, st)) != hipSuccess) return e;
    if ((e = hipStreamWaitEvent(f->aux, f->fork, 0)) != hipSuccess) return e;
    hipLaunchKernelGGL(nuq_zero, zgrid, dim3(256), 0, f->aux, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if ((e = hipEventRecord(f->zero, f->aux)) != hipSuccess) return e;
    if ((e = launch_values<BITS>(a, val_cpc, f->aux)) != hipSuccess) return e;
    if ((e = hipEventRecord(f->join, f->aux)) != hipSuccess) return e;
    if ((e = hipStreamWaitEvent(st, f->zero, 0)) != hipSuccess) return e;
    hipLaunchKernelGGL((nuq_key_quant<BITS>), dim3((unsigned)a.k_blk_x, a.BH), dim3(256), 0, st, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if ((e = hipStreamWaitEvent(st, f->join, 0)) != hipSuccess) return e;
  }
  const int64_t k_nblk = a.k_blk_x * (int64_t)a.BH;
  hipLaunchKernelGGL(nuq_place, dim3((unsigned)(k_nblk + a.v_nblk)), dim3(256), 0, st, a, k_nblk);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_nuq(const NuqArgs &a, int key_cpc, int val_cpc, bool fork, hipStream_t st) {
  switch (a.bits) {
    case 1: return launch_bits<1>(a, key_cpc, val_cpc, fork, st);
    case 2: return launch_bits<2>(a, key_cpc, val_cpc, fork, st);
    case 3: return launch_bits<3>(a, key_cpc, val_cpc, fork, st);
    default: return launch_bits<4>(a, key_cpc, val_cpc, fork, st);
  }
}

}  // namespace kvq
