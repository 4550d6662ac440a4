// CPU oracle for the KV-cache quantize -> pack -> unpack -> dequantize path.
//
// TEST INFRASTRUCTURE ONLY. This file is the slow, plain, single-threaded
// reference that the GPU library is checked against. Only the test suite, the
// smoke check and the CPU-baseline leg of the benchmark may load it; the
// product library never does, and the two share no code, header or table.
//
// Build: g++ -std=c++17 -O2 -ffp-contract=off -fPIC -shared (no fast-math), so
// every float operation below is one IEEE-754 binary32 operation rounded to
// nearest-even, in the order written.
//
// Sources (cited by page title and section):
//  [P1] MTPLX pull request #267, "feat(kv-cache): add q6 paged KV quantization"
//       -- PR description (symmetric quantizer, q6 byte equations, packed_dim,
//       storage arithmetic) and its "Summary"/"Implementation" blocks.
//  [P2] "veloxquant_mlx.cache.kvquant_cache module" -- module docstring
//       (quantization axes, level lifecycle, byte accounting, attention-sink
//       quantization) and the KVQuantKVCache class/property docs.
//  [P3] "veloxquant_mlx.cache.kivi_cache" module source -- KIVIKVCache,
//       methods _quant_dequant_along and _quantization_boundary.
//
// Where the pages leave a step open, the reading taken is stated at the
// function. Parity status of each function is listed in the test suite:
//  - fp16 conversion, symmetric, KIVI, NUQ: pinned (see tests/test_oracle_*).
//  - paged geometry, q8/q4 byte order, NUQ outlier-list order: parity
//    unpinned by the pages (fixed only by the readings stated here).

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <vector>

namespace {

// ---------------------------------------------------------------- fp16 <-> fp32
// IEEE binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits.

float h2f(uint16_t h) {
  uint32_t sign = (uint32_t)(h & 0x8000u) << 16;
  uint32_t e = (h >> 10) & 0x1fu;
  uint32_t m = h & 0x3ffu;
  uint32_t bits;
  if (e == 0) {
    if (m == 0) {
      bits = sign;
    } else {
      // subnormal: value = m * 2^-24; normalise into binary32.
      int shift = 0;
      while ((m & 0x400u) == 0) {
        m <<= 1;
        ++shift;
      }
      m &= 0x3ffu;
      bits = sign | ((uint32_t)(127 - 14 - shift) << 23) | (m << 13);
    }
  } else if (e == 31) {
    bits = sign | 0x7f800000u | (m << 13);
  } else {
    bits = sign | ((e - 15 + 127) << 23) | (m << 13);
  }
  float f;
  std::memcpy(&f, &bits, 4);
  return f;
}

// binary32 -> binary16, round to nearest, ties to even; gradual underflow;
// overflow to +-inf; NaN stays NaN.
uint16_t f2h(float f) {
  uint32_t x;
  std::memcpy(&x, &f, 4);
  uint32_t sign = (x >> 16) & 0x8000u;
  uint32_t e8 = (x >> 23) & 0xffu;
  uint32_t man = x & 0x7fffffu;
  if (e8 == 0xffu) return (uint16_t)(sign | 0x7c00u | (man ? 0x200u | (man >> 13) : 0u));
  if (e8 == 0) return (uint16_t)sign;  // binary32 zero/subnormal: far below 2^-25
  int e = (int)e8 - 127;
  if (e > 15) return (uint16_t)(sign | 0x7c00u);
  if (e >= -14) {
    uint32_t h = ((uint32_t)(e + 15) << 10) | (man >> 13);
    uint32_t rem = man & 0x1fffu;
    if (rem > 0x1000u || (rem == 0x1000u && (h & 1u))) ++h;  // may carry to inf
    return (uint16_t)(sign | h);
  }
  // result is a binary16 subnormal q * 2^-24 (or rounds to 0 / min normal)
  uint32_t m = man | 0x800000u;  // value = m * 2^(e-23)
  int shift = -e - 1;            // q = m * 2^(e+1) = m >> shift
  if (shift > 24) return (uint16_t)sign;
  uint32_t q = m >> shift;
  uint32_t rem = m & ((1u << shift) - 1u);
  uint32_t half = 1u << (shift - 1);
  if (rem > half || (rem == half && (q & 1u))) ++q;
  return (uint16_t)(sign | q);
}

// ---------------------------------------------------------------- symmetric
// [P1] PR description: one symmetric quantizer per (token, KV head) row with
// one fp16 scale; the clip bound is the only thing that changes between
// widths, and the width->bound map is an explicit table that rejects widths
// it does not know.
int sym_qmax(int bits) {
  switch (bits) {
    case 8: return 127;
    case 6: return 31;
    case 4: return 7;
    default: return -1;
  }
}

// [P1] PR description: packed_dim(D, bits) = D*bits/8 bytes per row; q6 needs
// D % 4 == 0 (four codes per three bytes); q4 stores two codes per byte
// ("Summary" block), so it needs an even D; q8 one code per byte.
long long packed_dim(int D, int bits) {
  if (D <= 0) return -1;
  if (bits == 8) return D;
  if (bits == 6) return (D % 4 == 0) ? (long long)D * 3 / 4 : -1;
  if (bits == 4) return (D % 2 == 0) ? D / 2 : -1;
  return -1;
}

// Quantise one row x[0..D) into its packed bytes and its fp16 scale.
// Reading (pages silent on the exact expression): the scale is the row's
// absolute maximum divided by qmax in binary32 and stored as fp16; codes are
// computed against that stored fp16 scale by multiplying with its binary32
// reciprocal, rounding half-to-even, then clipping to [-qmax, qmax]. An
// all-zero row (scale 0) gets all-zero codes.
void sym_quant_row(const uint16_t *x, int D, int bits, uint8_t *out, uint16_t *scale_out) {
  const int qmax = sym_qmax(bits);
  float amax = 0.0f;
  for (int i = 0; i < D; ++i) {
    float a = std::fabs(h2f(x[i]));
    if (a > amax) amax = a;
  }
  float s32 = amax / (float)qmax;
  uint16_t s16 = f2h(s32);
  float s = h2f(s16);
  std::vector<int> q(D, 0);
  if (s != 0.0f) {
    float r = 1.0f / s;
    for (int i = 0; i < D; ++i) {
      float t = h2f(x[i]) * r;
      float v = std::nearbyint(t);  // default rounding mode: nearest, ties to even
      if (v > (float)qmax) v = (float)qmax;
      if (v < (float)-qmax) v = (float)-qmax;
      q[i] = (int)v;
    }
  }
  *scale_out = s16;
  if (bits == 8) {
    // [P1] "Summary": q8 keeps one code per byte; stored as two's-complement int8.
    for (int i = 0; i < D; ++i) out[i] = (uint8_t)(int8_t)q[i];
  } else if (bits == 6) {
    // [P1] PR description: bias +32 into a 6-bit field, then each group of
    // four fields u0..u3 becomes three little-endian bytes per the page's
    // byte equations.
    for (int g = 0; g < D / 4; ++g) {
      unsigned u0 = (unsigned)(q[4 * g + 0] + 32), u1 = (unsigned)(q[4 * g + 1] + 32);
      unsigned u2 = (unsigned)(q[4 * g + 2] + 32), u3 = (unsigned)(q[4 * g + 3] + 32);
      out[3 * g + 0] = (uint8_t)((u0 | ((u1 & 0x03u) << 6)) & 0xffu);
      out[3 * g + 1] = (uint8_t)(((u1 >> 2) | ((u2 & 0x0fu) << 4)) & 0xffu);
      out[3 * g + 2] = (uint8_t)(((u2 >> 4) | ((u3 & 0x3fu) << 2)) & 0xffu);
    }
  } else {
    // Reading for q4 ("two per byte", layout not stated): bias +8 into a
    // nibble, even element in the low nibble (same little-endian order as q6).
    for (int j = 0; j < D / 2; ++j) {
      unsigned lo = (unsigned)(q[2 * j] + 8), hi = (unsigned)(q[2 * j + 1] + 8);
      out[j] = (uint8_t)(lo | (hi << 4));
    }
  }
}

// Unpack a row's codes back to signed integers (inverse of the packing above).
void sym_unpack_row(const uint8_t *in, int D, int bits, int *q) {
  if (bits == 8) {
    for (int i = 0; i < D; ++i) q[i] = (int)(int8_t)in[i];
  } else if (bits == 6) {
    for (int g = 0; g < D / 4; ++g) {
      unsigned b0 = in[3 * g], b1 = in[3 * g + 1], b2 = in[3 * g + 2];
      unsigned u0 = b0 & 0x3fu;
      unsigned u1 = (b0 >> 6) | ((b1 & 0x0fu) << 2);
      unsigned u2 = (b1 >> 4) | ((b2 & 0x03u) << 4);
      unsigned u3 = b2 >> 2;
      q[4 * g + 0] = (int)u0 - 32;
      q[4 * g + 1] = (int)u1 - 32;
      q[4 * g + 2] = (int)u2 - 32;
      q[4 * g + 3] = (int)u3 - 32;
    }
  } else {
    for (int j = 0; j < D / 2; ++j) {
      q[2 * j] = (int)(in[j] & 0x0fu) - 8;
      q[2 * j + 1] = (int)(in[j] >> 4) - 8;
    }
  }
}

// [P1] PR description: reading back dequantises code * scale to fp16 before
// attention. Product formed in binary32, stored with round-to-nearest-even.
void sym_dequant_row(const uint8_t *in, uint16_t scale, int D, int bits, uint16_t *out) {
  std::vector<int> q(D);
  sym_unpack_row(in, D, bits, q.data());
  float s = h2f(scale);
  for (int i = 0; i < D; ++i) out[i] = f2h((float)q[i] * s);
}

// ---------------------------------------------------------------- KIVI
// [P3] _quant_dequant_along: asymmetric min/max quantisation of groups of
// `gs` consecutive elements along one axis, in binary32, with levels = 2^b-1,
// scale = max((max-min)/levels, eps), code = clip(round((x-min)/scale), 0,
// levels) with round half-to-even, recon = code*scale + min (a product then a
// sum, not fused), cast back to fp16. A last group shorter than gs behaves as
// the page's edge-replicating pad does: the replicated element changes
// neither the min nor the max, and padded outputs are dropped.
void kivi_group(float *vals, int n, int levels, float eps, int *codes, float *scale_out,
                float *min_out) {
  float mn = vals[0], mx = vals[0];
  for (int i = 1; i < n; ++i) {
    if (vals[i] < mn) mn = vals[i];
    if (vals[i] > mx) mx = vals[i];
  }
  float scale = (mx - mn) / (float)levels;
  if (scale < eps) scale = eps;
  for (int i = 0; i < n; ++i) {
    float t = (vals[i] - mn) / scale;
    float c = std::nearbyint(t);
    if (c < 0.0f) c = 0.0f;
    if (c > (float)levels) c = (float)levels;
    codes[i] = (int)c;
    float prod = c * scale;
    vals[i] = prod + mn;
  }
  *scale_out = scale;
  *min_out = mn + 0.0f;  // reading: a zero group minimum is exported as +0
}

void put_code(uint8_t *row, int d, int bits, int code) {
  // codes packed LSB-first along the channel axis: element d occupies bits
  // [d*bits, (d+1)*bits) of the row read as one little-endian bit string
  for (int b = 0; b < bits; ++b) {
    long bit = (long)d * bits + b;
    if ((code >> b) & 1) row[bit / 8] = (uint8_t)(row[bit / 8] | (1u << (bit % 8)));
  }
}

// ---------------------------------------------------------------- NUQ helpers
// Exact fixed-point view of the numbers the NUQ fit compares: every fp16
// value and every level produced below is an integer multiple of 2^-90 of
// magnitude < 2^37, so distances are compared exactly as 128-bit integers.
typedef __int128 i128;

i128 to_fixed(double v) {
  double s = std::ldexp(v, 90);
  i128 r = (i128)s;
  if ((double)r != s) std::abort();  // outside the exact domain: refuse to guess
  return r;
}

i128 iabs(i128 v) { return v < 0 ? -v : v; }

// index of the nearest level to u; ties go to the lower index [reading]
int nearest_level(double u, const float *lev, int L) {
  i128 uf = to_fixed(u);
  int best = 0;
  i128 bd = iabs(uf - to_fixed((double)lev[0]));
  for (int j = 1; j < L; ++j) {
    i128 d = iabs(uf - to_fixed((double)lev[j]));
    if (d < bd) {
      bd = d;
      best = j;
    }
  }
  return best;
}

// round-to-nearest-even binary32 of the rational sum/count, sum in 2^-24
// units. long double (64-bit significand) holds any int64 sum exactly and its
// quotient rounded to 64 bits then to 24 bits equals the direct rounding
// (64 >= 2*24+2).
float mean_rn32(long long sum_units, long long count) {
  long double q = (long double)sum_units / (long double)count;
  float f = (float)q;
  return f * 0x1p-24f;
}

// [P2] module docstring, "Level lifecycle" / "Performance": levels are fit by
// Lloyd-Max iterations (the unweighted k-means special case). Steps, in the
// pages' order: quantile initialisation [reading: linear-interpolated sample
// quantiles at probabilities (j+1/2)/L, evaluated exactly in double and
// rounded once to binary32], then `iters` rounds of (assign every sample to
// its nearest level, ties to the lower index; replace every non-empty level
// by the binary32-rounded exact mean of its samples; an empty level keeps its
// value; then the table is sorted ascending). u: the inlier samples (fp16 bit
// patterns, any order).
void nuq_fit(const uint16_t *u_bits, int m, int L, int iters, float *lev) {
  if (m == 0) {
    for (int j = 0; j < L; ++j) lev[j] = 0.0f;
    return;
  }
  std::vector<double> u(m);
  for (int i = 0; i < m; ++i) u[i] = (double)h2f(u_bits[i]);
  std::sort(u.begin(), u.end());
  for (int j = 0; j < L; ++j) {
    // position (j + 1/2)/L * (m-1) = (2j+1)(m-1) / (2L), split exactly
    long long num = (long long)(2 * j + 1) * (long long)(m - 1);
    long long den = 2LL * L;
    long long i = num / den;
    double f = (double)(num % den) / (double)den;
    double v = u[i];
    if (f != 0.0) v = u[i] + f * (u[i + 1] - u[i]);
    lev[j] = (float)v + 0.0f;  // reading: a zero level is +0 (the sort does not order -0/+0)
  }
  std::vector<long long> sum(L), cnt(L);
  for (int it = 0; it < iters; ++it) {
    std::fill(sum.begin(), sum.end(), 0LL);
    std::fill(cnt.begin(), cnt.end(), 0LL);
    for (int i = 0; i < m; ++i) {
      int j = nearest_level(u[i], lev, L);
      sum[j] += (long long)std::ldexp(u[i], 24);
      cnt[j] += 1;
    }
    for (int j = 0; j < L; ++j)
      if (cnt[j] > 0) lev[j] = mean_rn32(sum[j], cnt[j]);
    // reading: the level table stays an ordered table ("signpost" table on
    // the kvquant_cache page). A cell left empty keeps its level, so when the
    // quantile initialisation produced duplicates the lower copy can move past
    // its frozen twin; re-sorting after each update keeps the order.
    std::stable_sort(lev, lev + L);
  }
}

// [P2] "dense-and-sparse" outlier isolation per vector: with n samples and a
// nominal fraction f, k = floor(f*n) [reading]; the threshold tau is the
// (k+1)-th largest |x| and a sample is an outlier when |x| > tau, so at most k
// samples per vector are isolated ("nominal" vs "realized" count). n == 0
// gives tau = 0. Returns tau as an fp16 bit pattern.
// The fraction is a binary64 number: the page's configuration field
// kvquant_outlier_fraction is a Python float (default 0.01), and f*n is one
// binary64 product, so 1% of 100 samples is exactly 1.
uint16_t nuq_threshold(const uint16_t *x_bits, int n, double frac) {
  if (n == 0) return 0;
  long long k = (long long)std::floor(frac * (double)n);
  if (k < 0 || k >= n) std::abort();  // callers keep 0 <= frac < 1
  std::vector<uint16_t> a(n);
  for (int i = 0; i < n; ++i) a[i] = (uint16_t)(x_bits[i] & 0x7fffu);
  // for non-negative finite fp16, bit-pattern order is numeric order
  std::sort(a.begin(), a.end(), [](uint16_t p, uint16_t q) { return p > q; });
  return a[(size_t)k];
}

bool is_outlier(uint16_t x, uint16_t tau) { return h2f((uint16_t)(x & 0x7fffu)) > h2f(tau); }

}  // namespace

extern "C" {

// ------------------------------------------------------------ exported: fp16
float orc_h2f(uint16_t h) { return h2f(h); }
uint16_t orc_f2h(float f) { return f2h(f); }
void orc_h2f_array(const uint16_t *h, float *f, long long n) {
  for (long long i = 0; i < n; ++i) f[i] = h2f(h[i]);
}
void orc_f2h_array(const float *f, uint16_t *h, long long n) {
  for (long long i = 0; i < n; ++i) h[i] = f2h(f[i]);
}

// ------------------------------------------------------------ exported: symmetric
int orc_sym_qmax(int bits) { return sym_qmax(bits); }
long long orc_packed_dim(int D, int bits) { return packed_dim(D, bits); }

// [P1] PR description, storage arithmetic: bytes of K+V per token for the
// whole cache, codes plus one fp16 scale per (token, head) row, or fp16 rows
// when bits == 16.
long long orc_sym_cache_bytes(long long tokens, int layers, int kv_heads, int D, int bits) {
  long long row = (bits == 16) ? 2LL * D : packed_dim(D, bits) + 2;
  if (bits != 16 && packed_dim(D, bits) < 0) return -1;
  return 2LL * tokens * layers * kv_heads * row;
}

// rows: n_rows independent rows of D fp16 values.
int orc_sym_quant_rows(const uint16_t *x, long long n_rows, int D, int bits, uint8_t *codes,
                       uint16_t *scales) {
  long long pd = packed_dim(D, bits);
  if (sym_qmax(bits) < 0 || pd < 0) return -1;
  for (long long r = 0; r < n_rows; ++r) sym_quant_row(x + r * D, D, bits, codes + r * pd, scales + r);
  return 0;
}

int orc_sym_dequant_rows(const uint8_t *codes, const uint16_t *scales, long long n_rows, int D,
                         int bits, uint16_t *out) {
  long long pd = packed_dim(D, bits);
  if (sym_qmax(bits) < 0 || pd < 0) return -1;
  for (long long r = 0; r < n_rows; ++r) sym_dequant_row(codes + r * pd, scales[r], D, bits, out + r * D);
  return 0;
}

int orc_sym_unpack_rows(const uint8_t *codes, long long n_rows, int D, int bits, int *q) {
  long long pd = packed_dim(D, bits);
  if (sym_qmax(bits) < 0 || pd < 0) return -1;
  for (long long r = 0; r < n_rows; ++r) sym_unpack_row(codes + r * pd, D, bits, q + r * D);
  return 0;
}

// Paged write for ONE layer. [P1] PR description: pages are allocated in
// packed_dim-sized rows. Reading (page geometry not stated): codes are laid
// out [page][slot][head][packed_dim] and scales [page][slot][head], addressed
// by a global slot index page*page_size + slot per token (slot_mapping); a
// negative entry or one beyond the pool marks a token that is not written.
// x: fp16 [n_tokens][H][D].
int orc_sym_quant_paged(const uint16_t *x, int n_tokens, int H, int D, int bits,
                        const int32_t *slot_mapping, long long n_slots, uint8_t *codes,
                        uint16_t *scales) {
  long long pd = packed_dim(D, bits);
  if (sym_qmax(bits) < 0 || pd < 0) return -1;
  for (int t = 0; t < n_tokens; ++t) {
    long long slot = slot_mapping[t];
    if (slot < 0 || slot >= n_slots) continue;
    for (int h = 0; h < H; ++h) {
      long long row = slot * H + h;
      sym_quant_row(x + ((long long)t * H + h) * D, D, bits, codes + row * pd, scales + row);
    }
  }
  return 0;
}

// Paged read for ONE layer: out fp16 [n_seqs][max_len][H][D]; position p of
// sequence s reads page block_table[s][p / page_size], slot p % page_size.
// Reading: positions at or beyond the sequence length, and positions whose
// page id is outside [0, num_pages), are written as +0.
int orc_sym_dequant_paged(const uint8_t *codes, const uint16_t *scales, int num_pages,
                          int page_size, int H, int D, int bits, const int32_t *block_table,
                          int max_blocks, const int32_t *seq_lens, int n_seqs, int max_len,
                          uint16_t *out) {
  long long pd = packed_dim(D, bits);
  if (sym_qmax(bits) < 0 || pd < 0) return -1;
  for (int s = 0; s < n_seqs; ++s) {
    for (int p = 0; p < max_len; ++p) {
      uint16_t *o = out + ((long long)s * max_len + p) * H * D;
      int blk = p / page_size;
      bool valid = p < seq_lens[s] && blk < max_blocks;
      long long page = valid ? block_table[(long long)s * max_blocks + blk] : -1;
      if (!valid || page < 0 || page >= num_pages) {
        std::memset(o, 0, sizeof(uint16_t) * H * D);
        continue;
      }
      long long slot = page * page_size + p % page_size;
      for (int h = 0; h < H; ++h)
        sym_dequant_row(codes + (slot * H + h) * pd, scales[slot * H + h], D, bits, o + (long long)h * D);
    }
  }
  return 0;
}

// ------------------------------------------------------------ exported: KIVI
// [P3] _quantization_boundary: tokens older than the residual window are
// eligible, snapped down to a whole number of groups.
long long orc_kivi_boundary(long long offset, int residual_length, int group_size) {
  long long aged = offset - residual_length;
  if (aged < 0) aged = 0;
  return (aged / group_size) * group_size;
}

// In-place KIVI round trip of the token slice [lo, hi) of x, fp16
// [B][H][S_cap][D]. per_channel = 1: keys, groups of gs tokens along the
// token axis, one group per channel ([P3] module docstring: keys per channel,
// values per token); per_channel = 0: values, groups of gs channels per token.
// Optional outputs (NULL to skip): codes packed LSB-first along D,
// [B][H][hi-lo][D*bits/8]; binary32 scale and min per group, laid out
// [B][H][ceil((hi-lo)/gs)][D] for keys and [B][H][hi-lo][ceil(D/gs)] for
// values.
int orc_kivi_round_trip(uint16_t *x, int B, int H, int S_cap, int D, int lo, int hi,
                        int per_channel, int bits, int gs, float eps, uint8_t *codes,
                        float *scale_out, float *min_out) {
  if (bits < 1 || bits > 8 || gs <= 0 || lo < 0 || hi < lo || hi > S_cap || D <= 0) return -1;
  const int levels = (1 << bits) - 1;
  const int n = hi - lo;
  const long long cpr = ((long long)D * bits + 7) / 8;  // code bytes per token row
  if (codes) std::memset(codes, 0, (size_t)((long long)B * H * n * cpr));
  std::vector<float> buf(std::max(gs, 1));
  std::vector<int> cbuf(std::max(gs, 1));
  for (int b = 0; b < B; ++b) {
    for (int h = 0; h < H; ++h) {
      long long bh = (long long)b * H + h;
      uint16_t *base = x + bh * S_cap * D;
      if (per_channel) {
        int ng = (n + gs - 1) / gs;
        for (int g = 0; g < ng; ++g) {
          int t0 = lo + g * gs, t1 = std::min(t0 + gs, hi);
          for (int d = 0; d < D; ++d) {
            int cnt = t1 - t0;
            for (int t = t0; t < t1; ++t) buf[t - t0] = h2f(base[(long long)t * D + d]);
            float sc, mn;
            kivi_group(buf.data(), cnt, levels, eps, cbuf.data(), &sc, &mn);
            for (int t = t0; t < t1; ++t) {
              base[(long long)t * D + d] = f2h(buf[t - t0]);
              if (codes) put_code(codes + (bh * n + (t - lo)) * cpr, d, bits, cbuf[t - t0]);
            }
            if (scale_out) scale_out[(bh * ng + g) * D + d] = sc;
            if (min_out) min_out[(bh * ng + g) * D + d] = mn;
          }
        }
      } else {
        int ng = (D + gs - 1) / gs;
        for (int t = lo; t < hi; ++t) {
          for (int g = 0; g < ng; ++g) {
            int d0 = g * gs, d1 = std::min(d0 + gs, D);
            for (int d = d0; d < d1; ++d) buf[d - d0] = h2f(base[(long long)t * D + d]);
            float sc, mn;
            kivi_group(buf.data(), d1 - d0, levels, eps, cbuf.data(), &sc, &mn);
            for (int d = d0; d < d1; ++d) {
              base[(long long)t * D + d] = f2h(buf[d - d0]);
              if (codes) put_code(codes + (bh * n + (t - lo)) * cpr, d, bits, cbuf[d - d0]);
            }
            long long pidx = (bh * n + (t - lo)) * ng + g;
            if (scale_out) scale_out[pidx] = sc;
            if (min_out) min_out[pidx] = mn;
          }
        }
      }
    }
  }
  return 0;
}

// ------------------------------------------------------ exported: KIVI packed
// Packed KIVI storage: b-bit codes plus one fp16 (scale, zero) pair per
// group, the layout the page's byte accounting charges for
// ["veloxquant_mlx.cache.kivi_cache", module docstring on per-token storage
// at bit-width b and group size g, and _quantized_bytes]. The group math is
// that of _quant_dequant_along with the parameters rounded to fp16 before
// use, so that the stored pair reproduces the codes:
//   scale = max(RN32((max - min)/levels), eps) rounded to fp16 toward zero,
//           so that the top level min + levels*scale never exceeds the
//           group's max (rounding to nearest can push it past the fp16
//           range: at b = 8 a group spanning +-65504 would reconstruct its
//           max as +inf); a result of 0 becomes 2^-24, the smallest positive
//           fp16 (the page's 1e-8 floor is not representable in fp16);
//   zero  = min (an fp16 value already, stored exactly; -0 as +0);
//   code  = clip(round_half_even(RN32(RN32(x - zero) / scale)), 0, levels);
//   recon = RN16(RN32(code * scale) + zero).
void kivi_group_p16(const float *vals, int n, int levels, float eps, int *codes, uint16_t *s16,
                    uint16_t *z16) {
  float mn = vals[0], mx = vals[0];
  for (int i = 1; i < n; ++i) {
    if (vals[i] < mn) mn = vals[i];
    if (vals[i] > mx) mx = vals[i];
  }
  float scale = (mx - mn) / (float)levels;
  if (scale < eps) scale = eps;
  uint16_t sh = f2h(scale);
  if (h2f(sh) > scale) --sh;  // toward zero (scale > 0: one step down the bit pattern)
  if (sh == 0) sh = 1;        // 2^-24
  const float s = h2f(sh);
  for (int i = 0; i < n; ++i) {
    float t = (vals[i] - mn) / s;
    float c = std::nearbyint(t);
    if (c < 0.0f) c = 0.0f;
    if (c > (float)levels) c = (float)levels;
    codes[i] = (int)c;
  }
  *s16 = sh;
  *z16 = f2h(mn + 0.0f);
}

// Quantize tokens [lo, hi) of x, fp16 [B][H][S_cap][D] (not modified), into
// packed storage indexed by absolute token: codes [B][H][S_cap][D*bits/8]
// (LSB-first along D), keys (per_channel = 1, groups of gs tokens from token
// 0; lo must be a multiple of gs) scale/zero fp16 [B][H][ceil(S_cap/gs)][D],
// values (per_channel = 0, groups of gs channels) scale/zero fp16
// [B][H][S_cap][ceil(D/gs)]. Codes outside [lo, hi) are left as they are.
int orc_kivi_pack(const uint16_t *x, int B, int H, int S_cap, int D, int lo, int hi, int per_channel,
                  int bits, int gs, float eps, uint8_t *codes, uint16_t *scale16, uint16_t *zero16) {
  if (bits < 1 || bits > 8 || gs <= 0 || lo < 0 || hi < lo || hi > S_cap || D <= 0) return -1;
  if ((long long)D * bits % 8) return -1;
  if (per_channel && lo % gs) return -1;
  const int levels = (1 << bits) - 1;
  const long long cpr = (long long)D * bits / 8;
  std::vector<float> buf(std::max(gs, 1));
  std::vector<int> cbuf(std::max(gs, 1));
  for (long long bh = 0; bh < (long long)B * H; ++bh) {
    const uint16_t *base = x + bh * S_cap * D;
    uint8_t *crow = codes + bh * S_cap * cpr;
    for (int t = lo; t < hi; ++t) std::memset(crow + (long long)t * cpr, 0, (size_t)cpr);
    if (per_channel) {
      const int ngc = (S_cap + gs - 1) / gs;
      for (int t0 = lo; t0 < hi; t0 += gs) {
        const int t1 = std::min(t0 + gs, hi);
        for (int d = 0; d < D; ++d) {
          for (int t = t0; t < t1; ++t) buf[t - t0] = h2f(base[(long long)t * D + d]);
          uint16_t sh, zh;
          kivi_group_p16(buf.data(), t1 - t0, levels, eps, cbuf.data(), &sh, &zh);
          for (int t = t0; t < t1; ++t) put_code(crow + (long long)t * cpr, d, bits, cbuf[t - t0]);
          scale16[(bh * ngc + t0 / gs) * D + d] = sh;
          zero16[(bh * ngc + t0 / gs) * D + d] = zh;
        }
      }
    } else {
      const int ng = (D + gs - 1) / gs;
      for (int t = lo; t < hi; ++t) {
        for (int g = 0; g < ng; ++g) {
          const int d0 = g * gs, d1 = std::min(d0 + gs, D);
          for (int d = d0; d < d1; ++d) buf[d - d0] = h2f(base[(long long)t * D + d]);
          uint16_t sh, zh;
          kivi_group_p16(buf.data(), d1 - d0, levels, eps, cbuf.data(), &sh, &zh);
          for (int d = d0; d < d1; ++d) put_code(crow + (long long)t * cpr, d, bits, cbuf[d - d0]);
          scale16[(bh * S_cap + t) * ng + g] = sh;
          zero16[(bh * S_cap + t) * ng + g] = zh;
        }
      }
    }
  }
  return 0;
}

// Reconstruct tokens [lo, hi) from packed storage (layouts as above) into
// out, fp16 [B][H][S_cap][D] at the same token positions:
// RN16(RN32(code * scale) + zero).
int orc_kivi_unpack(const uint8_t *codes, const uint16_t *scale16, const uint16_t *zero16, int B, int H,
                    int S_cap, int D, int lo, int hi, int per_channel, int bits, int gs, uint16_t *out) {
  if (bits < 1 || bits > 8 || gs <= 0 || lo < 0 || hi < lo || hi > S_cap || D <= 0) return -1;
  if ((long long)D * bits % 8) return -1;
  const long long cpr = (long long)D * bits / 8;
  const int ngc = (S_cap + gs - 1) / gs, ng = (D + gs - 1) / gs;
  for (long long bh = 0; bh < (long long)B * H; ++bh) {
    for (int t = lo; t < hi; ++t) {
      const uint8_t *row = codes + (bh * S_cap + t) * cpr;
      for (int d = 0; d < D; ++d) {
        int c = 0;
        for (int b = 0; b < bits; ++b) {
          const long bit = (long)d * bits + b;
          c |= ((row[bit / 8] >> (bit % 8)) & 1) << b;
        }
        const long long p = per_channel ? (bh * ngc + t / gs) * D + d : (bh * S_cap + t) * ng + d / gs;
        const float prod = (float)c * h2f(scale16[p]);
        out[(bh * S_cap + t) * D + d] = f2h(prod + h2f(zero16[p]));
      }
    }
  }
  return 0;
}

// ------------------------------------------------------------ exported: NUQ
// Lloyd fit of one vector of inlier samples (used directly by the pins).
void orc_nuq_fit(const uint16_t *u, int m, int L, int iters, float *levels) {
  nuq_fit(u, m, L, iters, levels);
}
uint16_t orc_nuq_threshold(const uint16_t *x, int n, double frac) { return nuq_threshold(x, n, frac); }
int orc_nuq_nearest(uint16_t u, const float *levels, int L) {
  return nearest_level((double)h2f(u), levels, L);
}

// One KVQuant-style call over fp16 keys/values [BH][S][D].
// [P2] module docstring: keys get per-channel levels (sample axis = tokens),
// values per-token levels (sample axis = channels); prefill fits key levels
// and the key |x| thresholds and freezes them, later tokens reuse them
// (fit_keys = 0); value levels are fit fresh on every call. Attention-sink
// tokens ("Attention Sink-Aware quantization"): the first n_sink tokens of a
// sequence -- present only in the call that starts it, start_pos == 0 --
// stay exact fp16 and are left out of every fit and threshold.
// Outputs: codes packed LSB-first along D ([BH][S][D*bits/8]); outliers and
// sinks take code 0. Outlier side channel [reading]: (int32 flat index into
// this call's [BH][S][D], fp16 value), ascending index, keys and values in
// separate lists, counts in out_counts[0..1]. Returns -2 when a list would
// exceed out_cap. recon (optional): inliers -> fp16 of their level,
// outliers and sinks -> x.
int orc_nuq_fit_quant(const uint16_t *keys, const uint16_t *values, int BH, int S, int D,
                      int start_pos, int bits, double frac, int iters, int n_sink, int fit_keys,
                      float *key_levels, uint16_t *key_thresh, float *value_levels,
                      uint8_t *k_codes, uint8_t *v_codes, int32_t *k_opos, uint16_t *k_oval,
                      int32_t *v_opos, uint16_t *v_oval, long long out_cap,
                      long long *out_counts, uint16_t *k_recon, uint16_t *v_recon) {
  if (bits < 1 || bits > 4 || BH <= 0 || S <= 0 || D <= 0 || ((long long)D * bits) % 8 != 0)
    return -1;
  if (!(frac >= 0.0 && frac < 1.0) || iters < 0) return -1;
  const int L = 1 << bits;
  const long long cpr = (long long)D * bits / 8;
  const int n_sink_eff = (start_pos == 0) ? std::min(std::max(n_sink, 0), S) : 0;
  std::memset(k_codes, 0, (size_t)((long long)BH * S * cpr));
  std::memset(v_codes, 0, (size_t)((long long)BH * S * cpr));
  std::vector<uint8_t> k_out((size_t)BH * S * D, 0), v_out((size_t)BH * S * D, 0);
  std::vector<int> k_code((size_t)BH * S * D, 0), v_code((size_t)BH * S * D, 0);
  std::vector<uint16_t> tmp;
  // ---- keys: per channel over the non-sink tokens of this call
  for (int bh = 0; bh < BH; ++bh) {
    for (int d = 0; d < D; ++d) {
      float *lev = key_levels + ((long long)bh * D + d) * L;
      auto at = [&](int s) { return ((long long)bh * S + s) * D + d; };
      if (fit_keys) {
        tmp.clear();
        for (int s = n_sink_eff; s < S; ++s) tmp.push_back(keys[at(s)]);
        uint16_t tau = nuq_threshold(tmp.data(), (int)tmp.size(), frac);
        std::vector<uint16_t> inl;
        for (uint16_t v : tmp)
          if (!is_outlier(v, tau)) inl.push_back(v);
        nuq_fit(inl.data(), (int)inl.size(), L, iters, lev);
        key_thresh[(long long)bh * D + d] = tau;
      }
      uint16_t tau = key_thresh[(long long)bh * D + d];
      for (int s = n_sink_eff; s < S; ++s) {
        uint16_t v = keys[at(s)];
        if (is_outlier(v, tau)) {
          k_out[at(s)] = 1;
        } else {
          k_code[at(s)] = nearest_level((double)h2f(v), lev, L);
        }
      }
    }
  }
  // ---- values: per token over its D channels, fit on every call
  for (int bh = 0; bh < BH; ++bh) {
    for (int s = 0; s < S; ++s) {
      float *lev = value_levels + ((long long)bh * S + s) * L;
      const uint16_t *row = values + ((long long)bh * S + s) * D;
      if (s < n_sink_eff) {
        for (int j = 0; j < L; ++j) lev[j] = 0.0f;
        continue;
      }
      uint16_t tau = nuq_threshold(row, D, frac);
      std::vector<uint16_t> inl;
      for (int d = 0; d < D; ++d)
        if (!is_outlier(row[d], tau)) inl.push_back(row[d]);
      nuq_fit(inl.data(), (int)inl.size(), L, iters, lev);
      for (int d = 0; d < D; ++d) {
        long long idx = ((long long)bh * S + s) * D + d;
        if (is_outlier(row[d], tau))
          v_out[idx] = 1;
        else
          v_code[idx] = nearest_level((double)h2f(row[d]), lev, L);
      }
    }
  }
  // ---- codes, side channel, reconstruction
  long long nk = 0, nv = 0;
  for (long long idx = 0; idx < (long long)BH * S * D; ++idx) {
    long long row = idx / D;
    int d = (int)(idx % D);
    int s = (int)(row % S);
    bool sink = s < n_sink_eff;
    put_code(k_codes + row * cpr, d, bits, k_code[idx]);
    put_code(v_codes + row * cpr, d, bits, v_code[idx]);
    if (k_out[idx]) {
      if (nk >= out_cap) return -2;
      k_opos[nk] = (int32_t)idx;
      k_oval[nk] = keys[idx];
      ++nk;
    }
    if (v_out[idx]) {
      if (nv >= out_cap) return -2;
      v_opos[nv] = (int32_t)idx;
      v_oval[nv] = values[idx];
      ++nv;
    }
    if (k_recon) {
      const float *lev = key_levels + ((row / S) * D + d) * L;
      k_recon[idx] = (sink || k_out[idx]) ? keys[idx] : f2h(lev[k_code[idx]]);
    }
    if (v_recon) {
      const float *lev = value_levels + row * L;
      v_recon[idx] = (sink || v_out[idx]) ? values[idx] : f2h(lev[v_code[idx]]);
    }
  }
  out_counts[0] = nk;
  out_counts[1] = nv;
  return 0;
}

}  // extern "C"
