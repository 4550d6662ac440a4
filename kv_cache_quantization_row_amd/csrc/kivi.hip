// KIVI asymmetric min/max group round trip, in place on fp16 [BH][S_cap][D].
//
// ["veloxquant_mlx.cache.kivi_cache" module source, KIVIKVCache and its
//  _quant_dequant_along] keys are grouped per channel along tokens, values
// per token along channels; per group in binary32: levels = 2^b - 1,
// scale = max((max - min)/levels, eps), code = clip(round_half_even((x -
// min)/scale), 0, levels), recon = code*scale + min (product, then sum),
// stored back as fp16. Only tokens [lo, hi) are touched; key groups start at
// lo. A short last group is its own group.
//
// Layout on the GPU (fast paths; D/8 a power of two dividing 64):
//  keys   one wave per (bh, group of gs tokens): the gs x D tile is read with
//         16-byte loads, lane l holding channels 8*(l % CL).. of tokens
//         l / CL + TPI*j (CL = D/8 lanes per token row, TPI = 64/CL rows per
//         load). Per-channel min/max reduce first over the lane's own tokens,
//         then across the lanes that share l % CL (DPP rotate for 8, lane
//         shuffles for 16/32).
//  values lane l holds channels 8*(l % CL).. of token row l / CL; a group of
//         gs channels is gs/8 consecutive lanes, reduced with DPP.
// Other shapes use one-thread-per-(vector, group) generic kernels.
//
// Packed storage (the b-bit codes and fp16 (scale, zero) per group that the
// page's byte accounting charges, module docstring and _quantized_bytes):
// the same kernels instantiated for packed storage round each scale toward zero to fp16
// (at least 2^-24) before computing the codes, write fp16 parameters and
// codes indexed by absolute token, and leave the fp16 input untouched;
// kivi_unpack rebuilds fp16(code*scale + zero) from them.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace kvq {

// One element: returns the fp16 reconstruction, writes the integer code.
__device__ __forceinline__ uint16_t kivi_elem(float x, float mn, float scale, float levels,
                                              uint32_t &code) {
  const float t = (x - mn) / scale;  // IEEE division, as the page computes it
  const float c = __builtin_amdgcn_fmed3f(__builtin_rintf(t), 0.0f, levels);
  code = (uint32_t)c;
  const float prod = c * scale;
  return f2h(prod + mn);
}

__device__ __forceinline__ float kivi_scale(float mn, float mx, float levels, float eps) {
  const float s = (mx - mn) / levels;
  return fmaxf(s, eps);
}

// Pack 8 codes of `bits` bits LSB-first into the low 8*bits bits.
template <int BITS>
__device__ __forceinline__ uint64_t pack8(const uint32_t *c) {
  uint64_t v = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) v |= (uint64_t)c[i] << (BITS * i);
  return v;
}

template <int BITS>
__device__ __forceinline__ void store_codes8(uint8_t *dst, const uint32_t *c) {
  const uint64_t v = pack8<BITS>(c);
  if constexpr (BITS == 2) *reinterpret_cast<uint16_t *>(dst) = (uint16_t)v;
  else if constexpr (BITS == 4) *reinterpret_cast<uint32_t *>(dst) = (uint32_t)v;
  else *reinterpret_cast<uint64_t *>(dst) = v;
}

// ----- exact quotient via the group's reciprocal
// t' = RN(a * RN(1/scale)) is within 2^-22 |a/scale| of the IEEE quotient
// RN(a/scale) (two roundings of 2^-24 each, plus the quotient's own). If t'
// is farther than (levels+2)*2^-21 from every half-integer, t' and the IEEE
// quotient round (ties-to-even) to the same integer, and beyond levels+1.5
// both clamp to levels. Otherwise the IEEE division is done; on this
// workload about 1e-4 of the elements take that branch.
// RN(x / levels) for x >= 0 without a division: x*RN(1/levels) corrected by
// one fused remainder step. Checked against IEEE division for every
// non-negative finite binary32 x and levels 3, 15 and 255 (all plain IEEE
// operations, so the check holds on any conforming device).
template <int BITS>
__device__ __forceinline__ float div_levels(float x) {
  constexpr float LEV = (float)((1 << BITS) - 1);
  constexpr float Y = 1.0f / LEV;
  const float q0 = x * Y;
  const float r = __builtin_fmaf(-q0, LEV, x);
  return __builtin_fmaf(r, Y, q0);
}
// reciprocal of a scale (>= eps) to within 2^-23 relative: hardware estimate
// plus one Newton step. Only used for the tie-guarded quotient below, whose
// margin covers that error.
__device__ __forceinline__ float recip(float s) {
  const float y0 = __builtin_amdgcn_rcpf(s);
  const float e = __builtin_fmaf(-s, y0, 1.0f);
  return __builtin_fmaf(e, y0, y0);
}
template <int BITS>
__device__ __forceinline__ float kivi_scale_c(float mn, float mx, float eps) {
  return fmaxf(div_levels<BITS>(mx - mn), eps);
}

// a binary32 scale rounded toward zero to fp16, at least 2^-24 (packed
// storage: the top level zero + levels*scale stays within the group's max)
__device__ __forceinline__ float scale_p16(float s) {
  uint16_t h = f2h(s);
  if (h2f(h) > s) --h;  // s > 0: one step down the bit pattern
  if (h == 0) h = 1;
  return h2f(h);
}

// Eight elements at a time: the quotients a[i]*inv[i] and their tie flags
// are computed branch-free; only if some lane of the wave has a flagged
// element in this group of eight does the wave redo the group with IEEE
// divisions (one wave-uniform branch per group).
template <int BITS>
__device__ __forceinline__ void kivi_codes8(const float *a, const float *scale, const float *inv, float *cf) {
  constexpr float LEV = (float)((1 << BITS) - 1);
  constexpr float MARGIN = (LEV + 2.0f) * 4.76837158203125e-07f;  // (levels+2) * 2^-21
  float t[8];
  bool near = false;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    t[i] = a[i] * inv[i];
    near |= __builtin_fabsf(__builtin_amdgcn_fractf(t[i]) - 0.5f) <= MARGIN;
  }
  if (__any(near)) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const bool ni = __builtin_fabsf(__builtin_amdgcn_fractf(t[i]) - 0.5f) <= MARGIN;
      t[i] = ni ? a[i] / scale[i] : t[i];
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) cf[i] = __builtin_amdgcn_fmed3f(__builtin_rintf(t[i]), 0.0f, LEV);
}

// packed 16-bit order keys of fp16 pairs (min/max without NaN canonicalisation)
__device__ __forceinline__ uint32_t kkey_pair(uint32_t w) {
  typedef short s2 __attribute__((ext_vector_type(2)));
  const s2 sg = __builtin_bit_cast(s2, w) >> (short)15;
  return w ^ 0x80008000u ^ (__builtin_bit_cast(uint32_t, sg) & 0x7fff7fffu);
}
__device__ __forceinline__ float kunkey_f(uint32_t k) {
  const uint32_t h = (k & 0x8000u) ? (k & 0x7fffu) : (~k & 0xffffu);
  return h2f((uint16_t)h);
}
__device__ __forceinline__ uint32_t pkmin(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_min(__builtin_bit_cast(u16x2, a), __builtin_bit_cast(u16x2, b)));
}
__device__ __forceinline__ uint32_t pkmax(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2, a), __builtin_bit_cast(u16x2, b)));
}

// ------------------------------------------------------------------ keys
template <int BITS, int CL, int NI, bool PK>
__global__ __launch_bounds__(256) void kivi_keys_fast(KiviArgs a) {
  constexpr int TPI = 64 / CL;  // token rows per load instruction
  const int D = CL * 8;
  const int n = a.hi - a.lo;
  const int ng = (n + a.gs - 1) / a.gs;
  const int lane = threadIdx.x & 63;
  const int g = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);  // group of this wave
  if (g >= ng) return;  // wave-uniform
  const int64_t bh = blockIdx.y;
  const int t0 = a.lo + g * a.gs;
  const int cnt = min(a.gs, a.hi - t0);
  const int ch = lane % CL, tr = lane / CL;
  uint16_t *base = a.keys + ((size_t)bh * a.x_rows + (t0 - a.x_t0)) * D + ch * 8;

  uint4 v[NI];
  bool ok[NI];
  // packing: loads without branches (rows past the group's end repeat its
  // last row, cnt >= 1), so every load issues before the first wait (+3.5%
  // measured); the in-place round trip measured 0.5-1% better with the
  // guarded loads
#pragma unroll
  for (int j = 0; j < NI; ++j) {
    const int t = tr + TPI * j;
    ok[j] = t < cnt;
    if constexpr (PK)
      v[j] = *reinterpret_cast<const uint4 *>(base + (size_t)min(t, cnt - 1) * D);
    else
      v[j] = ok[j] ? *reinterpret_cast<const uint4 *>(base + (size_t)t * D) : make_uint4(0, 0, 0, 0);
  }
  // per channel pair: packed min/max of order keys over this lane's tokens
  uint32_t kmn[4] = {0xffffffffu, 0xffffffffu, 0xffffffffu, 0xffffffffu};
  uint32_t kmx[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int j = 0; j < NI; ++j) {
    if (!ok[j]) continue;
    const uint32_t w[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t kk = kkey_pair(w[i]);
      kmn[i] = pkmin(kmn[i], kk);
      kmx[i] = pkmax(kmx[i], kk);
    }
  }
  // reduce across the lanes holding the same channels (lane bits >= log2(CL))
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (CL <= 8) {
      kmn[i] = pkmin(kmn[i], dpp<DPP_ROR8>(kmn[i]));
      kmx[i] = pkmax(kmx[i], dpp<DPP_ROR8>(kmx[i]));
    }
    if constexpr (CL <= 16) {
      kmn[i] = pkmin(kmn[i], (uint32_t)__shfl_xor((int)kmn[i], 16));
      kmx[i] = pkmax(kmx[i], (uint32_t)__shfl_xor((int)kmx[i], 16));
    }
    if constexpr (CL <= 32) {
      kmn[i] = pkmin(kmn[i], (uint32_t)__shfl_xor((int)kmn[i], 32));
      kmx[i] = pkmax(kmx[i], (uint32_t)__shfl_xor((int)kmx[i], 32));
    }
    if constexpr (CL <= 4) {
      kmn[i] = pkmin(kmn[i], dpp<0x124>(kmn[i]));  // row_ror:4
      kmx[i] = pkmax(kmx[i], dpp<0x124>(kmx[i]));
    }
    if constexpr (CL <= 2) {
      kmn[i] = pkmin(kmn[i], dpp<0x122>(kmn[i]));  // row_ror:2
      kmx[i] = pkmax(kmx[i], dpp<0x122>(kmx[i]));
    }
    if constexpr (CL <= 1) {
      kmn[i] = pkmin(kmn[i], dpp<0x121>(kmn[i]));  // row_ror:1
      kmx[i] = pkmax(kmx[i], dpp<0x121>(kmx[i]));
    }
  }
  // every lane of a channel chunk now holds the same 8 minima and maxima;
  // lane tr computes the scales of channels tr, tr + TPI, ... once and the
  // chunk's lanes gather the 8 scales and reciprocals with lane shuffles
  constexpr int SPL = TPI >= 8 ? 1 : 8 / TPI;  // scales computed per lane
  float mn[8], mxv[8], sc[8], inv[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    mn[i] = kunkey_f((kmn[i / 2] >> (16 * (i & 1))) & 0xffffu);
    mxv[i] = kunkey_f((kmx[i / 2] >> (16 * (i & 1))) & 0xffffu);
  }
  float s_own[SPL], i_own[SPL];
#pragma unroll
  for (int q = 0; q < SPL; ++q) {
    const int ci = (tr % 8) + q * TPI;  // channel of this lane's q-th scale
    float cmn = mn[0], cmx = mxv[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) {
      cmn = ci == i ? mn[i] : cmn;
      cmx = ci == i ? mxv[i] : cmx;
    }
    float sq = kivi_scale_c<BITS>(cmn, cmx, a.eps);
    if constexpr (PK) sq = scale_p16(sq);
    s_own[q] = sq;
    i_own[q] = recip(sq);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int src = ch + CL * (i % (TPI < 8 ? TPI : 8));  // the lane that computed channel i
    sc[i] = __shfl(s_own[TPI < 8 ? i / TPI : 0], src);
    inv[i] = __shfl(i_own[TPI < 8 ? i / TPI : 0], src);
  }

  const int64_t nrow0 = bh * a.code_rows + (t0 - a.code_t0);  // code row of token t0
#pragma unroll
  for (int j = 0; j < NI; ++j) {
    if (!ok[j]) continue;
    const uint32_t w[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
    uint32_t o[4], c[8];
    float ad[8], cf[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) ad[i] = ((i & 1) ? hi_h2f(w[i / 2]) : lo_h2f(w[i / 2])) - mn[i];
    kivi_codes8<BITS>(ad, sc, inv, cf);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      c[i] = (uint32_t)cf[i];
      const uint32_t r = f2h(cf[i] * sc[i] + mn[i]);
      if (i & 1) o[i / 2] |= r << 16; else o[i / 2] = r;
    }
    const int t = tr + TPI * j;
    if constexpr (!PK) *reinterpret_cast<uint4 *>(base + (size_t)t * D) = make_uint4(o[0], o[1], o[2], o[3]);
    if (a.k_codes)
      store_codes8<BITS>(a.k_codes + (size_t)(nrow0 + t) * (D * BITS / 8) + ch * BITS, c);
  }
  if (tr == 0) {
    const size_t p = ((size_t)bh * a.kgrp_rows + a.kgrp0 + g) * D + ch * 8;
    if constexpr (PK) {
      uint32_t sw[4], zw[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sw[i] = (uint32_t)f2h(sc[2 * i]) | ((uint32_t)f2h(sc[2 * i + 1]) << 16);
        zw[i] = (uint32_t)f2h(mn[2 * i] + 0.0f) | ((uint32_t)f2h(mn[2 * i + 1] + 0.0f) << 16);
      }
      *reinterpret_cast<uint4 *>(a.k_s16 + p) = make_uint4(sw[0], sw[1], sw[2], sw[3]);
      *reinterpret_cast<uint4 *>(a.k_z16 + p) = make_uint4(zw[0], zw[1], zw[2], zw[3]);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if (a.k_scale) a.k_scale[p + i] = sc[i];
        if (a.k_min) a.k_min[p + i] = mn[i] + 0.0f;
      }
    }
  }
}

// generic keys: one thread per (bh, group, chunk of C channels); C = 8 when
// D % 8 == 0 (then the chunk's codes are whole bytes), else 1 (no codes).
template <int C>
__global__ __launch_bounds__(256) void kivi_keys_generic(KiviArgs a) {
  const int D = a.D;
  const int nch = D / C;
  const int n = a.hi - a.lo;
  const int ng = (n + a.gs - 1) / a.gs;
  const int64_t id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (id >= a.BH * ng * nch) return;
  const int ck = (int)(id % nch);
  const int64_t tg = id / nch;
  const int g = (int)(tg % ng);
  const int64_t bh = tg / ng;
  const int t0 = a.lo + g * a.gs, t1 = min(t0 + a.gs, a.hi);
  const float lev = (float)((1 << a.bits) - 1);
  uint16_t *col = a.keys + (size_t)bh * a.x_rows * D + ck * C;  // row t - x_t0 holds token t
  float mn[C], mx[C], sc[C];
  for (int i = 0; i < C; ++i) {
    mn[i] = __builtin_inff();
    mx[i] = -__builtin_inff();
  }
  for (int t = t0; t < t1; ++t)
    for (int i = 0; i < C; ++i) {
      const float x = h2f(col[(size_t)(t - a.x_t0) * D + i]);
      mn[i] = fminf(mn[i], x);
      mx[i] = fmaxf(mx[i], x);
    }
  for (int i = 0; i < C; ++i) {
    sc[i] = kivi_scale(mn[i], mx[i], lev, a.eps);
    if (a.packed) sc[i] = scale_p16(sc[i]);
  }
  const int cpr = D * a.bits / 8;
  for (int t = t0; t < t1; ++t) {
    uint64_t packed = 0;
    for (int i = 0; i < C; ++i) {
      uint32_t c;
      const uint16_t r = kivi_elem(h2f(col[(size_t)(t - a.x_t0) * D + i]), mn[i], sc[i], lev, c);
      if (!a.packed) col[(size_t)(t - a.x_t0) * D + i] = r;
      packed |= (uint64_t)c << (a.bits * i);
    }
    if (C == 8 && a.k_codes) {
      uint8_t *dst = a.k_codes + ((size_t)bh * a.code_rows + (t - a.code_t0)) * cpr + ck * a.bits;
      for (int b = 0; b < a.bits; ++b) dst[b] = (uint8_t)(packed >> (8 * b));
    }
  }
  for (int i = 0; i < C; ++i) {
    const size_t p = ((size_t)bh * a.kgrp_rows + a.kgrp0 + g) * D + ck * C + i;
    if (a.packed) {
      a.k_s16[p] = f2h(sc[i]);
      a.k_z16[p] = f2h(mn[i] + 0.0f);
    } else {
      if (a.k_scale) a.k_scale[p] = sc[i];
      if (a.k_min) a.k_min[p] = mn[i] + 0.0f;  // a zero minimum is exported as +0
    }
  }
}

// ------------------------------------------------------------------ values
template <int BITS, int CL, int LPG, int U, bool PK>
__global__ __launch_bounds__(256) void kivi_values_fast(KiviArgs a) {
  constexpr int RPW = 64 / CL;  // token rows per wave
  const int D = CL * 8;
  const int n = a.hi - a.lo;
  const int lane = threadIdx.x & 63;
  const int wave = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  const int64_t bh = blockIdx.y;
  const int ch = lane % CL, tr = lane / CL;
  const int ng = D / (LPG * 8);
  if (n <= 0) return;
  uint16_t *vb = a.values + ((size_t)bh * a.x_rows + (a.lo - a.x_t0)) * D + ch * 8;

  uint4 v[U];
  int tok[U];  // token offset from lo
#pragma unroll
  for (int u = 0; u < U; ++u) {  // no branches, so every load issues before the first wait
    tok[u] = (wave * U + u) * RPW + tr;
    v[u] = *reinterpret_cast<const uint4 *>(vb + (size_t)min(tok[u], n - 1) * D);  // n >= 1
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const uint32_t w[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
    float x[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = lo_h2f(w[i]);
      x[2 * i + 1] = hi_h2f(w[i]);
    }
    uint32_t kp = kkey_pair(w[0]);
    uint32_t kq = kp;
#pragma unroll
    for (int i = 1; i < 4; ++i) {
      const uint32_t kk = kkey_pair(w[i]);
      kp = pkmin(kp, kk);
      kq = pkmax(kq, kk);
    }
    uint32_t kmn = min(kp & 0xffffu, kp >> 16), kmx = max(kq & 0xffffu, kq >> 16);
    kmn = group_min_u32<LPG>(kmn);
    kmx = group_max_u32<LPG>(kmx);
    const float mn = kunkey_f(kmn), mx = kunkey_f(kmx);
    float sc = kivi_scale_c<BITS>(mn, mx, a.eps);
    if constexpr (PK) sc = scale_p16(sc);
    const float inv = recip(sc);
    uint32_t o[4], c[8];
    float ad[8], scv[8], invv[8], cf[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      ad[i] = x[i] - mn;
      scv[i] = sc;
      invv[i] = inv;
    }
    kivi_codes8<BITS>(ad, scv, invv, cf);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      c[i] = (uint32_t)cf[i];
      const uint32_t r = f2h(cf[i] * sc + mn);
      if (i & 1) o[i / 2] |= r << 16; else o[i / 2] = r;
    }
    if (tok[u] < n) {
      const size_t rowid = (size_t)bh * a.code_rows + (a.lo + tok[u] - a.code_t0);  // code row
      if constexpr (!PK) *reinterpret_cast<uint4 *>(vb + (size_t)tok[u] * D) = make_uint4(o[0], o[1], o[2], o[3]);
      if (a.v_codes) store_codes8<BITS>(a.v_codes + rowid * (D * BITS / 8) + ch * BITS, c);
      if (ch % LPG == 0) {
        const size_t p = rowid * ng + ch / LPG;
        if constexpr (PK) {
          a.v_s16[p] = f2h(sc);
          a.v_z16[p] = f2h(mn + 0.0f);
        } else {
          if (a.v_scale) a.v_scale[p] = sc;
          if (a.v_min) a.v_min[p] = mn + 0.0f;
        }
      }
    }
  }
}

// generic values: one thread per (bh, token, group)
__global__ __launch_bounds__(256) void kivi_values_generic(KiviArgs a) {
  const int D = a.D;
  const int n = a.hi - a.lo;
  const int ng = (D + a.gs - 1) / a.gs;
  const int64_t id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (id >= a.BH * n * ng) return;
  const int g = (int)(id % ng);
  const int64_t row0 = id / ng;  // bh * n + (t - lo)
  const int64_t bh = row0 / n;
  const int t = a.lo + (int)(row0 - bh * n);
  const int64_t row = bh * a.code_rows + (t - a.code_t0);  // code / parameter row
  const int d0 = g * a.gs, d1 = min(d0 + a.gs, D);
  const float lev = (float)((1 << a.bits) - 1);
  uint16_t *r = a.values + ((size_t)bh * a.x_rows + (t - a.x_t0)) * D;
  float mn = __builtin_inff(), mx = -__builtin_inff();
  for (int d = d0; d < d1; ++d) {
    const float x = h2f(r[d]);
    mn = fminf(mn, x);
    mx = fmaxf(mx, x);
  }
  float sc = kivi_scale(mn, mx, lev, a.eps);
  if (a.packed) sc = scale_p16(sc);
  // codes (only requested when D % 8 == 0 and gs % 8 == 0): the group covers
  // whole 8-channel chunks, each chunk is `bits` whole bytes
  uint8_t *cr = a.v_codes ? a.v_codes + (size_t)row * (D * a.bits / 8) : nullptr;
  uint64_t packed = 0;
  for (int d = d0; d < d1; ++d) {
    uint32_t c;
    const uint16_t rec = kivi_elem(h2f(r[d]), mn, sc, lev, c);
    if (!a.packed) r[d] = rec;
    packed |= (uint64_t)c << (a.bits * (d % 8));
    if (cr && (d % 8 == 7 || d == d1 - 1)) {
      uint8_t *dst = cr + (d / 8) * a.bits;
      for (int b = 0; b < a.bits; ++b) dst[b] = (uint8_t)(packed >> (8 * b));
      packed = 0;
    }
  }
  const size_t p = (size_t)row * ng + g;
  if (a.packed) {
    a.v_s16[p] = f2h(sc);
    a.v_z16[p] = f2h(mn + 0.0f);
  } else {
    if (a.v_scale) a.v_scale[p] = sc;
    if (a.v_min) a.v_min[p] = mn + 0.0f;
  }
}

// ------------------------------------------------------------------ unpack
// One thread per (b, h, 8 consecutive tokens, 8 channels): BITS code bytes
// per token, the group's fp16 (scale, zero), 8 outputs
// fp16(RN32(code*scale) + zero) per token in one 16-byte store. Keys
// reload their group's parameters only when the group changes (never, when
// lo is a multiple of 8: the group size is); values take one pair per token
// and 8 channels.
constexpr int KIVI_UNPACK_ROWS = 8;
template <int BITS, bool PERCH>
__global__ __launch_bounds__(256) void kivi_unpack(KiviUnpackArgs a) {
  // grid: x = (8-token block, chunk) pairs of one (b, h) slice, y (+ 65535 z) = (b, h)
  const int chunks = a.D / 8, n = a.hi - a.lo;
  const int nblk = (n + KIVI_UNPACK_ROWS - 1) / KIVI_UNPACK_ROWS;
  const uint32_t i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (uint32_t)(nblk * chunks)) return;
  const int64_t bh = (int64_t)blockIdx.z * 65535 + blockIdx.y;
  if (bh >= a.BH) return;
  const int k = a.chunk_shift >= 0 ? (int)(i & (uint32_t)(chunks - 1)) : (int)(i % (uint32_t)chunks);
  const int tb = (int)(a.chunk_shift >= 0 ? i >> a.chunk_shift : i / (uint32_t)chunks);
  const int t0 = a.lo + tb * KIVI_UNPACK_ROWS;
  const int rows = min(KIVI_UNPACK_ROWS, a.hi - t0);
  const int64_t row0 = bh * a.S_cap + t0;                  // storage row of token t0
  const int64_t orow0 = bh * a.out_rows + (t0 - a.out_t0);  // output row of token t0
  const int ngv = (a.D + a.gs - 1) / a.gs;
  float s[8], z[8];
  int cur_tg = -1;  // key group whose parameters s, z hold
  const int64_t kg0 = bh * ((a.S_cap + a.gs - 1) / a.gs);
  const int vg = a.gs_shift >= 0 ? (8 * k) >> a.gs_shift : (8 * k) / a.gs;
  // every token's codes (and, for values, its group's parameters) are
  // loaded before the first store
  // (a register per value: packing two 16-bit values into one would wait
  // on the first load)
  typedef std::conditional_t<BITS == 2, uint16_t, std::conditional_t<BITS == 4, uint32_t, uint64_t>> CWT;
  typedef std::conditional_t<BITS == 8, uint64_t, uint32_t> CWR;
  CWR cwr[KIVI_UNPACK_ROWS];
  uint32_t s16[KIVI_UNPACK_ROWS], z16[KIVI_UNPACK_ROWS];
#pragma unroll
  for (int r = 0; r < KIVI_UNPACK_ROWS; ++r) {
    const int64_t row = row0 + min(r, rows - 1);  // rows >= 1; the rows past the block's end repeat its last
    cwr[r] = *reinterpret_cast<const CWT *>(a.codes + row * (a.D * BITS / 8) + k * BITS);
    if constexpr (!PERCH) {
      s16[r] = a.scale[row * ngv + vg];
      z16[r] = a.zero[row * ngv + vg];
    }
  }
#pragma unroll
  for (int r = 0; r < KIVI_UNPACK_ROWS; ++r) {
    if (r >= rows) break;
    if constexpr (PERCH) {  // the 8 tokens share a group unless lo % 8 != 0
      const int tg = a.gs_shift >= 0 ? (t0 + r) >> a.gs_shift : (t0 + r) / a.gs;
      if (tg != cur_tg) {
        cur_tg = tg;
        const int64_t p = (kg0 + tg) * a.D + 8 * k;
        const uint4 sv = *reinterpret_cast<const uint4 *>(a.scale + p);
        const uint4 zv = *reinterpret_cast<const uint4 *>(a.zero + p);
        const uint32_t sw[4] = {sv.x, sv.y, sv.z, sv.w}, zw[4] = {zv.x, zv.y, zv.z, zv.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          s[e] = (e & 1) ? hi_h2f(sw[e / 2]) : lo_h2f(sw[e / 2]);
          z[e] = (e & 1) ? hi_h2f(zw[e / 2]) : lo_h2f(zw[e / 2]);
        }
      }
    }
    const uint64_t cw = cwr[r];
    if constexpr (!PERCH) {
      const float s0 = h2f((uint16_t)s16[r]), z0 = h2f((uint16_t)z16[r]);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        s[e] = s0;
        z[e] = z0;
      }
    }
    // code*scale is exact in binary32 (at most 8 + 11 significant bits), so
    // RN32(RN32(code*scale) + zero) is one fma
    const uint32_t cw0 = (uint32_t)cw, cw1 = (uint32_t)(cw >> 32);
    uint32_t o[4];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float c;
      if constexpr (BITS == 8) c = (float)(uint32_t)(uint8_t)((e < 4 ? cw0 : cw1) >> (8 * (e % 4)));
      else c = (float)__builtin_amdgcn_ubfe(cw0, BITS * e, BITS);
      const uint32_t h = f2h(__builtin_fmaf(c, s[e], z[e]));
      if (e & 1) o[e / 2] |= h << 16; else o[e / 2] = h;
    }
    *reinterpret_cast<uint4 *>(a.out + (orow0 + r) * a.D + 8 * k) = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

// ------------------------------------------------------------------ launch
namespace {
// workgroup shapes measured on B=128 x 8 heads x 8064 tokens x D=64:
// keys 2 waves (key groups) per workgroup, values 1 wave with one row
// group (+4% keys, +10% values over 4 waves / 2 row groups)
#ifndef KVQ_KIVI_KWPB
#define KVQ_KIVI_KWPB 2  // waves (key groups) per workgroup
#endif
#ifndef KVQ_KIVI_VWPB
#define KVQ_KIVI_VWPB 1  // waves per workgroup, values
#endif
#ifndef KVQ_KIVI_VU
#define KVQ_KIVI_VU 1  // row groups per wave, values (in-place round trip)
#endif
#ifndef KVQ_KIVI_VU_PK
#define KVQ_KIVI_VU_PK 4  // row groups per wave, values (packing: +4-5% over one, measured)
#endif
template <int BITS, int CL, bool PK>
hipError_t keys_cl(const KiviArgs &a, int ng, hipStream_t st) {
  constexpr int TPI = 64 / CL, W = KVQ_KIVI_KWPB;
  const dim3 grid((unsigned)((ng + W - 1) / W), (unsigned)a.BH), blk(64 * W);
  switch (a.gs / TPI) {  // loads per lane; fast path only when gs % TPI == 0
    case 1: hipLaunchKernelGGL((kivi_keys_fast<BITS, CL, 1, PK>), grid, blk, 0, st, a); break;
    case 2: hipLaunchKernelGGL((kivi_keys_fast<BITS, CL, 2, PK>), grid, blk, 0, st, a); break;
    case 4: hipLaunchKernelGGL((kivi_keys_fast<BITS, CL, 4, PK>), grid, blk, 0, st, a); break;
    case 8: hipLaunchKernelGGL((kivi_keys_fast<BITS, CL, 8, PK>), grid, blk, 0, st, a); break;
    case 16: hipLaunchKernelGGL((kivi_keys_fast<BITS, CL, 16, PK>), grid, blk, 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

bool keys_fast_ok(const KiviArgs &a) {
  if (a.BH > 65535) return false;
  const int CL = a.D / 8;
  if (a.D % 8 || (CL & (CL - 1)) || CL > 32 || CL < 1) return false;
  const int TPI = 64 / CL;
  if (a.gs % TPI) return false;
  const int ni = a.gs / TPI;
  return ni == 1 || ni == 2 || ni == 4 || ni == 8 || ni == 16;
}

template <int BITS, bool PK>
hipError_t launch_keys(const KiviArgs &a, hipStream_t st) {
  const int n = a.hi - a.lo;
  const int ng = (n + a.gs - 1) / a.gs;
  if (keys_fast_ok(a)) {
    switch (a.D / 8) {
      case 1: return keys_cl<BITS, 1, PK>(a, ng, st);
      case 2: return keys_cl<BITS, 2, PK>(a, ng, st);
      case 4: return keys_cl<BITS, 4, PK>(a, ng, st);
      case 8: return keys_cl<BITS, 8, PK>(a, ng, st);
      case 16: return keys_cl<BITS, 16, PK>(a, ng, st);
      case 32: return keys_cl<BITS, 32, PK>(a, ng, st);
    }
  }
  if (a.D % 8 == 0) {
    const int64_t total = a.BH * ng * (a.D / 8);
    hipLaunchKernelGGL((kivi_keys_generic<8>), dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st, a);
  } else {
    const int64_t total = a.BH * ng * a.D;
    hipLaunchKernelGGL((kivi_keys_generic<1>), dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st, a);
  }
  return hipGetLastError();
}

template <int BITS, int CL, int LPG, bool PK>
hipError_t values_cfg(const KiviArgs &a, hipStream_t st) {
  constexpr int U = PK ? KVQ_KIVI_VU_PK : KVQ_KIVI_VU, RPW = 64 / CL, W = KVQ_KIVI_VWPB;
  const int64_t waves = ((a.hi - a.lo) + RPW * U - 1) / (RPW * U);  // per (b, h)
  hipLaunchKernelGGL((kivi_values_fast<BITS, CL, LPG, U, PK>), dim3((unsigned)((waves + W - 1) / W), (unsigned)a.BH),
                     dim3(64 * W), 0, st, a);
  return hipGetLastError();
}

template <int BITS, int CL, bool PK>
hipError_t values_cl(const KiviArgs &a, hipStream_t st) {
  switch (a.gs / 8) {
    case 1: return values_cfg<BITS, CL, 1, PK>(a, st);
    case 2: if constexpr (CL >= 2) return values_cfg<BITS, CL, 2, PK>(a, st); break;
    case 4: if constexpr (CL >= 4) return values_cfg<BITS, CL, 4, PK>(a, st); break;
    case 8: if constexpr (CL >= 8) return values_cfg<BITS, CL, 8, PK>(a, st); break;
    case 16: if constexpr (CL >= 16) return values_cfg<BITS, CL, 16, PK>(a, st); break;
    case 32: if constexpr (CL >= 32) return values_cfg<BITS, CL, 32, PK>(a, st); break;
    case 64: if constexpr (CL >= 64) return values_cfg<BITS, CL, 64, PK>(a, st); break;
  }
  return hipErrorInvalidValue;
}

bool values_fast_ok(const KiviArgs &a) {
  if (a.BH > 65535) return false;
  const int CL = a.D / 8;
  if (a.D % 8 || (CL & (CL - 1)) || CL > 64 || CL < 1) return false;
  if (a.gs % 8) return false;
  const int lpg = a.gs / 8;
  return (lpg & (lpg - 1)) == 0 && lpg <= CL && a.D % a.gs == 0;
}

template <int BITS, bool PK>
hipError_t launch_values(const KiviArgs &a, hipStream_t st) {
  if (values_fast_ok(a)) {
    switch (a.D / 8) {
      case 1: return values_cl<BITS, 1, PK>(a, st);
      case 2: return values_cl<BITS, 2, PK>(a, st);
      case 4: return values_cl<BITS, 4, PK>(a, st);
      case 8: return values_cl<BITS, 8, PK>(a, st);
      case 16: return values_cl<BITS, 16, PK>(a, st);
      case 32: return values_cl<BITS, 32, PK>(a, st);
      case 64: return values_cl<BITS, 64, PK>(a, st);
    }
  }
  const int n = a.hi - a.lo;
  const int ng = (a.D + a.gs - 1) / a.gs;
  const int64_t total = a.BH * n * (int64_t)ng;
  hipLaunchKernelGGL(kivi_values_generic, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st, a);
  return hipGetLastError();
}

template <int BITS, bool PK>
hipError_t launch_bits_p(const KiviArgs &a, hipStream_t st) {
  hipError_t e = hipSuccess;
  if (a.keys) e = launch_keys<BITS, PK>(a, st);
  if (e == hipSuccess && a.values) e = launch_values<BITS, PK>(a, st);
  return e;
}
template <int BITS>
hipError_t launch_bits(const KiviArgs &a, hipStream_t st) {
  return a.packed ? launch_bits_p<BITS, true>(a, st) : launch_bits_p<BITS, false>(a, st);
}
}  // namespace

hipError_t launch_kivi(const KiviArgs &a, hipStream_t st) {
  switch (a.bits) {
    case 2: return launch_bits<2>(a, st);
    case 4: return launch_bits<4>(a, st);
    default: return launch_bits<8>(a, st);
  }
}

namespace {
template <int BITS>
hipError_t unpack_b(const KiviUnpackArgs &a, hipStream_t st) {
  const int64_t per_bh = (int64_t)((a.hi - a.lo + KIVI_UNPACK_ROWS - 1) / KIVI_UNPACK_ROWS) * (a.D / 8);
  const dim3 grid((unsigned)((per_bh + 255) / 256), (unsigned)(a.BH < 65535 ? a.BH : 65535),
                  (unsigned)((a.BH + 65534) / 65535));
  if (a.per_channel) hipLaunchKernelGGL((kivi_unpack<BITS, true>), grid, dim3(256), 0, st, a);
  else hipLaunchKernelGGL((kivi_unpack<BITS, false>), grid, dim3(256), 0, st, a);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_kivi_unpack(KiviUnpackArgs a, hipStream_t st) {
  auto log2_or = [](int v) {
    int s = 0;
    while ((1 << s) < v) ++s;
    return (1 << s) == v ? s : -1;
  };
  a.chunk_shift = log2_or(a.D / 8);
  a.gs_shift = log2_or(a.gs);
  switch (a.bits) {
    case 2: return unpack_b<2>(a, st);
    case 4: return unpack_b<4>(a, st);
    default: return unpack_b<8>(a, st);
  }
}

}  // namespace kvq
