// Symmetric per-(token, head) q8 / q6 / q4 quantization on paged storage.
//
// [MTPLX pull request #267, "feat(kv-cache): add q6 paged KV quantization",
//  PR description] one fp16 scale per (token, KV head) row, qmax table
//  {8:127, 6:31, 4:7}, q6 codes biased +32 into 6-bit fields, four fields per
//  three little-endian bytes; q4 two codes per byte, q8 one ("Summary").
//
// Fast paths (head_dim a power of two in [16, 1024]). Large writes use
// sym_quant_v8: a row is handled by D/8 consecutive lanes, one 16-byte load of
// 8 fp16 values per lane, so every wave load is one contiguous 1 KiB run.
// Small writes (decode appends) and D = 1024 use sym_quant_fast, with
// LPR = D/16 lanes of 16 elements per row and several rows per wave. The
// row's |x| maximum is taken on fp16 bit patterns with packed 16-bit max,
// then across the row's lanes with DPP. The generic path (other head dims)
// runs one wave per row.
//
// Rounding: codes need rint(x * r) with ties-to-even, clipped to +-qmax. The
// clipped product c is added to 1.5*2^23 + bias: in [2^23, 2^24) the float
// spacing is 1, so that single IEEE addition rounds c to the nearest integer
// with ties to even (the addend is even) and leaves rint(c) + bias in the low
// mantissa bits.
#include <type_traits>

#include "common.h"
#include "kernels.h"

#ifndef KVQ_SYM_QUANT_U
#define KVQ_SYM_QUANT_U 2  // row groups per wave in the write path
#endif
#ifndef KVQ_SYM_QUANT_WPB
#define KVQ_SYM_QUANT_WPB 4  // waves per workgroup in the write path
#endif
#ifndef KVQ_SYM_DEQ_PPB
#define KVQ_SYM_DEQ_PPB 16  // most positions per workgroup in the read path (divides page_size)
#endif
#ifndef KVQ_SYM_DEQ_CHUNKS
#define KVQ_SYM_DEQ_CHUNKS 512  // most 8-element chunks per read-path workgroup (two per thread measured best)
#endif
#ifndef KVQ_NT_LOAD
#define KVQ_NT_LOAD 0  // 1: non-temporal hint on the streaming fp16 loads (write path)
#endif
#ifndef KVQ_NT_CODES
#define KVQ_NT_CODES 1  // non-temporal hint on the packed code stores of the write path (q6 +2%, q8 +0.5% measured)
#endif
#ifndef KVQ_NT_STORE
#define KVQ_NT_STORE 1  // non-temporal hint on the streaming fp16 stores of the read path (+3% measured)
#endif

namespace kvq {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld_stream(const uint4 *p) {
#if KVQ_NT_LOAD
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
#else
  return *p;
#endif
}
template <typename T>
__device__ __forceinline__ void st_codes(T *p, T v) {
#if KVQ_NT_CODES
  __builtin_nontemporal_store(v, p);
#else
  *p = v;
#endif
}
__device__ __forceinline__ void st_stream(uint4 *p, uint4 v) {
#if KVQ_NT_STORE
  const u32x4 w = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(w, reinterpret_cast<u32x4 *>(p));
#else
  *p = v;
#endif
}

template <int BITS>
struct SymFmt;
template <>
struct SymFmt<8> {
  static constexpr int QMAX = 127, BIAS = 0;
};
template <>
struct SymFmt<6> {
  static constexpr int QMAX = 31, BIAS = 32;
};
template <>
struct SymFmt<4> {
  static constexpr int QMAX = 7, BIAS = 8;
};

template <int BITS>
__device__ __forceinline__ uint32_t encode(float x, float r) {
  constexpr float Q = (float)SymFmt<BITS>::QMAX;
  float t = x * r;
  float c = __builtin_amdgcn_fmed3f(t, -Q, Q);
  float m = c + (12582912.0f + (float)SymFmt<BITS>::BIAS);
  return __builtin_bit_cast(uint32_t, m) - 0x4b400000u;
}

// Raw encoding of one element: the bit pattern of RN(x*r) + 1.5*2^23 + bias,
// i.e. 0x4b400000 + rint(x*r) + bias. x*r is formed as fma(x, r, +0), a
// single rounding of the exact product (only a zero's sign can differ, and
// it vanishes in the addition). CLAMP clips to +-qmax first; it is needed
// only when the row's fp16 scale is subnormal: with a normal scale
// s = RN16(RN32(a/qmax)) we have |x*r| <= qmax (1 + 2^-11 + 2^-22) < qmax + 1/2.
template <int BITS, bool CLAMP>
__device__ __forceinline__ uint32_t enc_raw(uint16_t h, float r) {
  constexpr float Q = (float)SymFmt<BITS>::QMAX;
  float t = __builtin_fmaf((float)__builtin_bit_cast(_Float16, h), r, 0.0f);
  if constexpr (CLAMP) t = __builtin_amdgcn_fmed3f(t, -Q, Q);
  return __builtin_bit_cast(uint32_t, t + (12582912.0f + (float)SymFmt<BITS>::BIAS));
}

// Pack 16 raw encodings (0x4b400000 + biased code) into BITS/2 dwords,
// LSB-first. The packing is done modulo 2^32 on the raw patterns and the
// constant contribution of 0x4b400000 is removed once per word: fields never
// overlap (biased codes are < 2^BITS), so no carries cross them.
template <int BITS>
__device__ __forceinline__ void pack16_raw(const uint32_t *m, uint32_t *o) {
  constexpr uint32_t K = 0x4b400000u;
  if constexpr (BITS == 8) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t lo = __builtin_amdgcn_perm(m[4 * j + 1], m[4 * j], 0x0c0c0400u);
      const uint32_t hi = __builtin_amdgcn_perm(m[4 * j + 3], m[4 * j + 2], 0x04000c0cu);
      o[j] = lo | hi;
    }
  } else if constexpr (BITS == 6) {
    constexpr uint32_t C = K + (K << 6) + (K << 12) + (K << 18);
    uint32_t g[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      g[j] = (m[4 * j] + (m[4 * j + 1] << 6) + (m[4 * j + 2] << 12) + (m[4 * j + 3] << 18)) - C;
    o[0] = g[0] | (g[1] << 24);
    o[1] = (g[1] >> 8) | (g[2] << 16);
    o[2] = (g[2] >> 16) | (g[3] << 8);
  } else {
    constexpr uint32_t C = K + (K << 4) + (K << 8) + (K << 12) + (K << 16) + (K << 20) + (K << 24) + (K << 28);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      uint32_t v = m[8 * j];
#pragma unroll
      for (int i = 1; i < 8; ++i) v += m[8 * j + i] << (4 * i);
      o[j] = v - C;
    }
  }
}

// Row scale: fp16(absmax / qmax) and the binary32 reciprocal of its value.
template <int BITS>
__device__ __forceinline__ void row_scale(uint32_t amax_bits, uint16_t &s16, float &r) {
  float a = h2f((uint16_t)amax_bits);
  s16 = f2h(a / (float)SymFmt<BITS>::QMAX);
  float s = h2f(s16);
  r = (s != 0.0f) ? 1.0f / s : 0.0f;
}

// Pack 16 biased codes (low bits of c[i]) into BITS/2 dwords, LSB-first.
template <int BITS>
__device__ __forceinline__ void pack16(const uint32_t *c, uint32_t *o) {
  if constexpr (BITS == 8) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      o[j] = (c[4 * j] & 0xffu) | ((c[4 * j + 1] & 0xffu) << 8) | ((c[4 * j + 2] & 0xffu) << 16) |
             (c[4 * j + 3] << 24);
  } else if constexpr (BITS == 6) {
    uint32_t g[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      g[j] = c[4 * j] | (c[4 * j + 1] << 6) | (c[4 * j + 2] << 12) | (c[4 * j + 3] << 18);
    o[0] = g[0] | (g[1] << 24);
    o[1] = (g[1] >> 8) | (g[2] << 16);
    o[2] = (g[2] >> 16) | (g[3] << 8);
  } else {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      uint32_t v = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) v |= c[8 * j + i] << (4 * i);
      o[j] = v;
    }
  }
}

// Unpack 16 biased codes from BITS/2 dwords.
template <int BITS>
__device__ __forceinline__ void unpack16(const uint32_t *w, uint32_t *u) {
  if constexpr (BITS == 8) {
#pragma unroll
    for (int i = 0; i < 16; ++i) u[i] = (w[i / 4] >> (8 * (i % 4))) & 0xffu;
  } else if constexpr (BITS == 6) {
    uint32_t g[4];
    g[0] = w[0] & 0xffffffu;
    g[1] = (w[0] >> 24) | ((w[1] & 0xffffu) << 8);
    g[2] = (w[1] >> 16) | ((w[2] & 0xffu) << 16);
    g[3] = w[2] >> 8;
#pragma unroll
    for (int i = 0; i < 16; ++i) u[i] = (g[i / 4] >> (6 * (i % 4))) & 63u;
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) u[i] = (w[i / 8] >> (4 * (i % 8))) & 15u;
  }
}

typedef _Float16 h2 __attribute__((ext_vector_type(2)));

// fp16 pair fp16(q0*s), fp16(q1*s) from two biased codes. q = u - bias is
// formed exactly in fp16 (1024 + u with spacing 1, minus 1024 + bias); the
// fp16 product is the single correctly rounded q*s (the binary32 product
// q*s is exact, so this equals rounding that product to fp16).
template <int BITS>
__device__ __forceinline__ uint32_t decode_pair(uint32_t u0, uint32_t u1, h2 ss) {
  uint32_t b;
  if constexpr (BITS == 8) {
    // int8 two's complement: u ^ 0x80 is q + 128 in [1, 255]
    b = ((u0 ^ 0x80u) | ((u1 ^ 0x80u) << 16)) | 0x64006400u;
    const h2 off = {(_Float16)(-1152.0f), (_Float16)(-1152.0f)};
    h2 q = __builtin_bit_cast(h2, b) + off;
    return __builtin_bit_cast(uint32_t, q * ss);
  } else {
    constexpr float O = -(1024.0f + (float)SymFmt<BITS>::BIAS);
    b = (u0 | (u1 << 16)) | 0x64006400u;
    const h2 off = {(_Float16)O, (_Float16)O};
    h2 q = __builtin_bit_cast(h2, b) + off;
    return __builtin_bit_cast(uint32_t, q * ss);
  }
}

// ----------------------------------------------------------------- write path
template <int BITS, int LPR, int U>
__global__ __launch_bounds__(256) void sym_quant_fast(SymQuantArgs a) {
  constexpr int D = LPR * 16, RPW = 64 / LPR, PD = D * BITS / 8, OW = BITS / 2;
  const int side = blockIdx.z;
  const uint16_t *x = side ? a.v : a.k;
  uint8_t *codes = side ? a.v_codes : a.k_codes;
  uint16_t *scales = side ? a.v_scales : a.k_scales;
  if (x == nullptr) return;
  const uint32_t layer = blockIdx.y;
  const uint32_t rows = a.rows_per_layer;
  const int lane = threadIdx.x & 63;
  const uint32_t wave = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  const int sub = lane / LPR, li = lane % LPR;
  const uint16_t *xl = x + (size_t)layer * rows * D;
  uint8_t *cl = codes + (size_t)(a.layer0 + layer) * a.code_layer_stride;
  uint16_t *sl = scales + (size_t)(a.layer0 + layer) * a.scale_layer_stride;

  uint32_t w[U][8];
  int64_t slot[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const uint32_t row = (wave * U + u) * RPW + sub;
    slot[u] = -1;
    if (row < rows) {
      slot[u] = a.slot_mapping[a.h_shift >= 0 ? (row >> a.h_shift) : row / a.H];
      const uint4 *p = reinterpret_cast<const uint4 *>(xl + (size_t)row * D + li * 16);
      uint4 v0 = ld_stream(p), v1 = ld_stream(p + 1);
      w[u][0] = v0.x; w[u][1] = v0.y; w[u][2] = v0.z; w[u][3] = v0.w;
      w[u][4] = v1.x; w[u][5] = v1.y; w[u][6] = v1.z; w[u][7] = v1.w;
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) w[u][i] = 0;
    }
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const uint32_t row = (wave * U + u) * RPW + sub;
    const uint32_t amax = group_max_u32<LPR>(absmax_bits(w[u], 8));
    uint16_t s16;
    float r;
    row_scale<BITS>(amax, s16, r);
    uint32_t c[16], o[OW];
    if (__any(s16 != 0 && s16 < 0x0400u)) {  // some row of the wave has a subnormal scale
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        c[2 * i] = enc_raw<BITS, true>((uint16_t)(w[u][i] & 0xffffu), r);
        c[2 * i + 1] = enc_raw<BITS, true>((uint16_t)(w[u][i] >> 16), r);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        c[2 * i] = enc_raw<BITS, false>((uint16_t)(w[u][i] & 0xffffu), r);
        c[2 * i + 1] = enc_raw<BITS, false>((uint16_t)(w[u][i] >> 16), r);
      }
    }
    pack16_raw<BITS>(c, o);
    if (row < rows && slot[u] >= 0 && slot[u] < a.n_slots) {
      const uint32_t t = a.h_shift >= 0 ? (row >> a.h_shift) : row / a.H;
      const uint32_t h = row - t * a.H;
      {
        const size_t orow = (size_t)slot[u] * a.H + h;
        uint32_t *dst = reinterpret_cast<uint32_t *>(cl + orow * PD + li * (OW * 4));
#pragma unroll
        for (int j = 0; j < OW; ++j) dst[j] = o[j];
        if (li == 0) sl[orow] = s16;
      }
    }
  }
}

// Write path, 8 elements per lane: a row of D is owned by L8 = D/8 lanes, one
// fully coalesced 16-byte load per lane; the wave holds 64/L8 rows and a
// 256-thread workgroup 256/L8 rows. Each lane packs 8 codes into BITS bytes;
// for q6 the odd lane hands its 6 bytes to the even lane (DPP), which stores
// 12 bytes.
template <int BITS, int L8, int U>
__global__ __launch_bounds__(256) void sym_quant_v8(SymQuantArgs a) {
  constexpr int D = L8 * 8, RPW = 64 / L8, PD = D * BITS / 8;
  const int side = blockIdx.z;
  const uint16_t *x = side ? a.v : a.k;
  uint8_t *codes = side ? a.v_codes : a.k_codes;
  uint16_t *scales = side ? a.v_scales : a.k_scales;
  if (x == nullptr) return;
  const uint32_t layer = blockIdx.y;
  const uint32_t rows = a.rows_per_layer;
  const int lane = threadIdx.x & 63;
  const uint32_t wave = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  const int sub = lane / L8, li = lane % L8;
  const uint16_t *xl = x + (size_t)layer * rows * D;
  uint8_t *cl = codes + (size_t)(a.layer0 + layer) * a.code_layer_stride;
  // U consecutive row groups per wave, all loads issued first
  uint4 in[U];
  int64_t slot[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const uint32_t row = (wave * U + u) * RPW + sub;
    in[u] = make_uint4(0, 0, 0, 0);
    slot[u] = -1;
    if (row < rows) {
      in[u] = ld_stream(reinterpret_cast<const uint4 *>(xl + (size_t)row * D + li * 8));
      slot[u] = a.slot_mapping[a.h_shift >= 0 ? (row >> a.h_shift) : row / a.H];
    }
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const uint32_t row = (wave * U + u) * RPW + sub;
    const uint32_t w[4] = {in[u].x, in[u].y, in[u].z, in[u].w};
    uint32_t amax = absmax_bits(w, 4);
    amax = group_max_u32<L8>(amax);
    uint16_t s16;
    float r;
    row_scale<BITS>(amax, s16, r);
    uint32_t m[8];
    if (__any(s16 != 0 && s16 < 0x0400u)) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        m[2 * i] = enc_raw<BITS, true>((uint16_t)(w[i] & 0xffffu), r);
        m[2 * i + 1] = enc_raw<BITS, true>((uint16_t)(w[i] >> 16), r);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        m[2 * i] = enc_raw<BITS, false>((uint16_t)(w[i] & 0xffffu), r);
        m[2 * i + 1] = enc_raw<BITS, false>((uint16_t)(w[i] >> 16), r);
      }
    }
    constexpr uint32_t K = 0x4b400000u;
    const bool ok = row < rows && slot[u] >= 0 && slot[u] < a.n_slots;
    const size_t orow =
        ok ? (size_t)slot[u] * a.H + (row - (a.h_shift >= 0 ? (row >> a.h_shift) : row / a.H) * a.H) : 0;
    if constexpr (BITS == 8) {
      const uint32_t o0 = __builtin_amdgcn_perm(m[1], m[0], 0x0c0c0400u) | __builtin_amdgcn_perm(m[3], m[2], 0x04000c0cu);
      const uint32_t o1 = __builtin_amdgcn_perm(m[5], m[4], 0x0c0c0400u) | __builtin_amdgcn_perm(m[7], m[6], 0x04000c0cu);
      if (ok) {
        typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
        st_codes(reinterpret_cast<u32x2 *>(cl + orow * PD + li * 8), u32x2{o0, o1});
      }
    } else if constexpr (BITS == 4) {
      constexpr uint32_t C = K + (K << 4) + (K << 8) + (K << 12) + (K << 16) + (K << 20) + (K << 24) + (K << 28);
      uint32_t v = m[0];
#pragma unroll
      for (int i = 1; i < 8; ++i) v += m[i] << (4 * i);
      if (ok) st_codes(reinterpret_cast<uint32_t *>(cl + orow * PD + li * 4), v - C);
    } else {
      constexpr uint32_t C = K + (K << 6) + (K << 12) + (K << 18);
      const uint32_t g0 = (m[0] + (m[1] << 6) + (m[2] << 12) + (m[3] << 18)) - C;
      const uint32_t g1 = (m[4] + (m[5] << 6) + (m[6] << 12) + (m[7] << 18)) - C;
      // this lane's 6 bytes: g0 (24 bits) then g1 (24 bits)
      const uint32_t lo = g0 | (g1 << 24), hi = g1 >> 8;  // 48 bits
      // the odd neighbour's 48 bits, moved to the even lane (quad_perm [1,1,3,3])
      const uint32_t nlo = dpp<0xf5>(lo), nhi = dpp<0xf5>(hi);
      if (ok && (li & 1) == 0) {
        uint32_t *dst = reinterpret_cast<uint32_t *>(cl + orow * PD + li * 6);
        st_codes(dst, lo);
        st_codes(dst + 1, hi | (nlo << 16));
        st_codes(dst + 2, (nlo >> 16) | (nhi << 16));
      }
    }
    if (ok && li == 0) scales[(size_t)(a.layer0 + layer) * a.scale_layer_stride + orow] = s16;
  }
}

// Generic write path: one wave per row, any head_dim valid for the width.
template <int BITS>
__global__ __launch_bounds__(256) void sym_quant_generic(SymQuantArgs a) {
  const int side = blockIdx.z;
  const uint16_t *x = side ? a.v : a.k;
  uint8_t *codes = side ? a.v_codes : a.k_codes;
  uint16_t *scales = side ? a.v_scales : a.k_scales;
  if (x == nullptr) return;
  const int D = a.D;
  const int PD = D * BITS / 8;
  const uint32_t layer = blockIdx.y;
  const uint32_t rows = a.rows_per_layer;
  const int lane = threadIdx.x & 63;
  const uint32_t row = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  if (row >= rows) return;  // wave-uniform
  const uint16_t *xr = x + ((size_t)layer * rows + row) * D;
  uint32_t m = 0;
  for (int i = lane; i < D; i += 64) m = max(m, (uint32_t)(xr[i] & 0x7fffu));
  m = group_max_u32<64>(m);
  uint16_t s16;
  float r;
  row_scale<BITS>(m, s16, r);
  const uint32_t t = row / a.H, h = row - t * a.H;
  const int64_t slot = a.slot_mapping[t];
  if (slot < 0 || slot >= a.n_slots) return;
  const size_t orow = (size_t)slot * a.H + h;
  uint8_t *dst = codes + (size_t)(a.layer0 + layer) * a.code_layer_stride + orow * PD;
  constexpr int G = BITS == 6 ? 4 : (BITS == 4 ? 2 : 1);  // elements per packing group
  for (int g = lane; g < D / G; g += 64) {
    uint32_t c[4];
#pragma unroll
    for (int i = 0; i < G; ++i) c[i] = encode<BITS>(h2f(xr[g * G + i]), r);
    if constexpr (BITS == 6) {
      uint32_t v = (c[0] & 63u) | ((c[1] & 63u) << 6) | ((c[2] & 63u) << 12) | ((c[3] & 63u) << 18);
      dst[3 * g] = (uint8_t)v;
      dst[3 * g + 1] = (uint8_t)(v >> 8);
      dst[3 * g + 2] = (uint8_t)(v >> 16);
    } else if constexpr (BITS == 4) {
      dst[g] = (uint8_t)((c[0] & 15u) | ((c[1] & 15u) << 4));
    } else {
      dst[g] = (uint8_t)c[0];
    }
  }
  if (lane == 0) scales[(size_t)(a.layer0 + layer) * a.scale_layer_stride + orow] = s16;
}

// ----------------------------------------------------------------- read path
__device__ __forceinline__ bool locate(const SymDequantArgs &a, uint32_t seq, uint32_t p,
                                       int32_t len, size_t &slot) {
  if ((int32_t)p >= len) return false;
  const uint32_t blk = p / (uint32_t)a.page_size;
  if ((int32_t)blk >= a.max_blocks) return false;
  const int32_t page = a.block_table[(size_t)seq * a.max_blocks + blk];
  if (page < 0 || page >= a.num_pages) return false;
  slot = (size_t)page * a.page_size + (p - blk * (uint32_t)a.page_size);
  return true;
}

template <int BITS, int LPR, int U>
__global__ __launch_bounds__(256) void sym_dequant_fast(SymDequantArgs a) {
  constexpr int D = LPR * 16, RPW = 64 / LPR, PD = D * BITS / 8, OW = BITS / 2;
  const int side = blockIdx.z & 1;
  const uint32_t layer = blockIdx.z >> 1;
  const uint8_t *codes = side ? a.v_codes : a.k_codes;
  const uint16_t *scales = side ? a.v_scales : a.k_scales;
  uint16_t *out = side ? a.v_out : a.k_out;
  if (out == nullptr) return;
  const uint32_t seq = blockIdx.y;
  const uint32_t rows = (uint32_t)a.max_len * a.H;  // rows per (layer, sequence)
  const int lane = threadIdx.x & 63;
  const uint32_t wave = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  const int sub = lane / LPR, li = lane % LPR;
  const int32_t len = a.seq_lens[seq];
  const uint8_t *cl = codes + (size_t)(a.layer0 + layer) * a.code_layer_stride;
  const uint16_t *sl = scales + (size_t)(a.layer0 + layer) * a.scale_layer_stride;
  uint16_t *ol = out + ((size_t)layer * a.n_seqs + seq) * rows * D;

  uint32_t w[U][OW];
  uint16_t s16[U];
  bool valid[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const uint32_t row = (wave * U + u) * RPW + sub;
    size_t slot = 0;
    const uint32_t p = a.h_shift >= 0 ? (row >> a.h_shift) : row / a.H;
    const uint32_t h = row - p * a.H;
    valid[u] = row < rows && locate(a, seq, p, len, slot);
    if (valid[u]) {
      const size_t irow = slot * a.H + h;
      const uint32_t *src = reinterpret_cast<const uint32_t *>(cl + irow * PD + li * (OW * 4));
#pragma unroll
      for (int j = 0; j < OW; ++j) w[u][j] = src[j];
      s16[u] = sl[irow];
    } else {
#pragma unroll
      for (int j = 0; j < OW; ++j) w[u][j] = 0;
      s16[u] = 0;
    }
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const uint32_t row = (wave * U + u) * RPW + sub;
    uint32_t cu[16], o[8];
    unpack16<BITS>(w[u], cu);
    if (!valid[u]) {  // +0 output: q = 0 with scale 0
#pragma unroll
      for (int i = 0; i < 16; ++i) cu[i] = SymFmt<BITS>::BIAS;
    }
    const _Float16 s = __builtin_bit_cast(_Float16, s16[u]);
    const h2 ss = {s, s};
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = decode_pair<BITS>(cu[2 * i], cu[2 * i + 1], ss);
    if (row < rows) {
      uint4 *dst = reinterpret_cast<uint4 *>(ol + (size_t)row * D + li * 16);
      dst[0] = make_uint4(o[0], o[1], o[2], o[3]);
      dst[1] = make_uint4(o[4], o[5], o[6], o[7]);
    }
  }
}

template <int BITS>
__global__ __launch_bounds__(256) void sym_dequant_generic(SymDequantArgs a) {
  const int side = blockIdx.z & 1;
  const uint32_t layer = blockIdx.z >> 1;
  const uint8_t *codes = side ? a.v_codes : a.k_codes;
  const uint16_t *scales = side ? a.v_scales : a.k_scales;
  uint16_t *out = side ? a.v_out : a.k_out;
  if (out == nullptr) return;
  const int D = a.D;
  const int PD = D * BITS / 8;
  const uint32_t seq = blockIdx.y;
  const uint32_t rows = (uint32_t)a.max_len * a.H;
  const int lane = threadIdx.x & 63;
  const uint32_t row = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  if (row >= rows) return;
  const uint32_t p = row / a.H, h = row - p * a.H;
  uint16_t *o = out + (((size_t)layer * a.n_seqs + seq) * rows + row) * D;
  size_t slot;
  if (!locate(a, seq, p, a.seq_lens[seq], slot)) {
    for (int i = lane; i < D; i += 64) o[i] = 0;
    return;
  }
  const size_t irow = slot * a.H + h;
  const uint8_t *src = codes + (size_t)(a.layer0 + layer) * a.code_layer_stride + irow * PD;
  const float s = h2f(scales[(size_t)(a.layer0 + layer) * a.scale_layer_stride + irow]);
  for (int i = lane; i < D; i += 64) {
    int q;
    if constexpr (BITS == 8) {
      q = (int)(int8_t)src[i];
    } else if constexpr (BITS == 6) {
      const int g = i / 4, k = i % 4;
      const uint32_t v = src[3 * g] | (src[3 * g + 1] << 8) | (src[3 * g + 2] << 16);
      q = (int)((v >> (6 * k)) & 63u) - 32;
    } else {
      q = (int)((src[i / 2] >> (4 * (i % 2))) & 15u) - 8;
    }
    o[i] = f2h((float)q * s);
  }
}

// Page-unit read path (power-of-two head_dim in [16, 1024]). One workgroup
// dequantizes a unit of positions inside one page of one sequence: the
// unit's codes are contiguous in the pool ([slot][head][packed_dim]) and its
// output rows are contiguous in the fp16 output, so 8-element chunk c of the
// unit (codes at byte c*bits, output at element 8c) is read and written by
// consecutive lanes: each wave load is one contiguous run of codes, each wave
// store one contiguous KiB. A thread takes chunks t, t + 256, ...; all its
// loads are issued before its first store. q6: a chunk's 6 bytes are read as
// the 8 bytes from the dword boundary at or below c*6 (c even: the chunk and
// 2 bytes of the next; c odd: 2 bytes of the previous and the chunk); the
// unit's last chunk has an odd index (D/8 is even), so no window leaves the
// unit. The block-table entry is read once per unit.
template <int BITS, int D>
__global__ __launch_bounds__(256) void sym_dequant_page(SymDequantArgs a) {
  constexpr int PD = D * BITS / 8;
  // load slots per batch (chunks t + 256k); q8 takes four slots, two of them
  // idle at 512 chunks per unit, which makes the compiler issue every load
  // before the first wait (measured at D = 256: +4% at q8 over two slots)
  constexpr int NC = BITS == 8 ? 4 : KVQ_SYM_DEQ_CHUNKS / 256;
  typedef std::conditional_t<BITS == 4, uint32_t, uint2> CW;
  const int side = blockIdx.z & 1;
  const uint32_t layer = blockIdx.z >> 1;
  const uint8_t *codes = side ? a.v_codes : a.k_codes;
  const uint16_t *scales = side ? a.v_scales : a.k_scales;
  uint16_t *out = side ? a.v_out : a.k_out;
  if (out == nullptr) return;
  const uint32_t seq = blockIdx.y;
  const int P = a.page_size, H = a.H;
  const int ppb = a.ppb;                   // positions per workgroup, divides P
  const int32_t len = a.seq_lens[seq];
  const int32_t p0 = (int32_t)blockIdx.x * ppb;  // first position of the unit
  const int32_t blk = p0 / P;
  int32_t page = -1;
  if (blk < a.max_blocks && p0 < len) page = a.block_table[(size_t)seq * a.max_blocks + blk];
  const bool have = page >= 0 && page < a.num_pages;
  const int valid_rows = have ? min(ppb, len - p0) * H : 0;
  const int32_t pos_end = min(ppb, a.max_len - p0);  // positions of this unit inside the output
  uint16_t *ob = out + (((size_t)layer * a.n_seqs + seq) * a.max_len + p0) * H * D;
  const int out_chunks = pos_end * H * (D / 8);
  // rows of positions p0.. of the page are contiguous: [slot][head][packed_dim]
  const size_t first_row = have ? (size_t)page * P * H + (size_t)(p0 - blk * P) * H : 0;
  const uint8_t *gb = codes + (size_t)(a.layer0 + layer) * a.code_layer_stride + first_row * PD;
  const uint16_t *sp = scales + (size_t)(a.layer0 + layer) * a.scale_layer_stride + first_row;
  for (int c0 = threadIdx.x; c0 < out_chunks; c0 += NC * 256) {
    CW w[NC];
    uint32_t sc[NC];  // a register each: packing two would wait on the first load
#pragma unroll
    for (int k = 0; k < NC; ++k) {
      const int c = c0 + k * 256;
      const int row = c / (D / 8);
      w[k] = CW{};
      sc[k] = 0;
      if (c < out_chunks && row < valid_rows) {
        if constexpr (BITS == 6) {  // two dwords at a 4-byte boundary
          const uint32_t *wp = reinterpret_cast<const uint32_t *>(gb + ((size_t)c * 6 & ~(size_t)3));
          w[k] = make_uint2(wp[0], wp[1]);
        } else {
          w[k] = *reinterpret_cast<const CW *>(gb + (size_t)c * BITS);
        }
        sc[k] = sp[row];
      }
    }
#pragma unroll
    for (int k = 0; k < NC; ++k) {
      const int c = c0 + k * 256;
      if (c >= out_chunks) break;
      uint32_t o[4] = {0, 0, 0, 0};
      if (c / (D / 8) < valid_rows) {
        uint32_t u[8];
        if constexpr (BITS == 8) {
#pragma unroll
          for (int i = 0; i < 8; ++i) u[i] = ((i < 4 ? w[k].x : w[k].y) >> (8 * (i % 4))) & 0xffu;
        } else if constexpr (BITS == 4) {
#pragma unroll
          for (int i = 0; i < 8; ++i) u[i] = (w[k] >> (4 * i)) & 15u;
        } else {
          const uint64_t q = ((uint64_t)w[k].y << 32 | w[k].x) >> (16 * (c & 1));
#pragma unroll
          for (int i = 0; i < 8; ++i) u[i] = (uint32_t)(q >> (6 * i)) & 63u;
        }
        const _Float16 sv = __builtin_bit_cast(_Float16, (uint16_t)sc[k]);
        const h2 ss = {sv, sv};
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = decode_pair<BITS>(u[2 * i], u[2 * i + 1], ss);
      }
      st_stream(reinterpret_cast<uint4 *>(ob) + c, make_uint4(o[0], o[1], o[2], o[3]));
    }
  }
}

// ----------------------------------------------------------------- launchers
namespace {
template <int BITS, int LPR, int U>
hipError_t launch_quant_u(const SymQuantArgs &a, int n_layers, hipStream_t st) {
  constexpr int RPW = 64 / LPR, WPB = KVQ_SYM_QUANT_WPB;
  const uint32_t per_block = RPW * U * WPB;
  dim3 grid((a.rows_per_layer + per_block - 1) / per_block, n_layers, 2);
  hipLaunchKernelGGL((sym_quant_fast<BITS, LPR, U>), grid, dim3(64 * WPB), 0, st, a);
  return hipGetLastError();
}
#ifndef KVQ_SYM_QUANT_V8
#define KVQ_SYM_QUANT_V8 1  // 8-elements-per-lane write path for large launches (+4..8% measured)
#endif
template <int BITS, int L8>
hipError_t launch_quant_v8(const SymQuantArgs &a, int n_layers, hipStream_t st) {
  // measured on the paged prefill: q6/q4 run best with two row groups per
  // wave and two waves per workgroup (+4% over one group and four waves),
  // q8 with one row group and four waves
  constexpr int RPW = 64 / L8, U = BITS == 8 ? 1 : 2, WPB = BITS == 8 ? 4 : 2;
  const uint32_t per_block = RPW * WPB * U;
  dim3 grid((a.rows_per_layer + per_block - 1) / per_block, n_layers, 2);
  hipLaunchKernelGGL((sym_quant_v8<BITS, L8, U>), grid, dim3(64 * WPB), 0, st, a);
  return hipGetLastError();
}
template <int BITS, int LPR>
hipError_t launch_quant_lpr(const SymQuantArgs &a, int n_layers, hipStream_t st) {
  if constexpr (LPR <= 32) {
    if (KVQ_SYM_QUANT_V8 && (int64_t)a.rows_per_layer * n_layers > 16384)
      return launch_quant_v8<BITS, 2 * LPR>(a, n_layers, st);
  }
  // small (decode-sized) launches: one row group per wave spreads the few rows
  // over more waves; large launches: several row groups per wave
  if ((int64_t)a.rows_per_layer * n_layers <= 16384) return launch_quant_u<BITS, LPR, 1>(a, n_layers, st);
  return launch_quant_u<BITS, LPR, KVQ_SYM_QUANT_U>(a, n_layers, st);
}
template <int BITS, int LPR>
hipError_t launch_dequant_lpr(const SymDequantArgs &a, int n_layers, hipStream_t st) {
  constexpr int U = 2, RPW = 64 / LPR, WPB = 4;
  const uint32_t per_block = RPW * U * WPB;
  const uint32_t rows = (uint32_t)a.max_len * a.H;
  dim3 grid((rows + per_block - 1) / per_block, a.n_seqs, 2 * n_layers);
  hipLaunchKernelGGL((sym_dequant_fast<BITS, LPR, U>), grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

template <int BITS>
hipError_t launch_quant_bits(const SymQuantArgs &a, int n_layers, hipStream_t st) {
  switch (a.D) {
    case 16: return launch_quant_lpr<BITS, 1>(a, n_layers, st);
    case 32: return launch_quant_lpr<BITS, 2>(a, n_layers, st);
    case 64: return launch_quant_lpr<BITS, 4>(a, n_layers, st);
    case 128: return launch_quant_lpr<BITS, 8>(a, n_layers, st);
    case 256: return launch_quant_lpr<BITS, 16>(a, n_layers, st);
    case 512: return launch_quant_lpr<BITS, 32>(a, n_layers, st);
    case 1024: return launch_quant_lpr<BITS, 64>(a, n_layers, st);
    default: {
      dim3 grid((a.rows_per_layer + 3) / 4, n_layers, 2);
      hipLaunchKernelGGL((sym_quant_generic<BITS>), grid, dim3(256), 0, st, a);
      return hipGetLastError();
    }
  }
}
// positions per workgroup: the largest divisor of page_size whose unit holds
// at most KVQ_SYM_DEQ_CHUNKS 8-element chunks (two per thread measured best
// at D = 256: fewer workgroups with more chunks each, or more with fewer,
// were slower), else one position
template <int BITS>
int pick_ppb(const SymDequantArgs &a) {
  for (int q = min(KVQ_SYM_DEQ_PPB, a.page_size); q > 1; --q)
    if (a.page_size % q == 0 && (int64_t)q * a.H * (a.D / 8) <= KVQ_SYM_DEQ_CHUNKS) return q;
  return 1;
}

template <int BITS, int D>
hipError_t launch_page(SymDequantArgs a, int n_layers, hipStream_t st) {
  a.ppb = pick_ppb<BITS>(a);
  dim3 grid((a.max_len + a.ppb - 1) / a.ppb, a.n_seqs, 2 * n_layers);
  hipLaunchKernelGGL((sym_dequant_page<BITS, D>), grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

// page path for power-of-two head dims in [16, 1024]
template <int BITS>
bool page_path_ok(const SymDequantArgs &a) {
  return a.D >= 16 && a.D <= 1024 && (a.D & (a.D - 1)) == 0;
}

template <int BITS>
hipError_t launch_dequant_bits(const SymDequantArgs &a, int n_layers, hipStream_t st) {
  if (page_path_ok<BITS>(a)) {
    switch (a.D) {
      case 16: return launch_page<BITS, 16>(a, n_layers, st);
      case 32: return launch_page<BITS, 32>(a, n_layers, st);
      case 64: return launch_page<BITS, 64>(a, n_layers, st);
      case 128: return launch_page<BITS, 128>(a, n_layers, st);
      case 256: return launch_page<BITS, 256>(a, n_layers, st);
      case 512: return launch_page<BITS, 512>(a, n_layers, st);
      case 1024: return launch_page<BITS, 1024>(a, n_layers, st);
    }
  }
  switch (a.D) {
    case 16: return launch_dequant_lpr<BITS, 1>(a, n_layers, st);
    case 32: return launch_dequant_lpr<BITS, 2>(a, n_layers, st);
    case 64: return launch_dequant_lpr<BITS, 4>(a, n_layers, st);
    case 128: return launch_dequant_lpr<BITS, 8>(a, n_layers, st);
    case 256: return launch_dequant_lpr<BITS, 16>(a, n_layers, st);
    case 512: return launch_dequant_lpr<BITS, 32>(a, n_layers, st);
    case 1024: return launch_dequant_lpr<BITS, 64>(a, n_layers, st);
    default: {
      const uint32_t rows = (uint32_t)a.max_len * a.H;
      dim3 grid((rows + 3) / 4, a.n_seqs, 2 * n_layers);
      hipLaunchKernelGGL((sym_dequant_generic<BITS>), grid, dim3(256), 0, st, a);
      return hipGetLastError();
    }
  }
}
}  // namespace

hipError_t launch_sym_quant(const SymQuantArgs &a, int bits, int n_layers, hipStream_t st) {
  switch (bits) {
    case 8: return launch_quant_bits<8>(a, n_layers, st);
    case 6: return launch_quant_bits<6>(a, n_layers, st);
    default: return launch_quant_bits<4>(a, n_layers, st);
  }
}

hipError_t launch_sym_dequant(const SymDequantArgs &a, int bits, int n_layers, hipStream_t st) {
  switch (bits) {
    case 8: return launch_dequant_bits<8>(a, n_layers, st);
    case 6: return launch_dequant_bits<6>(a, n_layers, st);
    default: return launch_dequant_bits<4>(a, n_layers, st);
  }
}

}  // namespace kvq
