// Paged decode attention reading the packed symmetric q8 / q6 / q4 codes.
//
// [MTPLX pull request #267, "feat(kv-cache): add q6 paged KV quantization",
//  PR description] the cached rows are dequantized to fp16 (code x fp16
//  scale) and handed to scaled-dot-product attention; here both steps are one
//  kernel that reads the codes and scales, so a decode step moves
//  D*bits/8 + 2 bytes per cached (token, head) row instead of 2*D.
//
// out[s][h] = sum_t softmax_t(scale * q[s][h] . k[t]) v[t] over the first
// min(seq_lens[s], max_len) positions of sequence s, with k, v the rows of KV
// head h / (q_heads / kv_heads), dequantized exactly as kvq_dequant_sym does
// (fp16(q * s)).
//
// Work split: a workgroup takes one sequence, a chunk of whole 16-position
// blocks and up to four KV heads, one wave per head. The chunk length is
// chosen at launch so that the grid is about one round of resident
// workgroups (never below 256 positions). Per block a wave computes the score
// tile S^T = K Q^T (16 positions x 16 query-head slots, G of them used) with
// 16x16x32 fp16 MFMAs (two k-steps of the lane's K piece each), the online
// softmax per head in fp32 (base 2; the accumulators are rescaled only when
// a running maximum grows), and O^T += V^T P^T with 16x16x16 fp16 MFMAs
// (the block's 16 positions are the contraction): the score tile's accumulator layout
// (lane l: positions 4*(l/16)+i, head l%16) is the B-operand layout of the
// second product, so the probabilities feed it from registers. Each chunk
// leaves (max, sum, unnormalised output) per head in the workspace; a second
// kernel merges the chunks.
//
// Decoding codes to fp16: a code c placed in mantissa bits [k, k+bits) of
// the fp16 1024 (0x6400) reads as 1024 + c*2^k; one exact fma
// x * 2^-k - (2^(10-k) + bias) gives the signed value, and one fp16 multiply
// by the scale rounds the exact product (= fp16(q * s)). Codes are masked
// out of the packed words two at a time (one per fp16 half, k <= 4) with one
// shift or byte permute and one and-or per pair. The order in which a lane's
// four k-values enter an MFMA is free as long as both operands agree, so Q
// is permuted once per wave to match the pairs.
//
// Loads: when the page size is a multiple of 16 a block lies in one page
// (block-table entries preloaded one per lane, 64 blocks at a time) and the
// rows are that page's base plus fixed lane offsets; other page sizes look
// pages up per position. Each block's codes and scales are loaded one block
// ahead of their use. Measured on this path: the loop is bound by VALU
// issue and latency with two waves per SIMD (about 2 VALU operations per
// code), not by HBM; staging K through LDS for whole-line loads and a
// deeper prefetch did not change the time, a third wave per SIMD does where
// the registers allow it without spilling.
#include <type_traits>

#include "common.h"
#include "kernels.h"

#ifndef KVQ_ATTN_X32
#define KVQ_ATTN_X32 1  // score tile from 16x16x32 fp16 MFMAs (pairs of k-steps)
#endif

namespace kvq {
namespace {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));

constexpr uint32_t MAG = 0x64006400u;  // fp16 1024.0 in both halves

// MAG held in a VGPR, so that (x & mask) | mag is one v_and_or_b32 (VOP3
// takes no literal on this target and one scalar operand at most)
__device__ __forceinline__ uint32_t mag_reg() {
  uint32_t m = MAG;
  asm volatile("" : "+v"(m));
  return m;
}

template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F &&f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

// offset between a stored code u and its value q = u - bias (q8 bytes are
// flipped to u = byte ^ 0x80 first)
template <int BITS>
constexpr int dbias() {
  return BITS == 8 ? 128 : (BITS == 6 ? 32 : 8);
}

// fp16 pair 1024 + c*2^K0 | 1024 + c*2^K1 (c < 2^BITS in the mantissa) ->
// exact c - bias per half
template <int BITS, int K0, int K1>
__device__ __forceinline__ h2 signed_codes(uint32_t r) {
  const h2 x = __builtin_bit_cast(h2, r);
  constexpr float a0 = -(float)((1024 >> K0) + dbias<BITS>());
  constexpr float a1 = -(float)((1024 >> K1) + dbias<BITS>());
  if constexpr (K0 == 0 && K1 == 0) {
    return x + h2{(_Float16)a0, (_Float16)a1};
  } else {
    constexpr float m0 = 1.0f / (float)(1 << K0), m1 = 1.0f / (float)(1 << K1);
    return __builtin_elementwise_fma(x, h2{(_Float16)m0, (_Float16)m1}, h2{(_Float16)a0, (_Float16)a1});
  }
}

__device__ __forceinline__ uint32_t funnel(uint32_t hi, uint32_t lo, int sh) {
  return __builtin_amdgcn_alignbit(hi, lo, sh);  // ((hi:lo) >> sh)[31:0]
}

template <int BITS, int D>
struct Shape {
  static constexpr int PD = D * BITS / 8;         // bytes of a packed row
  static constexpr int KS = D / 16;               // k-steps of S^T, tiles of O^T
  static constexpr int KW = (D / 4) * BITS / 32;  // dwords of a lane's K piece (D/4 dims)
  static constexpr int VB = (D / 16) * BITS / 8;  // bytes of a lane's V piece (D/16 dims)
  static constexpr int VW = (VB + 3) / 4;
};

// Dimension (within the lane's D/4-dim K piece) that k-slot i of k-step j
// carries; slots 0,1 are the halves of the first register, 2,3 the second.
template <int BITS>
__device__ __forceinline__ constexpr int kdim(int j, int i) {
  if constexpr (BITS == 4) {
    // word m holds codes 8m..8m+7; step 2m: (c0,c4),(c1,c5); step 2m+1: (c2,c6),(c3,c7)
    const int lo = 8 * (j >> 1) + 2 * (j & 1);
    return i == 0 ? lo : (i == 1 ? lo + 4 : (i == 2 ? lo + 1 : lo + 5));
  } else {
    // one 4-code group per step: (c0,c2),(c1,c3)
    return 4 * j + (i == 0 ? 0 : (i == 1 ? 2 : (i == 2 ? 1 : 3)));
  }
}

// A operand of k-step J of S^T = K Q^T from the lane's K piece
template <int BITS, int J>
__device__ __forceinline__ h4 k_operand(const uint32_t *kw, h2 ss, uint32_t mag) {
  h2 a, b;
  if constexpr (BITS == 8) {
    const uint32_t w = kw[J] ^ 0x80808080u;
    a = signed_codes<8, 0, 0>(__builtin_amdgcn_perm(0x64646464u, w, 0x04020400u));
    b = signed_codes<8, 0, 0>(__builtin_amdgcn_perm(0x64646464u, w, 0x04030401u));
  } else if constexpr (BITS == 4) {
    const uint32_t w = (J & 1) ? (kw[J >> 1] >> 8) : kw[J >> 1];
    a = signed_codes<4, 0, 0>((w & 0x000f000fu) | mag);
    b = signed_codes<4, 4, 4>((w & 0x00f000f0u) | mag);
  } else {
    // the group's 24 bits start at bit 24J of the piece; y = group << 4 puts
    // c0 at bits 4..9 and c2 at 16..21, z = group >> 2 puts c1 and c3 there
    constexpr int bit = 24 * J, wi = bit / 32, sh = bit % 32;
    uint32_t y, z;
    if constexpr (sh == 0) {
      y = kw[wi] << 4;
      z = kw[wi] >> 2;
    } else {
      const uint32_t hi = (sh + 24 > 32) ? kw[wi + 1] : 0u;
      y = funnel(hi, kw[wi], sh - 4);
      z = funnel(hi, kw[wi], sh + 2);
    }
    a = signed_codes<6, 4, 0>((y & 0x003f03f0u) | mag);
    b = signed_codes<6, 4, 0>((z & 0x003f03f0u) | mag);
  }
  a = a * ss;
  b = b * ss;
  return h4{a.x, a.y, b.x, b.y};
}

// fp16 pair (row A, row B) of code T of the lanes' V pieces, as exact signed
// values
template <int BITS, int T>
__device__ __forceinline__ h2 v_pair(const uint32_t *A, const uint32_t *B, uint32_t mag) {
  if constexpr (BITS == 8) {
    constexpr int wi = T / 4, b = T % 4;
    constexpr uint32_t sel = 0x0c000c00u | ((uint32_t)(4 + b) << 16) | (uint32_t)b;
    return signed_codes<8, 0, 0>(__builtin_amdgcn_perm(B[wi], A[wi], sel) ^ 0x64806480u);
  } else if constexpr (BITS == 4) {
    constexpr int j = T / 2, wi = j / 4, b = j % 4;
    constexpr uint32_t sel = 0x0c000c00u | ((uint32_t)(4 + b) << 16) | (uint32_t)b;
    const uint32_t p = __builtin_amdgcn_perm(B[wi], A[wi], sel);
    if constexpr (T & 1) return signed_codes<4, 4, 4>((p & 0x00f000f0u) | mag);
    else return signed_codes<4, 0, 0>((p & 0x000f000fu) | mag);
  } else {
    constexpr int bit = 6 * T, b0 = bit / 8, rr = bit % 8, wi = b0 / 4, b = b0 % 4;
    if constexpr (rr == 0 || rr == 2) {  // the code lies in one byte
      constexpr uint32_t sel = 0x0c000c00u | ((uint32_t)(4 + b) << 16) | (uint32_t)b;
      const uint32_t p = __builtin_amdgcn_perm(B[wi], A[wi], sel);
      if constexpr (rr == 0) return signed_codes<6, 0, 0>((p & 0x003f003fu) | mag);
      else return signed_codes<6, 2, 2>((p & 0x00fc00fcu) | mag);
    } else {  // bytes b0, b0+1: bits 4..9 (rr 4) or 6..11 (rr 6, shifted down 2)
      uint32_t p;
      if constexpr (b <= 2) {
        constexpr uint32_t sel = (uint32_t)b | ((uint32_t)(b + 1) << 8) | ((uint32_t)(4 + b) << 16) |
                                 ((uint32_t)(5 + b) << 24);
        p = __builtin_amdgcn_perm(B[wi], A[wi], sel);
      } else {
        const uint32_t a2 = funnel(A[wi + 1], A[wi], 24), b2 = funnel(B[wi + 1], B[wi], 24);
        p = __builtin_amdgcn_perm(b2, a2, 0x05040100u);
      }
      if constexpr (rr == 6) p >>= 2;
      return signed_codes<6, 4, 4>((p & 0x03f003f0u) | mag);
    }
  }
}

// The lane's V piece of one row: VB bytes at src, packed into words from byte 0
template <int VB, int VW>
__device__ __forceinline__ void load_vpiece(const uint8_t *src, uint32_t *w) {
  if constexpr (VB % 4 == 0) {
#pragma unroll
    for (int i = 0; i < VW; ++i) w[i] = reinterpret_cast<const uint32_t *>(src)[i];
  } else if constexpr (VB % 2 == 0) {
    const uint16_t *h = reinterpret_cast<const uint16_t *>(src);
#pragma unroll
    for (int i = 0; i < VW; ++i) {
      const uint32_t lo = h[2 * i];
      const uint32_t hi = (2 * i + 1 < VB / 2) ? (uint32_t)h[2 * i + 1] : 0u;
      w[i] = lo | (hi << 16);
    }
  } else {
#pragma unroll
    for (int i = 0; i < VW; ++i) {
      uint32_t v = 0;
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if (4 * i + k < VB) v |= (uint32_t)src[4 * i + k] << (8 * k);
      w[i] = v;
    }
  }
}

// Q slots of KV head hk's group for the lane (n, g): B operand of
// S^T = K Q^T, dims [g*D/4, (g+1)*D/4) in the order the K pairs use
template <int BITS, int D>
__device__ __forceinline__ void load_q(const AttnArgs &a, int s, int hk, int n, int g, h4 *qb) {
  constexpr int KS = D / 16;
  const bool on = n < a.group;
  const uint16_t *qr = a.q + ((size_t)s * a.q_heads + hk * a.group + (on ? n : 0)) * D + g * (D / 4);
  uint16_t qv[D / 4];
#pragma unroll
  for (int i = 0; i < D / 16; ++i) {
    const uint2 w = on ? reinterpret_cast<const uint2 *>(qr)[i] : make_uint2(0, 0);
    qv[4 * i] = (uint16_t)w.x;
    qv[4 * i + 1] = (uint16_t)(w.x >> 16);
    qv[4 * i + 2] = (uint16_t)w.y;
    qv[4 * i + 3] = (uint16_t)(w.y >> 16);
  }
#pragma unroll
  for (int j = 0; j < KS; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) qb[j][i] = __builtin_bit_cast(_Float16, qv[kdim<BITS>(j, i)]);
}

// Running state of one wave: per head n the maximum (base-2 units, equal in
// the column's four lanes), this lane's share of the sum, and O^T.
template <int D>
struct Softmax {
  f4 acc[D / 16];
  float m, l;
};

// One block of 16 positions: K piece kw (row n, dims of group g) with its
// scale, V pieces vw[i] (rows 4g+i, dims n*D/16..) with their scales (0 for
// absent rows), vmask bit i = position 4g+i present (some bit set in the wave);
// the Q operand of k-step j is qb[j * QS].
template <int BITS, int D, int QS>
__device__ __forceinline__ void block_step(const uint32_t *kw, uint32_t ksc,
                                           const uint32_t (*vw)[Shape<BITS, D>::VW], const uint32_t *vsc,
                                           uint32_t vmask, const h4 *qb, float sl2, uint32_t mag,
                                           Softmax<D> &sm) {
  constexpr int KS = D / 16;
  // ---- scores S^T (positions 4g+i, head n in this lane)
  const h2 kss = __builtin_bit_cast(h2, ksc | (ksc << 16));
  f4 st0 = {0.f, 0.f, 0.f, 0.f}, st1 = st0;  // two MFMA chains
#if KVQ_ATTN_X32
  // k-steps 2P and 2P+1 as one 16x16x32 product: both operands put the
  // first step's four k-values before the second's (the k order inside one
  // product is free while A and B agree)
  static_for<0, KS / 2>([&](auto P) {
    const h4 a0 = k_operand<BITS, 2 * P>(kw, kss, mag), a1 = k_operand<BITS, 2 * P + 1>(kw, kss, mag);
    const h4 b0 = qb[(2 * P) * QS], b1 = qb[(2 * P + 1) * QS];
    const h8 av = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
    const h8 bv = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
    if constexpr (P % 2 == 0)
      st0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, bv, st0, 0, 0, 0);
    else
      st1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, bv, st1, 0, 0, 0);
  });
#else
  static_for<0, KS>([&](auto J) {
    if constexpr (J % 2 == 0)
      st0 = __builtin_amdgcn_mfma_f32_16x16x16f16(k_operand<BITS, J>(kw, kss, mag), qb[J * QS], st0, 0, 0, 0);
    else
      st1 = __builtin_amdgcn_mfma_f32_16x16x16f16(k_operand<BITS, J>(kw, kss, mag), qb[J * QS], st1, 0, 0, 0);
  });
#endif
  const f4 st = st0 + st1;
  float sv[4], bm = -__builtin_inff();
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    sv[i] = (vmask >> i) & 1u ? st[i] * sl2 : -__builtin_inff();
    bm = fmaxf(bm, sv[i]);
  }
  bm = fmaxf(bm, __shfl_xor(bm, 16));
  bm = fmaxf(bm, __shfl_xor(bm, 32));
  // every column sees the same present positions, so bm is finite here
  if (__builtin_amdgcn_ballot_w64(bm > sm.m) != 0) {
    const float mnew = fmaxf(sm.m, bm);
    const float corr = sm.m == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(sm.m - mnew);
#pragma unroll
    for (int t = 0; t < KS; ++t) sm.acc[t] = sm.acc[t] * corr;
    sm.l *= corr;
    sm.m = mnew;
  }
  float pv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    pv[i] = (vmask >> i) & 1u ? __builtin_amdgcn_exp2f(sv[i] - sm.m) : 0.f;
    sm.l += pv[i];  // this lane's positions only; summed over the column at the end
  }
  const h4 pb = {(_Float16)pv[0], (_Float16)pv[1], (_Float16)pv[2], (_Float16)pv[3]};
  // ---- O^T += V^T P^T; in tile t, row m is dim m*(D/16) + t
  const h2 s01 = __builtin_bit_cast(h2, vsc[0] | (vsc[1] << 16));
  const h2 s23 = __builtin_bit_cast(h2, vsc[2] | (vsc[3] << 16));
  static_for<0, KS>([&](auto T) {
    const h2 x = v_pair<BITS, T>(vw[0], vw[1], mag) * s01;
    const h2 y = v_pair<BITS, T>(vw[2], vw[3], mag) * s23;
    sm.acc[T] = __builtin_amdgcn_mfma_f32_16x16x16f16(h4{x.x, x.y, y.x, y.y}, pb, sm.acc[T], 0, 0, 0);
  });
}

// chunk result of the lane's head slot n (< group): (max, sum) and the
// unnormalised output; lane (n, g) holds dims (4g + i)*(D/16) + t
template <int D>
__device__ __forceinline__ void store_chunk(const AttnArgs &a, int s, int c, int hk, int n, int g,
                                            Softmax<D> &sm) {
  constexpr int KS = D / 16;
  sm.l += __shfl_xor(sm.l, 16);
  sm.l += __shfl_xor(sm.l, 32);
  if (n >= a.group) return;
  float *w = a.ws + (((size_t)s * a.n_chunks + c) * a.q_heads + hk * a.group + n) * (D + 2);
  if (g == 0) {
    w[0] = sm.m;
    w[1] = sm.l;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int t = 0; t < KS; ++t) w[2 + (4 * g + i) * KS + t] = sm.acc[t][i];
}

}  // namespace

// codes and scales of one block as loaded for the lane (K row n, V rows 4g+i)
template <int KW, int VW>
struct BlockRegs {
  uint32_t kw[KW], vw[4][VW], ksc, vsc[4], vmask;
};

// ---------------------------------------------------------------------------
// Page size a multiple of 16: a block's 16 slots lie in one page, found from
// one block-table entry (entries preloaded one per lane, 64 blocks at a
// time). Row addresses are that page's base (wave-uniform) plus lane offsets
// fixed for the whole chunk.
// waves per SIMD the page kernel is compiled for: 3 where its registers fit
// that without spilling (measured: spills at q8/q6, D=256 cost more than
// the third wave gains)
template <int BITS, int D>
constexpr int pg_waves_per_simd() {
  return (D == 256 && BITS != 4) ? 2 : 3;
}

template <int BITS, int D>
__global__ __launch_bounds__(256, (pg_waves_per_simd<BITS, D>())) void attn_decode_chunk_pg(AttnArgs a) {
  using Sh = Shape<BITS, D>;
  constexpr int PD = Sh::PD, KS = Sh::KS, KW = Sh::KW, VB = Sh::VB, VW = Sh::VW;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hk = __builtin_amdgcn_readfirstlane(blockIdx.z * 4 + w);  // KV head of this wave
  if (hk >= a.kv_heads) return;  // no workgroup-wide barriers in this kernel
  const int s = blockIdx.y, c = blockIdx.x;
  const int len = min(a.seq_lens[s], a.max_len);
  const int nblk = (len + 15) >> 4;
  const int b_begin = c * a.chunk_blocks;
  if (b_begin >= nblk) return;
  const int b_end = min(b_begin + a.chunk_blocks, nblk);
  const int P = a.page_size, H = a.kv_heads;
  const int n = lane & 15, g = lane >> 4;
  const uint8_t *kc = a.k_codes + (size_t)a.layer * a.code_layer_stride;
  const uint8_t *vc = a.v_codes + (size_t)a.layer * a.code_layer_stride;
  const uint16_t *ksl = a.k_scales + (size_t)a.layer * a.scale_layer_stride;
  const uint16_t *vsl = a.v_scales + (size_t)a.layer * a.scale_layer_stride;
  const int32_t *bt = a.block_table + (size_t)s * a.max_blocks;
  const uint32_t mag = mag_reg();

  // Q operands: in registers, or in LDS ([k-step][lane], one 8-byte read per
  // step) where that saves the registers for a third wave per SIMD. The LDS
  // copy is written and read by the same wave only: no barrier.
  constexpr bool QLDS = D == 256 && BITS == 4;
  __shared__ h4 lq[QLDS ? 4 : 1][QLDS ? KS : 1][64];
  h4 qreg[QLDS ? 1 : KS];
  const h4 *qb;
  if constexpr (QLDS) {
    h4 qt[KS];
    load_q<BITS, D>(a, s, hk, n, g, qt);
#pragma unroll
    for (int j = 0; j < KS; ++j) lq[w][j][lane] = qt[j];
    qb = &lq[w][0][lane];
  } else {
    load_q<BITS, D>(a, s, hk, n, g, qreg);
    qb = qreg;
  }

  // lane offsets from the row (first slot of the block, head hk)
  const uint32_t koff = (uint32_t)(n * H) * PD + g * KW * 4;
  const uint32_t ksoff = (uint32_t)(n * H);
  uint32_t voff[4], vsoff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    voff[i] = (uint32_t)((4 * g + i) * H) * PD + n * VB;
    vsoff[i] = (uint32_t)((4 * g + i) * H);
  }

  int win = -(1 << 30), wpg = -1;
  auto block_page = [&](int b) -> int {
    if (b - win >= 64) {  // uniform: refill the window of 64 blocks
      win = b;
      const int pos = (b + lane) * 16;
      int pg = -1;
      if (pos < len && pos / P < a.max_blocks) {
        const int v = bt[pos / P];
        if (v >= 0 && v < a.num_pages) pg = v;
      }
      wpg = pg;
    }
    return __builtin_amdgcn_readlane(wpg, b - win);
  };
  using R = BlockRegs<KW, VW>;
  auto load = [&](int b, R &st) {
    const int pg = block_page(b);
    if (pg < 0) {  // uniform: an absent page contributes nothing
      st.vmask = 0;
      return;
    }
    const int pos0 = b * 16;
    const int64_t row0 = ((int64_t)pg * P + pos0 % P) * H + hk;  // uniform
    const uint32_t *ksrc = reinterpret_cast<const uint32_t *>(kc + row0 * PD + koff);
#pragma unroll
    for (int i = 0; i < KW; ++i) st.kw[i] = ksrc[i];
    st.ksc = ksl[row0 + ksoff];
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (pos0 + 4 * g + i < len) m |= 1u << i;
      load_vpiece<VB, VW>(vc + row0 * PD + voff[i], st.vw[i]);
      const uint32_t sv = vsl[row0 + vsoff[i]];
      st.vsc[i] = (m >> i) & 1u ? sv : 0u;
    }
    st.vmask = m;
  };

  Softmax<D> sm;
#pragma unroll
  for (int t = 0; t < KS; ++t) sm.acc[t] = f4{0.f, 0.f, 0.f, 0.f};
  sm.m = -__builtin_inff();
  sm.l = 0.f;
  const float sl2 = a.scale_log2;
  auto consume = [&](const R &st) {
    if (__builtin_amdgcn_ballot_w64(st.vmask != 0) == 0) return;  // no position of the block present
    block_step<BITS, D, QLDS ? 64 : 1>(st.kw, st.ksc, st.vw, st.vsc, st.vmask, qb, sl2, mag, sm);
  };
  R s0 = {}, s1 = {};
  load(b_begin, s0);
  for (int b = b_begin; b < b_end; b += 2) {
    if (b + 1 < b_end) load(b + 1, s1);
    consume(s0);
    if (b + 1 >= b_end) break;
    if (b + 2 < b_end) load(b + 2, s0);
    consume(s1);
  }
  store_chunk<D>(a, s, c, hk, n, g, sm);
}

// ---------------------------------------------------------------------------
// Other page sizes: the page of every position is looked up; a lane reads
// its own K and V pieces (absent rows at slot 0, scale 0), one block ahead.
template <int BITS, int D>
__global__ __launch_bounds__(256, 2) void attn_decode_chunk_pos(AttnArgs a) {
  using Sh = Shape<BITS, D>;
  constexpr int PD = Sh::PD, KS = Sh::KS, KW = Sh::KW, VB = Sh::VB, VW = Sh::VW;
  const int lane = threadIdx.x & 63;
  const int hk = __builtin_amdgcn_readfirstlane(blockIdx.z * 4 + (threadIdx.x >> 6));
  if (hk >= a.kv_heads) return;  // no workgroup-wide barriers in this kernel
  const int s = blockIdx.y, c = blockIdx.x;
  const int len = min(a.seq_lens[s], a.max_len);
  const int nblk = (len + 15) >> 4;
  const int b_begin = c * a.chunk_blocks;
  if (b_begin >= nblk) return;
  const int b_end = min(b_begin + a.chunk_blocks, nblk);
  const int P = a.page_size, H = a.kv_heads;
  const int n = lane & 15, g = lane >> 4;
  const uint8_t *kc = a.k_codes + (size_t)a.layer * a.code_layer_stride;
  const uint8_t *vc = a.v_codes + (size_t)a.layer * a.code_layer_stride;
  const uint16_t *ksl = a.k_scales + (size_t)a.layer * a.scale_layer_stride;
  const uint16_t *vsl = a.v_scales + (size_t)a.layer * a.scale_layer_stride;
  const int32_t *bt = a.block_table + (size_t)s * a.max_blocks;
  const uint32_t mag = mag_reg();
  h4 qb[KS];
  load_q<BITS, D>(a, s, hk, n, g, qb);

  auto lookup = [&](int pos, int64_t &slot) -> bool {
    slot = 0;
    if (pos >= len || pos / P >= a.max_blocks) return false;
    const int v = bt[pos / P];
    if (v < 0 || v >= a.num_pages) return false;
    slot = (int64_t)v * P + pos % P;
    return true;
  };
  using Stage = BlockRegs<KW, VW>;
  auto load = [&](int b, Stage &st) {
    const int pos0 = b * 16;
    int64_t kslot, vslot[4];
    uint32_t m = 0;
    lookup(pos0 + n, kslot);
    const uint32_t *ksrc =
        reinterpret_cast<const uint32_t *>(kc + (size_t)(kslot * H + hk) * PD + g * KW * 4);
#pragma unroll
    for (int i = 0; i < KW; ++i) st.kw[i] = ksrc[i];
    st.ksc = ksl[kslot * H + hk];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (lookup(pos0 + 4 * g + i, vslot[i])) m |= 1u << i;
      load_vpiece<VB, VW>(vc + (size_t)(vslot[i] * H + hk) * PD + n * VB, st.vw[i]);
      const uint32_t sv = vsl[vslot[i] * H + hk];
      st.vsc[i] = (m >> i) & 1u ? sv : 0u;
    }
    st.vmask = m;
  };

  Softmax<D> sm;
#pragma unroll
  for (int t = 0; t < KS; ++t) sm.acc[t] = f4{0.f, 0.f, 0.f, 0.f};
  sm.m = -__builtin_inff();
  sm.l = 0.f;
  const float sl2 = a.scale_log2;
  auto consume = [&](const Stage &st) {
    if (__builtin_amdgcn_ballot_w64(st.vmask != 0) == 0) return;  // no position of the block present
    block_step<BITS, D, 1>(st.kw, st.ksc, st.vw, st.vsc, st.vmask, qb, sl2, mag, sm);
  };
  Stage s0 = {}, s1 = {};
  load(b_begin, s0);
  for (int b = b_begin; b < b_end; b += 2) {
    if (b + 1 < b_end) load(b + 1, s1);
    consume(s0);
    if (b + 1 >= b_end) break;
    if (b + 2 < b_end) load(b + 2, s0);
    consume(s1);
  }
  store_chunk<D>(a, s, c, hk, n, g, sm);
}

// merge the chunks of one (sequence, head): weights 2^(m_c - M)
template <int D>
__global__ __launch_bounds__(D) void attn_decode_merge(AttnArgs a) {
  __shared__ float red[D / 64];
  const int h = blockIdx.x, s = blockIdx.y, d = threadIdx.x;
  const int len = min(a.seq_lens[s], a.max_len);
  const int span = a.chunk_blocks * 16;
  const int nc = (len + span - 1) / span;
  const float *w0 = a.ws + ((size_t)s * a.n_chunks * a.q_heads + h) * (D + 2);
  const size_t cstride = (size_t)a.q_heads * (D + 2);
  float M = -__builtin_inff();
  for (int c = d; c < nc; c += D) M = fmaxf(M, w0[c * cstride]);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
  if constexpr (D > 64) {
    if ((d & 63) == 0) red[d >> 6] = M;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < D / 64; ++i) M = fmaxf(M, red[i]);
  }
  float L = 0.f, o = 0.f;
  if (M != -__builtin_inff()) {
#pragma unroll 4
    for (int c = 0; c < nc; ++c) {
      const float *w = w0 + c * cstride;
      const float e = __builtin_amdgcn_exp2f(w[0] - M);  // 0 for a chunk without positions
      L += w[1] * e;
      o += w[2 + d] * e;
    }
  }
  a.out[((size_t)s * a.q_heads + h) * D + d] = f2h(L > 0.f ? o / L : 0.f);
}

namespace {

template <int BITS, int D, bool PG16>
hipError_t launch_attn_bdp(AttnArgs a, hipStream_t st) {
  constexpr auto kern_for = []() {
    if constexpr (PG16) return attn_decode_chunk_pg<BITS, D>;
    else return attn_decode_chunk_pos<BITS, D>;
  };
  // resident workgroups per device and workgroup size (1..4 waves), cached
  static int resident_cache[64][4] = {};
  const int waves = a.kv_heads < 4 ? a.kv_heads : 4;
  const int wg_heads = (a.kv_heads + 3) / 4;
  auto kern = kern_for();
  int dev = 0, resident = 0;
  if (hipGetDevice(&dev) == hipSuccess && dev >= 0 && dev < 64) {
    resident = resident_cache[dev][waves - 1];
    if (resident <= 0) {
      int cus = 0, per_cu = 0;
      if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
          hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, 64 * waves, 0) == hipSuccess)
        resident = resident_cache[dev][waves - 1] = cus * (per_cu > 0 ? per_cu : 1);
    }
  }
  // chunks per sequence: enough workgroups for about one resident round
  const int64_t nblk = ((int64_t)a.max_len + 15) / 16;
  const int64_t groups = (int64_t)a.n_seqs * wg_heads;
  int64_t per_seq = resident > 0 ? resident / groups : 1;
  if (per_seq < 1) per_seq = 1;
  int64_t cb = (nblk + per_seq - 1) / per_seq;
  if (cb < ATTN_MIN_CHUNK / 16) cb = ATTN_MIN_CHUNK / 16;
  a.chunk_blocks = (int32_t)cb;
  a.n_chunks = nblk > 0 ? (int32_t)((nblk + cb - 1) / cb) : 1;  // <= ceil(max_len / ATTN_MIN_CHUNK)
  hipLaunchKernelGGL(kern, dim3((unsigned)a.n_chunks, (unsigned)a.n_seqs, (unsigned)wg_heads), dim3(64 * waves),
                     0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((attn_decode_merge<D>), dim3((unsigned)a.q_heads, (unsigned)a.n_seqs), dim3(D), 0, st, a);
  return hipGetLastError();
}
template <int BITS, int D>
hipError_t launch_attn_bd(const AttnArgs &a, hipStream_t st) {
  return a.page_size % 16 == 0 ? launch_attn_bdp<BITS, D, true>(a, st) : launch_attn_bdp<BITS, D, false>(a, st);
}
template <int BITS>
hipError_t launch_attn_b(const AttnArgs &a, hipStream_t st) {
  switch (a.head_dim) {
    case 64: return launch_attn_bd<BITS, 64>(a, st);
    case 128: return launch_attn_bd<BITS, 128>(a, st);
    default: return launch_attn_bd<BITS, 256>(a, st);
  }
}
}  // namespace

hipError_t launch_attn_decode(AttnArgs a, hipStream_t st) {
  switch (a.bits) {
    case 8: return launch_attn_b<8>(a, st);
    case 6: return launch_attn_b<6>(a, st);
    default: return launch_attn_b<4>(a, st);
  }
}

}  // namespace kvq
