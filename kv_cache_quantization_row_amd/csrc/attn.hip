// Paged decode attention reading the packed symmetric q8 / q6 / q4 codes.
//
// [MTPLX pull request #267, "feat(kv-cache): add q6 paged KV quantization",
//  PR description] the cached rows are dequantized to fp16 (code x fp16
//  scale) and handed to scaled-dot-product attention; here both steps are one
//  kernel that reads the codes and scales, so a decode step moves
//  D*bits/8 + 2 bytes per cached (token, head) row instead of 2*D.
//
// out[s][h] = sum_t softmax_t(scale * q[s][h] . k[t]) v[t] over the first
// seq_lens[s] positions of sequence s, with k, v the rows of KV head
// h / (q_heads / kv_heads), dequantized exactly as kvq_dequant_sym does
// (fp16(q * s)).
//
// Work split: a workgroup takes one sequence, a chunk of ATTN_CHUNK
// positions and up to four KV heads, one wave per head (the page rows of
// neighbouring heads are read together). Per block of 16 positions a wave computes the score tile
// S^T = K Q^T (16 positions x 16 query-head slots, G = q_heads / kv_heads of
// them used) with 16x16x16 fp16 MFMAs, the online softmax per head in fp32,
// and O^T += V^T P^T with the same MFMA: the score tile's accumulator layout
// (lane l: positions 4*(l/16)+i, head l%16) is the B-operand layout of the
// second product, so the probabilities feed it from registers. Head
// dimensions are assigned to lanes so that every lane reads contiguous code
// bytes: in the score product lane group g = l/16 covers dims [g*D/4,
// (g+1)*D/4); in the value product output row m of tile t is dim
// m*(D/16) + t. Each chunk leaves (max, sum, unnormalised output) per head
// in the workspace; a second kernel merges the chunks.
#include "common.h"
#include "kernels.h"

namespace kvq {
namespace {

typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef float f4 __attribute__((ext_vector_type(4)));

// code bias of a width: q = u - bias (q8 codes are two's complement bytes)
template <int BITS>
constexpr int abias() {
  return BITS == 6 ? 32 : (BITS == 4 ? 8 : 0);
}

// the i-th biased code (0 <= i < n) of a little-endian LSB-first bit string
template <int BITS>
__device__ __forceinline__ uint32_t code_at(const uint32_t *w, int i) {
  if constexpr (BITS == 8) {
    return (w[i / 4] >> (8 * (i % 4))) & 0xffu;
  } else if constexpr (BITS == 4) {
    return (w[i / 8] >> (4 * (i % 8))) & 0xfu;
  } else {
    const int bit = 6 * i, wi = bit / 32, sh = bit % 32;
    uint32_t v = w[wi] >> sh;
    if (sh > 26) v |= w[wi + 1] << (32 - sh);
    return v & 63u;
  }
}

// fp16(q * s) for a biased code u: q is formed exactly in fp16 and one fp16
// multiply rounds the exact product
template <int BITS>
__device__ __forceinline__ _Float16 deq(uint32_t u, _Float16 s) {
  _Float16 q;
  if constexpr (BITS == 8) {
    q = (_Float16)(float)(int)(int8_t)(uint8_t)u;
  } else {
    q = (_Float16)(float)((int)u - abias<BITS>());
  }
  return q * s;
}

}  // namespace

template <int BITS, int D>
__global__ __launch_bounds__(256) void attn_decode_chunk(AttnArgs a) {
  constexpr int PD = D * BITS / 8;
  constexpr int KS = D / 16;               // k-steps of the score product, tiles of the value product
  constexpr int KW = (D / 4) * BITS / 32;  // words of a lane's score-product code piece (D/4 dims)
  constexpr int VB = (D / 16) * BITS / 8;  // bytes of a lane's value-product code piece (D/16 dims)
  constexpr int VW = (VB + 3) / 4;
  const int lane = threadIdx.x & 63;
  const int hk = blockIdx.z * 4 + (threadIdx.x >> 6);  // KV head of this wave
  if (hk >= a.kv_heads) return;  // no workgroup-wide barriers in this kernel
  const int s = blockIdx.y;
  const int c = blockIdx.x;
  const int G = a.group;
  const int P = a.page_size, H = a.kv_heads;
  const int len = min(a.seq_lens[s], a.max_len);
  const int p0 = c * ATTN_CHUNK;
  const int n = lane & 15, g = lane >> 4;
  const uint8_t *kc = a.k_codes + (size_t)a.layer * a.code_layer_stride;
  const uint8_t *vc = a.v_codes + (size_t)a.layer * a.code_layer_stride;
  const uint16_t *ks = a.k_scales + (size_t)a.layer * a.scale_layer_stride;
  const uint16_t *vs = a.v_scales + (size_t)a.layer * a.scale_layer_stride;
  // query slots of this wave's head group: B operand of S^T = K Q^T
  h4 qb[KS];
  {
    const bool on = n < G;
    const uint16_t *qr = a.q + ((size_t)s * a.q_heads + hk * G + (on ? n : 0)) * D + g * (D / 4);
#pragma unroll
    for (int j = 0; j < KS; ++j) {
      const uint2 w = on ? *reinterpret_cast<const uint2 *>(qr + 4 * j) : make_uint2(0, 0);
      qb[j] = __builtin_bit_cast(h4, w);
    }
  }
  f4 acc[KS];
#pragma unroll
  for (int t = 0; t < KS; ++t) acc[t] = f4{0.f, 0.f, 0.f, 0.f};
  float mrun = -__builtin_inff(), lrun = 0.f;  // per head n (same in the 4 lanes of a column)
  const float sc = a.scale;
  for (int b0 = p0; b0 < min(p0 + ATTN_CHUNK, len); b0 += 16) {
    // ---- K rows: lane (n, g) reads dims [g*D/4, (g+1)*D/4) of position b0 + n
    const int pk = b0 + n;
    int64_t rowk = -1;
    if (pk < len && pk / P < a.max_blocks) {
      const int32_t pg = a.block_table[(size_t)s * a.max_blocks + pk / P];
      if (pg >= 0 && pg < a.num_pages) rowk = ((int64_t)pg * P + pk % P) * H + hk;
    }
    uint32_t kw[KW + 1];
#pragma unroll
    for (int i = 0; i <= KW; ++i) kw[i] = 0;
    _Float16 ksc = (_Float16)0.f;
    if (rowk >= 0) {
      const uint32_t *src = reinterpret_cast<const uint32_t *>(kc + rowk * PD + g * (D / 4) * BITS / 8);
#pragma unroll
      for (int i = 0; i < KW; ++i) kw[i] = src[i];
      ksc = __builtin_bit_cast(_Float16, ks[rowk]);
    }
    f4 st = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < KS; ++j) {
      h4 ka;
#pragma unroll
      for (int i = 0; i < 4; ++i) ka[i] = deq<BITS>(code_at<BITS>(kw, 4 * j + i), ksc);
      st = __builtin_amdgcn_mfma_f32_16x16x16f16(ka, qb[j], st, 0, 0, 0);
    }
    // ---- rows of the positions this lane holds in the score tile and reads
    // in the value product: b0 + 4g + i (absent -> masked)
    int64_t rowv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      rowv[i] = -1;
      const int pvp = b0 + 4 * g + i;
      if (pvp < len && pvp / P < a.max_blocks) {
        const int32_t pg = a.block_table[(size_t)s * a.max_blocks + pvp / P];
        if (pg >= 0 && pg < a.num_pages) rowv[i] = ((int64_t)pg * P + pvp % P) * H + hk;
      }
    }
    // ---- online softmax per head (column n)
    float sv[4], bm = -__builtin_inff();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sv[i] = rowv[i] >= 0 ? st[i] * sc : -__builtin_inff();
      bm = fmaxf(bm, sv[i]);
    }
    bm = fmaxf(bm, __shfl_xor(bm, 16));
    bm = fmaxf(bm, __shfl_xor(bm, 32));
    if (bm == -__builtin_inff()) continue;  // a block without any present position (uniform over the wave)
    const float mnew = fmaxf(mrun, bm);
    const float corr = mrun == -__builtin_inff() ? 0.f : __expf(mrun - mnew);
    float pv[4], ps = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pv[i] = sv[i] == -__builtin_inff() ? 0.f : __expf(sv[i] - mnew);
      ps += pv[i];
    }
    ps += __shfl_xor(ps, 16);
    ps += __shfl_xor(ps, 32);
    lrun = lrun * corr + ps;
    mrun = mnew;
    h4 pb;
#pragma unroll
    for (int i = 0; i < 4; ++i) pb[i] = (_Float16)pv[i];
    // ---- V rows: lane (m = n, g) reads dims [m*D/16, (m+1)*D/16) of positions b0 + 4g + i
    uint32_t vw[4][VW + 1];
    _Float16 vsc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int w = 0; w <= VW; ++w) vw[i][w] = 0;
      vsc[i] = (_Float16)0.f;
      if (rowv[i] >= 0) {
        const uint8_t *src = vc + rowv[i] * PD + n * VB;
        if constexpr (VB % 4 == 0) {
#pragma unroll
          for (int w = 0; w < VW; ++w) vw[i][w] = reinterpret_cast<const uint32_t *>(src)[w];
        } else {  // 2-, 3- or 6-byte pieces (not dword aligned): byte loads
#pragma unroll
          for (int bb = 0; bb < VB; ++bb) vw[i][bb / 4] |= (uint32_t)src[bb] << (8 * (bb % 4));
        }
        vsc[i] = __builtin_bit_cast(_Float16, vs[rowv[i]]);
      }
    }
#pragma unroll
    for (int t = 0; t < KS; ++t) {
      h4 va;
#pragma unroll
      for (int i = 0; i < 4; ++i) va[i] = deq<BITS>(code_at<BITS>(vw[i], t), vsc[i]);
      acc[t] = acc[t] * corr;
      acc[t] = __builtin_amdgcn_mfma_f32_16x16x16f16(va, pb, acc[t], 0, 0, 0);
    }
  }
  // ---- chunk result: (max, sum) per head slot and the unnormalised output;
  // lane (n, g) holds dims t + (D/16)*(4g + i) of head n
  if (n < G) {
    float *w = a.ws + (((size_t)s * a.n_chunks + c) * a.q_heads + hk * G + n) * (D + 2);
    if (g == 0) {
      w[0] = mrun;
      w[1] = lrun;
    }
#pragma unroll
    for (int t = 0; t < KS; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) w[2 + (4 * g + i) * KS + t] = acc[t][i];
  }
}

// merge the chunks of one (sequence, head): weights exp(m_c - M)
template <int D>
__global__ __launch_bounds__(D) void attn_decode_merge(AttnArgs a) {
  const int h = blockIdx.x, s = blockIdx.y, d = threadIdx.x;
  const int len = min(a.seq_lens[s], a.max_len);
  const int nc = (len + ATTN_CHUNK - 1) / ATTN_CHUNK;
  const float *w0 = a.ws + ((size_t)s * a.n_chunks * a.q_heads + h) * (D + 2);
  const size_t cstride = (size_t)a.q_heads * (D + 2);
  float M = -__builtin_inff();
  for (int c = 0; c < nc; ++c) M = fmaxf(M, w0[c * cstride]);
  float L = 0.f, o = 0.f;
  for (int c = 0; c < nc; ++c) {
    const float *w = w0 + c * cstride;
    if (w[1] > 0.f) {
      const float e = __expf(w[0] - M);
      L += w[1] * e;
      o += w[2 + d] * e;
    }
  }
  a.out[((size_t)s * a.q_heads + h) * D + d] = f2h(L > 0.f ? o / L : 0.f);
}

namespace {
template <int BITS, int D>
hipError_t launch_attn_bd(const AttnArgs &a, hipStream_t st) {
  hipLaunchKernelGGL((attn_decode_chunk<BITS, D>),
                     dim3((unsigned)a.n_chunks, (unsigned)a.n_seqs, (unsigned)((a.kv_heads + 3) / 4)),
                     dim3(64 * (a.kv_heads < 4 ? a.kv_heads : 4)), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((attn_decode_merge<D>), dim3((unsigned)a.q_heads, (unsigned)a.n_seqs), dim3(D), 0, st, a);
  return hipGetLastError();
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

hipError_t launch_attn_decode(const AttnArgs &a, hipStream_t st) {
  switch (a.bits) {
    case 8: return launch_attn_b<8>(a, st);
    case 6: return launch_attn_b<6>(a, st);
    default: return launch_attn_b<4>(a, st);
  }
}

}  // namespace kvq
