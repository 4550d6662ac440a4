// Device helpers shared by the libkvq kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvq {

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float h2f(uint16_t h) {
  return (float)__builtin_bit_cast(_Float16, h);
}
// binary32 -> binary16 with the hardware conversion (mode register: round to
// nearest even, fp16 denormals kept).
__device__ __forceinline__ uint16_t f2h(float f) {
  return __builtin_bit_cast(uint16_t, (_Float16)f);
}
__device__ __forceinline__ float lo_h2f(uint32_t w) { return h2f((uint16_t)(w & 0xffffu)); }
__device__ __forceinline__ float hi_h2f(uint32_t w) { return h2f((uint16_t)(w >> 16)); }

// DPP lane moves inside a 16-lane row (all lanes must be active).
template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xf, 0xf, false);
}
template <int CTRL>
__device__ __forceinline__ float dppf(float v) {
  return __builtin_bit_cast(float, dpp<CTRL>(__builtin_bit_cast(uint32_t, v)));
}
constexpr int DPP_XOR1 = 0xb1;         // quad_perm [1,0,3,2]
constexpr int DPP_XOR2 = 0x4e;         // quad_perm [2,3,0,1]
constexpr int DPP_HALF_MIRROR = 0x141; // lane i <- 7-i within each 8-lane half row
constexpr int DPP_MIRROR = 0x140;      // lane i <- 15-i within the 16-lane row
constexpr int DPP_ROR8 = 0x128;        // rotate right by 8 within the row (= xor 8 for reductions)

// Max over groups of N consecutive lanes (N a power of two <= 64) of an
// unsigned value; every lane of the group receives the result.
template <int N>
__device__ __forceinline__ uint32_t group_max_u32(uint32_t v) {
  if constexpr (N >= 2) v = max(v, dpp<DPP_XOR1>(v));
  if constexpr (N >= 4) v = max(v, dpp<DPP_XOR2>(v));
  if constexpr (N >= 8) v = max(v, dpp<DPP_HALF_MIRROR>(v));
  if constexpr (N >= 16) v = max(v, dpp<DPP_MIRROR>(v));
  if constexpr (N >= 32) v = max(v, (uint32_t)__shfl_xor((int)v, 16));
  if constexpr (N >= 64) v = max(v, (uint32_t)__shfl_xor((int)v, 32));
  return v;
}

template <int N>
__device__ __forceinline__ uint32_t group_min_u32(uint32_t v) {
  if constexpr (N >= 2) v = min(v, dpp<DPP_XOR1>(v));
  if constexpr (N >= 4) v = min(v, dpp<DPP_XOR2>(v));
  if constexpr (N >= 8) v = min(v, dpp<DPP_HALF_MIRROR>(v));
  if constexpr (N >= 16) v = min(v, dpp<DPP_MIRROR>(v));
  if constexpr (N >= 32) v = min(v, (uint32_t)__shfl_xor((int)v, 16));
  if constexpr (N >= 64) v = min(v, (uint32_t)__shfl_xor((int)v, 32));
  return v;
}

// Min and max over groups of N consecutive lanes of a float.
template <int N>
__device__ __forceinline__ void group_minmax_f32(float &mn, float &mx) {
  if constexpr (N >= 2) { mn = fminf(mn, dppf<DPP_XOR1>(mn)); mx = fmaxf(mx, dppf<DPP_XOR1>(mx)); }
  if constexpr (N >= 4) { mn = fminf(mn, dppf<DPP_XOR2>(mn)); mx = fmaxf(mx, dppf<DPP_XOR2>(mx)); }
  if constexpr (N >= 8) { mn = fminf(mn, dppf<DPP_HALF_MIRROR>(mn)); mx = fmaxf(mx, dppf<DPP_HALF_MIRROR>(mx)); }
  if constexpr (N >= 16) { mn = fminf(mn, dppf<DPP_MIRROR>(mn)); mx = fmaxf(mx, dppf<DPP_MIRROR>(mx)); }
  if constexpr (N >= 32) { mn = fminf(mn, __shfl_xor(mn, 16)); mx = fmaxf(mx, __shfl_xor(mx, 16)); }
  if constexpr (N >= 64) { mn = fminf(mn, __shfl_xor(mn, 32)); mx = fmaxf(mx, __shfl_xor(mx, 32)); }
}

// |x| maximum of 8 packed fp16 pairs as an fp16 bit pattern (non-negative
// fp16 bit patterns order like their values).
__device__ __forceinline__ uint32_t absmax_bits(const uint32_t *w, int n) {
  u16x2 m = {0, 0};
  for (int i = 0; i < n; ++i) {
    u16x2 a = __builtin_bit_cast(u16x2, w[i] & 0x7fff7fffu);
    m = __builtin_elementwise_max(m, a);
  }
  return max((uint32_t)m.x, (uint32_t)m.y);
}

}  // namespace kvq
