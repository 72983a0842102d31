// Rebuilding key/value rows from cached factors, shared by the prefill
// kernels: k_t[d] = sum_r A[t,h,r] B[t,r,d] for an 8-wide slice of d, with the
// rank pairs on v_dot2_f32_bf16 ("Tensor Product Attention Is All You Need"
// review on coreui.cn, the K_t and V_t equations of 核心机制总结).
#pragma once

#include "common.h"

namespace tpa {

// R consecutive bf16 values, loaded as one 2R-byte word.
template <int R>
struct RankWordP;
template <>
struct RankWordP<1> { typedef uint16_t type; };
template <>
struct RankWordP<2> { typedef uint32_t type; };
template <>
struct RankWordP<4> { typedef uint2 type; };

typedef __bf16 bf16x2_v __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_v, a), __builtin_bit_cast(bf16x2_v, b), c, false);
}

// sum_r a_r * b_r[j] for the 8 elements j of one 16-byte slice per rank.
// Ranks are paired: word w of rank r holds elements (2w, 2w+1); v_perm_b32
// regroups them as (rank r, rank r+1) pairs for v_dot2_f32_bf16.  Rank 1 is a
// plain product.
template <int R>
__device__ __forceinline__ void factor_combine(typename RankWordP<R>::type a, const uint4 (&b)[R], float (&out)[8]) {
  static_assert(R == 1 || R == 2 || R == 4, "ranks 1, 2 and 4");
  if constexpr (R == 1) {
    const uint32_t w[4] = {b[0].x, b[0].y, b[0].z, b[0].w};
    const float a0 = bf16_to_f32(a);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      out[2 * q] = a0 * __uint_as_float(w[q] << 16);
      out[2 * q + 1] = a0 * __uint_as_float(w[q] & 0xffff0000u);
    }
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) out[j] = 0.f;
#pragma unroll
    for (int rp = 0; rp < R / 2; ++rp) {
      uint32_t apair;
      if constexpr (R == 2) apair = a;
      else apair = rp ? a.y : a.x;
      const uint32_t w0[4] = {b[2 * rp].x, b[2 * rp].y, b[2 * rp].z, b[2 * rp].w};
      const uint32_t w1[4] = {b[2 * rp + 1].x, b[2 * rp + 1].y, b[2 * rp + 1].z, b[2 * rp + 1].w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t lo = __builtin_amdgcn_perm(w1[q], w0[q], 0x05040100u);  // (r0[2q], r1[2q])
        const uint32_t hi = __builtin_amdgcn_perm(w1[q], w0[q], 0x07060302u);  // (r0[2q+1], r1[2q+1])
        out[2 * q] = dot2_bf16(lo, apair, out[2 * q]);
        out[2 * q + 1] = dot2_bf16(hi, apair, out[2 * q + 1]);
      }
    }
  }
}

}  // namespace tpa
