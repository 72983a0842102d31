// gfx950 matrix-core helpers: v_mfma_f32_16x16x32_bf16 and its operand types.
//
// Register layout of the 16x16x32 bf16 product D = A B + C for lane l
// (li = l % 16, lg = l / 16):
//   A (16 x 32): 8 values A[li][8*lg + j], j < 8
//   B (32 x 16): 8 values B[8*lg + j][li]
//   D (16 x 16): 4 values D[4*lg + i][li], i < 4
// Any bijection between the 32 k indices and the (lg, j) slots may be used, as
// long as A and B use the same one; the kernels use that freedom to keep each
// lane's loads contiguous.
#pragma once

#include "common.h"

namespace tpa {

typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef unsigned short u16x8_t __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f32x4_t mfma_bf16(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

// v_mfma_f32_32x32x16_bf16, D = A B + C for lane l (l32 = l % 32, lh = l / 32):
//   A (32 x 16): 8 values A[l32][8*lh + j];  B (16 x 32): 8 values B[8*lh + j][l32]
//   D (32 x 32): 16 values D[8*(i/4) + 4*lh + i%4][l32], i < 16
typedef float f32x16_t __attribute__((ext_vector_type(16)));

__device__ __forceinline__ f32x16_t mfma32_bf16(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;

// Transposed LDS read (ds_read_b64_tr_b16): the 16 lanes of a group each name
// an 8-byte piece (4 bf16) of a 4 x 16 block, lane 4r + c the piece at row r,
// columns 4c .. 4c + 3; lane i receives column i of each of the four rows.
__device__ __forceinline__ uint2 lds_read_tr16(const bf16_t* p) {
  const i16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(p));
  return __builtin_bit_cast(uint2, v);
}

__device__ __forceinline__ bf16x8_t pack8(const float* v) {
  const uint4 u = make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                             pack_bf16x2(v[6], v[7]));
  return __builtin_bit_cast(bf16x8_t, u);
}

// Maximum / sum of x over the lanes l, l^16, l^32, l^48 (the four lane groups
// that hold one column of a 16x16 tile), with the gfx950 half-wave swaps:
// after permlane32_swap(x, x) lane l holds x[l] and x[l^32]; after
// permlane16_swap(y, y) it holds y[l] and y[l^16].  The sum adds the pairs in
// the same order in every lane, so all four lanes get the same bits.
__device__ __forceinline__ float lane_group_max(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float y = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// max(a, b) for scores (finite or -inf): IEEE maximum, which propagates NaN
// instead of quieting its operands, so a swapped-in value needs no extra
// instruction.
__device__ __forceinline__ float max_nn(float a, float b) { return __builtin_elementwise_maximum(a, b); }

__device__ __forceinline__ float lane_group_max_nn(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float y = max_nn(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  return max_nn(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ float lane_group_sum(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float y = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Maximum / sum of x over the whole wave: DPP quad permutations and row
// mirrors combine each 16-lane row, the half-wave swaps combine the rows.
// Every lane ends with the result; the pairing order is fixed.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}

// Maximum / sum over the 16 lanes of a row (lanes 16k .. 16k + 15): pairs,
// then quads, then the mirrored halves of 8 and of 16.  Each step combines two
// partial results that every lane of the pair holds with the same bits, so all
// 16 lanes end with the same value.
__device__ __forceinline__ float row16_max(float x) {
  x = fmaxf(x, dpp_mov<0xB1>(x));    // quad_perm [1,0,3,2]
  x = fmaxf(x, dpp_mov<0x4E>(x));    // quad_perm [2,3,0,1]
  x = fmaxf(x, dpp_mov<0x141>(x));   // row_half_mirror
  x = fmaxf(x, dpp_mov<0x140>(x));   // row_mirror
  return x;
}

__device__ __forceinline__ float row16_sum(float x) {
  x += dpp_mov<0xB1>(x);
  x += dpp_mov<0x4E>(x);
  x += dpp_mov<0x141>(x);
  x += dpp_mov<0x140>(x);
  return x;
}

__device__ __forceinline__ float wave_max(float x) { return lane_group_max(row16_max(x)); }

__device__ __forceinline__ float wave_sum(float x) { return lane_group_sum(row16_sum(x)); }

}  // namespace tpa
