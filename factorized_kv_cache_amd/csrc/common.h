// Device helpers shared by the libtpa kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tpa {

typedef uint16_t bf16_t;

// ---------------------------------------------------------------------------
// bfloat16 <-> float32.  bf16 is the top half of an IEEE binary32; narrowing
// rounds to nearest, ties to even (the language conversion, which gfx950 does
// in one v_cvt_pk_bf16_f32 per pair).
// ---------------------------------------------------------------------------
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_to_f32(uint16_t v) { return __uint_as_float((uint32_t)v << 16); }

__device__ __forceinline__ uint16_t f32_to_bf16(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// Element load/store in float32 arithmetic, for either storage type.
__device__ __forceinline__ float ldf(const float* p, int64_t i) { return p[i]; }
__device__ __forceinline__ float ldf(const bf16_t* p, int64_t i) { return bf16_to_f32(p[i]); }
__device__ __forceinline__ void stf(float* p, int64_t i, float v) { p[i] = v; }
__device__ __forceinline__ void stf(bf16_t* p, int64_t i, float v) { p[i] = f32_to_bf16(v); }

// ---------------------------------------------------------------------------
// Rotary angles.  rev[i] = base^(-2i/d_h) / (2*pi), computed on the host in
// float64.  The angle pos*theta_i is formed in float64 as a number of turns,
// reduced to [-1/2, 1/2] turns, and only then narrowed to float32 (so large
// positions lose no precision to the narrowing).  v_sin_f32 / v_cos_f32 take
// their argument in turns; over [-1/2, 1/2] they agree with fp64 sin/cos to
// about 1.3e-7 (measured on gfx950 over 4M random angles).
// ---------------------------------------------------------------------------
constexpr int kMaxRopePairs = 128;  // head_dim <= 256

struct RopeTable {
  double rev[kMaxRopePairs];
};

// rev points at the table's frequencies; kernels whose lanes index it with
// differing pairs keep a copy in LDS and pass that.
__device__ __forceinline__ void rope_cos_sin(const double* rev, int64_t pos, int pair, float& c, float& s) {
  double turns = (double)pos * rev[pair];
  turns -= rint(turns);
  const float t = (float)turns;
  s = __builtin_amdgcn_sinf(t);
  c = __builtin_amdgcn_cosf(t);
}

__device__ __forceinline__ void rope_cos_sin(const RopeTable& tab, int64_t pos, int pair, float& c, float& s) {
  rope_cos_sin(tab.rev, pos, pair, c, s);
}

// Copies the first n_pairs frequencies into LDS; the caller's next barrier
// makes them visible to the workgroup.
__device__ __forceinline__ void rope_stage(const RopeTable& tab, int n_pairs, double* s_rev) {
  for (int i = threadIdx.x; i < n_pairs && i < kMaxRopePairs; i += blockDim.x) s_rev[i] = tab.rev[i];
}

// Softmax runs in base 2: scores are pre-multiplied by log2(e).
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace tpa
