// Standalone rotary embedding of dim factors, in place.
//
// b is [n_tok, rows, d_h]; token m = b_idx*S + s sits at position start_pos + s.
// Every (2i, 2i+1) pair turns by pos * base^(-2i/d_h) (pre-rotation of the
// key dim factors: "Tensor Product Attention Is All You Need" review on
// coreui.cn, question 2 of 关键问题及回答).
//
// The angles depend on the token and the pair only, so the main kernel gives a
// thread one 16-byte piece of d (four pairs in bf16, two in fp32) of one
// token: it forms those angles once and turns the piece in every row, one
// 16-byte load and store per row.  Consecutive threads take consecutive pieces
// of a token, so a row's d_h elements move as whole lines.  Other head sizes
// and unaligned tensors take the element kernel (one pair per thread).
#include "kernels.h"

namespace tpa {

template <typename T>
__global__ void __launch_bounds__(256) rope_kernel(RopeArgs a) {
  const int half = a.head_dim >> 1;
  const int64_t pairs_per_tok = (int64_t)a.rows * half;
  const int64_t total = a.n_tok * pairs_per_tok;
  T* b = reinterpret_cast<T*>(a.b);
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int64_t m = idx / pairs_per_tok;
    const int64_t rem = idx - m * pairs_per_tok;
    const int pair = (int)(rem % half);
    const int64_t pos = a.start_pos + (m % a.S);
    float c, s;
    rope_cos_sin(a.rope, pos, pair, c, s);
    const int64_t e = 2 * idx;  // element index of the pair's first element
    const float x0 = ldf(b, e), x1 = ldf(b, e + 1);
    stf(b, e, fmaf(x0, c, -(x1 * s)));   // the same operation order as the piece kernel
    stf(b, e + 1, fmaf(x0, s, x1 * c));
  }
}


template <typename T>
__global__ void __launch_bounds__(256) rope_piece_kernel(RopeArgs a) {
  constexpr int E = 16 / (int)sizeof(T), P = E / 2;   // elements and pairs of a piece
  const int G = a.head_dim / E;
  const int64_t total = a.n_tok * G;
  const int64_t row_stride = a.head_dim;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int64_t m = idx / G;
    const int g = (int)(idx - m * G);
    const int64_t pos = a.start_pos + (m % a.S);
    float c[P], sn[P];
#pragma unroll
    for (int p = 0; p < P; ++p) rope_cos_sin(a.rope, pos, g * P + p, c[p], sn[p]);
    T* row = reinterpret_cast<T*>(a.b) + m * a.rows * row_stride + g * E;
    for (int r = 0; r < a.rows; ++r, row += row_stride) {
      uint4 v = *reinterpret_cast<const uint4*>(row);
      float x[E];
      if constexpr (sizeof(T) == 2) {
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          x[2 * q] = __uint_as_float(w[q] << 16);
          x[2 * q + 1] = __uint_as_float(w[q] & 0xffff0000u);
        }
      } else {
        x[0] = __uint_as_float(v.x);
        x[1] = __uint_as_float(v.y);
        x[2] = __uint_as_float(v.z);
        x[3] = __uint_as_float(v.w);
      }
#pragma unroll
      for (int p = 0; p < P; ++p) {
        const float x0 = x[2 * p], x1 = x[2 * p + 1];
        x[2 * p] = fmaf(x0, c[p], -(x1 * sn[p]));
        x[2 * p + 1] = fmaf(x0, sn[p], x1 * c[p]);
      }
      if constexpr (sizeof(T) == 2)
        v = make_uint4(pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(x[4], x[5]),
                       pack_bf16x2(x[6], x[7]));
      else
        v = make_uint4(__float_as_uint(x[0]), __float_as_uint(x[1]), __float_as_uint(x[2]), __float_as_uint(x[3]));
      *reinterpret_cast<uint4*>(row) = v;
    }
  }
}

hipError_t launch_rope(int dtype, const RopeArgs& a, hipStream_t st) {
  const int es = dtype == kF32 ? 4 : 2;
  const int E = 16 / es;
  if (a.head_dim % E == 0 && ((uintptr_t)a.b & 15) == 0) {
    const int64_t total = a.n_tok * (a.head_dim / E);
    int64_t blocks = (total + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    if (blocks < 1) blocks = 1;
    if (dtype == kF32)
      hipLaunchKernelGGL(rope_piece_kernel<float>, dim3((unsigned)blocks), dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL(rope_piece_kernel<bf16_t>, dim3((unsigned)blocks), dim3(256), 0, st, a);
    return hipGetLastError();
  }
  const int64_t total = a.n_tok * (int64_t)a.rows * (a.head_dim / 2);
  int64_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (blocks < 1) blocks = 1;
  if (dtype == kF32)
    hipLaunchKernelGGL(rope_kernel<float>, dim3((unsigned)blocks), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(rope_kernel<bf16_t>, dim3((unsigned)blocks), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace tpa
