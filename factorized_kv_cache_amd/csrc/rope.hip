// Standalone rotary embedding of dim factors, in place.
//
// b is [n_tok, rows, d_h]; token m = b_idx*S + s sits at position start_pos + s.
// Each thread turns one (2i, 2i+1) pair by pos * base^(-2i/d_h)
// (pre-rotation of the key dim factors: "Tensor Product Attention Is All You
// Need" review on coreui.cn, question 2 of 关键问题及回答).
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
    stf(b, e, x0 * c - x1 * s);
    stf(b, e + 1, x0 * s + x1 * c);
  }
}

hipError_t launch_rope(int dtype, const RopeArgs& a, hipStream_t st) {
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
