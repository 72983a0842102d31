// Factor projection: F = X * W_packed^T, split into the factor tensors, with
// the rotary embedding of the query/key dim factors fused into the epilogue.
//
// "Tensor Product Attention Is All You Need" review on coreui.cn, code
// walk-through 前向传播: six bias-free linear layers produce A_q, A_k, A_v
// (viewed [h, R]) and B_q, B_k, B_v (viewed [R, d_h]); question 2 of
// 关键问题及回答: the key dim factors are rotated before they are cached.
//
// The packed weight stacks the rotated outputs first (W_B_q, W_B_k, then
// W_B_v, W_A_q, W_A_k, W_A_v), so the rotated columns are [0, rot_cols) and
// every rotary pair (2i, 2i+1) sits on an even column.
#include "kernels.h"

namespace tpa {

// Writes the pair of columns (n, n+1) of row m (n even); n+1 may be past N.
template <typename T>
__device__ __forceinline__ void proj_store_pair(const ProjArgs& a, int64_t m, int n, float v0, float v1) {
  const int64_t s = m % a.S;
  const int64_t b = m / a.S;
  if (n < a.rot_cols) {
    float c, sn;
    rope_cos_sin(a.rope, a.start_pos + s, (n % a.head_dim) >> 1, c, sn);
    const float r0 = v0 * c - v1 * sn;
    const float r1 = v0 * sn + v1 * c;
    v0 = r0;
    v1 = r1;
  }
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int col = n + q;
    if (col >= a.N) break;
    int e = 0;
    while (e + 1 < a.nseg && col >= a.seg_begin[e + 1]) ++e;
    T* d = reinterpret_cast<T*>(a.dst[e]);
    stf(d, b * a.bstride[e] + s * a.width[e] + (col - a.seg_begin[e]), q ? v1 : v0);
  }
}

// General tiled GEMM on the vector ALUs: 64x64 output tile per 256-thread
// workgroup, 4x4 outputs per thread, K staged through LDS in steps of 16.
template <typename T>
__global__ void __launch_bounds__(256) proj_generic_kernel(ProjArgs a) {
  constexpr int BM = 64, BN = 64, BK = 16;
  __shared__ float xs[BK][BM + 4];
  __shared__ float ws[BK][BN + 4];
  const T* X = reinterpret_cast<const T*>(a.x);
  const T* W = reinterpret_cast<const T*>(a.w);
  const int tid = threadIdx.x;
  const int tx = tid & 15, ty = tid >> 4;
  const int64_t m0 = (int64_t)blockIdx.x * BM;
  const int n0 = blockIdx.y * BN;
  float acc[4][4] = {};
  const int lr = tid >> 2;          // tile row loaded by this thread
  const int lk = (tid & 3) * 4;     // first k of its 4 loads
  for (int64_t k0 = 0; k0 < a.K; k0 += BK) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int64_t k = k0 + lk + q;
      const int64_t m = m0 + lr;
      const int n = n0 + lr;
      xs[lk + q][lr] = (m < a.M && k < a.K) ? ldf(X, m * a.K + k) : 0.f;
      ws[lk + q][lr] = (n < a.N && k < a.K) ? ldf(W, (int64_t)n * a.K + k) : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < BK; ++kk) {
      float av[4], bv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) av[i] = xs[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) bv[j] = ws[kk][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(av[i], bv[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t m = m0 + ty * 4 + i;
    if (m >= a.M) continue;
#pragma unroll
    for (int jp = 0; jp < 2; ++jp) {
      const int n = n0 + tx * 4 + 2 * jp;
      if (n < a.N) proj_store_pair<T>(a, m, n, acc[i][2 * jp], acc[i][2 * jp + 1]);
    }
  }
}

hipError_t launch_factor_proj(int dtype, const ProjArgs& a, hipStream_t st) {
  dim3 grid((unsigned)((a.M + 63) / 64), (unsigned)((a.N + 63) / 64));
  if (dtype == kF32)
    hipLaunchKernelGGL(proj_generic_kernel<float>, grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(proj_generic_kernel<bf16_t>, grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace tpa
