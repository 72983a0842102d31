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
#include "mfma.h"

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

// ---------------------------------------------------------------------------
// Few tokens (decode): bound by reading the weights once.  One workgroup owns
// 16 weight rows; its eight waves split K.  The product is taken as
// D[n, m] = W[n, :] . X[m, :], weight rows as the A operand and tokens as the B
// operand, both read straight from memory (K-contiguous), up to eight k-steps'
// loads issued together.  The eight partial tiles are summed in LDS in wave
// order, then the epilogue stores pairs.
// ---------------------------------------------------------------------------
constexpr int kSkinnyWaves = 8;

template <int MT>
__global__ void __launch_bounds__(64 * kSkinnyWaves) proj_skinny_kernel(ProjArgs a) {
  __shared__ float red[kSkinnyWaves][16][16 * MT + 1];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int li = lane & 15, lg = lane >> 4;
  const int n0 = blockIdx.x * 16;
  const int K = (int)a.K, M = (int)a.M, N = (int)a.N;
  const int kq = K / kSkinnyWaves;
  const bf16_t* X = reinterpret_cast<const bf16_t*>(a.x);
  const bf16_t* W = reinterpret_cast<const bf16_t*>(a.w);
  const int nrow = (n0 + li < N) ? n0 + li : N - 1;
  const bf16_t* wrow = W + (int64_t)nrow * K + wave * kq + lg * 8;
  const bf16_t* xrow[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int m = (mt * 16 + li < M) ? mt * 16 + li : M - 1;
    xrow[mt] = X + (int64_t)m * K + wave * kq + lg * 8;
  }
  f32x4_t acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // eight k-steps per trip (steps past kq repeat the last address, unused)
  for (int k = 0; k < kq; k += 256) {
    uint4 wv[8], xv[8][MT];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int ku = k + 32 * u < kq ? k + 32 * u : kq - 32;
      wv[u] = *reinterpret_cast<const uint4*>(wrow + ku);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) xv[u][mt] = *reinterpret_cast<const uint4*>(xrow[mt] + ku);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (k + 32 * u >= kq) break;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[mt] = mfma_bf16(as_bf16x8(wv[u]), as_bf16x8(xv[u][mt]), acc[mt]);
    }
  }
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) red[wave][4 * lg + i][mt * 16 + li] = acc[mt][i];
  __syncthreads();
  for (int item = threadIdx.x; item < 8 * 16 * MT; item += blockDim.x) {
    const int p = item & 7, m = item >> 3;   // rows 2p, 2p+1 of the tile, token m
    const int n = n0 + 2 * p;
    if (m >= M || n >= N) continue;
    float v0 = 0.f, v1 = 0.f;
#pragma unroll
    for (int w = 0; w < kSkinnyWaves; ++w) {
      v0 += red[w][2 * p][m];
      v1 += red[w][2 * p + 1][m];
    }
    proj_store_pair<bf16_t>(a, m, n, v0, v1);
  }
}

// ---------------------------------------------------------------------------
// Many tokens (prefill): 128 x 128 output tile per workgroup, four waves of
// 64 x 64, K staged through LDS 64 at a time with the next slab held in
// registers while the current one is multiplied.
// ---------------------------------------------------------------------------
constexpr int kPBM = 128, kPBN = 128, kPBK = 64, kPLDK = kPBK + 8;

__global__ void __launch_bounds__(256, 2) proj_mfma_kernel(ProjArgs a) {
  __shared__ __align__(16) bf16_t xs[kPBM * kPLDK];
  __shared__ __align__(16) bf16_t ws[kPBN * kPLDK];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = lane & 15, lg = lane >> 4;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t m0 = (int64_t)blockIdx.x * kPBM;
  const int n0 = blockIdx.y * kPBN;
  const int64_t M = a.M, K = a.K;
  const int N = (int)a.N;
  const bf16_t* X = reinterpret_cast<const bf16_t*>(a.x);
  const bf16_t* W = reinterpret_cast<const bf16_t*>(a.w);

  // This thread's four 16-byte pieces of each slab: row = idx / 8, piece = idx % 8.
  // Rows past M or N are clamped to the last row: they only feed outputs that
  // are never stored.
  const bf16_t* xsrc[4];
  const bf16_t* wsrc[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int idx = tid + 256 * q, row = idx >> 3, pc = idx & 7;
    const int64_t xm = m0 + row < M ? m0 + row : M - 1;
    const int64_t wn_ = n0 + row < N ? n0 + row : N - 1;
    xsrc[q] = X + xm * K + pc * 8;
    wsrc[q] = W + wn_ * K + pc * 8;
  }
  uint4 xr0 = *reinterpret_cast<const uint4*>(xsrc[0]), xr1 = *reinterpret_cast<const uint4*>(xsrc[1]);
  uint4 xr2 = *reinterpret_cast<const uint4*>(xsrc[2]), xr3 = *reinterpret_cast<const uint4*>(xsrc[3]);
  uint4 wr0 = *reinterpret_cast<const uint4*>(wsrc[0]), wr1 = *reinterpret_cast<const uint4*>(wsrc[1]);
  uint4 wr2 = *reinterpret_cast<const uint4*>(wsrc[2]), wr3 = *reinterpret_cast<const uint4*>(wsrc[3]);
  f32x4_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int srow = tid >> 3, spc = tid & 7;   // row of piece q is srow + 32 q
  for (int64_t k0 = 0; k0 < K; k0 += kPBK) {
    *reinterpret_cast<uint4*>(xs + (srow + 0) * kPLDK + spc * 8) = xr0;
    *reinterpret_cast<uint4*>(xs + (srow + 32) * kPLDK + spc * 8) = xr1;
    *reinterpret_cast<uint4*>(xs + (srow + 64) * kPLDK + spc * 8) = xr2;
    *reinterpret_cast<uint4*>(xs + (srow + 96) * kPLDK + spc * 8) = xr3;
    *reinterpret_cast<uint4*>(ws + (srow + 0) * kPLDK + spc * 8) = wr0;
    *reinterpret_cast<uint4*>(ws + (srow + 32) * kPLDK + spc * 8) = wr1;
    *reinterpret_cast<uint4*>(ws + (srow + 64) * kPLDK + spc * 8) = wr2;
    *reinterpret_cast<uint4*>(ws + (srow + 96) * kPLDK + spc * 8) = wr3;
    __syncthreads();
    // next slab (the last iteration reloads the final slab; it is never used)
    const int64_t kn = k0 + kPBK < K ? k0 + kPBK : k0;
    xr0 = *reinterpret_cast<const uint4*>(xsrc[0] + kn);
    xr1 = *reinterpret_cast<const uint4*>(xsrc[1] + kn);
    xr2 = *reinterpret_cast<const uint4*>(xsrc[2] + kn);
    xr3 = *reinterpret_cast<const uint4*>(xsrc[3] + kn);
    wr0 = *reinterpret_cast<const uint4*>(wsrc[0] + kn);
    wr1 = *reinterpret_cast<const uint4*>(wsrc[1] + kn);
    wr2 = *reinterpret_cast<const uint4*>(wsrc[2] + kn);
    wr3 = *reinterpret_cast<const uint4*>(wsrc[3] + kn);
#pragma unroll
    for (int ks = 0; ks < kPBK / 32; ++ks) {
      bf16x8_t af[4], bfr[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        af[t] = as_bf16x8(*reinterpret_cast<const uint4*>(xs + (wm * 64 + t * 16 + li) * kPLDK + ks * 32 + lg * 8));
        bfr[t] = as_bf16x8(*reinterpret_cast<const uint4*>(ws + (wn * 64 + t * 16 + li) * kPLDK + ks * 32 + lg * 8));
      }
#pragma unroll
      for (int tm = 0; tm < 4; ++tm)
#pragma unroll
        for (int tn = 0; tn < 4; ++tn) acc[tm][tn] = mfma_bf16(af[tm], bfr[tn], acc[tm][tn]);
    }
    __syncthreads();
  }
  // D[m][n] with n = ... + li: the rotary partner column n^1 is lane li^1.
#pragma unroll
  for (int tm = 0; tm < 4; ++tm)
#pragma unroll
    for (int tn = 0; tn < 4; ++tn)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float v = acc[tm][tn][i];
        const float partner = __shfl_xor(v, 1);
        const int64_t m = m0 + wm * 64 + tm * 16 + 4 * lg + i;
        const int n = n0 + wn * 64 + tn * 16 + li;
        if (!(li & 1) && m < M && n < N) proj_store_pair<bf16_t>(a, m, n, v, partner);
      }
}

static bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

hipError_t launch_factor_proj(int dtype, const ProjArgs& a, hipStream_t st) {
  if (dtype == kBF16 && aligned16(a.x) && aligned16(a.w) && a.K % 64 == 0) {
    if (a.M <= 64 && a.K % (32 * kSkinnyWaves) == 0) {
      const dim3 grid((unsigned)((a.N + 15) / 16)), block(64 * kSkinnyWaves);
      switch ((a.M + 15) / 16) {
        case 1: hipLaunchKernelGGL(proj_skinny_kernel<1>, grid, block, 0, st, a); break;
        case 2: hipLaunchKernelGGL(proj_skinny_kernel<2>, grid, block, 0, st, a); break;
        case 3: hipLaunchKernelGGL(proj_skinny_kernel<3>, grid, block, 0, st, a); break;
        default: hipLaunchKernelGGL(proj_skinny_kernel<4>, grid, block, 0, st, a); break;
      }
    } else {
      const dim3 grid((unsigned)((a.M + kPBM - 1) / kPBM), (unsigned)((a.N + kPBN - 1) / kPBN));
      hipLaunchKernelGGL(proj_mfma_kernel, grid, dim3(256), 0, st, a);
    }
    return hipGetLastError();
  }
  dim3 grid((unsigned)((a.M + 63) / 64), (unsigned)((a.N + 63) / 64));
  if (dtype == kF32)
    hipLaunchKernelGGL(proj_generic_kernel<float>, grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(proj_generic_kernel<bf16_t>, grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace tpa
