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
__device__ __forceinline__ void proj_store_pair(const ProjArgs& a, const double* rev, int64_t m, int n, float v0,
                                                float v1) {
  const int64_t s = m % a.S;
  const int64_t b = m / a.S;
  if (n < a.rot_cols) {
    float c, sn;
    rope_cos_sin(rev, a.start_pos + s, (n % a.head_dim) >> 1, c, sn);
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

// Writes columns n .. n+7 of row m = b*S + s (n a multiple of 8) from float32
// values v, rotating the pairs below rot_cols (frequencies from rev, in LDS).  With vec8 the piece lies in one
// segment and one head and goes out as a single 16-byte store; otherwise each
// column is placed on its own (columns past N are dropped).
__device__ __forceinline__ void proj_store_piece8(const ProjArgs& a, const double* rev, uint32_t b, uint32_t s, int n,
                                                  float* v) {
  const int64_t pos = a.start_pos + s;
  if (a.vec8) {
    if (n < a.rot_cols) {
      const int p0 = (n % a.head_dim) >> 1;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float c, sn;
        rope_cos_sin(rev, pos, p0 + j, c, sn);
        const float r0 = v[2 * j] * c - v[2 * j + 1] * sn;
        const float r1 = v[2 * j] * sn + v[2 * j + 1] * c;
        v[2 * j] = r0;
        v[2 * j + 1] = r1;
      }
    }
    int e = 0;
    while (e + 1 < a.nseg && n >= a.seg_begin[e + 1]) ++e;
    bf16_t* d = reinterpret_cast<bf16_t*>(a.dst[e]) + (int64_t)b * a.bstride[e] + (int64_t)s * a.width[e] +
                (n - a.seg_begin[e]);
    *reinterpret_cast<uint4*>(d) = make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                                              pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7]));
    return;
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int c0 = n + 2 * j;
    if (c0 < a.rot_cols) {
      float c, sn;
      rope_cos_sin(rev, pos, (c0 % a.head_dim) >> 1, c, sn);
      const float r0 = v[2 * j] * c - v[2 * j + 1] * sn;
      const float r1 = v[2 * j] * sn + v[2 * j + 1] * c;
      v[2 * j] = r0;
      v[2 * j + 1] = r1;
    }
  }
  for (int q = 0; q < 8; ++q) {
    const int col = n + q;
    if (col >= a.N) break;
    int e = 0;
    while (e + 1 < a.nseg && col >= a.seg_begin[e + 1]) ++e;
    bf16_t* d = reinterpret_cast<bf16_t*>(a.dst[e]);
    d[(int64_t)b * a.bstride[e] + (int64_t)s * a.width[e] + (col - a.seg_begin[e])] = f32_to_bf16(v[q]);
  }
}

// General tiled GEMM on the vector ALUs: 64x64 output tile per 256-thread
// workgroup, 4x4 outputs per thread, K staged through LDS in steps of 16.
template <typename T>
__global__ void __launch_bounds__(256) proj_generic_kernel(ProjArgs a) {
  constexpr int BM = 64, BN = 64, BK = 16;
  __shared__ float xs[BK][BM + 4];
  __shared__ float ws[BK][BN + 4];
  __shared__ double s_rev[kMaxRopePairs];
  rope_stage(a.rope, a.head_dim >> 1, s_rev);
  __syncthreads();
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
      if (n < a.N) proj_store_pair<T>(a, s_rev, m, n, acc[i][2 * jp], acc[i][2 * jp + 1]);
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

// U = k-steps of 32 whose loads are issued together; it divides K / (32 * 8).
template <int MT, int U>
__global__ void __launch_bounds__(64 * kSkinnyWaves) proj_skinny_kernel(ProjArgs a) {
  __shared__ float red[kSkinnyWaves][16][16 * MT + 1];
  __shared__ double s_rev[kMaxRopePairs];
  rope_stage(a.rope, a.head_dim >> 1, s_rev);
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
  for (int k = 0; k < kq; k += 32 * U) {
    uint4 wv[U], xv[U][MT];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      wv[u] = *reinterpret_cast<const uint4*>(wrow + k + 32 * u);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) xv[u][mt] = *reinterpret_cast<const uint4*>(xrow[mt] + k + 32 * u);
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[mt] = mfma_bf16(as_bf16x8(wv[u]), as_bf16x8(xv[u][mt]), acc[mt]);
  }
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) red[wave][4 * lg + i][mt * 16 + li] = acc[mt][i];
  __syncthreads();
  // one 8-column piece (half of the 16 weight rows) of one token per thread
  const int item = threadIdx.x;
  const int m = item >> 1, n = n0 + 8 * (item & 1);
  if (item >= 2 * 16 * MT || m >= M || n >= N) return;
  float v[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) v[q] = 0.f;
#pragma unroll
  for (int w = 0; w < kSkinnyWaves; ++w)
#pragma unroll
    for (int q = 0; q < 8; ++q) v[q] += red[w][8 * (item & 1) + q][m];
  const uint32_t S = (uint32_t)a.S;
  const uint32_t b = (uint32_t)m / S;
  proj_store_piece8(a, s_rev, b, (uint32_t)m - b * S, n, v);
}

// ---------------------------------------------------------------------------
// Many tokens (prefill): 128 x 128 output tile per workgroup, four waves of
// 64 x 64, K staged through one LDS slab buffer 64 at a time.  The buffer is
// single and nothing is prefetched into registers, so a workgroup needs 37 KB
// of LDS and 128 registers: four workgroups share a CU and hide each other's
// slab loads (the 896 tiles of a 16,384 x 800 projection then run in one
// round).  Measured against two buffers with the next slab prefetched into
// registers (two workgroups per CU): 61 against 68 us at 16,384 x 800 x 1024,
// 1.25 against 1.37 ms at 131,072 x 2240 x 1536.
// ---------------------------------------------------------------------------
constexpr int kPBM = 128, kPBN = 128, kPBK = 64, kPLDK = kPBK + 8;
constexpr int kPSlab = (kPBM + kPBN) * kPLDK;   // bf16 elements of one slab buffer

// The epilogue stages half of the fp32 tile (64 rows) at a time in the same
// LDS, then each thread rotates and stores 8-column pieces.
constexpr int kPLDT = kPBN + 4;
static_assert(64 * kPLDT * 4 <= kPSlab * 2, "epilogue tile must fit the slab buffer");

__global__ void __launch_bounds__(256, 4) proj_mfma_kernel(ProjArgs a) {
  __shared__ __align__(16) bf16_t lds[kPSlab];
  __shared__ double s_rev[kMaxRopePairs];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = lane & 15, lg = lane >> 4;
  const int wm = wave >> 1, wn = wave & 1;
  // Workgroups go to the eight XCDs round-robin by linear index.  The grid is
  // padded to a multiple of 8 row tiles and ordered so that each XCD takes its
  // row tiles in turn with all column tiles of one row tile back to back:
  // those share the X rows, which then come from that XCD's L2.
  const int n_ntiles = (int)((a.N + kPBN - 1) / kPBN);
  const int n_mtiles = (int)((a.M + kPBM - 1) / kPBM);
  const int xcd = blockIdx.x & 7, q = blockIdx.x >> 3;
  const int mtile = (q / n_ntiles) * 8 + xcd, ntile = q % n_ntiles;
  if (mtile >= n_mtiles) return;
  rope_stage(a.rope, a.head_dim >> 1, s_rev);   // visible after the first barrier
  const int64_t m0 = (int64_t)mtile * kPBM;
  const int n0 = ntile * kPBN;
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
  auto store_slab = [&](bf16_t* xs, bf16_t* ws) __attribute__((always_inline)) {
    *reinterpret_cast<uint4*>(xs + (srow + 0) * kPLDK + spc * 8) = xr0;
    *reinterpret_cast<uint4*>(xs + (srow + 32) * kPLDK + spc * 8) = xr1;
    *reinterpret_cast<uint4*>(xs + (srow + 64) * kPLDK + spc * 8) = xr2;
    *reinterpret_cast<uint4*>(xs + (srow + 96) * kPLDK + spc * 8) = xr3;
    *reinterpret_cast<uint4*>(ws + (srow + 0) * kPLDK + spc * 8) = wr0;
    *reinterpret_cast<uint4*>(ws + (srow + 32) * kPLDK + spc * 8) = wr1;
    *reinterpret_cast<uint4*>(ws + (srow + 64) * kPLDK + spc * 8) = wr2;
    *reinterpret_cast<uint4*>(ws + (srow + 96) * kPLDK + spc * 8) = wr3;
  };
  auto load_slab = [&](int64_t kn) __attribute__((always_inline)) {
    xr0 = *reinterpret_cast<const uint4*>(xsrc[0] + kn);
    xr1 = *reinterpret_cast<const uint4*>(xsrc[1] + kn);
    xr2 = *reinterpret_cast<const uint4*>(xsrc[2] + kn);
    xr3 = *reinterpret_cast<const uint4*>(xsrc[3] + kn);
    wr0 = *reinterpret_cast<const uint4*>(wsrc[0] + kn);
    wr1 = *reinterpret_cast<const uint4*>(wsrc[1] + kn);
    wr2 = *reinterpret_cast<const uint4*>(wsrc[2] + kn);
    wr3 = *reinterpret_cast<const uint4*>(wsrc[3] + kn);
  };
  store_slab(lds, lds + kPBM * kPLDK);
  __syncthreads();
  for (int64_t k0 = 0; k0 < K; k0 += kPBK) {
    const bf16_t* xs = lds;
    const bf16_t* ws = xs + kPBM * kPLDK;
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
    __syncthreads();   // every wave has read the slab
    if (k0 + kPBK < K) {
      load_slab(k0 + kPBK);
      store_slab(lds, lds + kPBM * kPLDK);
      __syncthreads();
    }
  }
  // Tile rows wm*64 + tm*16 + 4*lg + i, columns wn*64 + tn*16 + li.
  float* tile = reinterpret_cast<float*>(lds);
  const int pc = tid & 15;          // this thread's 8-column piece
  const int n = n0 + 8 * pc;
  const uint32_t S = (uint32_t)a.S;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    if (wm == half) {
#pragma unroll
      for (int tm = 0; tm < 4; ++tm)
#pragma unroll
        for (int tn = 0; tn < 4; ++tn)
#pragma unroll
          for (int i = 0; i < 4; ++i) tile[(tm * 16 + 4 * lg + i) * kPLDT + wn * 64 + tn * 16 + li] = acc[tm][tn][i];
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = (tid >> 4) + 16 * j;
      const int64_t m = m0 + half * 64 + r;
      if (m < M && n < N) {
        float v[8];
        const float4 lo = *reinterpret_cast<const float4*>(tile + r * kPLDT + 8 * pc);
        const float4 hi = *reinterpret_cast<const float4*>(tile + r * kPLDT + 8 * pc + 4);
        v[0] = lo.x; v[1] = lo.y; v[2] = lo.z; v[3] = lo.w;
        v[4] = hi.x; v[5] = hi.y; v[6] = hi.z; v[7] = hi.w;
        const uint32_t b = (uint32_t)m / S;
        proj_store_piece8(a, s_rev, b, (uint32_t)m - b * S, n, v);
      }
    }
    if (half == 0) __syncthreads();
  }
}

static bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

hipError_t launch_factor_proj(int dtype, const ProjArgs& a, hipStream_t st) {
  const int64_t mfma_grid = ((a.M + kPBM * 8 - 1) / (kPBM * 8)) * 8 * ((a.N + kPBN - 1) / kPBN);
  if (dtype == kBF16 && aligned16(a.x) && aligned16(a.w) && a.K % 64 == 0 && mfma_grid <= INT32_MAX) {
    if (a.M <= 64 && a.K % (32 * kSkinnyWaves) == 0) {
      const dim3 grid((unsigned)((a.N + 15) / 16)), block(64 * kSkinnyWaves);
      const int64_t steps = a.K / (32 * kSkinnyWaves);
      const int u = steps % 8 == 0 ? 8 : steps % 4 == 0 ? 4 : steps % 2 == 0 ? 2 : 1;
      const int mt = (int)((a.M + 15) / 16);
#define TPA_SKINNY(MT, U) hipLaunchKernelGGL((proj_skinny_kernel<MT, U>), grid, block, 0, st, a)
#define TPA_SKINNY_U(MT)               \
  switch (u) {                         \
    case 8: TPA_SKINNY(MT, 8); break;  \
    case 4: TPA_SKINNY(MT, 4); break;  \
    case 2: TPA_SKINNY(MT, 2); break;  \
    default: TPA_SKINNY(MT, 1); break; \
  }
      switch (mt) {
        case 1: TPA_SKINNY_U(1); break;
        case 2: TPA_SKINNY_U(2); break;
        case 3: TPA_SKINNY_U(3); break;
        default: TPA_SKINNY_U(4); break;
      }
#undef TPA_SKINNY_U
#undef TPA_SKINNY
    } else {
      const int64_t mt = (a.M + kPBM - 1) / kPBM, nt = (a.N + kPBN - 1) / kPBN;
      const dim3 grid((unsigned)(((mt + 7) / 8) * 8 * nt));
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
