// Prefill attention over the factor cache (causal or full), general kernel.
//
// Per (query block, head, sequence): the query block is formed from its
// factors, and for every key block the keys and values of this head are
// rebuilt from the cached factors in LDS, k_t = sum_r A_K[t,h,r] B~_K[t,r,:]
// (the 1/R_K is folded into the query scale, 1/R_V into the output), followed
// by an online softmax in base 2.  ("Tensor Product Attention Is All You
// Need" review on coreui.cn: the Q_t/K_t/V_t equations of 核心机制总结 and the
// masked softmax attention of the code walk-through 前向传播; the attention
// formula of the jieyibu.net explainer, section Ⅱ.1.)
#include "kernels.h"

namespace tpa {

constexpr int kPrefillThreads = 256;

template <typename T>
__device__ __forceinline__ float rebuild(const T* A, const T* Bm, int64_t tok, int hh, int h, int R, int dh, int d) {
  float v = 0.f;
  for (int r = 0; r < R; ++r) v = fmaf(ldf(A, (tok * h + hh) * R + r), ldf(Bm, (tok * R + r) * dh + d), v);
  return v;
}

// SHARED: the shared-basis cache.  a.c_bk / a.c_bv then point at the basis
// B_K [R_K, d_h] (unrotated) and B_V [R_V, d_h], and key t is rebuilt from its
// head factors and the basis, then rotated at its own position t.
template <typename T>
__device__ __forceinline__ float rebuild_basis(const T* A, const T* Bm, int64_t tok, int hh, int h, int R, int dh,
                                               int d) {
  float v = 0.f;
  for (int r = 0; r < R; ++r) v = fmaf(ldf(A, (tok * h + hh) * R + r), ldf(Bm, (int64_t)r * dh + d), v);
  return v;
}

template <typename T, int BM, int BN, bool SHARED>
__global__ void __launch_bounds__(kPrefillThreads) prefill_generic_kernel(AttnArgs a, RopeTable tab) {
  extern __shared__ float smem[];
  __shared__ double s_rev[SHARED ? kMaxRopePairs : 1];
  if constexpr (SHARED) rope_stage(tab, a.d_h >> 1, s_rev);   // visible after the next barrier
  constexpr int kOut = 16;  // BM * d_h / threads, at most (BM=32,d_h=128 or BM=16,d_h=256)
  const int h = a.h, dh = a.d_h;
  float* qs = smem;              // [BM][d_h]
  float* ks = qs + BM * dh;      // [BN][d_h]
  float* vs = ks + BN * dh;      // [BN][d_h]
  float* ss = vs + BN * dh;      // [BM][BN]
  float* mrow = ss + BM * BN;    // [BM]
  float* lrow = mrow + BM;       // [BM]
  float* alpha = lrow + BM;      // [BM]
  const int64_t q0 = (int64_t)blockIdx.x * BM;
  const int hh = blockIdx.y;
  const int64_t b = blockIdx.z;
  const T* AQ = reinterpret_cast<const T*>(a.a_q);
  const T* BQ = reinterpret_cast<const T*>(a.b_q);
  const T* AK = reinterpret_cast<const T*>(a.c_ak);
  const T* BK = reinterpret_cast<const T*>(a.c_bk);
  const T* AV = reinterpret_cast<const T*>(a.c_av);
  const T* BV = reinterpret_cast<const T*>(a.c_bv);
  const int64_t seq0 = b * a.max_seq;

  for (int idx = threadIdx.x; idx < BM * dh; idx += blockDim.x) {
    const int i = idx / dh, d = idx - i * dh;
    const int64_t s = q0 + i;
    float v = 0.f;
    if (s < a.S) {
      const int64_t tok = b * a.q_bstride_tok + s;
      v = (a.rq == 0) ? ldf(BQ, (tok * h + hh) * dh + d) : rebuild(AQ, BQ, tok, hh, h, a.rq, dh, d);
    }
    qs[idx] = v * a.q_scale;
  }
  for (int i = threadIdx.x; i < BM; i += blockDim.x) {
    mrow[i] = -INFINITY;
    lrow[i] = 0.f;
  }
  float acc[kOut];
#pragma unroll
  for (int j = 0; j < kOut; ++j) acc[j] = 0.f;
  __syncthreads();

  const int64_t n_keys = a.start_pos + a.S;
  const int64_t last_q = (q0 + BM < a.S ? q0 + BM : a.S) - 1;
  const int64_t kend = a.causal ? a.start_pos + last_q + 1 : n_keys;

  for (int64_t k0 = 0; k0 < kend; k0 += BN) {
    if constexpr (SHARED) {
      // one rotary pair (2i, 2i+1) of one key per item
      const int np = dh >> 1;
      for (int idx = threadIdx.x; idx < BN * np; idx += blockDim.x) {
        const int j = idx / np, i = idx - j * np;
        const int64_t t = k0 + j;
        float k0v = 0.f, k1v = 0.f, v0 = 0.f, v1 = 0.f;
        if (t < kend) {
          const float x0 = rebuild_basis(AK, BK, seq0 + t, hh, h, a.rk, dh, 2 * i);
          const float x1 = rebuild_basis(AK, BK, seq0 + t, hh, h, a.rk, dh, 2 * i + 1);
          float c, sn;
          rope_cos_sin(s_rev, t, i, c, sn);
          k0v = x0 * c - x1 * sn;
          k1v = x0 * sn + x1 * c;
          v0 = rebuild_basis(AV, BV, seq0 + t, hh, h, a.rv, dh, 2 * i);
          v1 = rebuild_basis(AV, BV, seq0 + t, hh, h, a.rv, dh, 2 * i + 1);
        }
        ks[j * dh + 2 * i] = k0v;
        ks[j * dh + 2 * i + 1] = k1v;
        vs[j * dh + 2 * i] = v0;
        vs[j * dh + 2 * i + 1] = v1;
      }
    } else {
      for (int idx = threadIdx.x; idx < BN * dh; idx += blockDim.x) {
        const int j = idx / dh, d = idx - j * dh;
        const int64_t t = k0 + j;
        float kv = 0.f, vv = 0.f;
        if (t < kend) {
          kv = rebuild(AK, BK, seq0 + t, hh, h, a.rk, dh, d);
          vv = rebuild(AV, BV, seq0 + t, hh, h, a.rv, dh, d);
        }
        ks[idx] = kv;
        vs[idx] = vv;
      }
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < BM * BN; idx += blockDim.x) {
      const int i = idx / BN, j = idx - i * BN;
      const int64_t t = k0 + j;
      const bool ok = t < kend && (!a.causal || t <= a.start_pos + q0 + i);
      float s = -INFINITY;
      if (ok) {
        s = 0.f;
        for (int d = 0; d < dh; ++d) s = fmaf(qs[i * dh + d], ks[j * dh + d], s);
      }
      ss[idx] = s;
    }
    __syncthreads();
    for (int i = threadIdx.x; i < BM; i += blockDim.x) {
      float mx = mrow[i];
      for (int j = 0; j < BN; ++j) mx = fmaxf(mx, ss[i * BN + j]);
      float al = 1.f, sum = 0.f;
      if (mx != -INFINITY) {
        al = fast_exp2(mrow[i] - mx);
        for (int j = 0; j < BN; ++j) {
          const float p = fast_exp2(ss[i * BN + j] - mx);
          ss[i * BN + j] = p;
          sum += p;
        }
      } else {
        for (int j = 0; j < BN; ++j) ss[i * BN + j] = 0.f;
      }
      lrow[i] = lrow[i] * al + sum;
      mrow[i] = mx;
      alpha[i] = al;
    }
    __syncthreads();
#pragma unroll
    for (int jo = 0; jo < kOut; ++jo) {
      const int idx = threadIdx.x + jo * kPrefillThreads;
      if (idx >= BM * dh) break;
      const int i = idx / dh, d = idx - i * dh;
      float o = acc[jo] * alpha[i];
      for (int j = 0; j < BN; ++j) o = fmaf(ss[i * BN + j], vs[j * dh + d], o);
      acc[jo] = o;
    }
    __syncthreads();
  }

  T* out = reinterpret_cast<T*>(a.out);
#pragma unroll
  for (int jo = 0; jo < kOut; ++jo) {
    const int idx = threadIdx.x + jo * kPrefillThreads;
    if (idx >= BM * dh) break;
    const int i = idx / dh, d = idx - i * dh;
    const int64_t s = q0 + i;
    if (s < a.S) stf(out, ((b * a.S + s) * h + hh) * (int64_t)dh + d, acc[jo] / lrow[i] * a.v_scale);
  }
}

template <typename T, bool SHARED>
static hipError_t launch_prefill_t(const AttnArgs& a, const RopeTable& tab, hipStream_t st) {
  if (a.d_h <= 128) {
    constexpr int BM = 32, BN = 32;
    const size_t lds = sizeof(float) * ((size_t)(BM + 2 * BN) * a.d_h + BM * BN + 3 * BM);
    dim3 grid((unsigned)((a.S + BM - 1) / BM), (unsigned)a.h, (unsigned)a.n_batch);
    hipLaunchKernelGGL((prefill_generic_kernel<T, BM, BN, SHARED>), grid, dim3(kPrefillThreads), lds, st, a, tab);
  } else {
    constexpr int BM = 16, BN = 16;
    const size_t lds = sizeof(float) * ((size_t)(BM + 2 * BN) * a.d_h + BM * BN + 3 * BM);
    dim3 grid((unsigned)((a.S + BM - 1) / BM), (unsigned)a.h, (unsigned)a.n_batch);
    hipLaunchKernelGGL((prefill_generic_kernel<T, BM, BN, SHARED>), grid, dim3(kPrefillThreads), lds, st, a, tab);
  }
  return hipGetLastError();
}

bool prefill_mfma_supported(int dtype, const AttnArgs& a);
hipError_t launch_prefill_mfma(const AttnArgs& a, hipStream_t st);
bool prefill_mfma32_supported(int dtype, const AttnArgs& a);
hipError_t launch_prefill_mfma32(const AttnArgs& a, hipStream_t st);
hipError_t launch_prefill_mfma32_shared(const AttnArgs& a, const RopeTable& tab, hipStream_t st);
bool prefill_material_shape_ok(int dtype, const AttnArgs& a);
bool prefill_material_supported(int dtype, const AttnArgs& a);
size_t prefill_material_bytes(const AttnArgs& a);
hipError_t launch_prefill_material(const AttnArgs& a, void* ws, const RopeTable* tab, hipStream_t st);

// d_h = 64 runs on the 32x32x16 matrix-core kernel, d_h = 128 on the 16x16x32
// one, every other shape (and fp32) on the general kernel.
hipError_t launch_prefill(int dtype, const AttnArgs& a, hipStream_t st) {
  if (prefill_mfma32_supported(dtype, a)) return launch_prefill_mfma32(a, st);
  if (prefill_mfma_supported(dtype, a)) return launch_prefill_mfma(a, st);
  static const RopeTable unused = {};
  return dtype == kF32 ? launch_prefill_t<float, false>(a, unused, st) : launch_prefill_t<bf16_t, false>(a, unused, st);
}

// With a workspace: where the 32x32x16 matrix-core kernel takes the shape, K
// and V are formed once into the workspace and the attention reads them;
// otherwise as launch_prefill.
size_t prefill_workspace_bytes(int dtype, const AttnArgs& a) {
  return prefill_material_shape_ok(dtype, a) ? prefill_material_bytes(a) : 0;
}

hipError_t launch_prefill_ws(int dtype, const AttnArgs& a, void* ws, hipStream_t st) {
  if (ws && prefill_material_supported(dtype, a)) return launch_prefill_material(a, ws, nullptr, st);
  return launch_prefill(dtype, a, st);
}

hipError_t launch_prefill_shared_ws(int dtype, const AttnArgs& a, const RopeTable& tab, void* ws, hipStream_t st) {
  if (ws && prefill_material_supported(dtype, a)) return launch_prefill_material(a, ws, &tab, st);
  return launch_prefill_shared(dtype, a, tab, st);
}

// Shared-basis cache: the 32x32x16 matrix-core kernel where it takes the shape
// (bf16, d_h = 64, R_K = R_V in {1, 2, 4}), the general kernel otherwise.
hipError_t launch_prefill_shared(int dtype, const AttnArgs& a, const RopeTable& tab, hipStream_t st) {
  if (prefill_mfma32_supported(dtype, a)) return launch_prefill_mfma32_shared(a, tab, st);
  return dtype == kF32 ? launch_prefill_t<float, true>(a, tab, st) : launch_prefill_t<bf16_t, true>(a, tab, st);
}

}  // namespace tpa
