// Backward of the prefill attention (training): gradients of the output with
// respect to the query factors and to the cached key/value factors, from an
// upstream gradient dO.  General kernels (fp32 arithmetic, any element type).
//
// The forward is the attention of the Q_t/K_t/V_t equations ("Tensor Product
// Attention Is All You Need" review on coreui.cn, 核心机制总结; the masked
// softmax attention of its code walk-through, 前向传播).  Its gradient by the
// chain rule: with P the softmax rows and s = q.k / sqrt(d_h),
//   dV = P^T dO,  dP = dO V^T,  dS = P * (dP - D),  D_i = sum_d dO_i O_i,
//   dQ = dS K / sqrt(d_h),  dK = dS^T Q / sqrt(d_h),
// then through the factor sums X = (1/R) sum_r a_r (x) b_r:
//   dA[t,h,r] = (1/R) dX[t,h,:] . B[t,r,:],  dB[t,r,:] = (1/R) sum_h A[t,h,r] dX[t,h,:].
//
// Four passes, each deterministic (no atomics):
//   1. per query: the base-2 log-sum-exp of its scores and D_i;
//   2. per key block: dK and dV, looping over the query blocks that see it;
//   3. per query block: dQ, looping over the key blocks it sees;
//   4. per token: the factor gradients from dQ, dK, dV.
// Keys and values are rebuilt from the factors in LDS as in the forward
// kernels (k^ = sum_r A_K B~_K without the 1/R_K, q^ carrying the forward's
// scale log2(e) / (R_Q R_K sqrt(d_h)), so z = q^.k^ is the score in base-2
// units).
#include "kernels.h"

namespace tpa {

constexpr int kBwdThreads = 256;
constexpr int kBwdOut = 16;   // BM (or BN) * d_h / threads, at most

template <typename T>
__device__ __forceinline__ float bwd_rebuild(const T* A, const T* Bm, int64_t row, int hh, int h, int R, int dh,
                                             int d) {
  float v = 0.f;
  for (int r = 0; r < R; ++r) v = fmaf(ldf(A, (row * h + hh) * R + r), ldf(Bm, (row * R + r) * dh + d), v);
  return v;
}

// q^ of query s (0-based in the block of S) for head hh, scaled like the forward.
template <typename T>
__device__ __forceinline__ float bwd_query(const AttnArgs& a, int64_t b, int64_t s, int hh, int d) {
  const T* AQ = reinterpret_cast<const T*>(a.a_q);
  const T* BQ = reinterpret_cast<const T*>(a.b_q);
  const int h = a.h, dh = a.d_h;
  const int64_t tok = b * a.q_bstride_tok + s;
  const float v = (a.rq == 0) ? ldf(BQ, (tok * h + hh) * dh + d) : bwd_rebuild(AQ, BQ, tok, hh, h, a.rq, dh, d);
  return v * a.q_scale;
}

// ---- pass 1: log-sum-exp (base 2) and D = dO . O per (sequence, query, head),
// O recomputed in fp32 (online softmax over the key blocks)
template <typename T, int BM, int BN>
__global__ void __launch_bounds__(kBwdThreads) bwd_stats_kernel(AttnArgs a, BwdArgs g) {
  extern __shared__ float smem[];
  const int h = a.h, dh = a.d_h;
  float* qs = smem;              // [BM][d_h]  q^, at the end O * dO
  float* ks = qs + BM * dh;      // [BN][d_h]
  float* vs = ks + BN * dh;      // [BN][d_h]
  float* ss = vs + BN * dh;      // [BM][BN]   scores, then p
  float* mrow = ss + BM * BN;    // [BM]
  float* lrow = mrow + BM;       // [BM]
  float* arow = lrow + BM;       // [BM]  rescale of the running sums
  const int64_t q0 = (int64_t)blockIdx.x * BM;
  const int hh = blockIdx.y;
  const int64_t b = blockIdx.z;
  const T* AK = reinterpret_cast<const T*>(a.c_ak);
  const T* BK = reinterpret_cast<const T*>(a.c_bk);
  const T* AV = reinterpret_cast<const T*>(a.c_av);
  const T* BV = reinterpret_cast<const T*>(a.c_bv);
  const T* dO = reinterpret_cast<const T*>(g.dout);
  const int64_t seq0 = b * a.max_seq;

  for (int idx = threadIdx.x; idx < BM * dh; idx += blockDim.x) {
    const int i = idx / dh, d = idx - i * dh;
    const int64_t s = q0 + i;
    qs[idx] = s < a.S ? bwd_query<T>(a, b, s, hh, d) : 0.f;
  }
  for (int i = threadIdx.x; i < BM; i += blockDim.x) {
    mrow[i] = -INFINITY;
    lrow[i] = 0.f;
  }
  // this thread's O outputs jo: query oi[jo], element od[jo] (n_out of them)
  float acc[kBwdOut];
  int oi[kBwdOut], od[kBwdOut];
  const int n_out = (BM * dh - (int)threadIdx.x + kBwdThreads - 1) / kBwdThreads;
#pragma unroll
  for (int jo = 0; jo < kBwdOut; ++jo) {
    const int idx = threadIdx.x + jo * kBwdThreads;
    oi[jo] = idx / dh;
    od[jo] = idx - oi[jo] * dh;
    acc[jo] = 0.f;
  }

  const int64_t last_q = (q0 + BM < a.S ? q0 + BM : a.S) - 1;
  const int64_t kend = a.causal ? a.start_pos + last_q + 1 : a.start_pos + a.S;
  for (int64_t k0 = 0; k0 < kend; k0 += BN) {
    __syncthreads();
    for (int idx = threadIdx.x; idx < BN * dh; idx += blockDim.x) {
      const int j = idx / dh, d = idx - j * dh;
      const int64_t t = k0 + j;
      const bool ok = t < kend;
      ks[idx] = ok ? bwd_rebuild(AK, BK, seq0 + t, hh, h, a.rk, dh, d) : 0.f;
      vs[idx] = ok ? bwd_rebuild(AV, BV, seq0 + t, hh, h, a.rv, dh, d) : 0.f;
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < BM * BN; idx += blockDim.x) {
      const int i = idx / BN, j = idx - i * BN;
      const int64_t t = k0 + j;
      const bool ok = t < kend && (!a.causal || t <= a.start_pos + q0 + i);
      float z = -INFINITY;
      if (ok) {
        z = 0.f;
        for (int d = 0; d < dh; ++d) z = fmaf(qs[i * dh + d], ks[j * dh + d], z);
      }
      ss[idx] = z;
    }
    __syncthreads();
    for (int i = threadIdx.x; i < BM; i += blockDim.x) {
      float mx = mrow[i];
      for (int j = 0; j < BN; ++j) mx = fmaxf(mx, ss[i * BN + j]);
      if (mx != -INFINITY) {
        float sum = 0.f;
        for (int j = 0; j < BN; ++j) {
          const float p = fast_exp2(ss[i * BN + j] - mx);
          ss[i * BN + j] = p;
          sum += p;
        }
        const float alpha = fast_exp2(mrow[i] - mx);   // 0 while nothing was seen
        lrow[i] = lrow[i] * alpha + sum;
        mrow[i] = mx;
        arow[i] = alpha;
      } else {
        for (int j = 0; j < BN; ++j) ss[i * BN + j] = 0.f;
        arow[i] = 1.f;
      }
    }
    __syncthreads();
#pragma unroll 1
    for (int j = 0; j < BN; ++j) {
#pragma unroll
      for (int jo = 0; jo < kBwdOut; ++jo) {
        if (jo >= n_out) break;
        const float a0 = j == 0 ? arow[oi[jo]] : 1.f;
        acc[jo] = fmaf(ss[oi[jo] * BN + j], vs[j * dh + od[jo]], acc[jo] * a0);
      }
    }
  }
  __syncthreads();
  // O = acc / l / R_V; each row's dO . O summed in a fixed order
  const float inv_rv = 1.f / (float)a.rv;
#pragma unroll
  for (int jo = 0; jo < kBwdOut; ++jo) {
    const int64_t s = q0 + oi[jo];
    if (jo < n_out) {
      const float o = acc[jo] / lrow[oi[jo]] * inv_rv;
      qs[oi[jo] * dh + od[jo]] = s < a.S ? o * ldf(dO, ((b * a.S + s) * h + hh) * (int64_t)dh + od[jo]) : 0.f;
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < BM; i += blockDim.x) {
    const int64_t s = q0 + i;
    if (s >= a.S) continue;
    float dsum = 0.f;
    for (int d = 0; d < dh; ++d) dsum += qs[i * dh + d];
    g.lse[(b * a.S + s) * h + hh] = mrow[i] + __log2f(lrow[i]);
    g.dvec[(b * a.S + s) * h + hh] = dsum;
  }
}

// ---- pass 2: dK and dV (true, i.e. with the 1/R scalings) per key block
template <typename T, int BM, int BN>
__global__ void __launch_bounds__(kBwdThreads) bwd_dkdv_kernel(AttnArgs a, BwdArgs g) {
  extern __shared__ float smem[];
  const int h = a.h, dh = a.d_h;
  float* ks = smem;              // [BN][d_h]  k^
  float* vs = ks + BN * dh;      // [BN][d_h]  v^
  float* qs = vs + BN * dh;      // [BM][d_h]  q^
  float* os = qs + BM * dh;      // [BM][d_h]  dO
  float* ps = os + BM * dh;      // [BM][BN]   p
  float* dss = ps + BM * BN;     // [BM][BN]   dS
  float* lse = dss + BM * BN;    // [BM]
  float* dv_ = lse + BM;         // [BM]
  const int64_t k0 = (int64_t)blockIdx.x * BN;
  const int hh = blockIdx.y;
  const int64_t b = blockIdx.z;
  const T* AK = reinterpret_cast<const T*>(a.c_ak);
  const T* BK = reinterpret_cast<const T*>(a.c_bk);
  const T* AV = reinterpret_cast<const T*>(a.c_av);
  const T* BV = reinterpret_cast<const T*>(a.c_bv);
  const T* dO = reinterpret_cast<const T*>(g.dout);
  const int64_t seq0 = b * a.max_seq;
  const int64_t n_keys = a.start_pos + a.S;
  const float inv_rv = 1.f / (float)a.rv;

  for (int idx = threadIdx.x; idx < BN * dh; idx += blockDim.x) {
    const int j = idx / dh, d = idx - j * dh;
    const int64_t t = k0 + j;
    const bool ok = t < n_keys;
    ks[idx] = ok ? bwd_rebuild(AK, BK, seq0 + t, hh, h, a.rk, dh, d) : 0.f;
    vs[idx] = ok ? bwd_rebuild(AV, BV, seq0 + t, hh, h, a.rv, dh, d) : 0.f;
  }
  // this thread's outputs jo: key oj[jo], element od[jo] (n_out of them)
  float dk[kBwdOut], dv[kBwdOut];
  int oj[kBwdOut], od[kBwdOut];
  const int n_out = (BN * dh - (int)threadIdx.x + kBwdThreads - 1) / kBwdThreads;
#pragma unroll
  for (int jo = 0; jo < kBwdOut; ++jo) {
    const int idx = threadIdx.x + jo * kBwdThreads;
    oj[jo] = idx / dh;
    od[jo] = idx - oj[jo] * dh;
    dk[jo] = dv[jo] = 0.f;
  }

  // the first query that can see this block's first key
  int64_t s_lo = 0;
  if (a.causal) s_lo = k0 - a.start_pos > 0 ? k0 - a.start_pos : 0;
  s_lo = (s_lo / BM) * BM;
  for (int64_t q0 = s_lo; q0 < a.S; q0 += BM) {
    __syncthreads();
    for (int idx = threadIdx.x; idx < BM * dh; idx += blockDim.x) {
      const int i = idx / dh, d = idx - i * dh;
      const int64_t s = q0 + i;
      const bool ok = s < a.S;
      qs[idx] = ok ? bwd_query<T>(a, b, s, hh, d) : 0.f;
      os[idx] = ok ? ldf(dO, ((b * a.S + s) * h + hh) * (int64_t)dh + d) : 0.f;
    }
    for (int i = threadIdx.x; i < BM; i += blockDim.x) {
      const int64_t s = q0 + i;
      lse[i] = s < a.S ? g.lse[(b * a.S + s) * h + hh] : 0.f;
      dv_[i] = s < a.S ? g.dvec[(b * a.S + s) * h + hh] : 0.f;
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < BM * BN; idx += blockDim.x) {
      const int i = idx / BN, j = idx - i * BN;
      const int64_t s = q0 + i, t = k0 + j;
      const bool ok = s < a.S && t < n_keys && (!a.causal || t <= a.start_pos + s);
      float p = 0.f, ds = 0.f;
      if (ok) {
        float z = 0.f, dp = 0.f;
        for (int d = 0; d < dh; ++d) {
          z = fmaf(qs[i * dh + d], ks[j * dh + d], z);
          dp = fmaf(os[i * dh + d], vs[j * dh + d], dp);
        }
        p = fast_exp2(z - lse[i]);
        ds = p * (dp * inv_rv - dv_[i]);
      }
      ps[idx] = p;
      dss[idx] = ds;
    }
    __syncthreads();
#pragma unroll 1
    for (int i = 0; i < BM; ++i) {
#pragma unroll
      for (int jo = 0; jo < kBwdOut; ++jo) {
        if (jo >= n_out) break;
        dv[jo] = fmaf(ps[i * BN + oj[jo]], os[i * dh + od[jo]], dv[jo]);
        dk[jo] = fmaf(dss[i * BN + oj[jo]], qs[i * dh + od[jo]], dk[jo]);
      }
    }
  }
  // dK = dS^T Q / sqrt(d_h) with Q = q^ * R_K sqrt(d_h) / log2(e)
  const float kscale = (float)a.rk / kLog2e;
#pragma unroll
  for (int jo = 0; jo < kBwdOut; ++jo) {
    const int idx = threadIdx.x + jo * kBwdThreads;
    if (idx >= BN * dh) break;
    const int j = idx / dh, d = idx - j * dh;
    const int64_t t = k0 + j;
    if (t >= n_keys) continue;
    const int64_t o = ((b * n_keys + t) * h + hh) * (int64_t)dh + d;
    g.dk[o] = dk[jo] * kscale;
    g.dv[o] = dv[jo];
  }
}

// ---- pass 3: dQ (true) per query block
template <typename T, int BM, int BN>
__global__ void __launch_bounds__(kBwdThreads) bwd_dq_kernel(AttnArgs a, BwdArgs g) {
  extern __shared__ float smem[];
  const int h = a.h, dh = a.d_h;
  float* qs = smem;              // [BM][d_h]  q^
  float* os = qs + BM * dh;      // [BM][d_h]  dO
  float* ks = os + BM * dh;      // [BN][d_h]  k^
  float* vs = ks + BN * dh;      // [BN][d_h]  v^
  float* dss = vs + BN * dh;     // [BM][BN]   dS
  float* lse = dss + BM * BN;    // [BM]
  float* dv_ = lse + BM;         // [BM]
  const int64_t q0 = (int64_t)blockIdx.x * BM;
  const int hh = blockIdx.y;
  const int64_t b = blockIdx.z;
  const T* AK = reinterpret_cast<const T*>(a.c_ak);
  const T* BK = reinterpret_cast<const T*>(a.c_bk);
  const T* AV = reinterpret_cast<const T*>(a.c_av);
  const T* BV = reinterpret_cast<const T*>(a.c_bv);
  const T* dO = reinterpret_cast<const T*>(g.dout);
  const int64_t seq0 = b * a.max_seq;
  const float inv_rv = 1.f / (float)a.rv;

  for (int idx = threadIdx.x; idx < BM * dh; idx += blockDim.x) {
    const int i = idx / dh, d = idx - i * dh;
    const int64_t s = q0 + i;
    const bool ok = s < a.S;
    qs[idx] = ok ? bwd_query<T>(a, b, s, hh, d) : 0.f;
    os[idx] = ok ? ldf(dO, ((b * a.S + s) * h + hh) * (int64_t)dh + d) : 0.f;
  }
  for (int i = threadIdx.x; i < BM; i += blockDim.x) {
    const int64_t s = q0 + i;
    lse[i] = s < a.S ? g.lse[(b * a.S + s) * h + hh] : 0.f;
    dv_[i] = s < a.S ? g.dvec[(b * a.S + s) * h + hh] : 0.f;
  }
  // this thread's outputs jo: query oi[jo], element od[jo] (n_out of them)
  float dq[kBwdOut];
  int oi[kBwdOut], od[kBwdOut];
  const int n_out = (BM * dh - (int)threadIdx.x + kBwdThreads - 1) / kBwdThreads;
#pragma unroll
  for (int jo = 0; jo < kBwdOut; ++jo) {
    const int idx = threadIdx.x + jo * kBwdThreads;
    oi[jo] = idx / dh;
    od[jo] = idx - oi[jo] * dh;
    dq[jo] = 0.f;
  }

  const int64_t last_q = (q0 + BM < a.S ? q0 + BM : a.S) - 1;
  const int64_t kend = a.causal ? a.start_pos + last_q + 1 : a.start_pos + a.S;
  for (int64_t k0 = 0; k0 < kend; k0 += BN) {
    __syncthreads();
    for (int idx = threadIdx.x; idx < BN * dh; idx += blockDim.x) {
      const int j = idx / dh, d = idx - j * dh;
      const int64_t t = k0 + j;
      const bool ok = t < kend;
      ks[idx] = ok ? bwd_rebuild(AK, BK, seq0 + t, hh, h, a.rk, dh, d) : 0.f;
      vs[idx] = ok ? bwd_rebuild(AV, BV, seq0 + t, hh, h, a.rv, dh, d) : 0.f;
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < BM * BN; idx += blockDim.x) {
      const int i = idx / BN, j = idx - i * BN;
      const int64_t s = q0 + i, t = k0 + j;
      const bool ok = s < a.S && t < kend && (!a.causal || t <= a.start_pos + s);
      float ds = 0.f;
      if (ok) {
        float z = 0.f, dp = 0.f;
        for (int d = 0; d < dh; ++d) {
          z = fmaf(qs[i * dh + d], ks[j * dh + d], z);
          dp = fmaf(os[i * dh + d], vs[j * dh + d], dp);
        }
        ds = fast_exp2(z - lse[i]) * (dp * inv_rv - dv_[i]);
      }
      dss[idx] = ds;
    }
    __syncthreads();
#pragma unroll 1
    for (int j = 0; j < BN; ++j) {
#pragma unroll
      for (int jo = 0; jo < kBwdOut; ++jo) {
        if (jo >= n_out) break;
        dq[jo] = fmaf(dss[oi[jo] * BN + j], ks[j * dh + od[jo]], dq[jo]);
      }
    }
  }
  // dQ = dS K / sqrt(d_h) with K = k^ / R_K
  const float qscale = 1.f / ((float)a.rk * sqrtf((float)dh));
#pragma unroll
  for (int jo = 0; jo < kBwdOut; ++jo) {
    const int idx = threadIdx.x + jo * kBwdThreads;
    if (idx >= BM * dh) break;
    const int i = idx / dh, d = idx - i * dh;
    const int64_t s = q0 + i;
    if (s < a.S) g.dq[((b * a.S + s) * h + hh) * (int64_t)dh + d] = dq[jo] * qscale;
  }
}

// ---- pass 4: factor gradients of one token, dX [h, d_h] -> dA [h, R], dB [R, d_h]
// With LDS: dX, A and B (rows padded by one float, so the R rows read
// together fall on different banks) are staged first, each read from global
// memory once.  Without (shapes too large for LDS): straight from memory.
template <typename T, bool LDS>
__device__ void bwd_factor_grads(const float* dX, const T* A, const T* Bm, int h, int R, int dh, float* dA,
                                 float* dB, float* lds) {
  const float inv_r = 1.f / (float)R;
  if constexpr (LDS) {
    float* xs = lds;              // [h][d_h]
    float* as = xs + h * dh;      // [h][R]
    float* bs = as + h * R;       // [R][d_h + 1]
    const int ldb = dh + 1;
    __syncthreads();              // the previous tensor's reads are done
    for (int idx = threadIdx.x; idx < h * dh; idx += blockDim.x) xs[idx] = dX[idx];
    for (int idx = threadIdx.x; idx < h * R; idx += blockDim.x) as[idx] = ldf(A, idx);
    for (int idx = threadIdx.x; idx < R * dh; idx += blockDim.x) {
      const int r = idx / dh, d = idx - r * dh;
      bs[r * ldb + d] = ldf(Bm, idx);
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < h * R; idx += blockDim.x) {
      const int hh = idx / R, r = idx - hh * R;
      float acc = 0.f;
      for (int d = 0; d < dh; ++d) acc = fmaf(xs[hh * dh + d], bs[r * ldb + d], acc);
      dA[idx] = acc * inv_r;
    }
    for (int idx = threadIdx.x; idx < R * dh; idx += blockDim.x) {
      const int r = idx / dh, d = idx - r * dh;
      float acc = 0.f;
      for (int hh = 0; hh < h; ++hh) acc = fmaf(as[hh * R + r], xs[hh * dh + d], acc);
      dB[idx] = acc * inv_r;
    }
  } else {
    for (int idx = threadIdx.x; idx < h * R; idx += blockDim.x) {
      const int hh = idx / R, r = idx - hh * R;
      float acc = 0.f;
      for (int d = 0; d < dh; ++d) acc = fmaf(dX[hh * dh + d], ldf(Bm, r * dh + d), acc);
      dA[idx] = acc * inv_r;
    }
    for (int idx = threadIdx.x; idx < R * dh; idx += blockDim.x) {
      const int r = idx / dh, d = idx - r * dh;
      float acc = 0.f;
      for (int hh = 0; hh < h; ++hh) acc = fmaf(ldf(A, hh * R + r), dX[hh * dh + d], acc);
      dB[idx] = acc * inv_r;
    }
  }
}

// One workgroup per (sequence, token): blockIdx.x < S: query token (when the
// query is factored); then the key/value tokens 0 .. n_keys-1.
template <typename T, bool LDS>
__global__ void __launch_bounds__(kBwdThreads) bwd_factor_kernel(AttnArgs a, BwdArgs g) {
  extern __shared__ float fsmem[];
  const int h = a.h, dh = a.d_h;
  const int64_t b = blockIdx.y;
  const int64_t n_keys = a.start_pos + a.S;
  const int64_t u = blockIdx.x;
  if (u < a.S) {
    const int64_t tok = b * a.q_bstride_tok + u;
    const float* dX = g.dq + (b * a.S + u) * h * (int64_t)dh;
    if (a.rq == 0) {
      float* out = g.d_bq + (b * g.dq_bstride + u) * h * (int64_t)dh;
      for (int idx = threadIdx.x; idx < h * dh; idx += blockDim.x) out[idx] = dX[idx];
    } else {
      bwd_factor_grads<T, LDS>(dX, reinterpret_cast<const T*>(a.a_q) + tok * h * a.rq,
                               reinterpret_cast<const T*>(a.b_q) + tok * a.rq * dh, h, a.rq, dh,
                               g.d_aq + (b * g.dq_bstride + u) * h * a.rq,
                               g.d_bq + (b * g.dq_bstride + u) * a.rq * dh, fsmem);
    }
    return;
  }
  const int64_t t = u - a.S;
  if (t >= n_keys) return;
  const int64_t row = b * a.max_seq + t;
  const int64_t drow = b * g.dkv_max_seq + t;
  const float* dK = g.dk + (b * n_keys + t) * h * (int64_t)dh;
  const float* dV = g.dv + (b * n_keys + t) * h * (int64_t)dh;
  bwd_factor_grads<T, LDS>(dK, reinterpret_cast<const T*>(a.c_ak) + row * h * a.rk,
                           reinterpret_cast<const T*>(a.c_bk) + row * a.rk * dh, h, a.rk, dh,
                           g.d_ak + drow * h * a.rk, g.d_bk + drow * a.rk * dh, fsmem);
  bwd_factor_grads<T, LDS>(dV, reinterpret_cast<const T*>(a.c_av) + row * h * a.rv,
                           reinterpret_cast<const T*>(a.c_bv) + row * a.rv * dh, h, a.rv, dh,
                           g.d_av + drow * h * a.rv, g.d_bv + drow * a.rv * dh, fsmem);
}

static size_t bwd_lds_limit() {
  int dev = 0, v = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess) return 0;
  return (size_t)v;
}

template <typename T>
static void launch_bwd_factor(const AttnArgs& a, const BwdArgs& g, hipStream_t st) {
  const int64_t n_keys = a.start_pos + a.S;
  const int R = a.rq > a.rk ? (a.rq > a.rv ? a.rq : a.rv) : (a.rk > a.rv ? a.rk : a.rv);
  const size_t lds = sizeof(float) * ((size_t)a.h * a.d_h + (size_t)a.h * R + (size_t)R * (a.d_h + 1));
  const dim3 grid((unsigned)(a.S + n_keys), (unsigned)a.n_batch);
  if (lds <= bwd_lds_limit())
    hipLaunchKernelGGL((bwd_factor_kernel<T, true>), grid, dim3(kBwdThreads), lds, st, a, g);
  else
    hipLaunchKernelGGL((bwd_factor_kernel<T, false>), grid, dim3(kBwdThreads), 0, st, a, g);
}

template <typename T, int BM, int BN>
static hipError_t launch_bwd_t(const AttnArgs& a, const BwdArgs& g, hipStream_t st) {
  const int dh = a.d_h;
  const int64_t n_keys = a.start_pos + a.S;
  const size_t lds1 = sizeof(float) * ((size_t)(BM + 2 * BN) * dh + (size_t)BM * BN + 3 * BM);
  const size_t lds2 = sizeof(float) * ((size_t)(2 * BN + 2 * BM) * dh + 2 * (size_t)BM * BN + 2 * BM);
  const size_t lds3 = sizeof(float) * ((size_t)(2 * BM + 2 * BN) * dh + (size_t)BM * BN + 2 * BM);
  const dim3 gq((unsigned)((a.S + BM - 1) / BM), (unsigned)a.h, (unsigned)a.n_batch);
  const dim3 gk((unsigned)((n_keys + BN - 1) / BN), (unsigned)a.h, (unsigned)a.n_batch);
  hipLaunchKernelGGL((bwd_stats_kernel<T, BM, BN>), gq, dim3(kBwdThreads), lds1, st, a, g);
  hipLaunchKernelGGL((bwd_dkdv_kernel<T, BM, BN>), gk, dim3(kBwdThreads), lds2, st, a, g);
  hipLaunchKernelGGL((bwd_dq_kernel<T, BM, BN>), gq, dim3(kBwdThreads), lds3, st, a, g);
  launch_bwd_factor<T>(a, g, st);
  return hipGetLastError();
}

size_t prefill_backward_workspace_bytes(const AttnArgs& a) {
  const int64_t n_keys = a.start_pos + a.S;
  const size_t per = (size_t)a.n_batch * a.h * a.d_h;
  // dQ, dK, dV in float32; q^ (hi, lo), k^ (hi, lo), v^ in bf16; lse and D
  return per * (size_t)(a.S + 2 * n_keys) * sizeof(float) + per * (size_t)(2 * a.S + 3 * n_keys) * sizeof(bf16_t) +
         2 * (size_t)a.n_batch * a.S * a.h * sizeof(float);
}

void prefill_backward_carve(const AttnArgs& a, void* ws, BwdArgs& g) {
  const int64_t n_keys = a.start_pos + a.S;
  const int64_t per = a.n_batch * a.h * (int64_t)a.d_h;
  float* p = reinterpret_cast<float*>(ws);
  g.dq = p;
  p += per * a.S;
  g.dk = p;
  p += per * n_keys;
  g.dv = p;
  p += per * n_keys;
  bf16_t* q = reinterpret_cast<bf16_t*>(p);
  g.q_hi = q;
  q += per * a.S;
  g.q_lo = q;
  q += per * a.S;
  g.k_hi = q;
  q += per * n_keys;
  g.k_lo = q;
  q += per * n_keys;
  g.v_hat = q;
  q += per * n_keys;
  p = reinterpret_cast<float*>(q);
  g.lse = p;
  p += a.n_batch * a.S * a.h;
  g.dvec = p;
}

bool backward_mfma_supported(int dtype, const AttnArgs& a, const BwdArgs& g);
hipError_t launch_backward_mfma(const AttnArgs& a, const BwdArgs& g, hipStream_t st);

hipError_t launch_prefill_backward(int dtype, const AttnArgs& a, const BwdArgs& g, hipStream_t st) {
  if (backward_mfma_supported(dtype, a, g)) {
    return launch_backward_mfma(a, g, st);
  }
  if (a.d_h <= 128) {
    return dtype == kF32 ? launch_bwd_t<float, 32, 32>(a, g, st) : launch_bwd_t<bf16_t, 32, 32>(a, g, st);
  }
  return dtype == kF32 ? launch_bwd_t<float, 16, 16>(a, g, st) : launch_bwd_t<bf16_t, 16, 16>(a, g, st);
}

}  // namespace tpa
