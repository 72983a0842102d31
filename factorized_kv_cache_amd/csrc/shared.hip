// Decode attention of the shared-basis variant: the dim factors of K and V are
// parameters common to every token (B_K [R_K, d_h] unrotated, B_V [R_V, d_h]),
// so the cache holds only the head factors A_K, A_V ("Tensor Product Attention
// Is All You Need" review on coreui.cn, 优点与创新 item 5, names the variant that
// shares basis vectors across tokens; the formula is this library's reading:
// key t of head h is RoPE_t((1/R_K) sum_r A_K[t,h,r] B_K[r]), value t is
// (1/R_V) sum_r A_V[t,h,r] B_V[r]).
//
// Score of key t for head h, with q the rotated query in pairs (q_2i, q_2i+1)
// and b = B_K[r]:
//   q . RoPE_t(b) = sum_i cos(t th_i) (q_2i b_2i + q_2i+1 b_2i+1)
//                       + sin(t th_i) (q_2i+1 b_2i - q_2i b_2i+1)
//                 = sum_i cos(t th_i) alpha[h,r,i] + sin(t th_i) beta[h,r,i],
// so per query alpha and beta are formed once, and a key costs its R_K head
// factors and the d_h/2 angle pairs of its position (shared by every head).
// Values never need B_V inside the loop: each head accumulates
// w[r] = sum_t p_t A_V[t,h,r], and the combine forms (1/R_V) sum_r w[r] B_V[r].
//
// One workgroup per (sequence, chunk of keys) covers every head.  A block of
// 32 keys: the angle pairs go to LDS (fp64 angles as in every rotation here);
// lane l of each half-wave takes key l of the block and the heads g, g+8, ...
// of its half-wave g, with an online softmax of its own; the 32 lanes merge
// at the end of the chunk, and a second pass merges the chunks in order.
#include "kernels.h"

namespace tpa {

constexpr int kShT = 32;   // keys per block: one per lane of a half-wave

template <typename T, int MJ, int MR>
__global__ void __launch_bounds__(256) shared_decode_kernel(AttnArgs a, RopeTable tab, int64_t ctx_len,
                                                            int64_t chunk, int n_chunks, float* ws) {
  extern __shared__ __align__(16) float sh[];
  const int h = a.h, dh = a.d_h, np = dh / 2, rk = a.rk, rv = a.rv;
  const int ldf2 = np + 1;                              // angle rows, padded (float2 units)
  float* qs = sh;                                       // [h][d_h] scaled query
  float2* ab = reinterpret_cast<float2*>(qs + h * dh);  // [h * R_K][d_h/2] (alpha, beta)
  float2* fb = ab + h * rk * np;                        // 2 x [kShT][d_h/2 + 1] (cos, sin)
  const int c = blockIdx.x;
  const int64_t b = blockIdx.y;
  const int64_t t0 = (int64_t)c * chunk;
  const int64_t t1 = t0 + chunk < ctx_len ? t0 + chunk : ctx_len;
  const T* AQ = reinterpret_cast<const T*>(a.a_q);
  const T* BQ = reinterpret_cast<const T*>(a.b_q);
  const T* BK = reinterpret_cast<const T*>(a.c_bk);
  const T* AK = reinterpret_cast<const T*>(a.c_ak);
  const T* AV = reinterpret_cast<const T*>(a.c_av);

  // ---- query (one token per sequence), scaled by log2(e) / (R_Q R_K sqrt(d_h))
  const int64_t tok = b * a.q_bstride_tok;
  for (int idx = threadIdx.x; idx < h * dh; idx += blockDim.x) {
    const int hh = idx / dh, d = idx - hh * dh;
    float v = 0.f;
    if (a.rq == 0) {
      v = ldf(BQ, (tok * h + hh) * dh + d);
    } else {
      for (int r = 0; r < a.rq; ++r) v = fmaf(ldf(AQ, (tok * h + hh) * a.rq + r), ldf(BQ, (tok * a.rq + r) * dh + d), v);
    }
    qs[idx] = v * a.q_scale;
  }
  __syncthreads();
  // ---- alpha, beta of every (head, rank, pair)
  for (int idx = threadIdx.x; idx < h * rk * np; idx += blockDim.x) {
    const int i = idx % np, hr = idx / np;
    const int hh = hr / rk, r = hr - hh * rk;
    const float q0 = qs[hh * dh + 2 * i], q1 = qs[hh * dh + 2 * i + 1];
    const float b0 = ldf(BK, (int64_t)r * dh + 2 * i), b1 = ldf(BK, (int64_t)r * dh + 2 * i + 1);
    ab[idx] = make_float2(fmaf(q0, b0, q1 * b1), fmaf(q1, b0, -q0 * b1));
  }

  const int tt = threadIdx.x % kShT, hg = threadIdx.x / kShT;   // key slot, head group (half-wave)
  const int n_heads = hg < h ? (h - hg + 7) / 8 : 0;            // heads hg, hg+8, ... of this lane
  float m[MJ], l[MJ], w[MJ][MR];
#pragma unroll
  for (int j = 0; j < MJ; ++j) {
    m[j] = -INFINITY;
    l[j] = 0.f;
#pragma unroll
    for (int r = 0; r < MR; ++r) w[j][r] = 0.f;
  }

  // angle pairs of the first block
  auto angles = [&](int64_t blk0, float2* f) {
    for (int idx = threadIdx.x; idx < kShT * np; idx += blockDim.x) {
      const int ti = idx / np, i = idx - ti * np;
      float cs, sn;
      rope_cos_sin(tab, blk0 + ti, i, cs, sn);
      f[ti * ldf2 + i] = make_float2(cs, sn);
    }
  };
  angles(t0, fb);
  __syncthreads();
  int buf = 0;
  for (int64_t blk0 = t0; blk0 < t1; blk0 += kShT) {
    const float2* f = fb + buf * kShT * ldf2;
    // the next block's angles into the other buffer (read after the barrier below)
    if (blk0 + kShT < t1) angles(blk0 + kShT, fb + (buf ^ 1) * kShT * ldf2);
    const int64_t t = blk0 + tt;
    const bool valid = t < t1;
    const int64_t row = b * a.max_seq + (valid ? t : t1 - 1);
    // g[j][r] = q_h . RoPE_t(B_K[r]) for this lane's key and heads
    float g[MJ][MR];
#pragma unroll
    for (int j = 0; j < MJ; ++j)
#pragma unroll
      for (int r = 0; r < MR; ++r) g[j][r] = 0.f;
    for (int i = 0; i < np; ++i) {
      const float2 fv = f[tt * ldf2 + i];
#pragma unroll
      for (int j = 0; j < MJ; ++j) {
        if (j < n_heads) {
          const float2* abh = ab + (hg + 8 * j) * rk * np + i;
#pragma unroll
          for (int r = 0; r < MR; ++r) {
            if (r < rk) {
              const float2 av = abh[r * np];
              g[j][r] = fmaf(fv.x, av.x, fmaf(fv.y, av.y, g[j][r]));
            }
          }
        }
      }
    }
    // scores and the lane's online softmax per head
#pragma unroll
    for (int j = 0; j < MJ; ++j) {
      if (j < n_heads && valid) {
        const int hh = hg + 8 * j;
        float s = 0.f;
#pragma unroll
        for (int r = 0; r < MR; ++r)
          if (r < rk) s = fmaf(ldf(AK, (row * h + hh) * rk + r), g[j][r], s);
        const float mn = fmaxf(m[j], s);
        const float alpha = fast_exp2(m[j] - mn);   // 0 for the lane's first key
        const float p = fast_exp2(s - mn);
        m[j] = mn;
        l[j] = fmaf(l[j], alpha, p);
#pragma unroll
        for (int r = 0; r < MR; ++r)
          if (r < rv) w[j][r] = fmaf(w[j][r], alpha, p * ldf(AV, (row * h + hh) * rv + r));
      }
    }
    __syncthreads();
    buf ^= 1;
  }

  // ---- merge the 32 key slots of each head (a half-wave), in a fixed order
#pragma unroll
  for (int j = 0; j < MJ; ++j) {
    float mx = m[j];
#pragma unroll
    for (int k = 1; k < kShT; k <<= 1) mx = fmaxf(mx, __shfl_xor(mx, k, kShT));
    const float sc = mx == -INFINITY ? 0.f : fast_exp2(m[j] - mx);
    float lt = l[j] * sc;
#pragma unroll
    for (int k = 1; k < kShT; k <<= 1) lt += __shfl_xor(lt, k, kShT);
    float wt[MR];
#pragma unroll
    for (int r = 0; r < MR; ++r) {
      wt[r] = w[j][r] * sc;
#pragma unroll
      for (int k = 1; k < kShT; k <<= 1) wt[r] += __shfl_xor(wt[r], k, kShT);
    }
    if (tt == 0 && j < n_heads) {
      const int hh = hg + 8 * j;
      float* p = ws + ((b * n_chunks + c) * h + hh) * (int64_t)(2 + rv);
      p[0] = mx;
      p[1] = lt;
#pragma unroll
      for (int r = 0; r < MR; ++r)
        if (r < rv) p[2 + r] = wt[r];
    }
  }
}

// Chunks merged in order per (sequence, head); out = (1/R_V) sum_r W[r] B_V[r] / L.
template <typename T, int MR>
__global__ void __launch_bounds__(64) shared_combine_kernel(AttnArgs a, int n_chunks, const float* ws) {
  const int hh = blockIdx.x;
  const int64_t b = blockIdx.y;
  const int h = a.h, dh = a.d_h, rv = a.rv;
  const float* p = ws + (b * n_chunks * h + hh) * (int64_t)(2 + rv);
  const int64_t cstride = (int64_t)h * (2 + rv);
  float M = -INFINITY;
  for (int c = 0; c < n_chunks; ++c) M = fmaxf(M, p[c * cstride]);
  float L = 0.f, W[MR];
#pragma unroll
  for (int r = 0; r < MR; ++r) W[r] = 0.f;
  for (int c = 0; c < n_chunks; ++c) {
    const float* q = p + c * cstride;
    const float s = q[0] == -INFINITY ? 0.f : fast_exp2(q[0] - M);
    L = fmaf(q[1], s, L);
#pragma unroll
    for (int r = 0; r < MR; ++r)
      if (r < rv) W[r] = fmaf(q[2 + r], s, W[r]);
  }
  const float inv = a.v_scale / L;
  const T* BV = reinterpret_cast<const T*>(a.c_bv);
  T* out = reinterpret_cast<T*>(a.out);
  for (int d = threadIdx.x; d < dh; d += blockDim.x) {
    float o = 0.f;
#pragma unroll
    for (int r = 0; r < MR; ++r)
      if (r < rv) o = fmaf(W[r], ldf(BV, (int64_t)r * dh + d), o);
    stf(out, (b * h + hh) * (int64_t)dh + d, o * inv);
  }
}

static size_t shared_lds_bytes(const AttnArgs& a) {
  const size_t np = a.d_h / 2;
  return sizeof(float) * ((size_t)a.h * a.d_h + (size_t)a.h * a.rk * a.d_h + 2 * kShT * (np + 1) * 2);
}

static size_t shared_device_lds() {
  int dev = 0, v = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess) return 0;
  return (size_t)v;
}

// Heads per lane and ranks the kernel instances hold in registers.
bool shared_decode_supported(const AttnArgs& a) {
  const int hpl = (a.h + 7) / 8;
  if (hpl > 8 || a.rk > 4 || a.rv > 4) return false;
  return shared_lds_bytes(a) <= shared_device_lds();
}

SharedPlan plan_shared_decode(const AttnArgs& a, int64_t ctx_len) {
  SharedPlan p;
  int64_t n = (512 + a.n_batch - 1) / a.n_batch;   // about two workgroups per CU in all
  const int64_t max_n = (ctx_len + kShT - 1) / kShT;
  n = n < 1 ? 1 : (n > max_n ? max_n : n);
  p.chunk_tokens = ((ctx_len + n - 1) / n + kShT - 1) / kShT * kShT;
  p.n_chunks = (ctx_len + p.chunk_tokens - 1) / p.chunk_tokens;
  return p;
}

size_t shared_decode_workspace_bytes(const SharedPlan& p, const AttnArgs& a) {
  return sizeof(float) * (size_t)a.n_batch * p.n_chunks * a.h * (2 + a.rv);
}

template <typename T, int MJ>
static void launch_shared_t(const AttnArgs& a, const RopeTable& tab, int64_t ctx_len, const SharedPlan& p,
                            float* ws, hipStream_t st) {
  const dim3 grid((unsigned)p.n_chunks, (unsigned)a.n_batch);
  hipLaunchKernelGGL((shared_decode_kernel<T, MJ, 4>), grid, dim3(256), shared_lds_bytes(a), st, a, tab, ctx_len,
                     p.chunk_tokens, (int)p.n_chunks, ws);
  hipLaunchKernelGGL((shared_combine_kernel<T, 4>), dim3((unsigned)a.h, (unsigned)a.n_batch), dim3(64), 0, st, a,
                     (int)p.n_chunks, ws);
}

hipError_t launch_shared_decode(int dtype, const AttnArgs& a, const RopeTable& tab, int64_t ctx_len,
                                const SharedPlan& p, void* ws, hipStream_t st) {
  float* w = reinterpret_cast<float*>(ws);
  const int hpl = (a.h + 7) / 8;
  if (dtype == kF32) {
    if (hpl <= 4) launch_shared_t<float, 4>(a, tab, ctx_len, p, w, st);
    else launch_shared_t<float, 8>(a, tab, ctx_len, p, w, st);
  } else {
    if (hpl <= 4) launch_shared_t<bf16_t, 4>(a, tab, ctx_len, p, w, st);
    else launch_shared_t<bf16_t, 8>(a, tab, ctx_len, p, w, st);
  }
  return hipGetLastError();
}

}  // namespace tpa
