// Decode attention over the factor cache on the matrix cores (bf16 MFMA).
//
// Same arithmetic as the general decode kernel (factored scores
// s_t = sum_r A_K[t,h,r] (B~_K[t,r,:] . q_h), values sum_t sum_r (p_t A_V[t,h,r]) B_V[t,r,:];
// "Tensor Product Attention Is All You Need" review on coreui.cn, K_t/V_t
// equations of 核心机制总结 and question 2 on the pre-rotated cache), mapped to
// v_mfma_f32_16x16x32_bf16 as follows.  A wave walks its share of the chunk in
// "value blocks" of 32 (token, rank) rows (32/R tokens):
//
//  * scores: P[(t,r), head] = B~_K[(t,r), :] . q[head, :] as two 16x16 tiles
//    per block, A operand = 16 cache rows read straight from HBM, B operand =
//    q^T held in registers for the whole kernel.  Each lane loads one
//    contiguous d_h/4 slice of its row; the same k-slot mapping is used for q,
//    so the contraction is unchanged.
//  * the head factor: every lane's 4 output rows of a tile are R whole tokens'
//    ranks (R in {1,2,4}), so s_t = sum_r A_K[t,head,r] P[(t,r),head] is
//    lane-local; the block maximum per head needs two cross-lane xor steps.
//  * values: O^T[d, head] += B_V^T[d, (t,r)] * C[(t,r), head] with
//    C = p_t * A_V[t,head,r].  The score tiles' output registers already sit
//    in the B-operand layout of this product (k-slot j of lane group g is row
//    4g+j of tile 0 for j<4, of tile 1 for j>=4); B_V goes through a
//    wave-private LDS tile to be read transposed.
//
// The four waves of a workgroup merge their (m, l, O) through LDS in a fixed
// order, and the workgroup writes one partial per head to the workspace; the
// combine pass is shared with the general kernel.
#include "kernels.h"

namespace tpa {

typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef unsigned short u16x8_t __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f32x4_t mfma_bf16(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

__device__ __forceinline__ bf16x8_t pack8(const float* v) {
  u16x8_t u;
#pragma unroll
  for (int j = 0; j < 8; ++j) u[j] = f32_to_bf16(v[j]);
  return __builtin_bit_cast(bf16x8_t, u);
}

// R consecutive bf16 values -> floats (R in {1, 2, 4}).
template <int R>
__device__ __forceinline__ void load_rank(const bf16_t* p, float* out) {
  if constexpr (R == 1) {
    out[0] = bf16_to_f32(*p);
  } else if constexpr (R == 2) {
    const uint32_t v = *reinterpret_cast<const uint32_t*>(p);
    out[0] = __uint_as_float(v << 16);
    out[1] = __uint_as_float(v & 0xffff0000u);
  } else {
    const uint2 v = *reinterpret_cast<const uint2*>(p);
    out[0] = __uint_as_float(v.x << 16);
    out[1] = __uint_as_float(v.x & 0xffff0000u);
    out[2] = __uint_as_float(v.y << 16);
    out[3] = __uint_as_float(v.y & 0xffff0000u);
  }
}

__device__ __forceinline__ void wave_lds_fence() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int DH, int R, int HT>
struct DecodeMfmaCfg {
  static constexpr int KS = DH / 32;     // k-steps of the score product
  static constexpr int DT = DH / 16;     // 16-wide d tiles of the value product
  static constexpr int NT = 4 / R;       // tokens per lane per score tile
  static constexpr int VBT = 32 / R;     // tokens per value block
  static constexpr int HP = HT * 16;     // padded head count
  static constexpr int LROW = DH + 4;    // LDS row stride (bf16): 4 rows apart = 8 banks apart
  static constexpr int OST = DH + 4;     // LDS row stride (f32) of the merge buffer
  static constexpr size_t kLoopBytes = 4 * 32 * LROW * sizeof(bf16_t);
  static constexpr size_t kMergeBytes = (8 * HP + 2 * HP * OST) * sizeof(float);
  static constexpr size_t kLds = kLoopBytes > kMergeBytes ? kLoopBytes : kMergeBytes;
};

template <int DH, int R, int HT>
__global__ void __launch_bounds__(256) decode_mfma_kernel(AttnArgs a, int64_t ctx_len, int64_t chunk,
                                                          int64_t n_chunks, float* ws) {
  using C = DecodeMfmaCfg<DH, R, HT>;
  constexpr int KS = C::KS, DT = C::DT, NT = C::NT, VBT = C::VBT, HP = C::HP, LROW = C::LROW, OST = C::OST;
  extern __shared__ __align__(16) unsigned char smem[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int li = lane & 15, lg = lane >> 4;
  const int h = a.h;
  const int64_t b = blockIdx.y, c = blockIdx.x;
  const int64_t t0 = c * chunk;
  const int64_t t1 = (t0 + chunk < ctx_len) ? t0 + chunk : ctx_len;
  const bf16_t* AK = reinterpret_cast<const bf16_t*>(a.c_ak);
  const bf16_t* BK = reinterpret_cast<const bf16_t*>(a.c_bk);
  const bf16_t* AV = reinterpret_cast<const bf16_t*>(a.c_av);
  const bf16_t* BV = reinterpret_cast<const bf16_t*>(a.c_bv);
  const int64_t seq0 = b * a.max_seq;

  // ---- query operand: lane (head = 16*ht + li, slice lg) holds
  //      q[head][lg*DH/4 + 8*ks + j], j < 8, scaled and rounded to bf16.
  bf16x8_t qop[HT][KS];
  {
    const bf16_t* AQ = reinterpret_cast<const bf16_t*>(a.a_q);
    const bf16_t* BQ = reinterpret_cast<const bf16_t*>(a.b_q);
    const int64_t tok = b * a.q_bstride_tok;
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
      const int head = ht * 16 + li;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int d0 = lg * (DH / 4) + 8 * ks;
        float v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = 0.f;
        if (head < h) {
          if (a.rq == 0) {
            const uint4 u = *reinterpret_cast<const uint4*>(BQ + (tok * h + head) * DH + d0);
            const bf16x8_t e = as_bf16x8(u);
#pragma unroll
            for (int j = 0; j < 8; ++j) v[j] = (float)e[j];
          } else {
            for (int r = 0; r < a.rq; ++r) {
              const float ar = bf16_to_f32(AQ[(tok * h + head) * a.rq + r]);
              const bf16x8_t e = as_bf16x8(*reinterpret_cast<const uint4*>(BQ + (tok * a.rq + r) * DH + d0));
#pragma unroll
              for (int j = 0; j < 8; ++j) v[j] = fmaf(ar, (float)e[j], v[j]);
            }
          }
#pragma unroll
          for (int j = 0; j < 8; ++j) v[j] *= a.q_scale;
        }
        qop[ht][ks] = pack8(v);
      }
    }
  }

  float m_run[HT], l_run[HT];
  f32x4_t oacc[HT][DT];
#pragma unroll
  for (int ht = 0; ht < HT; ++ht) {
    m_run[ht] = -INFINITY;
    l_run[ht] = 0.f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) oacc[ht][dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  bf16_t* lbv = reinterpret_cast<bf16_t*>(smem) + wave * 32 * LROW;
  const int64_t last = t1 - 1;
  const int nvb = (int)((t1 - t0 + VBT - 1) / VBT);

  for (int vb = wave; vb < nvb; vb += 4) {
    const int64_t tb = t0 + (int64_t)vb * VBT;

    // ---- B_V block (32 rows x DH) -> LDS: lane loads half of row lane/2.
    {
      const int row = lane >> 1, half = lane & 1;
      int64_t tok = tb + row / R;
      tok = tok < last ? tok : last;
      const uint4* src = reinterpret_cast<const uint4*>(BV + ((seq0 + tok) * R + row % R) * DH + half * (DH / 2));
      uint4 v[DH / 16];
#pragma unroll
      for (int u = 0; u < DH / 16; ++u) v[u] = src[u];
      uint2* dst = reinterpret_cast<uint2*>(lbv + row * LROW + half * (DH / 2));
#pragma unroll
      for (int u = 0; u < DH / 16; ++u) {
        dst[2 * u] = make_uint2(v[u].x, v[u].y);
        dst[2 * u + 1] = make_uint2(v[u].z, v[u].w);
      }
    }

    // ---- B~_K operand: tile st, row li, slice lg.
    bf16x8_t kop[2][KS];
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      const int row = st * 16 + li;
      int64_t tok = tb + row / R;
      tok = tok < last ? tok : last;
      const uint4* src = reinterpret_cast<const uint4*>(BK + ((seq0 + tok) * R + row % R) * DH + lg * (DH / 4));
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) kop[st][ks] = as_bf16x8(src[ks]);
    }

    // ---- head factors of the lane's rows: tokens (16*st + 4*lg)/R + k.
    float ak[2][HT][4], av[2][HT][4];
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int ht = 0; ht < HT; ++ht) {
        int head = ht * 16 + li;
        head = head < h ? head : h - 1;
#pragma unroll
        for (int k = 0; k < NT; ++k) {
          int64_t tok = tb + (st * 16 + lg * 4) / R + k;
          tok = tok < last ? tok : last;
          load_rank<R>(AK + ((seq0 + tok) * h + head) * R, &ak[st][ht][k * R]);
          load_rank<R>(AV + ((seq0 + tok) * h + head) * R, &av[st][ht][k * R]);
        }
      }

    // ---- scores on the matrix cores
    f32x4_t sacc[2][HT];
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int ht = 0; ht < HT; ++ht) {
        f32x4_t accv = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) accv = mfma_bf16(kop[st][ks], qop[ht][ks], accv);
        sacc[st][ht] = accv;
      }

    // ---- online softmax per head, and the value-product operand C
    bf16x8_t cop[HT];
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
      float s[2][NT];
      float bmax = -INFINITY;
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int k = 0; k < NT; ++k) {
          float v = 0.f;
#pragma unroll
          for (int rr = 0; rr < R; ++rr) v = fmaf(ak[st][ht][k * R + rr], sacc[st][ht][k * R + rr], v);
          const bool valid = tb + (st * 16 + lg * 4) / R + k <= last;
          s[st][k] = valid ? v : -INFINITY;
          bmax = fmaxf(bmax, s[st][k]);
        }
      bmax = fmaxf(bmax, __shfl_xor(bmax, 16));
      bmax = fmaxf(bmax, __shfl_xor(bmax, 32));
      const float m_new = fmaxf(m_run[ht], bmax);
      const float alpha = fast_exp2(m_run[ht] - m_new);
      m_run[ht] = m_new;
      float psum = 0.f;
      float cv[8];
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int k = 0; k < NT; ++k) {
          const float p = fast_exp2(s[st][k] - m_new);
          psum += p;
#pragma unroll
          for (int rr = 0; rr < R; ++rr) cv[st * 4 + k * R + rr] = p * av[st][ht][k * R + rr];
        }
      l_run[ht] = l_run[ht] * alpha + psum;
      cop[ht] = pack8(cv);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) oacc[ht][dt] *= alpha;
    }

    // ---- value product: A operand = B_V^T read from LDS in the k-slot order
    wave_lds_fence();
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const int d = dt * 16 + li;
      u16x8_t e;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int row = (j < 4) ? 4 * lg + j : 16 + 4 * lg + (j - 4);
        e[j] = lbv[row * LROW + d];
      }
      const bf16x8_t bvop = __builtin_bit_cast(bf16x8_t, e);
#pragma unroll
      for (int ht = 0; ht < HT; ++ht) oacc[ht][dt] = mfma_bf16(bvop, cop[ht], oacc[ht][dt]);
    }
    wave_lds_fence();
  }

  // ---- merge the four waves (fixed order) and write this chunk's partial
#pragma unroll
  for (int ht = 0; ht < HT; ++ht) {
    l_run[ht] += __shfl_xor(l_run[ht], 16);
    l_run[ht] += __shfl_xor(l_run[ht], 32);
  }
  __syncthreads();
  float* mbuf = reinterpret_cast<float*>(smem);  // [4][HP]
  float* lbuf = mbuf + 4 * HP;                    // [4][HP]
  float* obuf = lbuf + 4 * HP;                    // [2][HP][OST]
  if (lg == 0) {
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
      mbuf[wave * HP + ht * 16 + li] = m_run[ht];
      lbuf[wave * HP + ht * 16 + li] = l_run[ht];
    }
  }
  __syncthreads();
#pragma unroll
  for (int ht = 0; ht < HT; ++ht) {
    const int head = ht * 16 + li;
    float M = mbuf[head];
#pragma unroll
    for (int w = 1; w < 4; ++w) M = fmaxf(M, mbuf[w * HP + head]);
    const float sc = fast_exp2(m_run[ht] - M);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) oacc[ht][dt] *= sc;
  }
  const int slot = wave & 1;
  if (wave < 2) {
#pragma unroll
    for (int ht = 0; ht < HT; ++ht)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
        *reinterpret_cast<f32x4_t*>(obuf + (slot * HP + ht * 16 + li) * OST + dt * 16 + lg * 4) = oacc[ht][dt];
  }
  __syncthreads();
  if (wave >= 2) {
#pragma unroll
    for (int ht = 0; ht < HT; ++ht)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        f32x4_t* p = reinterpret_cast<f32x4_t*>(obuf + (slot * HP + ht * 16 + li) * OST + dt * 16 + lg * 4);
        *p = *p + oacc[ht][dt];
      }
  }
  __syncthreads();
  float* P = ws + ((b * n_chunks + c) * h) * (int64_t)(DH + 2);
  for (int idx = threadIdx.x; idx < h * DH; idx += blockDim.x) {
    const int head = idx / DH, d = idx - head * DH;
    P[head * (DH + 2) + 2 + d] = obuf[head * OST + d] + obuf[(HP + head) * OST + d];
  }
  for (int head = threadIdx.x; head < h; head += blockDim.x) {
    float M = mbuf[head];
    for (int w = 1; w < 4; ++w) M = fmaxf(M, mbuf[w * HP + head]);
    float L = 0.f;
    for (int w = 0; w < 4; ++w) L = fmaf(fast_exp2(mbuf[w * HP + head] - M), lbuf[w * HP + head], L);
    P[head * (DH + 2)] = M;
    P[head * (DH + 2) + 1] = L;
  }
}

bool decode_mfma_supported(int dtype, const AttnArgs& a) {
  if (dtype != kBF16) return false;
  if (a.rk != a.rv || !(a.rk == 1 || a.rk == 2 || a.rk == 4)) return false;
  if (!(a.d_h == 64 || a.d_h == 128)) return false;
  if (a.h > 64) return false;
  const void* ptrs[6] = {a.b_q, a.c_ak, a.c_bk, a.c_av, a.c_bv, a.a_q};
  for (int i = 0; i < 6; ++i)
    if (((uintptr_t)ptrs[i]) % 16) return false;
  return true;
}

// Value-block tokens times the four waves of a workgroup.
int64_t decode_mfma_wave_tokens(const AttnArgs& a) { return 4 * (32 / a.rk); }

template <int DH, int R, int HT>
static void launch_cfg(const AttnArgs& a, int64_t ctx_len, int64_t chunk, int64_t n_chunks, float* ws,
                       hipStream_t st) {
  using C = DecodeMfmaCfg<DH, R, HT>;
  hipLaunchKernelGGL((decode_mfma_kernel<DH, R, HT>), dim3((unsigned)n_chunks, (unsigned)a.n_batch), dim3(256),
                     C::kLds, st, a, ctx_len, chunk, n_chunks, ws);
}

template <int DH, int R>
static void launch_dh_r(const AttnArgs& a, int64_t ctx_len, int64_t chunk, int64_t n_chunks, float* ws,
                        hipStream_t st) {
  const int ht = (a.h + 15) / 16;
  switch (ht) {
    case 1: launch_cfg<DH, R, 1>(a, ctx_len, chunk, n_chunks, ws, st); break;
    case 2: launch_cfg<DH, R, 2>(a, ctx_len, chunk, n_chunks, ws, st); break;
    case 3: launch_cfg<DH, R, 3>(a, ctx_len, chunk, n_chunks, ws, st); break;
    default: launch_cfg<DH, R, 4>(a, ctx_len, chunk, n_chunks, ws, st); break;
  }
}

template <int DH>
static void launch_dh(const AttnArgs& a, int64_t ctx_len, int64_t chunk, int64_t n_chunks, float* ws,
                      hipStream_t st) {
  switch (a.rk) {
    case 1: launch_dh_r<DH, 1>(a, ctx_len, chunk, n_chunks, ws, st); break;
    case 2: launch_dh_r<DH, 2>(a, ctx_len, chunk, n_chunks, ws, st); break;
    default: launch_dh_r<DH, 4>(a, ctx_len, chunk, n_chunks, ws, st); break;
  }
}

hipError_t launch_decode_mfma(const AttnArgs& a, int64_t ctx_len, int64_t chunk, int64_t n_chunks, float* ws,
                              hipStream_t st) {
  if (a.d_h == 64)
    launch_dh<64>(a, ctx_len, chunk, n_chunks, ws, st);
  else
    launch_dh<128>(a, ctx_len, chunk, n_chunks, ws, st);
  return hipGetLastError();
}

}  // namespace tpa
