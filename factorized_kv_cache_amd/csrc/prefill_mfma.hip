// Causal prefill attention on the matrix cores (bf16 MFMA), with keys and
// values rebuilt from the cached factors in LDS.
//
// Arithmetic as the general prefill kernel ("Tensor Product Attention Is All
// You Need" review on coreui.cn: Q_t/K_t/V_t equations of 核心机制总结 and the
// masked softmax attention of the code walk-through 前向传播), mapped as follows.
// A workgroup owns 128 queries of one head of one sequence; each of its four
// waves owns 32 of them (two 16-query tiles).  For every block of 64 keys:
//
//  * rebuild: the whole workgroup forms k_t = sum_r A_K[t,h,r] B~_K[t,r,:] and
//    v_t = sum_r A_V[t,h,r] B_V[t,r,:] for the block in fp32, and stores K
//    row-major and V transposed (V^T[d][t]) in LDS as bf16; at d_h = 64 the
//    factors of the next block are loaded while this block is multiplied;
//  * scores, transposed: S^T[t, q] = K[t,:] . Q[q,:] with K as the A operand
//    (from LDS) and Q^T as the B operand (registers, formed once), so each
//    lane's scores belong to one query (its column);
//  * online softmax per query in base 2 (the scale log2(e) / (R_Q R_K sqrt(d_h))
//    is folded into Q), masking only on blocks that reach past a query;
//  * values, transposed: O^T[d, q] += V^T[d, t] P^T[t, q]; the score tiles'
//    output registers are already the B operand of this product (k-slot j of
//    lane group g is key 4g+j of one 16-key tile for j<4, of the next for j>=4),
//    and the matching V^T rows are two 8-byte LDS reads.
//
// Query blocks are scheduled heaviest (most keys) first, evenly across XCDs.
#include "kernels.h"
#include "mfma.h"

namespace tpa {

// R consecutive bf16 values, loaded as one 2R-byte word.
template <int R>
struct RankWordP;
template <>
struct RankWordP<1> { typedef uint16_t type; };
template <>
struct RankWordP<2> { typedef uint32_t type; };
template <>
struct RankWordP<4> { typedef uint2 type; };

template <int R>
__device__ __forceinline__ float rank_elem(typename RankWordP<R>::type v, int r) {
  if constexpr (R == 1) {
    return bf16_to_f32(v);
  } else if constexpr (R == 2) {
    return r ? __uint_as_float(v & 0xffff0000u) : __uint_as_float(v << 16);
  } else {
    const uint32_t w = (r < 2) ? v.x : v.y;
    return (r & 1) ? __uint_as_float(w & 0xffff0000u) : __uint_as_float(w << 16);
  }
}

template <int DH>
struct PrefillMfmaCfg {
  static constexpr int BM = 128;         // queries per workgroup
  static constexpr int BN = 64;          // keys per block
  static constexpr int QT = 2;           // 16-query tiles per wave
  static constexpr int KS = DH / 32;     // k-steps of the score product
  static constexpr int DT = DH / 16;     // d tiles of the value product
  static constexpr int LDK = DH + 8;     // K row stride in LDS (bf16)
  static constexpr int LDV = BN + 4;     // V^T row stride in LDS (bf16), 8-byte aligned rows
  static constexpr int IT = BN * DH / 8 / 256;  // rebuild items (key, 8 d's) per thread
  // the next block's factors are loaded during this block's products (d_h = 64;
  // at d_h = 128 those registers would spill)
  static constexpr bool kPipelined = DH == 64;
};

// The cached factors one thread needs to rebuild its items of one key block.
template <int DH, int R>
struct RebuildRegs {
  static constexpr int IT = PrefillMfmaCfg<DH>::IT;
  uint4 bk[IT][R];
  uint4 bv[IT][R];
  typename RankWordP<R>::type ak[IT];
  typename RankWordP<R>::type av[IT];
};

// Keys past kend are clamped to the last valid key: they are masked out of
// every score, so only finiteness matters.
template <int DH, int R>
__device__ __forceinline__ void load_rebuild(RebuildRegs<DH, R>& g, const AttnArgs& a, int64_t seq0, int hh,
                                             int64_t k0, int64_t kend) {
  using C = PrefillMfmaCfg<DH>;
  typedef typename RankWordP<R>::type W;
  const bf16_t* AK = reinterpret_cast<const bf16_t*>(a.c_ak);
  const bf16_t* BK = reinterpret_cast<const bf16_t*>(a.c_bk);
  const bf16_t* AV = reinterpret_cast<const bf16_t*>(a.c_av);
  const bf16_t* BV = reinterpret_cast<const bf16_t*>(a.c_bv);
#pragma unroll
  for (int it = 0; it < C::IT; ++it) {
    const int item = threadIdx.x + 256 * it;
    const int kl = item % C::BN, d0 = (item / C::BN) * 8;
    int64_t t = k0 + kl;
    t = t < kend ? t : kend - 1;
    const int64_t row = seq0 + t;
    g.ak[it] = *reinterpret_cast<const W*>(AK + (row * a.h + hh) * R);
    g.av[it] = *reinterpret_cast<const W*>(AV + (row * a.h + hh) * R);
#pragma unroll
    for (int r = 0; r < R; ++r) {
      g.bk[it][r] = *reinterpret_cast<const uint4*>(BK + (row * R + r) * DH + d0);
      g.bv[it][r] = *reinterpret_cast<const uint4*>(BV + (row * R + r) * DH + d0);
    }
  }
}

template <int DH, int R>
__device__ __forceinline__ void store_rebuild(const RebuildRegs<DH, R>& g, bf16_t* ks_lds, bf16_t* vt_lds) {
  using C = PrefillMfmaCfg<DH>;
#pragma unroll
  for (int it = 0; it < C::IT; ++it) {
    const int item = threadIdx.x + 256 * it;
    const int kl = item % C::BN, d0 = (item / C::BN) * 8;
    float kv[8], vv[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) kv[j] = vv[j] = 0.f;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const float ar = rank_elem<R>(g.ak[it], r), vr = rank_elem<R>(g.av[it], r);
      const bf16x8_t ek = as_bf16x8(g.bk[it][r]), ev = as_bf16x8(g.bv[it][r]);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        kv[j] = fmaf(ar, (float)ek[j], kv[j]);
        vv[j] = fmaf(vr, (float)ev[j], vv[j]);
      }
    }
    *reinterpret_cast<bf16x8_t*>(ks_lds + kl * C::LDK + d0) = pack8(kv);
#pragma unroll
    for (int j = 0; j < 8; ++j) vt_lds[(d0 + j) * C::LDV + kl] = f32_to_bf16(vv[j]);
  }
}

template <int DH, int R>
__global__ void __launch_bounds__(256, 2) prefill_mfma_kernel(AttnArgs a, int n_qblocks) {
  using C = PrefillMfmaCfg<DH>;
  constexpr int BM = C::BM, BN = C::BN, QT = C::QT, KS = C::KS, DT = C::DT, LDK = C::LDK, LDV = C::LDV;
  __shared__ __align__(16) bf16_t ks_lds[BN * LDK];
  __shared__ __align__(16) bf16_t vt_lds[DH * LDV];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int li = lane & 15, lg = lane >> 4;
  // One-dimensional grid.  Work items (query block, head, sequence) in order of
  // decreasing key count are numbered by the linear workgroup id; since
  // workgroups go to the XCDs round-robin by that id, every XCD gets an equal
  // share of every query block, heaviest first.
  const int h = a.h;
  const int64_t hb = (int64_t)h * a.n_batch;
  const int64_t L = blockIdx.x;
  const int qb = n_qblocks - 1 - (int)(L / hb);
  const int hh = (int)(L % h);
  const int64_t b = (L % hb) / h;
  const int64_t q0 = (int64_t)qb * BM;
  const int64_t seq0 = b * a.max_seq;
  const int64_t last_q = (q0 + BM < a.S ? q0 + BM : a.S) - 1;
  const int64_t kend = a.causal ? a.start_pos + last_q + 1 : a.start_pos + a.S;

  // The first key block's factors go out before the query is formed.
  RebuildRegs<DH, R> rg;
  if constexpr (C::kPipelined) load_rebuild<DH, R>(rg, a, seq0, hh, 0, kend);

  // ---- query operand: lane (query q0 + 32*wave + 16*qt + li, slice lg)
  bf16x8_t qop[QT][KS];
  {
    const bf16_t* AQ = reinterpret_cast<const bf16_t*>(a.a_q);
    const bf16_t* BQ = reinterpret_cast<const bf16_t*>(a.b_q);
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      const int64_t s = q0 + 32 * wave + 16 * qt + li;
      const int64_t tok = b * a.q_bstride_tok + (s < a.S ? s : a.S - 1);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int d0 = lg * (DH / 4) + 8 * ks;
        float v[8];
        if (a.rq == 0) {
          const bf16x8_t e = as_bf16x8(*reinterpret_cast<const uint4*>(BQ + (tok * h + hh) * DH + d0));
#pragma unroll
          for (int j = 0; j < 8; ++j) v[j] = (float)e[j] * a.q_scale;
        } else {
#pragma unroll
          for (int j = 0; j < 8; ++j) v[j] = 0.f;
          for (int r = 0; r < a.rq; ++r) {
            const float ar = bf16_to_f32(AQ[(tok * h + hh) * a.rq + r]);
            const bf16x8_t e = as_bf16x8(*reinterpret_cast<const uint4*>(BQ + (tok * a.rq + r) * DH + d0));
#pragma unroll
            for (int j = 0; j < 8; ++j) v[j] = fmaf(ar, (float)e[j], v[j]);
          }
#pragma unroll
          for (int j = 0; j < 8; ++j) v[j] *= a.q_scale;
        }
        qop[qt][ks] = pack8(v);
      }
    }
  }

  float m_run[QT], l_run[QT];
  f32x4_t oacc[QT][DT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    m_run[qt] = -INFINITY;
    l_run[qt] = 0.f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) oacc[qt][dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  // first position of this wave's queries
  const int64_t wpos0 = a.start_pos + q0 + 32 * wave;

  for (int64_t k0 = 0; k0 < kend; k0 += BN) {
    // ---- rebuild K and V^T of this head for keys k0 .. k0+63 from the
    //      registers, then start loading the next block's factors
    if constexpr (!C::kPipelined) load_rebuild<DH, R>(rg, a, seq0, hh, k0, kend);
    store_rebuild<DH, R>(rg, ks_lds, vt_lds);
    __syncthreads();
    if constexpr (C::kPipelined) {
      if (k0 + BN < kend) load_rebuild<DH, R>(rg, a, seq0, hh, k0 + BN, kend);
    }

    // ---- scores S^T[key, query] for the block's 4 key tiles
    f32x4_t sacc[4][QT];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      bf16x8_t kf[KS];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        kf[ks] = *reinterpret_cast<const bf16x8_t*>(ks_lds + (kt * 16 + li) * LDK + lg * (DH / 4) + 8 * ks);
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) {
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) acc = mfma_bf16(kf[ks], qop[qt][ks], acc);
        sacc[kt][qt] = acc;
      }
    }

    // ---- mask (only where the block reaches past a query of this wave)
    const bool need_mask = (a.causal && k0 + BN - 1 > wpos0) || (k0 + BN > kend);
    if (need_mask) {
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int qt = 0; qt < QT; ++qt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int64_t t = k0 + kt * 16 + 4 * lg + i;
            const int64_t p = wpos0 + 16 * qt + li;
            const bool ok = t < kend && (!a.causal || t <= p);
            if (!ok) sacc[kt][qt][i] = -INFINITY;
          }
    }

    // ---- online softmax per query, P^T operands
    bf16x8_t pop[QT][2];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      float bmax = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) bmax = fmaxf(bmax, sacc[kt][qt][i]);
      bmax = fmaxf(bmax, __shfl_xor(bmax, 16));
      bmax = fmaxf(bmax, __shfl_xor(bmax, 32));
      const float m_new = fmaxf(m_run[qt], bmax);
      // a query with no visible key yet keeps m = -inf; its p and alpha are 0 and 1
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = fast_exp2(m_run[qt] - m_use);
      m_run[qt] = m_new;
      float psum = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        float pv[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float p = fast_exp2(sacc[2 * kb + (j >> 2)][qt][j & 3] - m_use);
          pv[j] = p;
          psum += p;
        }
        pop[qt][kb] = pack8(pv);
      }
      l_run[qt] = l_run[qt] * alpha + psum;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) oacc[qt][dt] *= alpha;
    }

    // ---- O^T += V^T P^T
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16_t* vrow = vt_lds + (dt * 16 + li) * LDV + kb * 32 + 4 * lg;
        const uint2 lo = *reinterpret_cast<const uint2*>(vrow);
        const uint2 hi = *reinterpret_cast<const uint2*>(vrow + 16);
        const bf16x8_t vf = as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) oacc[qt][dt] = mfma_bf16(vf, pop[qt][kb], oacc[qt][dt]);
      }
    }
    __syncthreads();
  }

  // ---- normalise and store: lane holds d = 16*dt + 4*lg + i of its query
  bf16_t* out = reinterpret_cast<bf16_t*>(a.out);
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    float l = l_run[qt];
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    const float inv = a.v_scale / l;
    const int64_t s = q0 + 32 * wave + 16 * qt + li;
    if (s < a.S) {
      bf16_t* orow = out + ((b * a.S + s) * h + hh) * (int64_t)DH;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const f32x4_t o = oacc[qt][dt];
        const uint2 w = make_uint2(pack_bf16x2(o[0] * inv, o[1] * inv), pack_bf16x2(o[2] * inv, o[3] * inv));
        *reinterpret_cast<uint2*>(orow + dt * 16 + 4 * lg) = w;
      }
    }
  }
}

bool prefill_mfma_supported(int dtype, const AttnArgs& a) {
  if (dtype != kBF16) return false;
  if ((a.S + 127) / 128 * (int64_t)a.h * a.n_batch >= ((int64_t)1 << 31)) return false;
  if (!(a.d_h == 64 || a.d_h == 128)) return false;
  if (a.rk != a.rv || !(a.rk == 1 || a.rk == 2 || a.rk == 4)) return false;
  const void* ptrs[4] = {a.b_q, a.c_bk, a.c_bv, a.out};   // read/written 8 or 16 bytes at a time
  for (int i = 0; i < 4; ++i)
    if (((uintptr_t)ptrs[i]) % 16) return false;
  return true;
}

hipError_t launch_prefill_mfma(const AttnArgs& a, hipStream_t st) {
  const int nqb = (int)((a.S + 127) / 128);
  const dim3 grid((unsigned)((int64_t)nqb * a.h * a.n_batch));
#define TPA_PREFILL_LAUNCH(DH_, R_) \
  hipLaunchKernelGGL((prefill_mfma_kernel<DH_, R_>), grid, dim3(256), 0, st, a, nqb)
  if (a.d_h == 64) {
    if (a.rk == 1) TPA_PREFILL_LAUNCH(64, 1);
    else if (a.rk == 2) TPA_PREFILL_LAUNCH(64, 2);
    else TPA_PREFILL_LAUNCH(64, 4);
  } else {
    if (a.rk == 1) TPA_PREFILL_LAUNCH(128, 1);
    else if (a.rk == 2) TPA_PREFILL_LAUNCH(128, 2);
    else TPA_PREFILL_LAUNCH(128, 4);
  }
#undef TPA_PREFILL_LAUNCH
  return hipGetLastError();
}

}  // namespace tpa
