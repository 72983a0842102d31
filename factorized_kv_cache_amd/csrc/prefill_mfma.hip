// Causal prefill attention on the matrix cores (bf16 MFMA), with keys and
// values rebuilt from the cached factors in LDS.
//
// Arithmetic as the general prefill kernel ("Tensor Product Attention Is All
// You Need" review on coreui.cn: Q_t/K_t/V_t equations of 核心机制总结 and the
// masked softmax attention of the code walk-through 前向传播), mapped as follows.
// A workgroup owns BM queries of one head of one sequence and each of its four
// waves QT 16-query tiles (d_h = 64: 256 queries, 64 per wave, against 32-key
// blocks; d_h = 128: 128 queries, 32 per wave, against 64-key blocks).  For
// every key block:
//
//  * rebuild: the whole workgroup forms k_t = sum_r A_K[t,h,r] B~_K[t,r,:] and
//    v_t = sum_r A_V[t,h,r] B_V[t,r,:] for the block (rank pairs through
//    v_dot2_f32_bf16, fp32 sums), and stores K row-major and V transposed
//    (V^T[d][t]) in LDS as bf16.  The tiles are double-buffered: block i+1 is
//    rebuilt while block i is multiplied (at d_h = 64 from factors loaded one
//    block earlier still), so each block costs one barrier;
//  * scores, transposed: S^T[t, q] = K[t,:] . Q[q,:] with K as the A operand
//    (from LDS) and Q^T as the B operand (registers, formed once), so each
//    lane's scores belong to one query (its column);
//  * online softmax per query in base 2 (the scale log2(e) / (R_Q R_K sqrt(d_h))
//    is folded into Q), masking only on blocks that reach past a query.  The
//    running maximum moves only when a block's maximum exceeds it by more than
//    8 (then every probability stays below 2^8), so most blocks skip the
//    rescale; the result does not depend on the reference maximum.  The block
//    maximum crosses lane groups by half-wave swaps, not through LDS;
//  * values, transposed: O^T[d, q] += V^T[d, t] P^T[t, q]; the score tiles'
//    output registers are already the B operand of this product (k-slot j of
//    lane group g is key 4g+j of one 16-key tile for j<4, of the next for j>=4),
//    and the matching V^T rows are two 8-byte LDS reads.  One extra V^T tile
//    holds a row of ones, so the same product also yields sum_t p_t.
//
// Query blocks are scheduled heaviest (most keys) first, evenly across XCDs.
#include "kernels.h"
#include "mfma.h"
#include "rebuild.h"

namespace tpa {

// d_h = 64: 256 queries per workgroup (64 per wave) against 32-key blocks, so
// every K / V^T element read from LDS serves 64 queries; d_h = 128: 128
// queries (32 per wave) against 64-key blocks (wider rows leave registers for
// fewer query tiles).  Either way a wave does 36 (d_h = 64) or 72 matrix ops per
// block between barriers.
template <int DH>
struct PrefillMfmaCfg {
  static constexpr int QT = DH == 64 ? 4 : 2;     // 16-query tiles per wave
  static constexpr int BM = 4 * 16 * QT;          // queries per workgroup
  static constexpr int BN = DH == 64 ? 32 : 64;   // keys per block
  static constexpr int KT = BN / 16;              // 16-key tiles of the score product
  static constexpr int KB = BN / 32;              // 32-key steps of the value product
  static constexpr int KS = DH / 32;     // k-steps of the score product
  static constexpr int DT = DH / 16;     // d tiles of the value product (one more holds the ones row)
  static constexpr int LDK = DH + 8;     // K row stride in LDS (bf16)
  static constexpr int LDV = BN + 4;     // V^T row stride in LDS (bf16), 8-byte aligned rows
  // rebuild items: KPI consecutive keys x an 8-wide d slice, IT per thread
  static constexpr int KPI = BN * (DH / 8) >= 512 ? 2 : 1;
  static constexpr int IT = BN * (DH / 8) / KPI / 256;
  static constexpr int KTILE = BN * LDK;            // bf16 elements of one K buffer
  static constexpr int VTILE = (DH + 16) * LDV;     // bf16 elements of one V^T buffer
  static constexpr size_t kLds = (size_t)2 * (KTILE + VTILE) * sizeof(bf16_t);
  static constexpr float kRescaleSlack = 8.f;       // log2 units
};

// How far ahead of its rebuild a key block's factors are loaded: one block at
// d_h = 64; at d_h = 128 (two items per thread) those registers would spill,
// so each block's factors are loaded just before its rebuild.  (A second
// register set, two blocks ahead, spills at d_h = 64 as well.)
template <int DH, int R>
constexpr int prefill_prefetch_depth() {
  return DH == 64 ? 1 : 0;
}

// The cached factors one thread needs for its rebuild items of one key block:
// keys KPI*kg .. KPI*kg+KPI-1, d slice d0 .. d0+7.
template <int DH, int R>
struct RebuildRegs {
  static constexpr int IT = PrefillMfmaCfg<DH>::IT;
  static constexpr int KPI = PrefillMfmaCfg<DH>::KPI;
  uint4 bk[IT][KPI][R];
  uint4 bv[IT][KPI][R];
  typename RankWordP<R>::type ak[IT][KPI];
  typename RankWordP<R>::type av[IT][KPI];
};

// Item = (key group kg, 8-wide d slice d0).  Consecutive lanes take consecutive
// d slices of one key group, so the DH/8 lanes of a key read each rank row of
// B~_K / B_V as whole, contiguous cache lines.
template <int DH>
__device__ __forceinline__ void rebuild_item(int it, int& kg, int& d0) {
  const int item = threadIdx.x + 256 * it;
  kg = item / (DH / 8);
  d0 = (item % (DH / 8)) * 8;
}

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
    int kg, d0;
    rebuild_item<DH>(it, kg, d0);
#pragma unroll
    for (int k = 0; k < C::KPI; ++k) {
      int64_t t = k0 + C::KPI * kg + k;
      t = t < kend ? t : kend - 1;
      const int64_t row = seq0 + t;
      g.ak[it][k] = *reinterpret_cast<const W*>(AK + (row * a.h + hh) * R);
      g.av[it][k] = *reinterpret_cast<const W*>(AV + (row * a.h + hh) * R);
#pragma unroll
      for (int r = 0; r < R; ++r) {
        g.bk[it][k][r] = *reinterpret_cast<const uint4*>(BK + (row * R + r) * DH + d0);
        g.bv[it][k][r] = *reinterpret_cast<const uint4*>(BV + (row * R + r) * DH + d0);
      }
    }
  }
}

template <int DH, int R>
__device__ __forceinline__ void store_rebuild(const RebuildRegs<DH, R>& g, bf16_t* ks_lds, bf16_t* vt_lds) {
  using C = PrefillMfmaCfg<DH>;
#pragma unroll
  for (int it = 0; it < C::IT; ++it) {
    int kg, d0;
    rebuild_item<DH>(it, kg, d0);
    float kv[C::KPI][8], vv[C::KPI][8];
#pragma unroll
    for (int k = 0; k < C::KPI; ++k) {
      factor_combine<R>(g.ak[it][k], g.bk[it][k], kv[k]);
      factor_combine<R>(g.av[it][k], g.bv[it][k], vv[k]);
      *reinterpret_cast<bf16x8_t*>(ks_lds + (C::KPI * kg + k) * C::LDK + d0) = pack8(kv[k]);
    }
    if constexpr (C::KPI == 2) {
#pragma unroll
      for (int j = 0; j < 8; ++j)
        *reinterpret_cast<uint32_t*>(vt_lds + (d0 + j) * C::LDV + 2 * kg) = pack_bf16x2(vv[0][j], vv[1][j]);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) vt_lds[(d0 + j) * C::LDV + kg] = f32_to_bf16(vv[0][j]);
    }
  }
}

// One key block of the online-softmax attention for this wave's QT x 16 queries
// (positions wpos0 ..), reading K and V^T of the block from LDS.  EARLY_V:
// read all of the block's V^T operands right after the score products, so the
// softmax hides their latency (where the registers allow it).
template <int DH, bool EARLY_V>
__device__ __forceinline__ void attend_block(const bf16_t* ks_lds, const bf16_t* vt_lds, int64_t k0, int64_t kend,
                                             int64_t wpos0, bool causal, int li, int lg,
                                             const bf16x8_t (&qop)[PrefillMfmaCfg<DH>::QT][PrefillMfmaCfg<DH>::KS],
                                             float (&m_run)[PrefillMfmaCfg<DH>::QT],
                                             f32x4_t (&oacc)[PrefillMfmaCfg<DH>::QT][PrefillMfmaCfg<DH>::DT + 1]) {
  using C = PrefillMfmaCfg<DH>;
  constexpr int BN = C::BN, QT = C::QT, KS = C::KS, DT = C::DT, LDK = C::LDK, LDV = C::LDV;
  constexpr int KT = C::KT, KB = C::KB;
    // ---- scores S^T[key, query] for the block's key tiles
    f32x4_t sacc[KT][QT];
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
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

    // ---- V^T operands of the block
    auto read_vt = [&](int dt, int kb) __attribute__((always_inline)) {
      const bf16_t* vrow = vt_lds + (dt * 16 + li) * LDV + kb * 32 + 4 * lg;
      const uint2 lo = *reinterpret_cast<const uint2*>(vrow);
      const uint2 hi = *reinterpret_cast<const uint2*>(vrow + 16);
      return as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
    };
    bf16x8_t vfe[EARLY_V ? DT + 1 : 1][KB];
    if constexpr (EARLY_V) {
#pragma unroll
      for (int dt = 0; dt <= DT; ++dt)
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) vfe[dt][kb] = read_vt(dt, kb);
    }

    // ---- mask (only where the block reaches past a query of this wave, or
    //      past the keys; a uniform branch).  Value i of tile (kt, qt) is the
    //      key at offset 16*kt + 4*lg + i from k0; it is visible iff that
    //      offset is at most both kend - 1 - k0 and, when causal, the query's
    //      position - k0 (limits clamped to 32-bit values: the offsets are
    //      small).
    const bool need_mask = (causal && k0 + BN - 1 > wpos0) || (k0 + BN > kend);
    if (need_mask) {
      const int64_t krel = kend - 1 - k0, qrel = wpos0 - k0;
      const int klim = (int)(krel < 2 * BN ? krel : 2 * BN);
      const int qlim = (int)(qrel < 2 * BN ? (qrel > -2 * BN ? qrel : -2 * BN) : 2 * BN);
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) {
        int lim = causal ? min(klim, qlim + 16 * qt + li) : klim;
        lim -= 4 * lg;
#pragma unroll
        for (int kt = 0; kt < KT; ++kt)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (kt * 16 + i > lim) sacc[kt][qt][i] = -INFINITY;
      }
    }

    // ---- online softmax per query (lazy rescale), P^T operands
    bf16x8_t pop[QT][KB];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      float bmax = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < KT; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) bmax = max_nn(bmax, sacc[kt][qt][i]);
      bmax = lane_group_max_nn(bmax);
      const bool grow = bmax > m_run[qt] + C::kRescaleSlack;
      if (__any(grow)) {
        const float m_new = grow ? bmax : m_run[qt];
        const float alpha = fast_exp2(m_run[qt] - m_new);   // 0 on the first block, 1 where m stays
        m_run[qt] = m_new;
#pragma unroll
        for (int dt = 0; dt <= DT; ++dt) oacc[qt][dt] *= alpha;
      }
      // a query with no visible key yet keeps m = -inf; its probabilities are 0
      const float m_use = m_run[qt] == -INFINITY ? 0.f : m_run[qt];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        float pv[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) pv[j] = fast_exp2(sacc[2 * kb + (j >> 2)][qt][j & 3] - m_use);
        pop[qt][kb] = pack8(pv);
      }
    }

    // ---- O^T += V^T P^T (and the ones row: sum_t p_t)
#pragma unroll
    for (int dt = 0; dt <= DT; ++dt) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        bf16x8_t vf;
        if constexpr (EARLY_V) vf = vfe[dt][kb];
        else vf = read_vt(dt, kb);
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) oacc[qt][dt] = mfma_bf16(vf, pop[qt][kb], oacc[qt][dt]);
      }
    }

}

template <int DH, int R>
__global__ void __launch_bounds__(256, 2) prefill_mfma_kernel(AttnArgs a, int n_qblocks) {
  using C = PrefillMfmaCfg<DH>;
  constexpr int BM = C::BM, BN = C::BN, QT = C::QT, KS = C::KS, DT = C::DT, LDV = C::LDV;
  extern __shared__ __align__(16) unsigned char smem[];
  bf16_t* const lds = reinterpret_cast<bf16_t*>(smem);
  // buffer i: K at lds + i*KTILE, V^T at lds + 2*KTILE + i*VTILE
#define KS_BUF(i) (lds + (i) * C::KTILE)
#define VT_BUF(i) (lds + 2 * C::KTILE + (i) * C::VTILE)
  // the wave index is uniform: kept scalar, so the per-block tests on the
  // wave's positions (skip, mask) are scalar branches
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int li = lane & 15, lg = lane >> 4;
  // One-dimensional grid.  Work items (query block, head, sequence) in order of
  // decreasing key count are numbered by the linear workgroup id; since
  // workgroups go to the XCDs round-robin by that id, every XCD gets an equal
  // share of every query block, heaviest first.  When the (sequence, head)
  // pairs split evenly over the eight XCDs, XCD x takes the x-th contiguous
  // range of them (sequence-major), so the factors it reads span as few
  // sequences as possible and stay in its L2.
  const int h = a.h;
  const int64_t hb = (int64_t)h * a.n_batch;
  const int64_t L = blockIdx.x;
  const int qb = n_qblocks - 1 - (int)(L / hb);
  int64_t u = L % hb;
  if (hb % 8 == 0) u = (u & 7) * (hb >> 3) + (u >> 3);
  const int hh = (int)(u % h);
  const int64_t b = u / h;
  const int64_t q0 = (int64_t)qb * BM;
  const int64_t seq0 = b * a.max_seq;
  const int64_t last_q = (q0 + BM < a.S ? q0 + BM : a.S) - 1;
  const int64_t kend = a.causal ? a.start_pos + last_q + 1 : a.start_pos + a.S;
  const int nblk = (int)((kend + BN - 1) / BN);

  // The first key block's factors go out before anything else.
  RebuildRegs<DH, R> rg;
  load_rebuild<DH, R>(rg, a, seq0, hh, 0, kend);

  // The ones row (and fifteen zero rows) of the extra V^T tile, in both buffers.
  for (int i = threadIdx.x; i < 16 * BN; i += blockDim.x) {
    const int rr = i / BN, col = i % BN;
    const bf16_t v = rr == 0 ? (bf16_t)0x3f80 : (bf16_t)0;
    VT_BUF(0)[(DH + rr) * LDV + col] = v;
    VT_BUF(1)[(DH + rr) * LDV + col] = v;
  }

  // ---- query operand: lane (query q0 + 16*QT*wave + 16*qt + li, slice lg)
  bf16x8_t qop[QT][KS];
  {
    const bf16_t* AQ = reinterpret_cast<const bf16_t*>(a.a_q);
    const bf16_t* BQ = reinterpret_cast<const bf16_t*>(a.b_q);
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      const int64_t s = q0 + 16 * QT * wave + 16 * qt + li;
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

  float m_run[QT];
  f32x4_t oacc[QT][DT + 1];     // tile DT: row 0 accumulates sum_t p_t
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    m_run[qt] = -INFINITY;
#pragma unroll
    for (int dt = 0; dt <= DT; ++dt) oacc[qt][dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  constexpr int kDepth = prefill_prefetch_depth<DH, R>();
  const int64_t wpos0 = a.start_pos + q0 + 16 * QT * wave;   // first position of this wave's queries
  const bool causal = a.causal != 0;
  // Block i is rebuilt into buffer i & 1 while block i - 1 is attended to.
  store_rebuild<DH, R>(rg, KS_BUF(0), VT_BUF(0));
  if constexpr (kDepth == 1) {
    if (nblk > 1) load_rebuild<DH, R>(rg, a, seq0, hh, BN, kend);
  }
  __syncthreads();
  for (int blk = 0; blk < nblk; ++blk) {
    const int64_t k0 = (int64_t)blk * BN;
    attend_block<DH, DH == 64 && R <= 2>(KS_BUF(blk & 1), VT_BUF(blk & 1), k0, kend, wpos0, causal, li, lg, qop,
                                          m_run, oacc);
    // rebuild the next block into the other buffer; with depth 1 its factors
    // were loaded a block ago and the block after it starts loading now
    if (blk + 1 < nblk) {
      if constexpr (kDepth == 0) load_rebuild<DH, R>(rg, a, seq0, hh, k0 + BN, kend);
      store_rebuild<DH, R>(rg, KS_BUF((blk + 1) & 1), VT_BUF((blk + 1) & 1));
      if constexpr (kDepth == 1) {
        if (blk + 2 < nblk) load_rebuild<DH, R>(rg, a, seq0, hh, k0 + 2 * BN, kend);
      }
    }
    __syncthreads();
  }
#undef KS_BUF
#undef VT_BUF

  // ---- normalise and store: lane holds d = 16*dt + 4*lg + i of its query;
  //      sum_t p_t of query li sits in lane li (row 0 of the ones tile)
  bf16_t* out = reinterpret_cast<bf16_t*>(a.out);
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const float l = __shfl(oacc[qt][DT][0], li);
    const float inv = a.v_scale / l;
    const int64_t s = q0 + 16 * QT * wave + 16 * qt + li;
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

// LDS a workgroup may allocate on the current device.
static size_t device_lds_per_block() {
  int dev = 0, v = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess) return 0;
  return (size_t)v;
}

bool prefill_mfma_supported(int dtype, const AttnArgs& a) {
  if (dtype != kBF16) return false;
  const size_t lds = a.d_h == 64 ? PrefillMfmaCfg<64>::kLds : PrefillMfmaCfg<128>::kLds;
  if (lds > device_lds_per_block()) return false;
  const int bm = a.d_h == 64 ? PrefillMfmaCfg<64>::BM : PrefillMfmaCfg<128>::BM;
  if ((a.S + bm - 1) / bm * (int64_t)a.h * a.n_batch >= ((int64_t)1 << 31)) return false;
  if (!(a.d_h == 64 || a.d_h == 128)) return false;
  if (a.rk != a.rv || !(a.rk == 1 || a.rk == 2 || a.rk == 4)) return false;
  if (a.d_h == 128 && a.rk == 4) return false;   // its registers would spill
  const void* ptrs[4] = {a.b_q, a.c_bk, a.c_bv, a.out};   // read/written 8 or 16 bytes at a time
  for (int i = 0; i < 4; ++i)
    if (((uintptr_t)ptrs[i]) % 16) return false;
  return true;
}

hipError_t launch_prefill_mfma(const AttnArgs& a, hipStream_t st) {
  const int bm = a.d_h == 64 ? PrefillMfmaCfg<64>::BM : PrefillMfmaCfg<128>::BM;
  const int nqb = (int)((a.S + bm - 1) / bm);
  const dim3 grid((unsigned)((int64_t)nqb * a.h * a.n_batch));
#define TPA_PREFILL_LAUNCH(DH_, R_)                                                               \
  hipLaunchKernelGGL((prefill_mfma_kernel<DH_, R_>), grid, dim3(256), PrefillMfmaCfg<DH_>::kLds, st, a, \
                     nqb)
  if (a.d_h == 64) {
    if (a.rk == 1) TPA_PREFILL_LAUNCH(64, 1);
    else if (a.rk == 2) TPA_PREFILL_LAUNCH(64, 2);
    else TPA_PREFILL_LAUNCH(64, 4);
  } else {
    if (a.rk == 1) TPA_PREFILL_LAUNCH(128, 1);
    else TPA_PREFILL_LAUNCH(128, 2);
  }
#undef TPA_PREFILL_LAUNCH
  return hipGetLastError();
}

}  // namespace tpa
