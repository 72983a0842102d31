// Causal prefill attention at d_h = 64 on v_mfma_f32_32x32x16_bf16 (on gfx950
// this form sustains about twice the rate of the 16x16x32 one), with keys and
// values rebuilt from the cached factors in LDS.
//
// Arithmetic as the general prefill kernel ("Tensor Product Attention Is All
// You Need" review on coreui.cn: Q_t/K_t/V_t equations of 核心机制总结 and the
// masked softmax attention of the code walk-through 前向传播).  A workgroup owns
// 256 queries of one head of one sequence; each of its four waves owns 64 of
// them as two 32-query tiles.  For every key block (64 keys at ranks 1 and 2;
// 32 at rank 4, whose factors would spill registers at 64):
//
//  * rebuild: the whole workgroup forms k_t = sum_r A_K[t,h,r] B~_K[t,r,:] and
//    v_t likewise (rank pairs through v_dot2_f32_bf16, fp32 sums) and stores
//    both row-major in LDS as bf16, 16 bytes per store.  Two buffers: block
//    i+1 is rebuilt (from factors loaded a block earlier) while block i is
//    multiplied, so each block costs one barrier;
//  * scores, transposed: S^T[t, q] = K[t,:] . Q[q,:], K as the A operand (LDS,
//    16-byte reads of rows padded to 72 elements) and Q^T as the B operand
//    (registers, formed once); each lane's 16 scores of a tile belong to one
//    query, and the two lanes that share a query swap once per block for the
//    block maximum;
//  * online softmax per query in base 2 (the scale log2(e) / (R_Q R_K sqrt(d_h))
//    is folded into Q); the running maximum moves only when a block's maximum
//    exceeds it by more than 8, so most blocks skip the rescale; masking only
//    on blocks that reach past a query; a wave skips blocks that lie wholly
//    after its queries;
//  * values, transposed: O^T[d, q] += V^T[d, t] P^T[t, q].  The score tiles'
//    output registers, rounded to bf16, are the B operand as they are (k-slot
//    j of lane half g is key 4g+j for j<4, 8+4g+(j-4) for j>=4, of a 16-key
//    step); the matching V^T operand comes straight from the row-major V tile
//    with two ds_read_b64_tr_b16 (each gives the lanes of a 16-lane group four
//    consecutive keys of their own column d);
//  * the softmax denominators are the sums of the same bf16 probabilities
//    (v_dot2 against ones), accumulated per lane and joined at the end.
//    (Taking them on the matrix cores with a ones row measured slower; so did
//    forming the next block's scores a step ahead from a third buffer, with
//    or without scheduling groups that interleave the matrix products with
//    the softmax and rebuild: 4-9% slower at 4 x 4096 tokens.)
//
// Query blocks are scheduled heaviest (most keys) first, evenly across XCDs.
//
// The same kernel also reads K and V formed once for the whole call into a
// workspace (kv_material32_kernel, same arithmetic and rounding as the
// rebuild, for the standard and the shared-basis cache): each block is then two 16-byte loads and LDS stores per thread
// instead of the rebuild's rank sums, which a 256-query workgroup would
// otherwise repeat for every key it attends to.
#include "kernels.h"
#include "mfma.h"
#include "rebuild.h"

namespace tpa {

// max of x over the lanes l and l ^ 32
__device__ __forceinline__ float half_swap_max(float x) {
  const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return max_nn(__uint_as_float(s[0]), __uint_as_float(s[1]));
}

template <int R>
struct Pf32Cfg {
  static constexpr int DH = 64;
  static constexpr int NW = 4;                 // waves per workgroup
  static constexpr int NT = 64 * NW;           // threads per workgroup
  static constexpr int OCC = 2;                // waves per SIMD to fit (registers <= 512 / OCC)
  static constexpr int QT = 2;                 // 32-query tiles per wave
  static constexpr int BM = NW * 32 * QT;      // queries per workgroup
  static constexpr int BN = R == 4 ? 32 : 64;  // keys per block
  static constexpr int KT = BN / 32;           // 32-key tiles of the score product
  static constexpr int KS = BN / 16;           // 16-key steps of the value product
  static constexpr int LD = DH + 8;            // LDS row stride (bf16) of K and V
  static constexpr int TILE = BN * LD;         // bf16 elements of one K or V buffer
  static constexpr int IT = BN * (DH / 8) / NT;    // rebuild items per thread
  static constexpr size_t kLds = (size_t)4 * TILE * sizeof(bf16_t);
  static constexpr float kRescaleSlack = 8.f;  // log2 units
};

// The cached factors one thread needs for its rebuild items of one key block:
// item = (key, 8-wide d slice), consecutive lanes on consecutive slices of one
// key, so each rank row of B~_K / B_V is read as whole cache lines.
template <int R>
struct Rebuild32 {
  static constexpr int IT = Pf32Cfg<R>::IT;
  uint4 bk[IT][R];
  uint4 bv[IT][R];
  typename RankWordP<R>::type ak[IT];
  typename RankWordP<R>::type av[IT];
};

// The factor rows of one (sequence, head), as uniform bases: a key's
// addresses are then one 32 x 32 -> 64-bit multiply-add from its index.
struct RebuildBase32 {
  const bf16_t* ak;    // A_K row of key 0, head hh
  const bf16_t* av;
  const bf16_t* bk;    // B~_K row of key 0 (in the shared mode, unused)
  const bf16_t* bv;
  uint32_t a_stride;   // elements per key of A_K / A_V (h * R)
};

template <int R>
__device__ __forceinline__ RebuildBase32 rebuild_base32(const AttnArgs& a, int64_t seq0, int hh) {
  RebuildBase32 r;
  r.ak = reinterpret_cast<const bf16_t*>(a.c_ak) + (seq0 * a.h + hh) * R;
  r.av = reinterpret_cast<const bf16_t*>(a.c_av) + (seq0 * a.h + hh) * R;
  r.bk = reinterpret_cast<const bf16_t*>(a.c_bk) + seq0 * R * 64;
  r.bv = reinterpret_cast<const bf16_t*>(a.c_bv) + seq0 * R * 64;
  r.a_stride = (uint32_t)(a.h * R);
  return r;
}

// Keys past klast (the last valid key) are clamped to it: they are masked out
// of every score, so only finiteness matters.  Key indices are below 2^31.
template <int R, bool SHARED = false>
__device__ __forceinline__ void load_rebuild32(Rebuild32<R>& g, const RebuildBase32& p, int k0, int klast) {
  typedef typename RankWordP<R>::type W;
#pragma unroll
  for (int it = 0; it < Rebuild32<R>::IT; ++it) {
    const int item = threadIdx.x + Pf32Cfg<R>::NT * it;
    const int key = item >> 3, d0 = (item & 7) * 8;
    const uint32_t t = (uint32_t)min(k0 + key, klast);
    const uint64_t aoff = (uint64_t)t * p.a_stride;
    g.ak[it] = *reinterpret_cast<const W*>(p.ak + aoff);
    g.av[it] = *reinterpret_cast<const W*>(p.av + aoff);
    if constexpr (!SHARED) {   // (the shared bases are loaded once, by load_basis32)
      const uint64_t boff = (uint64_t)t * (R * 64) + (uint32_t)d0;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        g.bk[it][r] = *reinterpret_cast<const uint4*>(p.bk + boff + r * 64);
        g.bv[it][r] = *reinterpret_cast<const uint4*>(p.bv + boff + r * 64);
      }
    }
  }
}

// The shared bases' slices of this thread: every rebuild item of a thread has
// the same 8-wide d slice (items differ by multiples of 8), so one load each.
template <int R>
__device__ __forceinline__ void load_basis32(Rebuild32<R>& g, const AttnArgs& a) {
  const bf16_t* BK = reinterpret_cast<const bf16_t*>(a.c_bk);
  const bf16_t* BV = reinterpret_cast<const bf16_t*>(a.c_bv);
  const int d0 = (threadIdx.x & 7) * 8;
#pragma unroll
  for (int it = 0; it < Rebuild32<R>::IT; ++it)
#pragma unroll
    for (int r = 0; r < R; ++r) {
      g.bk[it][r] = *reinterpret_cast<const uint4*>(BK + r * 64 + d0);
      g.bv[it][r] = *reinterpret_cast<const uint4*>(BV + r * 64 + d0);
    }
}

// One rotary pair turned by (c, s), contractions written out so every kernel
// that forms shared-basis keys rounds them the same way.
__device__ __forceinline__ void rotate_pair(float& x0, float& x1, float c, float s) {
  const float y0 = fmaf(x0, c, -(x1 * s));
  const float y1 = fmaf(x0, s, x1 * c);
  x0 = y0;
  x1 = y1;
}

// SHARED: k0 is the block's first key (= its position) and s_rev the rotary
// frequencies; each key is rotated at its own position after the rank sum.
template <int R, bool SHARED = false>
__device__ __forceinline__ void store_rebuild32(const Rebuild32<R>& g, bf16_t* k_lds, bf16_t* v_lds, int64_t k0 = 0,
                                                const double* s_rev = nullptr) {
  constexpr int LD = Pf32Cfg<R>::LD;
#pragma unroll
  for (int it = 0; it < Rebuild32<R>::IT; ++it) {
    const int item = threadIdx.x + Pf32Cfg<R>::NT * it;
    const int key = item >> 3, d0 = (item & 7) * 8;
    float kv[8], vv[8];
    factor_combine<R>(g.ak[it], g.bk[it], kv);
    factor_combine<R>(g.av[it], g.bv[it], vv);
    if constexpr (SHARED) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float c, sn;
        rope_cos_sin(s_rev, k0 + key, (d0 >> 1) + q, c, sn);
        rotate_pair(kv[2 * q], kv[2 * q + 1], c, sn);
      }
    }
    *reinterpret_cast<bf16x8_t*>(k_lds + key * LD + d0) = pack8(kv);
    *reinterpret_cast<bf16x8_t*>(v_lds + key * LD + d0) = pack8(vv);
  }
}

// Materialised keys and values ([B][h][T][64] bf16, formed by
// kv_material32_kernel): the thread's 16-byte row pieces of one 64-key block,
// items as in the rebuild (consecutive lanes on consecutive slices of a row).
struct KvRows32 {
  static constexpr int IT = Pf32Cfg<2>::IT;
  bf16x8_t k[IT];   // (native vectors: HIP's uint4 struct here went through scratch)
  bf16x8_t v[IT];
};

__device__ __forceinline__ void load_kv32(KvRows32& g, const bf16_t* kb, const bf16_t* vb, int k0, int klast) {
#pragma unroll
  for (int it = 0; it < KvRows32::IT; ++it) {
    const int item = threadIdx.x + Pf32Cfg<2>::NT * it;
    const int key = item >> 3, d0 = (item & 7) * 8;
    const uint64_t off = (uint64_t)(uint32_t)min(k0 + key, klast) * 64 + (uint32_t)d0;
    g.k[it] = *reinterpret_cast<const bf16x8_t*>(kb + off);
    g.v[it] = *reinterpret_cast<const bf16x8_t*>(vb + off);
  }
}

__device__ __forceinline__ void store_kv32(const KvRows32& g, bf16_t* k_lds, bf16_t* v_lds) {
  constexpr int LD = Pf32Cfg<2>::LD;
#pragma unroll
  for (int it = 0; it < KvRows32::IT; ++it) {
    const int item = threadIdx.x + Pf32Cfg<2>::NT * it;
    const int key = item >> 3, d0 = (item & 7) * 8;
    *reinterpret_cast<bf16x8_t*>(k_lds + key * LD + d0) = g.k[it];
    *reinterpret_cast<bf16x8_t*>(v_lds + key * LD + d0) = g.v[it];
  }
}

// One key block for this wave's QT x 32 queries (positions wpos0 ..).
template <int R>
__device__ __forceinline__ void attend_block32(const bf16_t* k_lds, const bf16_t* v_lds, int64_t k0, int64_t kend,
                                               int64_t wpos0, bool causal, int lane,
                                               const bf16x8_t (&qop)[Pf32Cfg<R>::QT][4],
                                               float (&m_run)[Pf32Cfg<R>::QT], float (&lsum)[Pf32Cfg<R>::QT],
                                               f32x16_t (&oacc)[Pf32Cfg<R>::QT][2]) {
  using C = Pf32Cfg<R>;
  constexpr int QT = C::QT, KT = C::KT, KS = C::KS, LD = C::LD, BN = C::BN;
  const int l32 = lane & 31, lh = lane >> 5;

  // ---- scores S^T[key, query] for the block's 32-key tiles.  With two key
  //      tiles (BN 64) each product starts from minus the query's running
  //      maximum (0 while it has none): one start block per query tile serves
  //      both key tiles, so the exponentials below need no subtraction.  With
  //      one key tile the start block would cost as many moves as it saves.
  constexpr bool kFromMinusM = KT > 1;
  float m_use[QT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) m_use[qt] = m_run[qt] == -INFINITY ? 0.f : m_run[qt];
  f32x16_t sacc[KT][QT];
#pragma unroll
  for (int kt = 0; kt < KT; ++kt) {
    bf16x8_t kf[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      kf[ks] = *reinterpret_cast<const bf16x8_t*>(k_lds + (kt * 32 + l32) * LD + ks * 16 + lh * 8);
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      f32x16_t acc;
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[e] = kFromMinusM ? -m_use[qt] : 0.f;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) acc = mfma32_bf16(kf[ks], qop[qt][ks], acc);
      sacc[kt][qt] = acc;
    }
  }

  // ---- mask (only where the block reaches past a query of this wave, or
  //      past the keys; a uniform branch).  Value e of tile kt is the key at
  //      offset 32*kt + 8*(e/4) + 4*lh + e%4 from k0; it is visible iff that
  //      offset is at most both kend - 1 - k0 and, when causal, the query's
  //      position - k0.  The offsets are small, so the limits are clamped to
  //      32-bit values and each element costs one compare against a constant.
  const bool need_mask = (causal && k0 + BN - 1 > wpos0) || (k0 + BN > kend);
  if (need_mask) {
    const int64_t krel = kend - 1 - k0, qrel = wpos0 - k0;
    const int klim = (int)(krel < 2 * BN ? krel : 2 * BN);
    const int qlim = (int)(qrel < 2 * BN ? (qrel > -2 * BN ? qrel : -2 * BN) : 2 * BN);
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      int lim = causal ? min(klim, qlim + 32 * qt + l32) : klim;
      lim -= 4 * lh;
#pragma unroll
      for (int kt = 0; kt < KT; ++kt)
#pragma unroll
        for (int e = 0; e < 16; ++e)
          if (32 * kt + 8 * (e >> 2) + (e & 3) > lim) sacc[kt][qt][e] = -INFINITY;
    }
  }

  // ---- online softmax per query (lazy rescale), P^T operands, row sums
  constexpr uint32_t kOnes = 0x3f803f80u;   // (1, 1) in bf16
  bf16x8_t pop[QT][KS];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    float bmax = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
#pragma unroll
      for (int e = 0; e < 16; ++e) bmax = max_nn(bmax, sacc[kt][qt][e]);
    bmax = half_swap_max(bmax);   // kFromMinusM: relative to m_use
    // The first visible key sets the maximum; later it moves only past the slack.
    bool grow;
    if constexpr (kFromMinusM)
      grow = bmax > (m_run[qt] == -INFINITY ? -INFINITY : C::kRescaleSlack);
    else
      grow = bmax > m_run[qt] + C::kRescaleSlack;
    if (__any(grow)) {
      const float m_new = grow ? (kFromMinusM ? m_use[qt] + bmax : bmax) : m_run[qt];
      const float alpha = grow ? fast_exp2(m_run[qt] - m_new) : 1.f;   // 0 on the first block
      m_run[qt] = m_new;
      lsum[qt] *= alpha;
#pragma unroll
      for (int dt = 0; dt < 2; ++dt) oacc[qt][dt] *= alpha;
      if constexpr (kFromMinusM) {
        const float shift = grow ? bmax : 0.f;
#pragma unroll
        for (int kt = 0; kt < KT; ++kt)
#pragma unroll
          for (int e = 0; e < 16; ++e) sacc[kt][qt][e] -= shift;
      }
    }
    // A query with no visible key yet keeps m = -inf: its scores are -inf and
    // its probabilities 0.
    const float m_sub = kFromMinusM ? 0.f : (m_run[qt] == -INFINITY ? 0.f : m_run[qt]);
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      float pv[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float x = sacc[s >> 1][qt][8 * (s & 1) + j];
        pv[j] = fast_exp2(kFromMinusM ? x : x - m_sub);
      }
      pop[qt][s] = pack8(pv);
      const uint4 w = __builtin_bit_cast(uint4, pop[qt][s]);
      float l = lsum[qt];
      l = dot2_bf16(w.x, kOnes, l);
      l = dot2_bf16(w.y, kOnes, l);
      l = dot2_bf16(w.z, kOnes, l);
      l = dot2_bf16(w.w, kOnes, l);
      lsum[qt] = l;
    }
  }

  // ---- O^T += V^T P^T.  Lane l of a 16-lane group reads the piece at key row
  //      4*lh + (l%16)/4 (+8 for the second half of the k-slots), columns
  //      16*((l/16)%2) + 4*(l%4) .. of the d tile.
  const int grp = lane & 15;
  const bf16_t* vbase = v_lds + (4 * lh + (grp >> 2)) * LD + 16 * ((lane >> 4) & 1) + 4 * (grp & 3);
#pragma unroll
  for (int dt = 0; dt < 2; ++dt) {
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const bf16_t* vp = vbase + s * 16 * LD + dt * 32;
      const uint2 lo = lds_read_tr16(vp);
      const uint2 hi = lds_read_tr16(vp + 8 * LD);
      const bf16x8_t vf = __builtin_bit_cast(bf16x8_t, make_uint4(lo.x, lo.y, hi.x, hi.y));
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) oacc[qt][dt] = mfma32_bf16(vf, pop[qt][s], oacc[qt][dt]);
    }
  }
}

// Where a block's keys and values come from: rebuilt from the cached factors,
// rebuilt from a shared-basis cache (c_bk / c_bv are the bases; keys rotated at
// their positions with tab), or read as formed by kv_material32_kernel (kmat,
// vmat: mat_len keys per (sequence, head); instantiated with R = 2, whose
// 64-key blocks it uses).
enum KvSource : int { kFromFactors = 0, kFromSharedBasis = 1, kFromMaterial = 2 };

template <int R, int SRC>
__global__ void __launch_bounds__(Pf32Cfg<R>::NT, Pf32Cfg<R>::OCC)
    prefill_mfma32_kernel(AttnArgs a, int n_qblocks, RopeTable tab, const bf16_t* kmat, const bf16_t* vmat,
                          int64_t mat_len, int mat_group) {
  constexpr bool SHARED = SRC == kFromSharedBasis, MAT = SRC == kFromMaterial;
  static_assert(!MAT || R == 2, "materialised blocks use the 64-key configuration");
  using C = Pf32Cfg<R>;
  constexpr int DH = 64, QT = C::QT, BM = C::BM, BN = C::BN, TILE = C::TILE;
  extern __shared__ __align__(16) unsigned char smem[];
  bf16_t* const lds = reinterpret_cast<bf16_t*>(smem);
  // buffer i: K at lds + i*TILE, V at lds + (2 + i)*TILE
  // the wave index is uniform: kept scalar, so the per-block tests on the
  // wave's positions (skip, mask) are scalar branches
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l32 = lane & 31, lh = lane >> 5;
  // One-dimensional grid.  Work items (query block, head, sequence) in order of
  // decreasing key count are numbered by the linear workgroup id; since
  // workgroups go to the XCDs round-robin by that id, every XCD gets an equal
  // share of every query block, heaviest first.  When the (sequence, head)
  // pairs split evenly over the eight XCDs, XCD x takes the x-th contiguous
  // range of them (sequence-major), so the factors it reads span as few
  // sequences as possible and stay in its L2.
  //
  // Materialised K and V are per head.  With many query blocks per pair that
  // order would leave every resident workgroup of an XCD on another pair, each
  // reading its own K and V from HBM.  So (mat_group > 0) an XCD's range of
  // pairs is taken in groups of mat_group pairs, one group after another, each
  // group in the order above (query block major, heaviest first): a group's
  // K and V are then read by about mat_group * n_qblocks workgroups that run
  // together.  The host picks mat_group so that a group spans about two
  // rounds of an XCD's resident workgroups (all of its pairs when they fit).
  const int h = a.h;
  const int64_t hb = (int64_t)h * a.n_batch;
  const int64_t L = blockIdx.x;
  int qb;
  int64_t u;
  if (MAT && mat_group > 0 && hb % 8 == 0) {
    const int64_t s = L >> 3, span = (int64_t)mat_group * n_qblocks;
    const int64_t r = s % span;
    qb = n_qblocks - 1 - (int)(r / mat_group);
    u = (L & 7) * (hb >> 3) + s / span * mat_group + r % mat_group;
  } else {
    qb = n_qblocks - 1 - (int)(L / hb);
    u = L % hb;
    if (hb % 8 == 0) u = (u & 7) * (hb >> 3) + (u >> 3);
  }
  const int hh = (int)(u % h);
  const int64_t b = u / h;
  const int64_t q0 = (int64_t)qb * BM;
  const int64_t seq0 = b * a.max_seq;
  const int64_t last_q = (q0 + BM < a.S ? q0 + BM : a.S) - 1;
  const int64_t kend = a.causal ? a.start_pos + last_q + 1 : a.start_pos + a.S;
  const int nblk = (int)((kend + BN - 1) / BN);

  // The first key block's loads go out before anything else.
  typename std::conditional<MAT, KvRows32, Rebuild32<R>>::type rg;
  __shared__ double s_rev[SHARED ? 32 : 1];   // d_h = 64: 32 rotary pairs
  if constexpr (SHARED) {
    rope_stage(tab, 32, s_rev);
    load_basis32<R>(rg, a);
  }
  const RebuildBase32 rbase = rebuild_base32<R>(a, seq0, hh);
  const bf16_t* const kb = MAT ? kmat + ((b * h + hh) * mat_len) * 64 : nullptr;
  const bf16_t* const vb = MAT ? vmat + ((b * h + hh) * mat_len) * 64 : nullptr;
  const int klast = (int)(kend - 1);
#define TPA_PF32_LOAD(k0)                       \
  do {                                          \
    if constexpr (MAT)                          \
      load_kv32(rg, kb, vb, k0, klast);         \
    else                                        \
      load_rebuild32<R, SHARED>(rg, rbase, k0, klast); \
  } while (0)
#define TPA_PF32_STORE(k_lds, v_lds, k0)                       \
  do {                                                         \
    if constexpr (MAT)                                         \
      store_kv32(rg, k_lds, v_lds);                            \
    else                                                       \
      store_rebuild32<R, SHARED>(rg, k_lds, v_lds, k0, s_rev); \
  } while (0)
  TPA_PF32_LOAD(0);

  // ---- query operand: lane (query q0 + 32*QT*wave + 32*qt + l32, d slice
  //      16*ks + 8*lh .. +8), pre-scaled
  bf16x8_t qop[QT][4];
  {
    const bf16_t* AQ = reinterpret_cast<const bf16_t*>(a.a_q);
    const bf16_t* BQ = reinterpret_cast<const bf16_t*>(a.b_q);
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      const int64_t s = q0 + 32 * QT * wave + 32 * qt + l32;
      const int64_t tok = b * a.q_bstride_tok + (s < a.S ? s : a.S - 1);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int d0 = ks * 16 + lh * 8;
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

  float m_run[QT], lsum[QT];   // lsum: this lane's half of each row sum
  f32x16_t oacc[QT][2];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    m_run[qt] = -INFINITY;
    lsum[qt] = 0.f;
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
      for (int e = 0; e < 16; ++e) oacc[qt][dt][e] = 0.f;
  }

  const int64_t wpos0 = a.start_pos + q0 + 32 * QT * wave;   // position of this wave's first query
  const bool causal = a.causal != 0;
  // Block i is rebuilt into buffer i & 1 while block i - 1 is attended to; its
  // factors were loaded a block earlier.
  if constexpr (SHARED) __syncthreads();   // the staged frequencies are visible
  TPA_PF32_STORE(lds, lds + 2 * TILE, 0);
  if (nblk > 1) TPA_PF32_LOAD(BN);
  __syncthreads();
  for (int blk = 0; blk < nblk; ++blk) {
    const int64_t k0 = (int64_t)blk * BN;
    // a block wholly after every query of this wave contributes nothing
    if (!causal || k0 <= wpos0 + 32 * QT - 1)
      attend_block32<R>(lds + (blk & 1) * TILE, lds + (2 + (blk & 1)) * TILE, k0, kend, wpos0, causal, lane, qop,
                        m_run, lsum, oacc);
    if (blk + 1 < nblk) {
      TPA_PF32_STORE(lds + ((blk + 1) & 1) * TILE, lds + (2 + ((blk + 1) & 1)) * TILE, k0 + BN);
      if (blk + 2 < nblk) TPA_PF32_LOAD((int)k0 + 2 * BN);
    }
    __syncthreads();
  }

#undef TPA_PF32_LOAD
#undef TPA_PF32_STORE

  // ---- normalise and store: value e of tile (qt, dt) is d = 32*dt + 8*(e/4)
  //      + 4*lh + e%4 of query l32; its two lanes (l32, l32 + 32) hold the
  //      halves of its row sum
  bf16_t* out = reinterpret_cast<bf16_t*>(a.out);
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(lsum[qt]), __float_as_uint(lsum[qt]), false,
                                                     false);
    const float lrow = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    const float inv = a.v_scale / lrow;
    const int64_t s = q0 + 32 * QT * wave + 32 * qt + l32;
    if (s < a.S) {
      bf16_t* orow = out + ((b * a.S + s) * h + hh) * (int64_t)DH;
#pragma unroll
      for (int dt = 0; dt < 2; ++dt)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x16_t o = oacc[qt][dt];
          const uint2 w = make_uint2(pack_bf16x2(o[4 * g] * inv, o[4 * g + 1] * inv),
                                     pack_bf16x2(o[4 * g + 2] * inv, o[4 * g + 3] * inv));
          *reinterpret_cast<uint2*>(orow + dt * 32 + 8 * g + 4 * lh) = w;
        }
    }
  }
}

// LDS a workgroup may allocate on the current device.
static size_t lds_per_block32() {
  int dev = 0, v = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess) return 0;
  return (size_t)v;
}

bool prefill_mfma32_supported(int dtype, const AttnArgs& a) {
  if (dtype != kBF16 || a.d_h != 64) return false;
  if (a.rk != a.rv || !(a.rk == 1 || a.rk == 2 || a.rk == 4)) return false;
  if (Pf32Cfg<4>::kLds > lds_per_block32() || Pf32Cfg<2>::kLds > lds_per_block32()) return false;
  constexpr int bm = Pf32Cfg<2>::BM;
  if ((a.S + bm - 1) / bm * (int64_t)a.h * a.n_batch >= ((int64_t)1 << 31)) return false;
  // key indices, and a block's first key plus its width, stay 32-bit
  if (a.start_pos + a.S > ((int64_t)1 << 31) - 256) return false;
  const void* ptrs[4] = {a.b_q, a.c_bk, a.c_bv, a.out};   // read/written 8 or 16 bytes at a time
  for (int i = 0; i < 4; ++i)
    if (((uintptr_t)ptrs[i]) % 16) return false;
  return true;
}

// K and V of every (sequence, head) and key 0 .. T-1, formed once:
// km[b][h][t][:] = bf16(sum_r A_K[b,t,h,r] B~_K[b,t,r,:]) and vm likewise, the
// same arithmetic and rounding as the rebuild in LDS.  One thread per (group
// of kMatHeads heads, key, 8-wide slice) of sequence blockIdx.y, group-major:
// a thread loads the key's dim-factor slices once for its heads, and a wave's
// stores for one head are 1 KB runs.
constexpr int kMatHeads = 4;

// SHARED: the shared-basis cache (c_bk / c_bv are the bases); each key is
// rotated at its own position after the rank sum, as the shared rebuild does.
template <int R, bool SHARED>
__global__ void __launch_bounds__(256) kv_material32_kernel(AttnArgs a, int64_t T, bf16_t* km, bf16_t* vm,
                                                            RopeTable tab) {
  typedef typename RankWordP<R>::type W;
  __shared__ double s_rev[SHARED ? 32 : 1];   // d_h = 64: 32 rotary pairs
  if constexpr (SHARED) {
    rope_stage(tab, 32, s_rev);
    __syncthreads();
  }
  const int h = a.h;
  const int i = (int)(blockIdx.x * 256 + threadIdx.x);
  const int T32 = (int)T, groups = (h + kMatHeads - 1) / kMatHeads;
  if ((int64_t)i >= T * 8 * groups) return;
  const int64_t b = blockIdx.y;
  const int slice = i & 7, r = i >> 3;
  const int t = r % T32, h0 = (r / T32) * kMatHeads;
  const int64_t row = b * a.max_seq + t;
  const int64_t brow = SHARED ? 0 : row;   // the shared bases have one row
  uint4 bk[R], bv[R];
#pragma unroll
  for (int q = 0; q < R; ++q) {
    bk[q] = *reinterpret_cast<const uint4*>(reinterpret_cast<const bf16_t*>(a.c_bk) + (brow * R + q) * 64 + slice * 8);
    bv[q] = *reinterpret_cast<const uint4*>(reinterpret_cast<const bf16_t*>(a.c_bv) + (brow * R + q) * 64 + slice * 8);
  }
  float cs[4], sn[4];
  if constexpr (SHARED) {
#pragma unroll
    for (int q = 0; q < 4; ++q) rope_cos_sin(s_rev, t, 4 * slice + q, cs[q], sn[q]);
  }
  const bf16_t* ak = reinterpret_cast<const bf16_t*>(a.c_ak) + row * h * R;
  const bf16_t* av = reinterpret_cast<const bf16_t*>(a.c_av) + row * h * R;
  const int64_t hstride = T * 64;
  bf16_t* ko = km + b * h * hstride + (int64_t)t * 64 + slice * 8;
  bf16_t* vo = vm + b * h * hstride + (int64_t)t * 64 + slice * 8;
#pragma unroll
  for (int j = 0; j < kMatHeads; ++j) {
    const int hh = h0 + j;
    if (hh < h) {
      float kv[8], vv[8];
      factor_combine<R>(*reinterpret_cast<const W*>(ak + hh * R), bk, kv);
      factor_combine<R>(*reinterpret_cast<const W*>(av + hh * R), bv, vv);
      if constexpr (SHARED) {
#pragma unroll
        for (int q = 0; q < 4; ++q) rotate_pair(kv[2 * q], kv[2 * q + 1], cs[q], sn[q]);
      }
      *reinterpret_cast<bf16x8_t*>(ko + hh * hstride) = pack8(kv);
      *reinterpret_cast<bf16x8_t*>(vo + hh * hstride) = pack8(vv);
    }
  }
}

// Pairs per group for the materialised order: the largest divisor of an XCD's
// pair count whose group holds at most about two rounds of the XCD's resident
// workgroups (32 CUs x 2), at least 1.
static int material_group(int64_t pairs, int nqb) {
  if (pairs % 8) return 0;
  const int64_t per_xcd = pairs / 8, budget = 128;
  int64_t g = budget / nqb < 1 ? 1 : budget / nqb;
  if (g > per_xcd) g = per_xcd;
  while (per_xcd % g) --g;
  return (int)g;
}

template <int SRC>
static hipError_t launch_pf32(const AttnArgs& a, const RopeTable& tab, const bf16_t* kmat, const bf16_t* vmat,
                              int64_t mat_len, hipStream_t st) {
  constexpr int bm = Pf32Cfg<2>::BM;
  const int nqb = (int)((a.S + bm - 1) / bm);
  const dim3 grid((unsigned)((int64_t)nqb * a.h * a.n_batch));
  const int grp = SRC == kFromMaterial ? material_group((int64_t)a.h * a.n_batch, nqb) : 0;
  if (SRC == kFromMaterial || a.rk == 2)
    hipLaunchKernelGGL((prefill_mfma32_kernel<2, SRC>), grid, dim3(Pf32Cfg<2>::NT), (Pf32Cfg<2>::kLds), st, a, nqb,
                       tab, kmat, vmat, mat_len, grp);
  else if (a.rk == 1)
    hipLaunchKernelGGL((prefill_mfma32_kernel<1, SRC == kFromMaterial ? kFromFactors : SRC>), grid,
                       dim3(Pf32Cfg<1>::NT), (Pf32Cfg<1>::kLds), st, a, nqb, tab, kmat, vmat, mat_len, grp);
  else
    hipLaunchKernelGGL((prefill_mfma32_kernel<4, SRC == kFromMaterial ? kFromFactors : SRC>), grid,
                       dim3(Pf32Cfg<4>::NT), (Pf32Cfg<4>::kLds), st, a, nqb, tab, kmat, vmat, mat_len, grp);
  return hipGetLastError();
}

hipError_t launch_prefill_mfma32(const AttnArgs& a, hipStream_t st) {
  static const RopeTable unused = {};
  return launch_pf32<kFromFactors>(a, unused, nullptr, nullptr, 0, st);
}

hipError_t launch_prefill_mfma32_shared(const AttnArgs& a, const RopeTable& tab, hipStream_t st) {
  return launch_pf32<kFromSharedBasis>(a, tab, nullptr, nullptr, 0, st);
}

// The shapes the workspace path takes, from sizes alone (no device or pointer
// checks: the workspace is sized and validated by these).
bool prefill_material_shape_ok(int dtype, const AttnArgs& a) {
  if (dtype != kBF16 || a.d_h != 64) return false;
  if (a.rk != a.rv || !(a.rk == 1 || a.rk == 2 || a.rk == 4)) return false;
  constexpr int bm = Pf32Cfg<2>::BM;
  if ((a.S + bm - 1) / bm * (int64_t)a.h * a.n_batch >= ((int64_t)1 << 31)) return false;
  // the materialising kernel indexes (key, head, slice) of a sequence in 32 bits
  return (a.start_pos + a.S) * a.h * 8 < ((int64_t)1 << 31) - 256;
}

bool prefill_material_supported(int dtype, const AttnArgs& a) {
  return prefill_material_shape_ok(dtype, a) && prefill_mfma32_supported(dtype, a);
}

size_t prefill_material_bytes(const AttnArgs& a) {
  return (size_t)2 * a.n_batch * a.h * (a.start_pos + a.S) * 64 * sizeof(bf16_t);
}

template <bool SHARED>
static void launch_material(const AttnArgs& a, int64_t T, bf16_t* km, bf16_t* vm, const RopeTable& tab,
                            hipStream_t st) {
  const int64_t groups = (a.h + kMatHeads - 1) / kMatHeads;
  const dim3 mgrid((unsigned)((T * 8 * groups + 255) / 256), (unsigned)a.n_batch);
  if (a.rk == 1)
    hipLaunchKernelGGL((kv_material32_kernel<1, SHARED>), mgrid, dim3(256), 0, st, a, T, km, vm, tab);
  else if (a.rk == 2)
    hipLaunchKernelGGL((kv_material32_kernel<2, SHARED>), mgrid, dim3(256), 0, st, a, T, km, vm, tab);
  else
    hipLaunchKernelGGL((kv_material32_kernel<4, SHARED>), mgrid, dim3(256), 0, st, a, T, km, vm, tab);
}

// tab: the rotary table for a shared-basis cache, nullptr for the standard one.
hipError_t launch_prefill_material(const AttnArgs& a, void* ws, const RopeTable* tab, hipStream_t st) {
  const int64_t T = a.start_pos + a.S;
  bf16_t* km = reinterpret_cast<bf16_t*>(ws);
  bf16_t* vm = km + a.n_batch * a.h * T * 64;
  static const RopeTable unused = {};
  if (tab)
    launch_material<true>(a, T, km, vm, *tab, st);
  else
    launch_material<false>(a, T, km, vm, unused, st);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_pf32<kFromMaterial>(a, unused, km, vm, T, st);
}

}  // namespace tpa
