// Backward of the prefill attention on the matrix cores (bf16 operands, fp32
// accumulation; d_h = 64 or 128).  Same gradient as the general kernels
// ("Tensor Product Attention Is All You Need" review on coreui.cn: the Q_t/K_t/
// V_t equations of 核心机制总结 and the masked softmax attention of the code
// walk-through 前向传播, differentiated by the chain rule):
//   dV = P^T dO,  dP = dO V^T,  dS = P * (dP - D),  dK = dS^T Q,  dQ = dS K,
// in the base-2 units of the forward (q^ carries log2(e) / (R_Q R_K sqrt(d_h)),
// k^ = sum_r A_K B~_K and v^ = sum_r A_V B_V carry no 1/R).
//
// Precision.  The gradients cancel strongly (every row of dS sums to zero), so
// plain bf16 operands lose too much: the scores take q^ and k^ as bf16 hi + lo
// pairs (x = hi + lo to 2^-17 relative; three products hi*hi + lo*hi + hi*lo),
// and D is formed from the statistics pass's own fp32 O (built from the same
// bf16 v^ that dP uses and normalised by the sum of the same bf16 p), which
// keeps sum_t P_t dP_t = D, not from a bf16-rounded output.  v^, dO, P and dS,
// and q^ and k^ where they multiply dS, enter their products as plain bf16:
// pairs there as well bought about a third of the remaining error for four
// more products per tile, and the 5e-3 relative L2 bound holds without them.
//
// Passes (all deterministic):
//  1. rebuild: q^ (hi, lo) of every query, k^ (hi, lo) and v^ of every key,
//     [B, *, h, d_h] (the lo halves serve the score products only);
//  2. statistics, per query block: lse (base 2, fp32 row sums), D;
//  3. dK, dV: a workgroup owns 64 (d_h = 64: 128) keys of one head, each wave
//     16 KW of them with k^ and v^ in registers.  32-query tiles stream through
//     LDS, row-major and transposed, double-buffered; a wave forms S = q^ k^T
//     and dP = dO v^T (queries down the lane groups, its keys across the lanes),
//     then P and dS, whose output registers are directly the B operands of
//     dV^T += dO^T P and dK^T += q^T dS (k-slot j of lane group g is query 4g+j
//     of the first 16-query tile for j<4, of the second for j>=4; the matching
//     transposed rows are two 8-byte LDS reads);
//  4. dQ, per query block of 128 (32 per wave, q^ and dO in registers): 32-key
//     tiles stream through LDS as k^, v^ row-major and k^ transposed; S^T and
//     dP^T put one query per lane, and dQ^T += k^T dS^T takes the dS^T
//     registers as its B operand.
// The epilogues of 3 and 4 also form each head's factor gradients
// dA[t, h, r] = (1/R) dX[t, h, :] . B[t, r, :] from the registers; pass 5 forms
// the dim-factor gradients, which sum over the heads, per token.
#include "kernels.h"
#include "mfma.h"

namespace tpa {

// x = hi + lo, both bf16 (round to nearest even each time).
__device__ __forceinline__ void split8(const float (&x)[8], bf16x8_t& hi, bf16x8_t& lo) {
  float h[8], l[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    h[j] = bf16_to_f32(f32_to_bf16(x[j]));
    l[j] = x[j] - h[j];
  }
  hi = pack8(h);
  lo = pack8(l);
}

// ---- pass 1: q^ (hi, lo), k^ (hi, lo), v^ ----------------------------------------
// One thread per (sequence, token, head, 8-wide d slice): the S query tokens
// first, then the n_keys key tokens.  fp32 sums.
__global__ void __launch_bounds__(256) bwd_rebuild_kernel(AttnArgs a, BwdArgs g, int64_t n_keys) {
  const int h = a.h, dh = a.d_h, slices = dh / 8;
  const int64_t nq = a.n_batch * a.S * h * slices;
  const int64_t total = nq + a.n_batch * n_keys * h * slices;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const bool is_q = idx < nq;
    const int64_t j = is_q ? idx : idx - nq;
    const int c = (int)(j % slices);
    const int64_t r = j / slices;   // (b * n + t) * h + hh, n = S or n_keys
    const int hh = (int)(r % h);
    const int64_t bt = r / h;
    const int64_t n = is_q ? a.S : n_keys;
    const int64_t b = bt / n, t = bt - b * n;
    float x[8], y[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = y[e] = 0.f;
    bf16x8_t hi, lo;
    if (is_q) {
      const bf16_t* AQ = reinterpret_cast<const bf16_t*>(a.a_q);
      const bf16_t* BQ = reinterpret_cast<const bf16_t*>(a.b_q);
      const int64_t tok = b * a.q_bstride_tok + t;
      if (a.rq == 0) {
        const bf16x8_t e8 = as_bf16x8(*reinterpret_cast<const uint4*>(BQ + (tok * h + hh) * dh + 8 * c));
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = (float)e8[e];
      } else {
        for (int q = 0; q < a.rq; ++q) {
          const float ar = bf16_to_f32(AQ[(tok * h + hh) * a.rq + q]);
          const bf16x8_t e8 = as_bf16x8(*reinterpret_cast<const uint4*>(BQ + (tok * a.rq + q) * dh + 8 * c));
#pragma unroll
          for (int e = 0; e < 8; ++e) x[e] = fmaf(ar, (float)e8[e], x[e]);
        }
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] *= a.q_scale;
      split8(x, hi, lo);
      *reinterpret_cast<bf16x8_t*>(g.q_hi + r * dh + 8 * c) = hi;
      *reinterpret_cast<bf16x8_t*>(g.q_lo + r * dh + 8 * c) = lo;
    } else {
      const bf16_t* AK = reinterpret_cast<const bf16_t*>(a.c_ak);
      const bf16_t* BK = reinterpret_cast<const bf16_t*>(a.c_bk);
      const bf16_t* AV = reinterpret_cast<const bf16_t*>(a.c_av);
      const bf16_t* BV = reinterpret_cast<const bf16_t*>(a.c_bv);
      const int64_t row = b * a.max_seq + t;
      for (int q = 0; q < a.rk; ++q) {
        const float ar = bf16_to_f32(AK[(row * h + hh) * a.rk + q]);
        const bf16x8_t e8 = as_bf16x8(*reinterpret_cast<const uint4*>(BK + (row * a.rk + q) * dh + 8 * c));
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = fmaf(ar, (float)e8[e], x[e]);
      }
      for (int q = 0; q < a.rv; ++q) {
        const float ar = bf16_to_f32(AV[(row * h + hh) * a.rv + q]);
        const bf16x8_t e8 = as_bf16x8(*reinterpret_cast<const uint4*>(BV + (row * a.rv + q) * dh + 8 * c));
#pragma unroll
        for (int e = 0; e < 8; ++e) y[e] = fmaf(ar, (float)e8[e], y[e]);
      }
      split8(x, hi, lo);
      *reinterpret_cast<bf16x8_t*>(g.k_hi + r * dh + 8 * c) = hi;
      *reinterpret_cast<bf16x8_t*>(g.k_lo + r * dh + 8 * c) = lo;
      *reinterpret_cast<bf16x8_t*>(g.v_hat + r * dh + 8 * c) = pack8(y);
    }
  }
}

// ---- LDS staging helpers -------------------------------------------------------
// Staged rows are held as native 4 x u32 vectors (HIP's uint4 is a struct,
// which the compiler may keep in scratch memory when selected or passed around).
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32x4_t ld16(const bf16_t* p) { return *reinterpret_cast<const u32x4_t*>(p); }

// Pairs element j of two 8-element bf16 rows into one 32-bit word (row a low).
__device__ __forceinline__ uint32_t pair_elem(u32x4_t a, u32x4_t b, int j) {
  return (j & 1) ? __builtin_amdgcn_perm(b[j >> 1], a[j >> 1], 0x07060302u)
                 : __builtin_amdgcn_perm(b[j >> 1], a[j >> 1], 0x05040100u);
}

// Rows `row`, `row`+1 (8-wide slice at column d0) into a row-major tile.
__device__ __forceinline__ void put_rows(u32x4_t r0, u32x4_t r1, bf16_t* tile, int ld, int row, int d0) {
  *reinterpret_cast<u32x4_t*>(tile + row * ld + d0) = r0;
  *reinterpret_cast<u32x4_t*>(tile + (row + 1) * ld + d0) = r1;
}

// The same two rows into a transposed tile (column `row`, `row`+1 of rows d0..d0+7).
__device__ __forceinline__ void put_tr(u32x4_t r0, u32x4_t r1, bf16_t* tile, int ld, int row, int d0) {
#pragma unroll
  for (int j = 0; j < 8; ++j) *reinterpret_cast<uint32_t*>(tile + (d0 + j) * ld + row) = pair_elem(r0, r1, j);
}

// A operand of a product contracting over 32 columns c0.. of a transposed
// tile's row: lane (li, lg) takes columns c0 + 4lg .. +3 and c0 + 16 + 4lg .. +3.
__device__ __forceinline__ bf16x8_t tr_operand(const bf16_t* tr_row, int c0, int lg) {
  const uint2 lo = *reinterpret_cast<const uint2*>(tr_row + c0 + 4 * lg);
  const uint2 hi = *reinterpret_cast<const uint2*>(tr_row + c0 + 16 + 4 * lg);
  return as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
}

__device__ __forceinline__ bf16x8_t ld8(const bf16_t* p) { return *reinterpret_cast<const bf16x8_t*>(p); }

// Makes the wave wait here for the loads of a value the tile loop reads.  The
// memory counter is in order, so a wait for such a value inside the loop would
// also hold every iteration until the next tile's staged loads had arrived.
template <typename T>
__device__ __forceinline__ void settle(const T& v) {
  asm volatile("" ::"v"(v));
}

// v where ok, else zeros.
__device__ __forceinline__ u32x4_t keep_if(bool ok, u32x4_t v) {
  const u32x4_t z = {0u, 0u, 0u, 0u};
  return ok ? v : z;
}

// Work item order shared by the passes: blocks of the outer index in the
// given order, (sequence, head) pairs spread evenly over the eight XCDs.
__device__ __forceinline__ void bwd_item(int64_t hb, int h, int& blk, int& hh, int64_t& b) {
  const int64_t L = blockIdx.x;
  blk = (int)(L / hb);
  int64_t u = L % hb;
  if (hb % 8 == 0) u = (u & 7) * (hb >> 3) + (u >> 3);
  hh = (int)(u % h);
  b = u / h;
}

// dA[r] = (1/R) sum_d x[d] Bm[r][d] for the row whose d = 16dt + 4lg + i values
// (i < 4, dt < DH/16) this lane holds in acc[dt][col] (the lane's 16-lane
// column); the four lane groups are summed, lane group 0 stores when ok.
template <int DH, int NC>
__device__ __forceinline__ void head_factor_grad(const f32x4_t (&acc)[DH / 16][NC], int col, const bf16_t* Bm, int R,
                                                 int lg, bool ok, float* dA) {
  const float inv_r = 1.f / (float)R;
  for (int r = 0; r < R; ++r) {
    float part = 0.f;
#pragma unroll
    for (int dt = 0; dt < DH / 16; ++dt) {
      const uint2 w = *reinterpret_cast<const uint2*>(Bm + r * DH + 16 * dt + 4 * lg);
      part = fmaf(acc[dt][col][0], __uint_as_float(w.x << 16), part);
      part = fmaf(acc[dt][col][1], __uint_as_float(w.x & 0xffff0000u), part);
      part = fmaf(acc[dt][col][2], __uint_as_float(w.y << 16), part);
      part = fmaf(acc[dt][col][3], __uint_as_float(w.y & 0xffff0000u), part);
    }
    part = lane_group_sum(part);
    if (ok && lg == 0) dA[r] = part * inv_r;
  }
}

// ---- pass 3: dK and dV --------------------------------------------------------------
template <int DH>
struct BwdKvCfg {
  static constexpr int KW = DH == 64 ? 2 : 1;   // 16-key tiles per wave
  static constexpr int BN = 64 * KW;            // keys per workgroup
  static constexpr int BQ = 32;                 // queries per staged tile
  static constexpr int KS = DH / 32;            // k-steps over d
  static constexpr int DT = DH / 16;            // d tiles of dK^T, dV^T
  static constexpr int LDR = DH + 8;            // row-major tile stride (bf16)
  static constexpr int LDT = BQ + 4;            // transposed tile stride (bf16)
  static constexpr int ROWT = BQ * LDR;
  static constexpr int TRT = DH * LDT;
  // q^ hi, q^ lo, dO row-major; q^ hi and dO transposed; lse and D (2 x BQ floats)
  static constexpr int BUF = 3 * ROWT + 2 * TRT + 4 * BQ;
  static constexpr int NP = DH / 8;             // 8-wide slices per row
  static constexpr int ITEMS = (BQ / 2) * NP;   // staging items (row pairs x slices)
  static constexpr size_t kLds = (size_t)2 * BUF * sizeof(bf16_t);
  static_assert(ITEMS % 64 == 0 && ITEMS <= 256, "staging by whole waves");
};

// Rows past the last query are loaded clamped and zeroed only when stored, so
// that nothing consumes the loads before the next tile's store: their latency
// then overlaps a whole tile of products.
struct KvStage {
  u32x4_t qh0, qh1, ql0, ql1, o0, o1;
  float lse, dv;
  bool ok0, ok1, ok;
};

template <int DH>
__device__ __forceinline__ void kv_stage_load(KvStage& r, const AttnArgs& a, const BwdArgs& g, int64_t b, int hh,
                                              int64_t s0) {
  using C = BwdKvCfg<DH>;
  if (threadIdx.x < C::ITEMS) {
    const int c = threadIdx.x % C::NP, p = threadIdx.x / C::NP;
    const bf16_t* dO = reinterpret_cast<const bf16_t*>(g.dout);
    const int64_t s = s0 + 2 * p;
    const bool ok0 = s < a.S, ok1 = s + 1 < a.S;
    const int64_t off0 = ((b * a.S + (ok0 ? s : a.S - 1)) * a.h + hh) * (int64_t)DH + 8 * c;
    const int64_t off1 = ((b * a.S + (ok1 ? s + 1 : a.S - 1)) * a.h + hh) * (int64_t)DH + 8 * c;
    r.qh0 = ld16(g.q_hi + off0);
    r.qh1 = ld16(g.q_hi + off1);
    r.ql0 = ld16(g.q_lo + off0);
    r.ql1 = ld16(g.q_lo + off1);
    r.o0 = ld16(dO + off0);
    r.o1 = ld16(dO + off1);
    r.ok0 = ok0;
    r.ok1 = ok1;
  }
  if (threadIdx.x < C::BQ) {
    const int64_t s = s0 + threadIdx.x;
    const bool ok = s < a.S;
    const int64_t i = (b * a.S + (ok ? s : a.S - 1)) * a.h + hh;
    r.lse = g.lse[i];
    r.dv = g.dvec[i];
    r.ok = ok;
  }
}

template <int DH>
__device__ __forceinline__ void kv_stage_store(const KvStage& r, bf16_t* buf) {
  using C = BwdKvCfg<DH>;
  if (threadIdx.x < C::ITEMS) {
    const int c = threadIdx.x % C::NP, p = threadIdx.x / C::NP;
    const u32x4_t qh0 = keep_if(r.ok0, r.qh0), qh1 = keep_if(r.ok1, r.qh1);
    const u32x4_t ql0 = keep_if(r.ok0, r.ql0), ql1 = keep_if(r.ok1, r.ql1);
    const u32x4_t o0 = keep_if(r.ok0, r.o0), o1 = keep_if(r.ok1, r.o1);
    put_rows(qh0, qh1, buf, C::LDR, 2 * p, 8 * c);
    put_rows(ql0, ql1, buf + C::ROWT, C::LDR, 2 * p, 8 * c);
    put_rows(o0, o1, buf + 2 * C::ROWT, C::LDR, 2 * p, 8 * c);
    bf16_t* tr = buf + 3 * C::ROWT;
    put_tr(qh0, qh1, tr, C::LDT, 2 * p, 8 * c);
    put_tr(o0, o1, tr + C::TRT, C::LDT, 2 * p, 8 * c);
  }
  if (threadIdx.x < C::BQ) {
    float* st = reinterpret_cast<float*>(buf + 3 * C::ROWT + 2 * C::TRT);
    st[threadIdx.x] = r.ok ? r.lse : 0.f;
    st[C::BQ + threadIdx.x] = r.ok ? r.dv : 0.f;
  }
}

template <int DH>
__global__ void __launch_bounds__(256, 2) bwd_dkdv_mfma_kernel(AttnArgs a, BwdArgs g) {
  using C = BwdKvCfg<DH>;
  constexpr int KW = C::KW, BN = C::BN, BQ = C::BQ, KS = C::KS, DT = C::DT, LDR = C::LDR, LDT = C::LDT;
  extern __shared__ __align__(16) unsigned char smem[];
  bf16_t* const lds = reinterpret_cast<bf16_t*>(smem);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int li = lane & 15, lg = lane >> 4;
  const int h = a.h;
  const int64_t n_keys = a.start_pos + a.S;
  // key blocks in increasing order: the first ones see the most queries
  int kb, hh;
  int64_t b;
  bwd_item((int64_t)h * a.n_batch, h, kb, hh, b);
  const int64_t k0 = (int64_t)kb * BN;
  const int64_t kw0 = k0 + 16 * KW * wave;   // this wave's first key
  const bool causal = a.causal != 0;

  // the first query tile that can see the block's first key
  int64_t s_lo = causal ? k0 - a.start_pos : 0;
  s_lo = s_lo > 0 ? (s_lo / BQ) * BQ : 0;
  const int ntiles = (int)((a.S - s_lo + BQ - 1) / BQ);

  KvStage sr;
  kv_stage_load<DH>(sr, a, g, b, hh, s_lo);

  // k^ (hi, lo), v^ of this wave's keys as B operands: lane (key li of tile kt, d 32ks + 8lg ..)
  bf16x8_t kh[KW][KS], kl[KW][KS], vo[KW][KS];
#pragma unroll
  for (int kt = 0; kt < KW; ++kt) {
    int64_t t = kw0 + 16 * kt + li;
    t = t < n_keys ? t : n_keys - 1;   // outputs of keys past the end are not stored
    const int64_t off = ((b * n_keys + t) * h + hh) * (int64_t)DH + 8 * lg;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      kh[kt][ks] = ld8(g.k_hi + off + 32 * ks);
      kl[kt][ks] = ld8(g.k_lo + off + 32 * ks);
      vo[kt][ks] = ld8(g.v_hat + off + 32 * ks);
    }
  }
  f32x4_t dk[DT][KW], dv[DT][KW];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int kt = 0; kt < KW; ++kt) dk[dt][kt] = dv[dt][kt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const float inv_rv = 1.f / (float)a.rv;

  kv_stage_store<DH>(sr, lds);
#pragma unroll
  for (int kt = 0; kt < KW; ++kt)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      settle(kh[kt][ks]);
      settle(kl[kt][ks]);
      settle(vo[kt][ks]);
    }
  if (ntiles > 1) kv_stage_load<DH>(sr, a, g, b, hh, s_lo + BQ);
  __syncthreads();
  for (int tile = 0; tile < ntiles; ++tile) {
    const bf16_t* buf = lds + (tile & 1) * C::BUF;
    const bf16_t* tr = buf + 3 * C::ROWT;
    const float* st = reinterpret_cast<const float*>(tr + 2 * C::TRT);
    const int64_t s0 = s_lo + (int64_t)tile * BQ;
    const int64_t pos0 = a.start_pos + s0;
    // wave-uniform skip: every key of the wave after every query of the tile
    if (!(causal && kw0 > pos0 + BQ - 1)) {
      f32x4_t sacc[2][KW], pacc[2][KW];
#pragma unroll
      for (int q2 = 0; q2 < 2; ++q2) {
        bf16x8_t qa[KS], qb[KS], oa[KS];
        const int rofs = (16 * q2 + li) * LDR + 8 * lg;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          qa[ks] = ld8(buf + rofs + 32 * ks);
          qb[ks] = ld8(buf + C::ROWT + rofs + 32 * ks);
          oa[ks] = ld8(buf + 2 * C::ROWT + rofs + 32 * ks);
        }
#pragma unroll
        for (int kt = 0; kt < KW; ++kt) {
          f32x4_t s = {0.f, 0.f, 0.f, 0.f}, p = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) {
            s = mfma_bf16(qa[ks], kh[kt][ks], s);
            s = mfma_bf16(qb[ks], kh[kt][ks], s);
            s = mfma_bf16(qa[ks], kl[kt][ks], s);
            p = mfma_bf16(oa[ks], vo[kt][ks], p);
          }
          sacc[q2][kt] = s;
          pacc[q2][kt] = p;
        }
      }
      // P and dS: lane holds queries 16q2 + 4lg + i of the tile against key 16kt + li
      const bool need_mask = causal && kw0 + 16 * KW - 1 > pos0;
      bf16x8_t pop[KW], dsh[KW];
#pragma unroll
      for (int kt = 0; kt < KW; ++kt) {
        float pv[8], dsv[8];
#pragma unroll
        for (int q2 = 0; q2 < 2; ++q2) {
          const float4 l4 = *reinterpret_cast<const float4*>(st + 16 * q2 + 4 * lg);
          const float4 d4 = *reinterpret_cast<const float4*>(st + BQ + 16 * q2 + 4 * lg);
          const float lse[4] = {l4.x, l4.y, l4.z, l4.w};
          const float dd[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float p = fast_exp2(sacc[q2][kt][i] - lse[i]);
            if (need_mask) {
              const int64_t t = kw0 + 16 * kt + li;
              p = t <= pos0 + 16 * q2 + 4 * lg + i ? p : 0.f;
            }
            pv[4 * q2 + i] = p;
            dsv[4 * q2 + i] = p * (pacc[q2][kt][i] * inv_rv - dd[i]);
          }
        }
        pop[kt] = pack8(pv);
        dsh[kt] = pack8(dsv);
      }
      // dV^T += dO^T P,  dK^T += q^T dS  (both plain bf16)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const int tofs = (16 * dt + li) * LDT;
        const bf16x8_t qa = tr_operand(tr + tofs, 0, lg);
        const bf16x8_t oa = tr_operand(tr + C::TRT + tofs, 0, lg);
#pragma unroll
        for (int kt = 0; kt < KW; ++kt) {
          dv[dt][kt] = mfma_bf16(oa, pop[kt], dv[dt][kt]);
          dk[dt][kt] = mfma_bf16(qa, dsh[kt], dk[dt][kt]);
        }
      }
    }
    if (tile + 1 < ntiles) {
      kv_stage_store<DH>(sr, lds + ((tile + 1) & 1) * C::BUF);
      if (tile + 2 < ntiles) kv_stage_load<DH>(sr, a, g, b, hh, s0 + 2 * BQ);
    }
    __syncthreads();
  }

  // lane holds d = 16dt + 4lg + i of key 16kt + li.  dK = dS^T Q / sqrt(d_h)
  // with Q = q^ R_K sqrt(d_h) / log2(e).
  const float kscale = (float)a.rk / kLog2e;
#pragma unroll
  for (int kt = 0; kt < KW; ++kt) {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) dk[dt][kt] *= kscale;
    const int64_t t = kw0 + 16 * kt + li;
    const bool ok = t < n_keys;
    const int64_t tc = ok ? t : n_keys - 1;
    // this head's factor gradients dA[t, h, r] = (1/R) dX[t, h, :] . B[t, r, :]
    head_factor_grad<DH>(dk, kt, reinterpret_cast<const bf16_t*>(a.c_bk) + (b * a.max_seq + tc) * a.rk * DH, a.rk,
                         lg, ok, g.d_ak + ((b * g.dkv_max_seq + tc) * h + hh) * a.rk);
    head_factor_grad<DH>(dv, kt, reinterpret_cast<const bf16_t*>(a.c_bv) + (b * a.max_seq + tc) * a.rv * DH, a.rv,
                         lg, ok, g.d_av + ((b * g.dkv_max_seq + tc) * h + hh) * a.rv);
    if (!ok) continue;
    const int64_t o = ((b * n_keys + t) * h + hh) * (int64_t)DH + 4 * lg;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      *reinterpret_cast<float4*>(g.dk + o + 16 * dt) =
          make_float4(dk[dt][kt][0], dk[dt][kt][1], dk[dt][kt][2], dk[dt][kt][3]);
      *reinterpret_cast<float4*>(g.dv + o + 16 * dt) =
          make_float4(dv[dt][kt][0], dv[dt][kt][1], dv[dt][kt][2], dv[dt][kt][3]);
    }
  }
}

// ---- passes 2 and 4: per query block (statistics; dQ) ------------------------------
template <int DH, bool STATS>
struct BwdQCfg {
  static constexpr int QT = (DH == 128 && !STATS) ? 1 : 2;   // 16-query tiles per wave
  static constexpr int BM = 64 * QT;             // queries per workgroup
  static constexpr int BN = 32;                  // keys per staged tile
  static constexpr int KT = BN / 16;
  static constexpr int KS = DH / 32;
  static constexpr int DT = DH / 16;
  static constexpr int LDR = DH + 8;
  static constexpr int LDT = BN + 4;
  static constexpr int ROWT = BN * LDR;
  static constexpr int TRT = DH * LDT;
  // statistics: k^ hi, lo row-major, v^ transposed with a ones row (DH + 16 rows);
  // dQ: k^ hi, lo, v^ row-major, k^ hi transposed
  static constexpr int BUF = STATS ? 2 * ROWT + (DH + 16) * LDT : 3 * ROWT + TRT;
  static constexpr int NP = DH / 8;
  static constexpr int ITEMS = (BN / 2) * NP;
  static constexpr size_t kLds = (size_t)2 * BUF * sizeof(bf16_t);
  static constexpr float kRescaleSlack = 8.f;    // log2 units
  static_assert(ITEMS % 64 == 0 && ITEMS <= 256, "staging by whole waves");
};

struct QStage {
  u32x4_t kh0, kh1, kl0, kl1, v0, v1;
};

template <int DH, bool STATS>
__device__ __forceinline__ void q_stage_load(QStage& r, const BwdArgs& g, int64_t b, int hh, int h, int64_t n_keys,
                                             int64_t k0) {
  using C = BwdQCfg<DH, STATS>;
  if (threadIdx.x >= C::ITEMS) return;
  const int c = threadIdx.x % C::NP, p = threadIdx.x / C::NP;
  int64_t t0 = k0 + 2 * p, t1 = t0 + 1;
  t0 = t0 < n_keys ? t0 : n_keys - 1;   // keys past the end are masked out of every score
  t1 = t1 < n_keys ? t1 : n_keys - 1;
  const int64_t off0 = ((b * n_keys + t0) * h + hh) * (int64_t)DH + 8 * c;
  const int64_t off1 = ((b * n_keys + t1) * h + hh) * (int64_t)DH + 8 * c;
  r.kh0 = ld16(g.k_hi + off0);
  r.kh1 = ld16(g.k_hi + off1);
  r.kl0 = ld16(g.k_lo + off0);
  r.kl1 = ld16(g.k_lo + off1);
  r.v0 = ld16(g.v_hat + off0);
  r.v1 = ld16(g.v_hat + off1);
}

template <int DH, bool STATS>
__device__ __forceinline__ void q_stage_store(const QStage& r, bf16_t* buf) {
  using C = BwdQCfg<DH, STATS>;
  if (threadIdx.x >= C::ITEMS) return;
  const int c = threadIdx.x % C::NP, p = threadIdx.x / C::NP;
  put_rows(r.kh0, r.kh1, buf, C::LDR, 2 * p, 8 * c);
  put_rows(r.kl0, r.kl1, buf + C::ROWT, C::LDR, 2 * p, 8 * c);
  if constexpr (STATS) {
    put_tr(r.v0, r.v1, buf + 2 * C::ROWT, C::LDT, 2 * p, 8 * c);
  } else {
    put_rows(r.v0, r.v1, buf + 2 * C::ROWT, C::LDR, 2 * p, 8 * c);
    put_tr(r.kh0, r.kh1, buf + 3 * C::ROWT, C::LDT, 2 * p, 8 * c);
  }
}

template <int DH, bool STATS>
__global__ void __launch_bounds__(256, 2) bwd_query_mfma_kernel(AttnArgs a, BwdArgs g, int n_qblocks) {
  using C = BwdQCfg<DH, STATS>;
  constexpr int QT = C::QT, BM = C::BM, BN = C::BN, KT = C::KT, KS = C::KS, DT = C::DT;
  constexpr int LDR = C::LDR, LDT = C::LDT;
  // dQ at d_h = 64 reads its k^T operands ahead of the dS step (221 registers);
  // in the statistics pass the extra registers would cost the third wave per
  // SIMD, which is worth more there than the early reads
  constexpr bool kEarlyT = DH == 64 && !STATS;
  extern __shared__ __align__(16) unsigned char smem[];
  bf16_t* const lds = reinterpret_cast<bf16_t*>(smem);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int li = lane & 15, lg = lane >> 4;
  const int h = a.h;
  const int64_t n_keys = a.start_pos + a.S;
  int L, hh;
  int64_t b;
  bwd_item((int64_t)h * a.n_batch, h, L, hh, b);
  const int qb = n_qblocks - 1 - L;   // heaviest first
  const int64_t q0 = (int64_t)qb * BM;
  const int64_t last_q = (q0 + BM < a.S ? q0 + BM : a.S) - 1;
  const bool causal = a.causal != 0;
  const int64_t kend = causal ? a.start_pos + last_q + 1 : n_keys;
  const int nblk = (int)((kend + BN - 1) / BN);

  QStage sr;
  q_stage_load<DH, STATS>(sr, g, b, hh, h, n_keys, 0);
  if constexpr (STATS) {
    // the ones row (and fifteen zero rows) below v^T, in both buffers
    for (int i = threadIdx.x; i < 16 * BN; i += blockDim.x) {
      const int rr = i / BN, col = i % BN;
      const bf16_t v = rr == 0 ? (bf16_t)0x3f80 : (bf16_t)0;
      lds[2 * C::ROWT + (DH + rr) * LDT + col] = v;
      lds[C::BUF + 2 * C::ROWT + (DH + rr) * LDT + col] = v;
    }
  }

  // q^ (hi, lo) and dO of this wave's queries as B operands (lane: query li, d 32ks + 8lg ..)
  const bf16_t* dO = reinterpret_cast<const bf16_t*>(g.dout);
  bf16x8_t qh[QT][KS], ql[QT][KS], dop[QT][KS];
  float lse[QT], dd[QT];
  const int64_t sw0 = q0 + 16 * QT * wave;
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    int64_t s = sw0 + 16 * qt + li;
    s = s < a.S ? s : a.S - 1;   // rows past the end are computed but not stored
    const int64_t i = (b * a.S + s) * h + hh;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      qh[qt][ks] = ld8(g.q_hi + i * DH + 32 * ks + 8 * lg);
      ql[qt][ks] = ld8(g.q_lo + i * DH + 32 * ks + 8 * lg);
      if constexpr (!STATS) dop[qt][ks] = ld8(dO + i * DH + 32 * ks + 8 * lg);
    }
    if constexpr (!STATS) {
      lse[qt] = g.lse[i];
      dd[qt] = g.dvec[i];
    }
  }
  // STATS: O^T (DT tiles) and sum_t bf16(p_t) (tile DT, row 0); dQ: dQ^T
  constexpr int NACC = STATS ? DT + 1 : DT;
  f32x4_t acc[QT][NACC];
  float m_run[QT], l_part[QT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    m_run[qt] = -INFINITY;
    l_part[qt] = 0.f;
#pragma unroll
    for (int dt = 0; dt < NACC; ++dt) acc[qt][dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  const float inv_rv = 1.f / (float)a.rv;
  const int64_t wpos0 = a.start_pos + sw0;   // first position of this wave's queries

  q_stage_store<DH, STATS>(sr, lds);
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      settle(qh[qt][ks]);
      settle(ql[qt][ks]);
      if constexpr (!STATS) settle(dop[qt][ks]);
    }
    if constexpr (!STATS) {
      settle(lse[qt]);
      settle(dd[qt]);
    }
  }
  if (nblk > 1) q_stage_load<DH, STATS>(sr, g, b, hh, h, n_keys, BN);
  __syncthreads();
  for (int blk = 0; blk < nblk; ++blk) {
    const bf16_t* buf = lds + (blk & 1) * C::BUF;
    const int64_t k0 = (int64_t)blk * BN;
    // wave-uniform skip: every key of the block after every query of the wave
    if (!(causal && k0 > wpos0 + 16 * QT - 1) && sw0 < a.S) {
      // S^T (and dP^T): lane holds keys k0 + 16kt + 4lg + i of query 16qt + li
      f32x4_t sacc[KT][QT], pacc[KT][QT];
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) {
        bf16x8_t ka[KS], kb[KS], va[KS];
        const int rofs = (16 * kt + li) * LDR + 8 * lg;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          ka[ks] = ld8(buf + rofs + 32 * ks);
          kb[ks] = ld8(buf + C::ROWT + rofs + 32 * ks);
          if constexpr (!STATS) va[ks] = ld8(buf + 2 * C::ROWT + rofs + 32 * ks);
        }
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) {
          f32x4_t s = {0.f, 0.f, 0.f, 0.f}, p = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) {
            s = mfma_bf16(ka[ks], qh[qt][ks], s);
            s = mfma_bf16(kb[ks], qh[qt][ks], s);
            s = mfma_bf16(ka[ks], ql[qt][ks], s);
            if constexpr (!STATS) p = mfma_bf16(va[ks], dop[qt][ks], p);
          }
          sacc[kt][qt] = s;
          pacc[kt][qt] = p;
        }
      }
      // the transposed operands of the second product (statistics: v^T with its
      // ones row; dQ: k^T hi), read now so the elementwise step hides their
      // latency
      constexpr int NE = !kEarlyT ? 1 : STATS ? DT + 1 : DT;
      bf16x8_t tre[NE];
      if constexpr (kEarlyT) {
#pragma unroll
        for (int e = 0; e < NE; ++e) {
          const int dt = e;
          const bf16_t* base = STATS ? buf + 2 * C::ROWT : buf + 3 * C::ROWT;
          tre[e] = tr_operand(base + (16 * dt + li) * LDT, 0, lg);
        }
      }
      const bool need_mask = (causal && k0 + BN - 1 > wpos0) || (k0 + BN > kend);
      if (need_mask) {
#pragma unroll
        for (int kt = 0; kt < KT; ++kt)
#pragma unroll
          for (int qt = 0; qt < QT; ++qt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int64_t t = k0 + 16 * kt + 4 * lg + i;
              const bool ok = t < kend && (!causal || t <= wpos0 + 16 * qt + li);
              if (!ok) sacc[kt][qt][i] = -INFINITY;
            }
      }
      if constexpr (STATS) {
        // online softmax (the maximum moves only when a block exceeds it by
        // more than the slack), fp32 row sums, O^T += v^T P^T with bf16 P
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
            const float alpha = fast_exp2(m_run[qt] - m_new);
            m_run[qt] = m_new;
            l_part[qt] *= alpha;
#pragma unroll
            for (int dt = 0; dt < NACC; ++dt) acc[qt][dt] *= alpha;
          }
          const float m_use = m_run[qt] == -INFINITY ? 0.f : m_run[qt];
          float pv[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            pv[j] = fast_exp2(sacc[j >> 2][qt][j & 3] - m_use);
            l_part[qt] += pv[j];
          }
          const bf16x8_t pop = pack8(pv);
          const bf16_t* vt = buf + 2 * C::ROWT;
#pragma unroll
          for (int dt = 0; dt <= DT; ++dt)
            acc[qt][dt] = mfma_bf16(kEarlyT ? tre[kEarlyT ? dt : 0] : tr_operand(vt + (16 * dt + li) * LDT, 0, lg),
                                    pop, acc[qt][dt]);
        }
      } else {
        // dS^T = P^T (dP^T - D); dQ^T += k^T dS^T (both plain bf16)
        bf16x8_t dsh[QT];
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) {
          float dsv[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const int kt = j >> 2, i = j & 3;
            const float p = fast_exp2(sacc[kt][qt][i] - lse[qt]);
            dsv[j] = p * (pacc[kt][qt][i] * inv_rv - dd[qt]);
          }
          dsh[qt] = pack8(dsv);
        }
        const bf16_t* kt_hi = buf + 3 * C::ROWT;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const bf16x8_t ka = kEarlyT ? tre[kEarlyT ? dt : 0] : tr_operand(kt_hi + (16 * dt + li) * LDT, 0, lg);
#pragma unroll
          for (int qt = 0; qt < QT; ++qt) {
            acc[qt][dt] = mfma_bf16(ka, dsh[qt], acc[qt][dt]);
          }
        }
      }
    }
    if (blk + 1 < nblk) {
      q_stage_store<DH, STATS>(sr, lds + ((blk + 1) & 1) * C::BUF);
      if (blk + 2 < nblk) q_stage_load<DH, STATS>(sr, g, b, hh, h, n_keys, k0 + 2 * BN);
    }
    __syncthreads();
  }

  if constexpr (STATS) {
    // lse = m + log2(sum_t p_t); O = (sum_t bf16(p_t) v^_t) / sum_t bf16(p_t) / R_V;
    // D = dO . O.  Lane holds d = 16dt + 4lg + i of query 16qt + li.
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      const float l32 = lane_group_sum(l_part[qt]);
      const float inv = a.v_scale / __shfl(acc[qt][DT][0], li);
      const int64_t s = sw0 + 16 * qt + li;
      const int64_t row = ((b * a.S + (s < a.S ? s : a.S - 1)) * h + hh) * (int64_t)DH;
      float dsum = 0.f;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const uint2 d = *reinterpret_cast<const uint2*>(dO + row + dt * 16 + 4 * lg);
        dsum = fmaf(acc[qt][dt][0] * inv, __uint_as_float(d.x << 16), dsum);
        dsum = fmaf(acc[qt][dt][1] * inv, __uint_as_float(d.x & 0xffff0000u), dsum);
        dsum = fmaf(acc[qt][dt][2] * inv, __uint_as_float(d.y << 16), dsum);
        dsum = fmaf(acc[qt][dt][3] * inv, __uint_as_float(d.y & 0xffff0000u), dsum);
      }
      dsum = lane_group_sum(dsum);
      if (s < a.S && lg == 0) {
        g.lse[(b * a.S + s) * h + hh] = m_run[qt] + __log2f(l32);
        g.dvec[(b * a.S + s) * h + hh] = dsum;
      }
    }
  } else {
    // lane holds d = 16dt + 4lg + i of query 16qt + li.  dQ = dS K / sqrt(d_h)
    // with K = k^ / R_K.  KV-only: dQ is the query gradient itself; factored:
    // this head's dA_Q here, dQ to the workspace for dB_Q.
    const float qscale = 1.f / ((float)a.rk * sqrtf((float)DH));
    f32x4_t dqt[DT][QT];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) dqt[dt][qt] = acc[qt][dt] * qscale;
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      const int64_t s = sw0 + 16 * qt + li;
      const bool ok = s < a.S;
      const int64_t sc = ok ? s : a.S - 1;
      float* o;
      if (a.rq == 0) {
        o = g.d_bq + ((b * g.dq_bstride + sc) * h + hh) * (int64_t)DH + 4 * lg;
      } else {
        const int64_t tok = b * a.q_bstride_tok + sc;
        head_factor_grad<DH>(dqt, qt, reinterpret_cast<const bf16_t*>(a.b_q) + tok * a.rq * DH, a.rq, lg, ok,
                             g.d_aq + ((b * g.dq_bstride + sc) * h + hh) * a.rq);
        o = g.dq + ((b * a.S + sc) * h + hh) * (int64_t)DH + 4 * lg;
      }
      if (!ok) continue;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
        *reinterpret_cast<float4*>(o + 16 * dt) = make_float4(dqt[dt][qt][0], dqt[dt][qt][1], dqt[dt][qt][2],
                                                              dqt[dt][qt][3]);
    }
  }
}

// ---- pass 5: dim-factor gradients dB[t, r, :] = (1/R) sum_h A[t, h, r] dX[t, h, :]
// One wave per (token, tensor): the query tokens (factored queries only), then
// each key token's K and V.  The wave stages its A [h, R] in its own LDS
// slice (read back as broadcasts); lanes run over d, reading dX coalesced,
// and the rank goes in chunks of 8.
constexpr int kMaxHR = 1024;   // h * R this pass takes (larger: general kernel)

template <int DH>
__global__ void __launch_bounds__(256) bwd_dim_factor_kernel(AttnArgs a, BwdArgs g, int64_t n_items) {
  __shared__ float a_lds[4][kMaxHR + 8];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t item = (int64_t)blockIdx.x * 4 + wave;
  const int h = a.h;
  const int64_t n_keys = a.start_pos + a.S;
  const int64_t nq = a.rq > 0 ? a.n_batch * a.S : 0;
  const float* dX = nullptr;
  const bf16_t* A = nullptr;
  float* dB = nullptr;
  int R = 1;
  if (item < nq) {
    const int64_t b = item / a.S, s = item - b * a.S;
    const int64_t tok = b * a.q_bstride_tok + s;
    R = a.rq;
    dX = g.dq + (b * a.S + s) * h * (int64_t)DH;
    A = reinterpret_cast<const bf16_t*>(a.a_q) + tok * h * R;
    dB = g.d_bq + (b * g.dq_bstride + s) * R * (int64_t)DH;
  } else if (item < n_items) {
    const int64_t k = (item - nq) >> 1;
    const bool is_v = (item - nq) & 1;
    const int64_t b = k / n_keys, t = k - b * n_keys;
    const int64_t row = b * a.max_seq + t, drow = b * g.dkv_max_seq + t;
    R = is_v ? a.rv : a.rk;
    dX = (is_v ? g.dv : g.dk) + (b * n_keys + t) * h * (int64_t)DH;
    A = reinterpret_cast<const bf16_t*>(is_v ? a.c_av : a.c_ak) + row * h * R;
    dB = (is_v ? g.d_bv : g.d_bk) + drow * R * (int64_t)DH;
  }
  float* as = a_lds[wave];
  if (A) {
    for (int e = lane; e < h * R; e += 64) as[e] = bf16_to_f32(A[e]);
    if (lane < 8) as[h * R + lane] = 0.f;   // read past the last rank chunk, never stored
  }
  __syncthreads();
  if (!A) return;
  const float inv_r = 1.f / (float)R;
#pragma unroll
  for (int c = lane; c < DH; c += 64) {
    for (int r0 = 0; r0 < R; r0 += 8) {
      float acc[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] = 0.f;
      for (int hh = 0; hh < h; ++hh) {
        const float x = dX[hh * DH + c];
        const float* ar = as + hh * R + r0;
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] = fmaf(ar[j], x, acc[j]);
      }
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (r0 + j < R) dB[(r0 + j) * DH + c] = acc[j] * inv_r;
    }
  }
}

// LDS a workgroup may allocate on the current device.
static size_t bwd_device_lds() {
  int dev = 0, v = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess) return 0;
  return (size_t)v;
}

template <int DH>
static size_t bwd_max_lds() {
  size_t m = BwdKvCfg<DH>::kLds;
  if (BwdQCfg<DH, true>::kLds > m) m = BwdQCfg<DH, true>::kLds;
  if (BwdQCfg<DH, false>::kLds > m) m = BwdQCfg<DH, false>::kLds;
  return m;
}

bool backward_mfma_supported(int dtype, const AttnArgs& a, const BwdArgs& g) {
  if (dtype != kBF16 || !(a.d_h == 64 || a.d_h == 128)) return false;
  const int r_max = a.rq > a.rk ? (a.rq > a.rv ? a.rq : a.rv) : (a.rk > a.rv ? a.rk : a.rv);
  if (a.h * r_max > kMaxHR) return false;
  if ((a.d_h == 64 ? bwd_max_lds<64>() : bwd_max_lds<128>()) > bwd_device_lds()) return false;
  const int64_t n_keys = a.start_pos + a.S;
  const int64_t hb = (int64_t)a.h * a.n_batch;
  if ((n_keys / 64 + 1) * hb >= ((int64_t)1 << 31) || (a.S / 64 + 1) * hb >= ((int64_t)1 << 31)) return false;
  // 16-byte loads and stores
  const void* p16[12] = {a.b_q, a.c_bk, a.c_bv, g.dout, g.q_hi, g.q_lo, g.k_hi, g.k_lo, g.v_hat, g.dk, g.dv, g.dq};
  for (int i = 0; i < 12; ++i)
    if (((uintptr_t)p16[i]) % 16) return false;
  // KV-only: dQ is written straight into the caller's tensor, 16 bytes at a time
  return a.rq > 0 || (((uintptr_t)g.d_bq) % 16 == 0 && (g.dq_bstride * a.h * a.d_h) % 4 == 0);
}

template <int DH>
static void launch_bwd_mfma_dh(const AttnArgs& a, const BwdArgs& g, hipStream_t st) {
  using K = BwdKvCfg<DH>;
  using QS = BwdQCfg<DH, true>;
  using QD = BwdQCfg<DH, false>;
  const int64_t n_keys = a.start_pos + a.S;
  const int64_t hb = (int64_t)a.h * a.n_batch;
  const int nkb = (int)((n_keys + K::BN - 1) / K::BN);
  const int nqs = (int)((a.S + QS::BM - 1) / QS::BM), nqd = (int)((a.S + QD::BM - 1) / QD::BM);
  hipLaunchKernelGGL((bwd_query_mfma_kernel<DH, true>), dim3((unsigned)(nqs * hb)), dim3(256), QS::kLds, st, a, g,
                     nqs);
  hipLaunchKernelGGL(bwd_dkdv_mfma_kernel<DH>, dim3((unsigned)(nkb * hb)), dim3(256), K::kLds, st, a, g);
  hipLaunchKernelGGL((bwd_query_mfma_kernel<DH, false>), dim3((unsigned)(nqd * hb)), dim3(256), QD::kLds, st, a, g,
                     nqd);
}

// All five passes.
hipError_t launch_backward_mfma(const AttnArgs& a, const BwdArgs& g, hipStream_t st) {
  const int64_t n_keys = a.start_pos + a.S;
  const int64_t items = a.n_batch * (a.S + n_keys) * a.h * (a.d_h / 8);
  int64_t blocks = (items + 255) / 256;
  blocks = blocks > 65536 ? 65536 : (blocks < 1 ? 1 : blocks);
  hipLaunchKernelGGL(bwd_rebuild_kernel, dim3((unsigned)blocks), dim3(256), 0, st, a, g, n_keys);
  if (a.d_h == 64) launch_bwd_mfma_dh<64>(a, g, st);
  else launch_bwd_mfma_dh<128>(a, g, st);
  const int64_t n_items = (a.rq > 0 ? a.n_batch * a.S : 0) + 2 * a.n_batch * n_keys;
  const dim3 grid((unsigned)((n_items + 3) / 4));
  if (a.d_h == 64) hipLaunchKernelGGL(bwd_dim_factor_kernel<64>, grid, dim3(256), 0, st, a, g, n_items);
  else hipLaunchKernelGGL(bwd_dim_factor_kernel<128>, grid, dim3(256), 0, st, a, g, n_items);
  return hipGetLastError();
}

}  // namespace tpa
