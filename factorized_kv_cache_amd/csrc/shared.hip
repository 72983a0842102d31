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
// One workgroup per (sequence, chunk of keys) covers every head.  It forms
// alpha/beta of every (head, rank) once, as bf16 hi + lo rows in LDS, and then
// walks the chunk in blocks of 64 keys with no barrier: wave w takes keys
// 16 (w % 4) .. + 15 of each block and a group of 16-column tiles (w / 4).
// The products run transposed on the matrix cores,
//   G^T[(h, r), t] = sum_i alpha[h,r,i] cos(t th_i) + beta[h,r,i] sin(t th_i),
// with each lane forming its key's angle features in registers as one complex
// product each: the wave's anchor (cos, sin)(t0 th_i) at its first key t0 of
// the block (one fp64-reduced angle per lane per block, in a wave-private LDS
// slot) turned by (cos, sin)(j th_i) for the key's offset j < 16 from a table
// built once per workgroup (features and alpha/beta both as hi + lo, three
// products: fp32-level accuracy).  Lane (li, lg) then holds key li and the four
// consecutive columns 16 n0 + 4 lg .. + 3 of tile n0.  Columns are numbered
// head * RKP + rank, RKP in {1, 2, 4} the smallest power of two >= R_K (ranks
// past R_K are zero), so the lane holds whole heads (HPL = 4 / RKP per tile):
// the rank sum of a score stays in the lane, and the head factors it needs are
// contiguous in its key's cache row, loaded straight into registers ahead of
// the products.  Each lane keeps an online softmax per head over its own keys;
// the 16 keys of a wave merge through DPP, the four waves of a tile group
// through LDS, and a second pass merges the chunks in a fixed order (one wave
// per sequence and head).
#include "kernels.h"
#include "mfma.h"

namespace tpa {

constexpr int kShB = 64;      // keys per block: 16 per wave of a tile group
constexpr int kShMaxKS = 4;   // d_h / 32 k-steps of the products, d_h up to 128
constexpr int kShMaxG = 4;    // tile groups (waves / 4) per workgroup

typedef uint32_t sh_u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t sh_u32x4 __attribute__((ext_vector_type(4)));

// LDS carve of the decode kernel (in bytes from the start).
struct SharedLds {
  size_t rev, stage, bhi, blo, rot, anch, end;
  int np, nt, ldb;
};

// Keys per wave of a block: the features of key t0 + j (j < kShSub) are the
// wave's anchor (cos, sin)(t0 th_i) turned by (cos, sin)(j th_i) from a table
// laid out [pair i][j] with rows of kShRotLd entries: the 16 lanes of a lane
// group read one row's 128 contiguous bytes, and the four groups' rows (4
// pairs apart) start 16 banks apart.
constexpr int kShSub = 16;
constexpr int kShRotLd = 18;

__host__ __device__ inline int shared_rkp(int rk) { return rk <= 1 ? 1 : (rk <= 2 ? 2 : 4); }

__host__ __device__ inline SharedLds shared_carve(int h, int dh, int rq, int rk, int waves) {
  SharedLds c;
  c.np = dh / 2;
  c.nt = (h * shared_rkp(rk) + 15) / 16;   // 16-column tiles of G^T
  c.ldb = dh + 8;                          // alpha/beta rows (bf16), padded
  const int rqq = rq > 0 ? rq : 1;
  size_t o = 0;
  c.rev = o; o += sizeof(double) * c.np;
  // the query factors and B_K in the prologue, the four waves' per-head
  // partials [4][h][2 + 4] at the end
  const size_t st_in = (size_t)h * rqq + (rq > 0 ? (size_t)rqq * dh : 0) + (size_t)rk * dh;
  const size_t st_out = (size_t)4 * h * 6;
  c.stage = o; o += sizeof(float) * (st_in > st_out ? st_in : st_out);
  o = (o + 15) / 16 * 16;
  c.bhi = o; o += sizeof(bf16_t) * c.nt * 16 * c.ldb;
  c.blo = o; o += sizeof(bf16_t) * c.nt * 16 * c.ldb;
  c.rot = o; o += sizeof(float) * 2 * kShRotLd * c.np;   // [i][j] (cos, sin)(j th_i)
  c.anch = o; o += sizeof(float) * 2 * waves * c.np;     // [wave][i] (cos, sin)(t0 th_i)
  c.end = o;
  return c;
}

// Element e of a run of head factors held as raw words (bf16 pairs or fp32).
template <typename T>
__device__ __forceinline__ float raw_elem(const uint32_t* w, int e) {
  if constexpr (sizeof(T) == 4) return __uint_as_float(w[e]);
  else return __uint_as_float((e & 1) ? (w[e >> 1] & 0xffff0000u) : (w[e >> 1] << 16));
}

template <typename T>
__device__ __forceinline__ void raw_put(uint32_t* w, int e, const T* p, int64_t i) {
  if constexpr (sizeof(T) == 4) {
    w[e] = __float_as_uint(p[i]);
  } else {
    const uint32_t bits = reinterpret_cast<const uint16_t*>(p)[i];
    w[e >> 1] |= (e & 1) ? bits << 16 : bits;
  }
}

// W contiguous, W*4-byte aligned words.
template <int W>
__device__ __forceinline__ void load_words(uint32_t (&r)[W], const void* p) {
  if constexpr (W == 1) {
    r[0] = *reinterpret_cast<const uint32_t*>(p);
  } else if constexpr (W == 2) {
    const sh_u32x2 v = *reinterpret_cast<const sh_u32x2*>(p);
    r[0] = v.x;
    r[1] = v.y;
  } else {
    static_assert(W % 4 == 0, "runs of 1, 2 or 4k words");
#pragma unroll
    for (int i = 0; i < W / 4; ++i) {
      const sh_u32x4 v = reinterpret_cast<const sh_u32x4*>(p)[i];
      r[4 * i] = v.x;
      r[4 * i + 1] = v.y;
      r[4 * i + 2] = v.z;
      r[4 * i + 3] = v.w;
    }
  }
}

// The head factors one lane needs from one cache row for one tile: the HPL
// heads hh0 .. hh0 + HPL - 1, A_K as [HPL][RKP] and A_V as [HPL][MRV] (zeros
// past R_K, R_V and past the last head).  Runs that are whole and aligned go
// as one vector load each.
template <typename T, int HPL, int MRV>
struct TileFactors {
  static constexpr int RKP = 4 / HPL;
  static constexpr int KW = (4 * (int)sizeof(T) + 3) / 4;
  static constexpr int VW = (HPL * MRV * (int)sizeof(T) + 3) / 4;
  uint32_t k[KW];
  uint32_t v[VW];

  __device__ __forceinline__ void load(const T* AK, const T* AV, int64_t row, int hh0, int h, int rk, int rv,
                                       bool vk, bool vv) {
    const bool whole = hh0 + HPL <= h;
    if (vk && whole) {
      load_words<KW>(k, AK + row * h * rk + (int64_t)hh0 * rk);
    } else {
#pragma unroll
      for (int i = 0; i < KW; ++i) k[i] = 0u;
#pragma unroll
      for (int j = 0; j < HPL; ++j)
#pragma unroll
        for (int r = 0; r < RKP; ++r)
          if (hh0 + j < h && r < rk) raw_put<T>(k, j * RKP + r, AK, row * h * rk + (int64_t)(hh0 + j) * rk + r);
    }
    if (vv && whole) {
      load_words<VW>(v, AV + row * h * rv + (int64_t)hh0 * rv);
    } else {
#pragma unroll
      for (int i = 0; i < VW; ++i) v[i] = 0u;
#pragma unroll
      for (int j = 0; j < HPL; ++j)
#pragma unroll
        for (int r = 0; r < MRV; ++r)
          if (hh0 + j < h && r < rv) raw_put<T>(v, j * MRV + r, AV, row * h * rv + (int64_t)(hh0 + j) * rv + r);
    }
  }
};

// LDS written by lanes of a wave made visible to the other lanes of that wave.
__device__ __forceinline__ void shared_wave_lds_fence() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// x = hi + lo as bf16 pairs (round to nearest even each).
__device__ __forceinline__ void split_pair8(const float (&x)[8], bf16x8_t& hi, bf16x8_t& lo) {
  float h[8], l[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    h[e] = bf16_to_f32(f32_to_bf16(x[e]));
    l[e] = x[e] - h[e];
  }
  hi = pack8(h);
  lo = pack8(l);
}

// Slack (log2 units) by which a score may pass a lane's running maximum
// before the lane's sums are rescaled (p <= 2^8 meanwhile).
constexpr float kShSlack = 8.f;

// NT tiles per wave at most, HPL heads per lane per tile (RKP = 4 / HPL
// columns each), MRV >= R_V value ranks.  blockDim = 256 x tile groups.
// WIDE: four tiles of two heads per lane in one tile group (256 threads), which
// needs up to 168 registers: three resident waves per SIMD instead of four,
// but each key's features are formed once instead of once per tile group.
template <typename T, int NT, int HPL, int MRV, bool WIDE>
__global__ void __launch_bounds__(WIDE ? 256 : 64 * 4 * kShMaxG, WIDE ? 3 : 1) shared_decode_kernel(AttnArgs a, RopeTable tab,
                                                                        int64_t ctx_len, int64_t chunk,
                                                                        int n_chunks, float* part) {
  constexpr int RKP = 4 / HPL;
  using TF = TileFactors<T, HPL, MRV>;
  extern __shared__ __align__(16) unsigned char shb[];
  const int h = a.h, dh = a.d_h, rk = a.rk, rv = a.rv, rq = a.rq > 0 ? a.rq : 1;
  const SharedLds L = shared_carve(h, dh, a.rq, rk, blockDim.x >> 6);
  const int np = L.np, nt = L.nt, ldb = L.ldb;
  double* s_rev = reinterpret_cast<double*>(shb + L.rev);
  float* s_aq = reinterpret_cast<float*>(shb + L.stage);     // [h][R_Q]
  float* s_bq = s_aq + h * rq;                                 // [R_Q][d_h]
  float* s_bk = s_bq + (a.rq > 0 ? rq * dh : 0);               // [R_K][d_h]
  float* s_red = reinterpret_cast<float*>(shb + L.stage);      // [4][h][2 + MRV] after the loop
  bf16_t* bhi = reinterpret_cast<bf16_t*>(shb + L.bhi);        // [nt*16][d_h + 8] alpha/beta rows, hi
  bf16_t* blo = reinterpret_cast<bf16_t*>(shb + L.blo);        //                                  lo
  float2* s_rot = reinterpret_cast<float2*>(shb + L.rot);      // [np][kShRotLd]
  const int c = blockIdx.x;
  const int64_t b = blockIdx.y;
  const int64_t t0 = (int64_t)c * chunk;
  const int64_t t1 = t0 + chunk < ctx_len ? t0 + chunk : ctx_len;
  const int lane = threadIdx.x & 63, li = lane & 15, lg = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int mt = wave & 3, grp = wave >> 2, n_grp = blockDim.x >> 8;
  const T* AQ = reinterpret_cast<const T*>(a.a_q);
  const T* BQ = reinterpret_cast<const T*>(a.b_q);
  const T* BK = reinterpret_cast<const T*>(a.c_bk);
  const T* AK = reinterpret_cast<const T*>(a.c_ak);
  const T* AV = reinterpret_cast<const T*>(a.c_av);
  const int64_t row0 = b * a.max_seq;

  // whole runs go as vector loads when the rows and the base keep them aligned
  const bool vk = rk == RKP && (h * rk) % 4 == 0 && ((uintptr_t)AK % (4 * sizeof(T) < 16 ? 4 * sizeof(T) : 16)) == 0;
  constexpr int VB = HPL * MRV * (int)sizeof(T);
  const bool vv = VB >= 4 && rv == MRV && (h * rv) % (HPL * MRV) == 0 && ((uintptr_t)AV % (VB < 16 ? VB : 16)) == 0;

  for (int i = threadIdx.x; i < np; i += blockDim.x) s_rev[i] = tab.rev[i];
  const int64_t tok = b * a.q_bstride_tok;
  if (a.rq > 0) {
    for (int idx = threadIdx.x; idx < h * rq; idx += blockDim.x) s_aq[idx] = ldf(AQ, tok * h * rq + idx);
    for (int idx = threadIdx.x; idx < rq * dh; idx += blockDim.x) s_bq[idx] = ldf(BQ, tok * rq * dh + idx);
  }
  for (int idx = threadIdx.x; idx < rk * dh; idx += blockDim.x) s_bk[idx] = ldf(BK, idx);
  __syncthreads();
  // ---- the key-offset rotations (cos, sin)(j th_i), j < kShSub, angles
  //      reduced in fp64 as everywhere
  for (int idx = threadIdx.x; idx < kShSub * np; idx += blockDim.x) {
    const int i = idx / kShSub, j = idx - i * kShSub;
    double turns = (double)j * s_rev[i];
    turns -= rint(turns);
    const float ang = (float)turns;
    s_rot[i * kShRotLd + j] = make_float2(__builtin_amdgcn_cosf(ang), __builtin_amdgcn_sinf(ang));
  }
  // ---- alpha/beta rows, column n = head RKP + r, feature 2i (alpha_i) and
  //      2i+1 (beta_i), as bf16 hi + lo; columns with r >= R_K or past the last
  //      head are zero.  The query pair (scaled by log2(e) / (R_Q R_K sqrt(d_h)))
  //      is formed on the way.
  for (int idx = threadIdx.x; idx < nt * 16 * np; idx += blockDim.x) {
    const int n = idx / np, i = idx - n * np;
    const int hh = n / RKP, r = n - hh * RKP;
    float al = 0.f, be = 0.f;
    if (hh < h && r < rk) {
      float q0 = 0.f, q1 = 0.f;
      if (a.rq == 0) {
        q0 = ldf(BQ, (tok * h + hh) * dh + 2 * i);
        q1 = ldf(BQ, (tok * h + hh) * dh + 2 * i + 1);
      } else {
        for (int rr = 0; rr < rq; ++rr) {
          const float aq = s_aq[hh * rq + rr];
          q0 = fmaf(aq, s_bq[rr * dh + 2 * i], q0);
          q1 = fmaf(aq, s_bq[rr * dh + 2 * i + 1], q1);
        }
      }
      q0 *= a.q_scale;
      q1 *= a.q_scale;
      const float b0 = s_bk[r * dh + 2 * i], b1 = s_bk[r * dh + 2 * i + 1];
      al = fmaf(q0, b0, q1 * b1);
      be = fmaf(q1, b0, -q0 * b1);
    }
    const float ah = bf16_to_f32(f32_to_bf16(al)), bh = bf16_to_f32(f32_to_bf16(be));
    *reinterpret_cast<uint32_t*>(bhi + n * ldb + 2 * i) = pack_bf16x2(ah, bh);
    *reinterpret_cast<uint32_t*>(blo + n * ldb + 2 * i) = pack_bf16x2(al - ah, be - bh);
  }
  __syncthreads();

  float m[NT][HPL], l[NT][HPL], w[NT][HPL][MRV];
#pragma unroll
  for (int k = 0; k < NT; ++k)
#pragma unroll
    for (int j = 0; j < HPL; ++j) {
      m[k][j] = -INFINITY;
      l[k][j] = 0.f;
#pragma unroll
      for (int r = 0; r < MRV; ++r) w[k][j][r] = 0.f;
    }
  const int ksn = dh / 32;
  float2* s_anch = reinterpret_cast<float2*>(shb + L.anch) + wave * np;   // this wave's anchors
  const float2* rot_j = s_rot + li;                                       // key offset li
  for (int64_t blk0 = t0; blk0 < t1; blk0 += kShB) {
    const int64_t key = blk0 + 16 * mt + li;
    const bool valid = key < t1;
    // the wave's anchors (cos, sin)(t0 th_i) at its first key t0 = blk0 + 16 mt,
    // one pair per lane (the previous block's reads are done first)
    shared_wave_lds_fence();
    for (int i = lane; i < np; i += 64) {
      double turns = (double)(blk0 + 16 * mt) * s_rev[i];
      turns -= rint(turns);
      const float ang = (float)turns;
      s_anch[i] = make_float2(__builtin_amdgcn_cosf(ang), __builtin_amdgcn_sinf(ang));
    }
    shared_wave_lds_fence();
    // the head factors of the lane's key go out first; the products hide them
    TF cur[NT];
#pragma unroll
    for (int k = 0; k < NT; ++k) {
      const int n0 = grp + n_grp * k;
      if (n0 < nt && valid) cur[k].load(AK, AV, row0 + key, (16 * n0 + 4 * lg) / RKP, h, rk, rv, vk, vv);
    }
    // ---- per k-step: the features of key li, 32 ks + 8 lg .. + 7 = (cos, sin)
    //      of pairs 16 ks + 4 lg .. + 3 (the anchor turned by li th_i: one
    //      complex product each), then that step of every tile's product
    f32x4_t acc[NT];
#pragma unroll
    for (int k = 0; k < NT; ++k) acc[k] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < kShMaxKS; ++ks) {
      if (ks >= ksn) break;
      float x[8];
      const int p0 = 16 * ks + 4 * lg;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float2 an = s_anch[p0 + e], ro = rot_j[(p0 + e) * kShRotLd];
        x[2 * e] = fmaf(an.x, ro.x, -an.y * ro.y);       // cos((t0 + li) th)
        x[2 * e + 1] = fmaf(an.y, ro.x, an.x * ro.y);    // sin((t0 + li) th)
      }
      bf16x8_t fh, fl;
      split_pair8(x, fh, fl);
#pragma unroll
      for (int k = 0; k < NT; ++k) {
        const int n0 = grp + n_grp * k;
        if (n0 >= nt) break;
        const int boff = (16 * n0 + li) * ldb + 32 * ks + 8 * lg;
        const bf16x8_t bh = *reinterpret_cast<const bf16x8_t*>(bhi + boff);
        const bf16x8_t bl = *reinterpret_cast<const bf16x8_t*>(blo + boff);
        acc[k] = mfma_bf16(bh, fh, acc[k]);
        acc[k] = mfma_bf16(bl, fh, acc[k]);
        acc[k] = mfma_bf16(bh, fl, acc[k]);
      }
    }
#pragma unroll
    for (int k = 0; k < NT; ++k) {
      const int n0 = grp + n_grp * k;
      if (n0 >= nt) break;
      // acc[k][i] = G^T[column 16 n0 + 4 lg + i][key li]
      if (valid) {
#pragma unroll
        for (int j = 0; j < HPL; ++j) {
          float s = 0.f;
#pragma unroll
          for (int r = 0; r < RKP; ++r) s = fmaf(raw_elem<T>(cur[k].k, j * RKP + r), acc[k][j * RKP + r], s);
          // The lane's running maximum moves only when a score passes it by
          // more than kShSlack (always at the lane's first key), so the
          // terms are rescaled rarely and each key costs one exponential.
          const bool up = s > m[k][j] + kShSlack;
          if (__any(up)) {
            const float mn = up ? s : m[k][j];
            const float alpha = up ? fast_exp2(m[k][j] - mn) : 1.f;   // 0 at the first key
            m[k][j] = mn;
            l[k][j] *= alpha;
#pragma unroll
            for (int r = 0; r < MRV; ++r) w[k][j][r] *= alpha;
          }
          const float p = fast_exp2(s - m[k][j]);
          l[k][j] += p;
#pragma unroll
          for (int r = 0; r < MRV; ++r) w[k][j][r] = fmaf(p, raw_elem<T>(cur[k].v, j * MRV + r), w[k][j][r]);
        }
      }
    }
  }

  // ---- merge the wave's 16 keys per head (DPP), then the four waves of the
  //      tile group through LDS, in a fixed order
#pragma unroll
  for (int k = 0; k < NT; ++k) {
    const int n0 = grp + n_grp * k;
    if (n0 >= nt) break;
#pragma unroll
    for (int j = 0; j < HPL; ++j) {
      const float mx = row16_max(m[k][j]);
      const float sc = m[k][j] == -INFINITY ? 0.f : fast_exp2(m[k][j] - mx);
      const float lt = row16_sum(l[k][j] * sc);
      float wt[MRV];
#pragma unroll
      for (int r = 0; r < MRV; ++r) wt[r] = row16_sum(w[k][j][r] * sc);
      const int hh = (16 * n0 + 4 * lg) / RKP + j;
      if (li == 0 && hh < h) {
        float* q = s_red + ((int64_t)mt * h + hh) * (2 + MRV);
        q[0] = mx;
        q[1] = lt;
#pragma unroll
        for (int r = 0; r < MRV; ++r) q[2 + r] = wt[r];
      }
    }
  }
  __syncthreads();
  for (int hh = threadIdx.x; hh < h; hh += blockDim.x) {
    float mx = -INFINITY;
#pragma unroll
    for (int q = 0; q < 4; ++q) mx = fmaxf(mx, s_red[((int64_t)q * h + hh) * (2 + MRV)]);
    float lt = 0.f, wt[MRV];
#pragma unroll
    for (int r = 0; r < MRV; ++r) wt[r] = 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float* e = s_red + ((int64_t)q * h + hh) * (2 + MRV);
      const float sc = e[0] == -INFINITY ? 0.f : fast_exp2(e[0] - mx);
      lt = fmaf(e[1], sc, lt);
#pragma unroll
      for (int r = 0; r < MRV; ++r) wt[r] = fmaf(e[2 + r], sc, wt[r]);
    }
    float* p = part + ((b * n_chunks + c) * h + hh) * (int64_t)(2 + rv);
    p[0] = mx;
    p[1] = lt;
#pragma unroll
    for (int r = 0; r < MRV; ++r)
      if (r < rv) p[2 + r] = wt[r];
  }
}

// Chunks merged per (sequence, head), one wave each: lane l merges chunks
// l, l + 64, ... in order, then the 64 lanes merge over DPP and the half-wave
// swaps, a fixed order; out = (1/R_V) sum_r W[r] B_V[r] / L.
constexpr int kShCombWaves = 4;

template <typename T, int MR>
__global__ void __launch_bounds__(64 * kShCombWaves) shared_combine_kernel(AttnArgs a, int n_chunks,
                                                                          const float* ws) {
  const int lane = threadIdx.x & 63;
  const int hh = blockIdx.x * kShCombWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t b = blockIdx.y;
  const int h = a.h, dh = a.d_h, rv = a.rv;
  if (hh >= h) return;   // a whole wave
  const float* p = ws + (b * n_chunks * h + hh) * (int64_t)(2 + rv);
  const int64_t cstride = (int64_t)h * (2 + rv);
  float mt = -INFINITY, lt = 0.f, wt[MR];
#pragma unroll
  for (int r = 0; r < MR; ++r) wt[r] = 0.f;
  for (int c = lane; c < n_chunks; c += 64) {
    const float* q = p + c * cstride;
    const float mc = q[0], lc = q[1];
    const float mn = fmaxf(mt, mc);
    const float sa = mt == -INFINITY ? 0.f : fast_exp2(mt - mn);
    const float sb = mc == -INFINITY ? 0.f : fast_exp2(mc - mn);
    mt = mn;
    lt = lt * sa + lc * sb;
#pragma unroll
    for (int r = 0; r < MR; ++r) wt[r] = wt[r] * sa + (r < rv ? q[2 + r] : 0.f) * sb;
  }
  const float M = wave_max(mt);
  const float sc = mt == -INFINITY ? 0.f : fast_exp2(mt - M);
  const float L = wave_sum(lt * sc);
  float W[MR];
#pragma unroll
  for (int r = 0; r < MR; ++r) W[r] = wave_sum(wt[r] * sc);
  const float inv = a.v_scale / L;
  const T* BV = reinterpret_cast<const T*>(a.c_bv);
  T* out = reinterpret_cast<T*>(a.out);
  for (int d = lane; d < dh; d += 64) {
    float o = 0.f;
#pragma unroll
    for (int r = 0; r < MR; ++r)
      if (r < rv) o = fmaf(W[r], ldf(BV, (int64_t)r * dh + d), o);
    stf(out, (b * h + hh) * (int64_t)dh + d, o * inv);
  }
}

static size_t shared_device_lds() {
  int dev = 0, v = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess) return 0;
  return (size_t)v;
}

// The kernel's shape for a layer: heads per lane per tile, value ranks, tile
// groups and tiles per wave.  A wave keeps, per tile, HPL (2 + MRV) softmax
// registers, one key's head factors, four accumulators and about eight
// registers of alpha/beta operands in flight.  The tile groups grow until the
// instance's tiles (a power of two) cost at most 76 such registers, or 88 for
// four tiles of one head per lane: the bounds under which every instance fits
// the 128 registers of four resident waves per SIMD without spills.  Four
// tiles of two heads per lane in bf16 (up to two value ranks) fit 168
// registers as one 256-thread tile group (three waves per SIMD); that form is
// taken when one group covers the layer, so each feature is formed once.
struct SharedShape {
  int hpl, mrv, groups, ntw, nt_max;
};

__host__ __device__ constexpr bool shared_fits(int es, int nt_max, int hpl, int mrv) {
  const int per_tile = hpl * (2 + mrv) + (4 * es + 3) / 4 + (hpl * mrv * es + 3) / 4 + 12;
  return (nt_max >= 1 && nt_max <= 2 && nt_max * per_tile <= 76) ||
         (nt_max == 4 && hpl == 1 && nt_max * per_tile <= 88);
}

__host__ __device__ constexpr bool shared_wide(int es, int nt_max, int hpl, int mrv) {
  return nt_max == 4 && hpl == 2 && es == 2 && mrv <= 2;
}

static SharedShape shared_shape(int dtype, const AttnArgs& a) {
  SharedShape s;
  const int es = dtype == kF32 ? 4 : 2;
  const int rkp = shared_rkp(a.rk);
  s.hpl = 4 / rkp;
  s.mrv = a.rv <= 1 ? 1 : (a.rv <= 2 ? 2 : 4);
  const int nt = (a.h * rkp + 15) / 16;
  s.groups = 0;
  s.ntw = 0;
  s.nt_max = 0;
  for (int g = 1; g <= kShMaxG; g *= 2) {
    const int ntw = (nt + g - 1) / g;
    const int ntm = ntw <= 1 ? 1 : (ntw <= 2 ? 2 : (ntw <= 4 ? 4 : 0));
    if (shared_fits(es, ntm, s.hpl, s.mrv) || (g == 1 && shared_wide(es, ntm, s.hpl, s.mrv))) {
      s.groups = g;
      s.ntw = ntw;
      s.nt_max = ntm;
      break;
    }
  }
  return s;
}

// Chunks of whole 64-key blocks.  The grid is sized to one round of resident
// workgroups: 256 CUs times the workgroups a CU holds (three for the wide
// form, else four waves per SIMD over the tile groups; fewer if LDS runs
// out).  Each sequence gets floor(slots / B) chunks and its blocks are spread
// evenly over them, so no partial second round trails the first (at
// 8 x 131,073 keys, h 32: 968 workgroups over 768 slots took 131 us, 752 in
// one round 112 us).
SharedPlan plan_shared_decode(int dtype, const AttnArgs& a, int64_t ctx_len) {
  SharedPlan p;
  const SharedShape s = shared_shape(dtype, a);
  const bool wide = s.groups == 1 && shared_wide(dtype == kF32 ? 4 : 2, s.nt_max, s.hpl, s.mrv);
  const int groups = s.groups > 0 ? s.groups : 1;
  int64_t per_cu = wide ? 3 : 4 / groups;
  const size_t lds = shared_carve(a.h, a.d_h, a.rq, a.rk, 4 * groups).end;
  const size_t cu_lds = shared_device_lds();
  if (lds > 0 && cu_lds > 0 && (int64_t)(cu_lds / lds) < per_cu) per_cu = (int64_t)(cu_lds / lds);
  if (per_cu < 1) per_cu = 1;
  int64_t per_seq = 256 * per_cu / a.n_batch;
  if (per_seq < 1) per_seq = 1;
  const int64_t blocks = (ctx_len + kShB - 1) / kShB;
  const int64_t per_chunk = (blocks + per_seq - 1) / per_seq;
  p.chunk_tokens = per_chunk * kShB;
  p.n_chunks = (ctx_len + p.chunk_tokens - 1) / p.chunk_tokens;
  return p;
}

// The matrix-core products take d_h a multiple of 32, up to 128; R_K and R_V
// up to 4; the per-query alpha/beta rows must fit the device's LDS.
bool shared_decode_supported(int dtype, const AttnArgs& a) {
  if (a.d_h % 32 || a.d_h > 32 * kShMaxKS || a.rk < 1 || a.rk > 4 || a.rv < 1 || a.rv > 4) return false;
  const SharedShape sh = shared_shape(dtype, a);
  if (sh.groups == 0) return false;
  return shared_carve(a.h, a.d_h, a.rq, a.rk, 4 * sh.groups).end <= shared_device_lds();
}

size_t shared_decode_workspace_bytes(const SharedPlan& p, const AttnArgs& a) {
  return sizeof(float) * (size_t)a.n_batch * p.n_chunks * a.h * (2 + a.rv);
}

template <typename T, int NT, int HPL, int MRV>
static void launch_shared_t(const AttnArgs& a, const RopeTable& tab, int64_t ctx_len, const SharedPlan& p,
                            int groups, float* ws, hipStream_t st) {
  // only the instances the shape rule can pick are built; the wide form runs
  // as a single tile group
  constexpr bool WIDE = shared_wide((int)sizeof(T), NT, HPL, MRV);
  if constexpr (shared_fits((int)sizeof(T), NT, HPL, MRV) || WIDE) {
    if (WIDE && groups != 1) return;
    const dim3 grid((unsigned)p.n_chunks, (unsigned)a.n_batch);
    hipLaunchKernelGGL((shared_decode_kernel<T, NT, HPL, MRV, WIDE>), grid, dim3(256 * groups),
                       shared_carve(a.h, a.d_h, a.rq, a.rk, 4 * groups).end, st, a, tab, ctx_len, p.chunk_tokens,
                       (int)p.n_chunks, ws);
    hipLaunchKernelGGL((shared_combine_kernel<T, MRV>),
                       dim3((unsigned)((a.h + kShCombWaves - 1) / kShCombWaves), (unsigned)a.n_batch),
                       dim3(64 * kShCombWaves), 0, st, a, (int)p.n_chunks, ws);
  }
}

template <typename T, int NT, int HPL>
static void launch_shared_v(const AttnArgs& a, const RopeTable& tab, int64_t ctx_len, const SharedPlan& p,
                            const SharedShape& s, float* ws, hipStream_t st) {
  if (s.mrv == 1) launch_shared_t<T, NT, HPL, 1>(a, tab, ctx_len, p, s.groups, ws, st);
  else if (s.mrv == 2) launch_shared_t<T, NT, HPL, 2>(a, tab, ctx_len, p, s.groups, ws, st);
  else launch_shared_t<T, NT, HPL, 4>(a, tab, ctx_len, p, s.groups, ws, st);
}

template <typename T, int NT>
static void launch_shared_h(const AttnArgs& a, const RopeTable& tab, int64_t ctx_len, const SharedPlan& p,
                            const SharedShape& s, float* ws, hipStream_t st) {
  if (s.hpl == 4) launch_shared_v<T, NT, 4>(a, tab, ctx_len, p, s, ws, st);
  else if (s.hpl == 2) launch_shared_v<T, NT, 2>(a, tab, ctx_len, p, s, ws, st);
  else launch_shared_v<T, NT, 1>(a, tab, ctx_len, p, s, ws, st);
}

template <typename T>
static void launch_shared_dt(const AttnArgs& a, const RopeTable& tab, int64_t ctx_len, const SharedPlan& p,
                             const SharedShape& s, float* ws, hipStream_t st) {
  if (s.nt_max == 1) launch_shared_h<T, 1>(a, tab, ctx_len, p, s, ws, st);
  else if (s.nt_max == 2) launch_shared_h<T, 2>(a, tab, ctx_len, p, s, ws, st);
  else launch_shared_h<T, 4>(a, tab, ctx_len, p, s, ws, st);
}

hipError_t launch_shared_decode(int dtype, const AttnArgs& a, const RopeTable& tab, int64_t ctx_len,
                                const SharedPlan& p, void* ws, hipStream_t st) {
  const SharedShape s = shared_shape(dtype, a);
  float* w = reinterpret_cast<float*>(ws);
  if (dtype == kF32) launch_shared_dt<float>(a, tab, ctx_len, p, s, w, st);
  else launch_shared_dt<bf16_t>(a, tab, ctx_len, p, s, w, st);
  return hipGetLastError();
}

}  // namespace tpa
