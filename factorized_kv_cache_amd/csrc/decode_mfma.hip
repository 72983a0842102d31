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
//    q^T held in registers for the whole kernel as a bf16 hi + lo pair (two
//    products; the cache rows are bf16 already, so the scores carry
//    fp32-level accuracy: a bf16 query alone costs ~2^-9 of each score, which
//    sharp heads at long context turn into output errors near 5e-3).  In
//    k-step ks lane group lg loads d = 32*ks + 8*lg .. +7 of its row, so each
//    load instruction reads whole 64-byte pieces of 16 rows; the same k-slot
//    mapping is used for q, so the contraction is unchanged.
//  * the head factor: every lane's 4 output rows of a tile are R whole tokens'
//    ranks (R in {1,2,4}), so s_t = sum_r A_K[t,head,r] P[(t,r),head] is
//    lane-local; the block maximum per head crosses the four lane groups with
//    two half-wave swaps.
//  * values: O^T[d, head] += B_V^T[d, (t,r)] * C[(t,r), head] with
//    C = p_t * A_V[t,head,r].  The score tiles' output registers already sit
//    in the B-operand layout of this product (k-slot j of lane group g is row
//    4g+j of tile 0 for j<4, of tile 1 for j>=4); B_V goes through a
//    wave-private LDS tile (16-byte stores of whole-line loads) and comes back
//    as the A operand with ds_read_b64_tr_b16.
//
// At d_h = 64 (up to 32 heads, 16 at rank 1) each wave keeps two blocks' loads
// in flight, both issued before the query is formed; at d_h = 128 or with more
// heads the registers go to a second resident wave instead, and the single
// register set is reloaded with the wave's next block part by part as soon as
// the current block has consumed a part (B_V once it is in LDS; where the
// registers allow, B~_K after the score products and the head factors after
// the softmax), so the wave keeps loads in flight through its compute: at
// 8 x 131073 keys, h 32, d_h 128 the call went from 260-263 to 255 us.
// The waves of a workgroup (eight at d_h = 128, four at 64) merge their
// (m, l, O) through LDS in a fixed order and write one partial per head to the
// workspace; the combine pass,
// shared with the general kernel, merges the chunks in index order.  (Merging
// in the last workgroup to finish would need an agent-scope release per
// workgroup, which writes back the whole L2 of its XCD: far slower than a
// second launch.)
#include "kernels.h"
#include "mfma.h"

namespace tpa {

// Narrowing to bf16 (round to nearest, ties to even, NaNs kept quiet) with
// integer operations, for the d_h = 128 value operand: with the packed
// hardware conversion the compiler schedules that value loop past the
// two-waves-per-SIMD register budget (spills), with this form it fits.  At
// d_h = 64 the hardware conversion fits and is cheaper (two values per
// instruction, no per-value branch).
__device__ __forceinline__ uint16_t bf16_rne_int(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ bf16x8_t pack8_int(const float* v) {
  u16x8_t u;
#pragma unroll
  for (int j = 0; j < 8; ++j) u[j] = bf16_rne_int(v[j]);
  return __builtin_bit_cast(bf16x8_t, u);
}

// The B rows of the factor cache are streamed once per call and read with
// the non-temporal hint, whole 16-byte pieces per lane, so they pass through
// without displacing other lines from the L2 and the last-level cache (at
// 8 x 131,073 keys the call went from about 237 to 212 us). The head-factor
// rows keep ordinary loads: neighbouring lanes take parts of one cache line
// in separate instructions, and with the hint each of those reads went back
// to memory (about 20 us slower at that size).
__device__ __forceinline__ uint4 ld_stream16(const bf16_t* p) {
  typedef unsigned int v4u __attribute__((ext_vector_type(4)));
  const v4u v = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// R consecutive bf16 values, loaded as one 2R-byte word.
template <int R>
struct RankWord;
template <>
struct RankWord<1> { typedef uint16_t type; };
template <>
struct RankWord<2> { typedef uint32_t type; };
template <>
struct RankWord<4> { typedef uint2 type; };

template <int R>
__device__ __forceinline__ void unpack_rank(typename RankWord<R>::type v, float* out) {
  if constexpr (R == 1) {
    out[0] = bf16_to_f32(v);
  } else if constexpr (R == 2) {
    out[0] = __uint_as_float(v << 16);
    out[1] = __uint_as_float(v & 0xffff0000u);
  } else {
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

// Waves per workgroup.  At d_h = 128 one eight-wave workgroup per CU, so that
// all the waves of a CU start together: two four-wave workgroups on a CU ran
// unevenly (the one dispatched second fell behind), and eight waves measured
// 241 against 245 us at 8 x 131,073 keys.  At d_h = 64 two four-wave
// workgroups (eight waves measured 146 against 141 us at 32 x 16,385 keys).
__host__ __device__ constexpr int decode_waves(int dh) { return dh == 128 ? 8 : 4; }

template <int DH, int R, int HT>
struct DecodeMfmaCfg {
  static constexpr int NW = decode_waves(DH);
  static constexpr int THREADS = 64 * NW;
  static constexpr int KS = DH / 32;     // k-steps of the score product
  static constexpr int DT = DH / 16;     // 16-wide d tiles of the value product
  static constexpr int NT = 4 / R;       // tokens per lane per score tile
  static constexpr int VBT = 32 / R;     // tokens per value block
  static constexpr int HP = HT * 16;     // padded head count
  // LDS row stride (bf16): 16-byte aligned rows, and the four rows one lane
  // group reads with a transposed read fall on disjoint banks
  static constexpr int LROW = DH + 16;
  static constexpr int OST = DH + 4;     // LDS row stride (f32) of the merge buffer
  // a second block in flight (its registers spill beyond these sizes)
  static constexpr bool kPrefetch = DH == 64 && (R == 1 ? HT == 1 : HT <= 2);
  static constexpr size_t kLoopBytes = (size_t)NW * 32 * LROW * sizeof(bf16_t);
  // the query's lo half in LDS instead of registers (lane-major, 16 bytes a
  // lane per (head tile, k-step)) where the registers would spill
  static constexpr bool kQloLds = (DH == 64 && HT == 4) || (DH == 128 && HT == 2);
  // which parts of the next block are loaded during the current one's compute
  // (each keeps its registers live through the rest of the block)
  // (bit 0: B_V, bit 1: B~_K, bit 2: head factors; chosen so none spills).
  // Only where a wave has a single register set: with two sets in flight the
  // rolling loads measured no better (147 against 146 us at 32 x 16385 keys).
  static constexpr int kRoll = kPrefetch ? 0
                               : DH == 128 ? (HT == 2 ? (R == 1 ? 0 : R == 2 ? 1 : 7) : 7)
                               : (R == 1 && HT == 3 ? 1 : 7);
  static constexpr size_t kQloBytes = kQloLds ? (size_t)NW * HT * KS * 64 * 16 : 0;
  static constexpr size_t kMergeBytes = (2 * NW * HP + (size_t)NW * HP * OST) * sizeof(float);
  static constexpr size_t kLds =
      kLoopBytes + kQloBytes > kMergeBytes ? kLoopBytes + kQloBytes : kMergeBytes;
  static_assert(kLds <= 160 * 1024, "LDS per workgroup (gfx950: 160 KB)");
};

// LDS the host checks before choosing this kernel: staged query factors (bytes).
constexpr size_t kDecodeMfmaQueryLds = 16384;

// Everything one value block needs from HBM, in registers.
template <int DH, int R, int HT>
struct BlockRegs {
  using C = DecodeMfmaCfg<DH, R, HT>;
  uint4 bv[DH / 16];                                 // B_V pieces, for the LDS tile
  uint4 bk[2][C::KS];                                // B~_K operand slices
  typename RankWord<R>::type ak[2][HT][C::NT];       // head factors of the lane's tokens
  typename RankWord<R>::type av[2][HT][C::NT];
};

// Uniform base pointers of the cache rows a block is read from (the chunk's
// first row, or with a paged cache the block's own first row: a page holds a
// whole number of value blocks); per-lane offsets from them are 32-bit (the
// plan keeps a chunk under 2^31 elements per tensor).
struct ChunkBase {
  const bf16_t* ak;
  const bf16_t* bk;
  const bf16_t* av;
  const bf16_t* bv;
};

// The three parts of a value block's loads: B_V (40% of the bytes at R = 2),
// the B~_K operand slices, the head factors.  Rows past `last` are clamped to
// it (their scores are masked).
template <int DH, int R, int HT>
__device__ __forceinline__ void load_bv(BlockRegs<DH, R, HT>& g, const ChunkBase& cb, int tb, int last, int lane) {
  // B_V rows of the block, 16-byte piece u*64 + lane of the block's 64*DH
  // bytes: every load instruction reads whole contiguous cache lines.
#pragma unroll
  for (int u = 0; u < DH / 16; ++u) {
    const int piece = u * 64 + lane;
    const int row = piece / (DH / 8), col = (piece % (DH / 8)) * 8;
    int tok = tb + row / R;
    tok = tok < last ? tok : last;
    g.bv[u] = ld_stream16(cb.bv + ((tok * R + row % R) * DH + col));
  }
}

template <int DH, int R, int HT>
__device__ __forceinline__ void load_bk(BlockRegs<DH, R, HT>& g, const ChunkBase& cb, int tb, int last, int lane) {
  using C = DecodeMfmaCfg<DH, R, HT>;
  const int li = lane & 15, lg = lane >> 4;
#pragma unroll
  for (int st = 0; st < 2; ++st) {
    const int row = st * 16 + li;
    int tok = tb + row / R;
    tok = tok < last ? tok : last;
    // k-step ks takes d = 32*ks .. 32*ks + 31, lane group lg its 8-wide slice
    // 8*lg: one load instruction reads 64 contiguous bytes of each of the
    // tile's 16 rows
    const bf16_t* src = cb.bk + ((tok * R + row % R) * DH + 8 * lg);
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) g.bk[st][ks] = ld_stream16(src + 32 * ks);
  }
}

template <int DH, int R, int HT>
__device__ __forceinline__ void load_heads(BlockRegs<DH, R, HT>& g, const ChunkBase& cb, int h, int tb, int last,
                                           int lane) {
  using C = DecodeMfmaCfg<DH, R, HT>;
  const int li = lane & 15, lg = lane >> 4;
  typedef typename RankWord<R>::type W;
#pragma unroll
  for (int st = 0; st < 2; ++st)
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
      int head = ht * 16 + li;
      head = head < h ? head : h - 1;
#pragma unroll
      for (int k = 0; k < C::NT; ++k) {
        int tok = tb + (st * 16 + lg * 4) / R + k;
        tok = tok < last ? tok : last;
        g.ak[st][ht][k] = *reinterpret_cast<const W*>(cb.ak + (tok * h + head) * R);
        g.av[st][ht][k] = *reinterpret_cast<const W*>(cb.av + (tok * h + head) * R);
      }
    }
}

template <int DH, int R, int HT>
__device__ __forceinline__ void load_block(BlockRegs<DH, R, HT>& g, const ChunkBase& cb, int h, int tb, int last,
                                           int lane) {
  load_bv<DH, R, HT>(g, cb, tb, last, lane);
  load_bk<DH, R, HT>(g, cb, tb, last, lane);
  load_heads<DH, R, HT>(g, cb, h, tb, last, lane);
}

// Where the next value block's loads come from, for the rolling prefetch:
// each part of the block's registers is reloaded with the next block as soon
// as the current block has consumed it.
struct NextBlock {
  bool valid;
  ChunkBase cb;
  int tb, last;
};

template <int DH, int R, int HT, int ROLL>
__device__ __forceinline__ void compute_block(BlockRegs<DH, R, HT>& g, bf16_t* lbv, int tb, int last,
                                              const NextBlock& nx, int h,
                                              int lane, const bf16x8_t (&qop)[HT][DecodeMfmaCfg<DH, R, HT>::KS],
                                              const bf16x8_t (&qlo)[HT][DecodeMfmaCfg<DH, R, HT>::KS],
                                              const bf16x8_t* qlo_lds,
                                              float (&m_run)[HT], float (&l_run)[HT],
                                              f32x4_t (&oacc)[HT][DecodeMfmaCfg<DH, R, HT>::DT]) {
  using C = DecodeMfmaCfg<DH, R, HT>;
  constexpr int KS = C::KS, DT = C::DT, NT = C::NT, LROW = C::LROW;
  const int li = lane & 15, lg = lane >> 4;

  // B_V pieces -> wave-private LDS tile, one 16-byte store each
#pragma unroll
  for (int u = 0; u < DH / 16; ++u) {
    const int piece = u * 64 + lane;
    const int row = piece / (DH / 8), col = (piece % (DH / 8)) * 8;
    *reinterpret_cast<bf16x8_t*>(lbv + row * LROW + col) = as_bf16x8(g.bv[u]);
  }
  if ((ROLL & 1) && nx.valid) load_bv<DH, R, HT>(g, nx.cb, nx.tb, nx.last, lane);

  // scores on the matrix cores
  f32x4_t sacc[2][HT];
#pragma unroll
  for (int st = 0; st < 2; ++st)
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
      // hi and lo products in two independent chains summed at the end (one
      // chain from three head tiles on, where the second would spill)
      constexpr bool kTwoChains = HT <= 2;
      f32x4_t acch = {0.f, 0.f, 0.f, 0.f}, accl = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        acch = mfma_bf16(as_bf16x8(g.bk[st][ks]), qop[ht][ks], acch);
        f32x4_t& al = kTwoChains ? accl : acch;
        if constexpr (DecodeMfmaCfg<DH, R, HT>::kQloLds)
          al = mfma_bf16(as_bf16x8(g.bk[st][ks]), qlo_lds[(ht * KS + ks) * 64 + lane], al);
        else
          al = mfma_bf16(as_bf16x8(g.bk[st][ks]), qlo[ht][ks], al);
      }
      sacc[st][ht] = kTwoChains ? acch + accl : acch;
    }
  if ((ROLL & 2) && nx.valid) load_bk<DH, R, HT>(g, nx.cb, nx.tb, nx.last, lane);

  // online softmax per head, and the value-product operand C
  bf16x8_t cop[HT];
#pragma unroll
  for (int ht = 0; ht < HT; ++ht) {
    float s[2][NT];
    float av[2][4];
    float bmax = -INFINITY;
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int k = 0; k < NT; ++k) {
        float ak[R];
        unpack_rank<R>(g.ak[st][ht][k], ak);
        unpack_rank<R>(g.av[st][ht][k], &av[st][k * R]);
        float v = 0.f;
#pragma unroll
        for (int rr = 0; rr < R; ++rr) v = fmaf(ak[rr], sacc[st][ht][k * R + rr], v);
        const bool valid = tb + (st * 16 + lg * 4) / R + k <= last;
        s[st][k] = valid ? v : -INFINITY;
        bmax = max_nn(bmax, s[st][k]);
      }
    bmax = lane_group_max_nn(bmax);
    const float m_new = max_nn(m_run[ht], bmax);
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
        for (int rr = 0; rr < R; ++rr) cv[st * 4 + k * R + rr] = p * av[st][k * R + rr];
      }
    l_run[ht] = l_run[ht] * alpha + psum;
    if constexpr (DH == 64) cop[ht] = pack8(cv);
    else cop[ht] = pack8_int(cv);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) oacc[ht][dt] *= alpha;
  }
  if ((ROLL & 4) && nx.valid) load_heads<DH, R, HT>(g, nx.cb, h, nx.tb, nx.last, lane);

  // value product: A operand = B_V^T in the k-slot order of the C operand
  // (slot j of lane group lg: row 4*lg + j for j < 4, row 16 + 4*lg + j - 4
  // after), two transposed reads of four rows at column 16*dt + li each
  wave_lds_fence();
  const bf16_t* vrow = lbv + (4 * lg + (li >> 2)) * LROW + 4 * (li & 3);
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    const uint2 lo = lds_read_tr16(vrow + dt * 16);
    const uint2 hi = lds_read_tr16(vrow + 16 * LROW + dt * 16);
    const bf16x8_t bvop = as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) oacc[ht][dt] = mfma_bf16(bvop, cop[ht], oacc[ht][dt]);
  }
  wave_lds_fence();
  // the parts of the next block not loaded above
  if (nx.valid) {
    if constexpr (!(ROLL & 1)) load_bv<DH, R, HT>(g, nx.cb, nx.tb, nx.last, lane);
    if constexpr (!(ROLL & 2)) load_bk<DH, R, HT>(g, nx.cb, nx.tb, nx.last, lane);
    if constexpr (!(ROLL & 4)) load_heads<DH, R, HT>(g, nx.cb, h, nx.tb, nx.last, lane);
  }
}

// Issue priority by progress: a wave that has done fewer of its blocks than
// the others keeps a higher priority, so the waves of a CU (two workgroups)
// finish together.  With equal priorities the arbiter favours the oldest
// waves, and the workgroups dispatched second on each CU ran about 18 %
// behind the first ones, leaving a tail in which half the CU's waves stream.
__device__ __forceinline__ void prio_by_progress(int done, int total) {
  const int ph = (4 * done) / total;   // 0..3, uniform
  if (ph == 0) __builtin_amdgcn_s_setprio(3);
  else if (ph == 1) __builtin_amdgcn_s_setprio(2);
  else if (ph == 2) __builtin_amdgcn_s_setprio(1);
  else __builtin_amdgcn_s_setprio(0);
}

// PAGED: cache rows through the block table, and per-sequence key counts.
template <int DH, int R, int HT, bool PAGED>
__global__ void __launch_bounds__(64 * decode_waves(DH), 2) decode_mfma_kernel(AttnArgs a, int64_t ctx_len, int64_t chunk,
                                                          int64_t n_chunks, float* ws) {
  using C = DecodeMfmaCfg<DH, R, HT>;
  constexpr int KS = C::KS, DT = C::DT, VBT = C::VBT, HP = C::HP, LROW = C::LROW, OST = C::OST;
  extern __shared__ __align__(16) unsigned char smem[];
  // the wave index is uniform within a wave: keep it scalar, so per-block
  // addresses (and page lookups) stay on the scalar unit
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int li = lane & 15, lg = lane >> 4;
  const int h = a.h;
  const int64_t b = blockIdx.y, c = blockIdx.x;
  const int64_t t0 = c * chunk;
  const int64_t len = PAGED ? seq_keys(a, b, ctx_len) : ctx_len;
  if (PAGED && t0 >= len) {                  // past this sequence's keys: an empty partial
    float* P = ws + (b * n_chunks + c) * (int64_t)h * (DH + 2);
    for (int i = threadIdx.x; i < h * (DH + 2); i += blockDim.x) P[i] = i % (DH + 2) ? 0.f : -INFINITY;
    return;
  }
  const int64_t t1 = (t0 + chunk < len) ? t0 + chunk : len;
  const int64_t row0 = b * a.max_seq + t0;   // first cache row of this chunk (dense)
  const ChunkBase cb = {reinterpret_cast<const bf16_t*>(a.c_ak) + row0 * h * R,
                        reinterpret_cast<const bf16_t*>(a.c_bk) + row0 * R * DH,
                        reinterpret_cast<const bf16_t*>(a.c_av) + row0 * h * R,
                        reinterpret_cast<const bf16_t*>(a.c_bv) + row0 * R * DH};
  const int last = (int)(t1 - t0) - 1;      // chunk-local index of the last token
  // Loads of value block vb: dense, from the chunk's base at token vb*VBT;
  // paged, from the block's own first row (so its tokens count from 0).
  auto load = [&](BlockRegs<DH, R, HT>& g, int vb) {
    if constexpr (PAGED) {
      const int64_t row = paged_row(a.pm, b, t0 + (int64_t)vb * VBT);
      const ChunkBase pb = {reinterpret_cast<const bf16_t*>(a.c_ak) + row * h * R,
                            reinterpret_cast<const bf16_t*>(a.c_bk) + row * R * DH,
                            reinterpret_cast<const bf16_t*>(a.c_av) + row * h * R,
                            reinterpret_cast<const bf16_t*>(a.c_bv) + row * R * DH};
      load_block<DH, R, HT>(g, pb, h, 0, last - vb * VBT, lane);
    } else {
      load_block<DH, R, HT>(g, cb, h, vb * VBT, last, lane);
    }
  };
  const int nvb = (last + VBT) / VBT;
  // The load source of value block vb (valid when the block exists).
  auto next_of = [&](int vb) {
    NextBlock nx;
    nx.valid = vb < nvb;
    if constexpr (PAGED) {
      const int64_t row = paged_row(a.pm, b, t0 + (int64_t)(nx.valid ? vb : 0) * VBT);
      nx.cb = {reinterpret_cast<const bf16_t*>(a.c_ak) + row * h * R,
               reinterpret_cast<const bf16_t*>(a.c_bk) + row * R * DH,
               reinterpret_cast<const bf16_t*>(a.c_av) + row * h * R,
               reinterpret_cast<const bf16_t*>(a.c_bv) + row * R * DH};
      nx.tb = 0;
      nx.last = last - vb * VBT;
    } else {
      nx.cb = cb;
      nx.tb = vb * VBT;
      nx.last = last;
    }
    return nx;
  };

  // The query factors ([h][rq] then [rq][DH], or the plain Q [h][DH]) are
  // staged in LDS.  Their first 4 * THREADS elements are loaded before the first
  // cache blocks' loads (two blocks per wave at d_h = 64, one at d_h = 128), so
  // they do not queue behind them; the rest after.
  const bf16_t* AQ = reinterpret_cast<const bf16_t*>(a.a_q);
  const bf16_t* BQ = reinterpret_cast<const bf16_t*>(a.b_q);
  const int64_t qtok = b * a.q_bstride_tok;
  const int rq = a.rq;
  const int nqa = rq ? h * rq : h * DH, nq = nqa + (rq ? rq * DH : 0);
  auto q_elem = [&](int i) {
    return i < nqa ? (rq ? AQ[qtok * h * rq + i] : BQ[qtok * h * DH + i]) : BQ[qtok * rq * DH + (i - nqa)];
  };
  bf16_t qv[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int i = threadIdx.x + C::THREADS * j;
    qv[j] = i < nq ? q_elem(i) : bf16_t(0);
  }
  BlockRegs<DH, R, HT> r0;
  BlockRegs<DH, R, HT> r1;
  if (wave < nvb) load(r0, wave);
  if constexpr (C::kPrefetch) {
    if (wave + C::NW < nvb) load(r1, wave + C::NW);
  }

  // ---- query operand, via the query factors staged in LDS (one round trip).
  //      Lane (head = 16*ht + li, slice lg) holds q[head][lg*DH/4 + 8*ks + j].
  bf16x8_t qop[HT][KS], qlo[HT][KS];   // q = hi + lo
  // the wave's lo halves in LDS, past the loop's B_V tiles (not the staged factors)
  bf16x8_t* qlo_lds = reinterpret_cast<bf16x8_t*>(smem + C::kLoopBytes) + wave * HT * KS * 64;
  {
    bf16_t* qa = reinterpret_cast<bf16_t*>(smem);     // [h][rq], or the plain Q [h][DH]
    bf16_t* qb = qa + nqa;                             // [rq][DH]
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int i = threadIdx.x + C::THREADS * j;
      if (i < nq) qa[i] = qv[j];
    }
    for (int i = threadIdx.x + 4 * C::THREADS; i < nq; i += C::THREADS) qa[i] = q_elem(i);
    __syncthreads();
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
      const int head = ht * 16 + li;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int d0 = 32 * ks + 8 * lg;   // the slot mapping of the B~_K operand
        float v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = 0.f;
        if (head < h) {
          if (rq == 0) {
#pragma unroll
            for (int j = 0; j < 8; ++j) v[j] = bf16_to_f32(qa[head * DH + d0 + j]);
          } else {
            for (int r = 0; r < rq; ++r) {
              const float ar = bf16_to_f32(qa[head * rq + r]);
#pragma unroll
              for (int j = 0; j < 8; ++j) v[j] = fmaf(ar, bf16_to_f32(qb[r * DH + d0 + j]), v[j]);
            }
          }
#pragma unroll
          for (int j = 0; j < 8; ++j) v[j] *= a.q_scale;
        }
        // q = hi + lo with the hardware conversion (the prologue has registers
        // to spare, and it sits on every workgroup's latency path)
        float vl[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) vl[j] = v[j] - bf16_to_f32(f32_to_bf16(v[j]));
        qop[ht][ks] = pack8(v);
        if constexpr (C::kQloLds)
          qlo_lds[(ht * KS + ks) * 64 + lane] = pack8(vl);
        else
          qlo[ht][ks] = pack8(vl);
      }
    }
    __syncthreads();
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
  // the paged form's page lookups leave no registers for a rolled B_V at
  // d_h = 128 with two head tiles and rank 2
  constexpr int kRoll = (PAGED && DH == 128 && HT == 2 && R == 2) ? 0 : C::kRoll;
  // Each register set is reloaded with its next block part by part while the
  // current block is computed (compute_block), so loads stay in flight.
  const NextBlock none = {false, cb, 0, 0};
  const int wtotal = (nvb - wave + C::NW - 1) / C::NW;   // this wave's blocks (at least 1 where it has any)
  if constexpr (C::kPrefetch) {
    // two register sets in flight: blocks vb and vb+4 of this wave
    for (int vb = wave; vb < nvb; vb += 2 * C::NW) {
      prio_by_progress((vb - wave) / C::NW, wtotal);
      compute_block<DH, R, HT, kRoll>(r0, lbv, vb * VBT, last, none, h, lane, qop, qlo, qlo_lds, m_run, l_run, oacc);
      if (vb + 2 * C::NW < nvb) load(r0, vb + 2 * C::NW);
      if (vb + C::NW < nvb) {
        compute_block<DH, R, HT, kRoll>(r1, lbv, (vb + C::NW) * VBT, last, none, h, lane, qop, qlo, qlo_lds, m_run, l_run,
                                 oacc);
        if (vb + 3 * C::NW < nvb) load(r1, vb + 3 * C::NW);
      }
    }
  } else if constexpr (kRoll == 0) {
    for (int vb = wave; vb < nvb; vb += C::NW) {
      // (not with a paged cache at d_h = 128, whose registers it would spill)
      if constexpr (!(PAGED && DH == 128)) prio_by_progress((vb - wave) / C::NW, wtotal);
      if (vb != wave) load(r0, vb);
      compute_block<DH, R, HT, kRoll>(r0, lbv, vb * VBT, last, none, h, lane, qop, qlo, qlo_lds, m_run, l_run, oacc);
    }
  } else {
    // one register set, reloaded with the wave's next block part by part
    for (int vb = wave; vb < nvb; vb += C::NW) {
      prio_by_progress((vb - wave) / C::NW, wtotal);
      compute_block<DH, R, HT, kRoll>(r0, lbv, vb * VBT, last, next_of(vb + C::NW), h, lane, qop, qlo, qlo_lds, m_run,
                                      l_run, oacc);
    }
  }

  __builtin_amdgcn_s_setprio(0);
  // ---- merge the waves (fixed order) and write this chunk's partial
#pragma unroll
  for (int ht = 0; ht < HT; ++ht) {
    l_run[ht] = lane_group_sum(l_run[ht]);
  }
  __syncthreads();
  float* mbuf = reinterpret_cast<float*>(smem);  // [NW][HP]
  float* lbuf = mbuf + C::NW * HP;                // [NW][HP]
  float* obuf = lbuf + C::NW * HP;                // [NW][HP][OST]
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
    for (int w = 1; w < C::NW; ++w) M = fmaxf(M, mbuf[w * HP + head]);
    const float sc = fast_exp2(m_run[ht] - M);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) oacc[ht][dt] *= sc;
  }
  // every wave's accumulators to its own slot; the partial is their sum in
  // wave order
#pragma unroll
  for (int ht = 0; ht < HT; ++ht)
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
      *reinterpret_cast<f32x4_t*>(obuf + (wave * HP + ht * 16 + li) * OST + dt * 16 + lg * 4) = oacc[ht][dt];
  __syncthreads();
  const int64_t cstride = (int64_t)h * (DH + 2);
  float* P = ws + (b * n_chunks + c) * cstride;
  for (int idx = threadIdx.x; idx < h * DH; idx += blockDim.x) {
    const int head = idx / DH, d = idx - head * DH;
    float o = obuf[head * OST + d];
#pragma unroll
    for (int w = 1; w < C::NW; ++w) o += obuf[(w * HP + head) * OST + d];
    P[head * (DH + 2) + 2 + d] = o;
  }
  for (int head = threadIdx.x; head < h; head += blockDim.x) {
    float M = mbuf[head];
    for (int w = 1; w < C::NW; ++w) M = fmaxf(M, mbuf[w * HP + head]);
    float L = 0.f;
    for (int w = 0; w < C::NW; ++w) L = fmaf(fast_exp2(mbuf[w * HP + head] - M), lbuf[w * HP + head], L);
    P[head * (DH + 2)] = M;
    P[head * (DH + 2) + 1] = L;
  }

}

// The shape conditions of the matrix-core decode: everything but the operand
// alignment, which depends on the caller's pointers.
bool decode_mfma_shape_ok(int dtype, const AttnArgs& a) {
  if (dtype != kBF16) return false;
  if (a.rk != a.rv || !(a.rk == 1 || a.rk == 2 || a.rk == 4)) return false;
  if (!(a.d_h == 64 || a.d_h == 128)) return false;
  if (a.h > 64) return false;
  if (a.d_h == 128 && a.h > 32) return false;  // three head tiles at d_h = 128 spill registers
  if (a.rk == 1 && a.h > 48) return false;     // so do four at rank 1
  const size_t qbytes = (a.rq ? (size_t)a.rq * (a.h + a.d_h) : (size_t)a.h * a.d_h) * sizeof(bf16_t);
  if (qbytes > kDecodeMfmaQueryLds) return false;
  if (a.pm.block_table && a.pm.page_tokens % 32) return false;   // pages of whole value blocks
  return true;
}

bool decode_mfma_supported(int dtype, const AttnArgs& a) {
  if (!decode_mfma_shape_ok(dtype, a)) return false;
  const void* ptrs[5] = {a.b_q, a.c_ak, a.c_bk, a.c_av, a.c_bv};
  for (int i = 0; i < 5; ++i)
    if (((uintptr_t)ptrs[i]) % 16) return false;
  return true;
}

// Tokens one workgroup covers per step (one value block per wave).
int64_t decode_mfma_wave_tokens(const AttnArgs& a) { return decode_waves(a.d_h) * (32 / a.rk); }

// Workgroups the plan aims for: one round of the CUs' resident waves (eight
// per CU).
int64_t decode_mfma_target_workgroups(const AttnArgs& a) { return 2048 / decode_waves(a.d_h); }

template <int DH, int R, int HT>
static void launch_cfg(const AttnArgs& a, int64_t ctx_len, int64_t chunk, int64_t n_chunks, float* ws,
                       hipStream_t st) {
  using C = DecodeMfmaCfg<DH, R, HT>;
  static_assert(C::kLds >= kDecodeMfmaQueryLds, "LDS area of the staged query factors");
  const dim3 grid((unsigned)n_chunks, (unsigned)a.n_batch);
  if (a.pm.block_table)
    hipLaunchKernelGGL((decode_mfma_kernel<DH, R, HT, true>), grid, dim3(C::THREADS), C::kLds, st, a, ctx_len, chunk,
                       n_chunks, ws);
  else
    hipLaunchKernelGGL((decode_mfma_kernel<DH, R, HT, false>), grid, dim3(C::THREADS), C::kLds, st, a, ctx_len, chunk,
                       n_chunks, ws);
}

template <int DH, int R>
static void launch_dh_r(const AttnArgs& a, int64_t ctx_len, int64_t chunk, int64_t n_chunks, float* ws,
                        hipStream_t st) {
  const int ht = (a.h + 15) / 16;
  switch (ht) {
    case 1: launch_cfg<DH, R, 1>(a, ctx_len, chunk, n_chunks, ws, st); break;
    case 2: launch_cfg<DH, R, 2>(a, ctx_len, chunk, n_chunks, ws, st); break;
    default:
      if constexpr (DH == 64) {
        if (ht == 3)
          launch_cfg<DH, R, 3>(a, ctx_len, chunk, n_chunks, ws, st);
        else if constexpr (R > 1)
          launch_cfg<DH, R, 4>(a, ctx_len, chunk, n_chunks, ws, st);
      }
      break;
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
