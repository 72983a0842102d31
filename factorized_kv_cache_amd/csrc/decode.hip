// Decode attention over the factor cache: one new query per sequence.
//
// Scores use the factored form s_t = sum_r A_K[t,h,r] (B~_K[t,r,:] . q_h) with
// q pre-scaled by log2(e) / (R_Q R_K sqrt(d_h)), so keys are never rebuilt;
// values are accumulated as sum_t sum_r (p_t A_V[t,h,r]) B_V[t,r,:] and scaled
// by 1/R_V at the end.  ("Tensor Product Attention Is All You Need" review on
// coreui.cn: the K_t and V_t equations of 核心机制总结 and the attention of the
// code walk-through 前向传播; question 2: the cached key factors are already
// rotated, so decode does no rotation.)
//
// The context is split into chunks, one workgroup per (sequence, chunk); each
// writes its partial (running max m, sum l, unnormalised acc[d_h]) per head to
// the workspace, and a combine pass merges the chunks in index order, so the
// result does not depend on scheduling.  With ragged lengths, chunks past a
// sequence's keys write an empty partial (m = -inf, l = 0, acc = 0), which the
// combine weighs by 0; with a paged cache every token's row goes through the
// block table.
#include <mutex>

#include "kernels.h"
#include "mfma.h"

namespace tpa {

constexpr int kDecodeThreads = 256;
constexpr int kDecodeTile = 16;        // tokens per inner step
constexpr int kMaxHeadElems = 8192;    // h * d_h limit of this library
constexpr int kMaxOutPerThread = kMaxHeadElems / kDecodeThreads;

// Query formation for sequence b into LDS, fp32, pre-scaled.
template <typename T>
__device__ void form_query(const AttnArgs& a, int64_t b, int64_t s, float* qs) {
  const int h = a.h, dh = a.d_h;
  const T* AQ = reinterpret_cast<const T*>(a.a_q);
  const T* BQ = reinterpret_cast<const T*>(a.b_q);
  const int64_t tok = b * a.q_bstride_tok + s;
  for (int idx = threadIdx.x; idx < h * dh; idx += blockDim.x) {
    const int hh = idx / dh, d = idx - hh * dh;
    float v;
    if (a.rq == 0) {
      v = ldf(BQ, tok * h * dh + idx);
    } else {
      v = 0.f;
      for (int r = 0; r < a.rq; ++r)
        v = fmaf(ldf(AQ, (tok * h + hh) * a.rq + r), ldf(BQ, (tok * a.rq + r) * dh + d), v);
    }
    qs[idx] = v * a.q_scale;
  }
}

template <typename T>
__global__ void __launch_bounds__(kDecodeThreads) decode_generic_kernel(AttnArgs a, int64_t ctx_len,
                                                                        int64_t chunk, int64_t n_chunks,
                                                                        float* ws) {
  extern __shared__ float smem[];
  const int h = a.h, dh = a.d_h;
  float* qs = smem;                      // [h][d_h]
  float* sc = qs + h * dh;               // [tile][h] scores, then probabilities
  float* mrow = sc + kDecodeTile * h;    // [h] running max (base-2 units)
  float* lrow = mrow + h;                // [h] running sum
  float* alpha = lrow + h;               // [h] rescale of this step
  __shared__ int64_t rows[kDecodeTile];   // cache rows of the tile's tokens
  const int64_t b = blockIdx.y;
  const int64_t c = blockIdx.x;
  const int64_t len = seq_keys(a, b, ctx_len);
  const int64_t t0 = c * chunk;
  if (t0 >= len) {                       // past this sequence's keys: an empty partial
    float* P = ws + ((b * n_chunks + c) * h) * (int64_t)(dh + 2);
    for (int i = threadIdx.x; i < h * (dh + 2); i += blockDim.x) P[i] = i % (dh + 2) ? 0.f : -INFINITY;
    return;
  }
  const int64_t t1 = (t0 + chunk < len) ? t0 + chunk : len;
  const T* AK = reinterpret_cast<const T*>(a.c_ak);
  const T* BK = reinterpret_cast<const T*>(a.c_bk);
  const T* AV = reinterpret_cast<const T*>(a.c_av);
  const T* BV = reinterpret_cast<const T*>(a.c_bv);

  form_query<T>(a, b, 0, qs);
  for (int hh = threadIdx.x; hh < h; hh += blockDim.x) {
    mrow[hh] = -INFINITY;
    lrow[hh] = 0.f;
  }
  float acc[kMaxOutPerThread];
#pragma unroll
  for (int j = 0; j < kMaxOutPerThread; ++j) acc[j] = 0.f;
  __syncthreads();

  for (int64_t tt0 = t0; tt0 < t1; tt0 += kDecodeTile) {
    if (threadIdx.x < kDecodeTile && tt0 + threadIdx.x < t1) rows[threadIdx.x] = cache_row(a, b, tt0 + threadIdx.x);
    __syncthreads();
    for (int item = threadIdx.x; item < kDecodeTile * h; item += blockDim.x) {
      const int tl = item / h, hh = item - tl * h;
      const int64_t t = tt0 + tl;
      float s = -INFINITY;
      if (t < t1) {
        const int64_t row = rows[tl];
        s = 0.f;
        for (int r = 0; r < a.rk; ++r) {
          const int64_t brow = (row * a.rk + r) * dh;
          float dot = 0.f;
          for (int d = 0; d < dh; ++d) dot = fmaf(ldf(BK, brow + d), qs[hh * dh + d], dot);
          s = fmaf(ldf(AK, (row * h + hh) * a.rk + r), dot, s);
        }
      }
      sc[item] = s;
    }
    __syncthreads();
    for (int hh = threadIdx.x; hh < h; hh += blockDim.x) {
      float mx = mrow[hh];
      for (int tl = 0; tl < kDecodeTile; ++tl) mx = fmaxf(mx, sc[tl * h + hh]);
      const float al = fast_exp2(mrow[hh] - mx);
      float sum = 0.f;
      for (int tl = 0; tl < kDecodeTile; ++tl) {
        const float p = fast_exp2(sc[tl * h + hh] - mx);
        sc[tl * h + hh] = p;
        sum += p;
      }
      lrow[hh] = lrow[hh] * al + sum;
      mrow[hh] = mx;
      alpha[hh] = al;
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kMaxOutPerThread; ++j) {
      const int idx = threadIdx.x + j * kDecodeThreads;
      if (idx >= h * dh) break;
      const int hh = idx / dh, d = idx - hh * dh;
      float o = acc[j] * alpha[hh];
      for (int tl = 0; tl < kDecodeTile; ++tl) {
        const int64_t t = tt0 + tl;
        if (t >= t1) break;
        const float p = sc[tl * h + hh];
        const int64_t row = rows[tl];
        for (int r = 0; r < a.rv; ++r)
          o = fmaf(p * ldf(AV, (row * h + hh) * a.rv + r), ldf(BV, (row * a.rv + r) * dh + d), o);
      }
      acc[j] = o;
    }
    __syncthreads();
  }

  float* P = ws + ((b * n_chunks + c) * h) * (int64_t)(dh + 2);
  for (int hh = threadIdx.x; hh < h; hh += blockDim.x) {
    P[hh * (dh + 2)] = mrow[hh];
    P[hh * (dh + 2) + 1] = lrow[hh];
  }
#pragma unroll
  for (int j = 0; j < kMaxOutPerThread; ++j) {
    const int idx = threadIdx.x + j * kDecodeThreads;
    if (idx >= h * dh) break;
    const int hh = idx / dh, d = idx - hh * dh;
    P[hh * (dh + 2) + 2 + d] = acc[j];
  }
}

// Log-sum-exp merge of the chunk partials of one (head, sequence); one
// workgroup per (head, sequence).  Thread (d, g) sums the chunks c = g, g+G, ...
// of element d (G = 256 / d_h groups) in that order, loading 32 of its
// partial values at a time, so that the merge costs one memory round trip per
// 32 chunks of a group (loaded one by one, the 32 chunks of a group at
// 8 x 131073 keys and d_h 128 took 10.8 us); groups are then added in order
// g = 0..G-1.  The chunk maxima and sums are loaded first, so waiting for them
// leaves the partial values in flight, and the overall maximum M and the sum
// L = sum_c 2^(m_c - M) l_c are wave reductions (every wave forms the same
// bits: the pairing order is fixed).
constexpr int kCombineThreads = 256;
constexpr int kCombineRegs = 32;
constexpr int kCombineMaxChunks = 2048;   // LDS: maxima and sums of the chunks

template <typename T>
__global__ void __launch_bounds__(kCombineThreads) decode_combine_kernel(AttnArgs a, int64_t n_chunks,
                                                                         const float* ws) {
  __shared__ float mloc[kCombineMaxChunks];
  __shared__ float lloc[kCombineMaxChunks];
  __shared__ float part[kCombineThreads];
  const int h = a.h, dh = a.d_h;
  const int hh = blockIdx.x;
  const int64_t b = blockIdx.y;
  const float* P = ws + (b * n_chunks * h + hh) * (int64_t)(dh + 2);
  const int64_t cstride = (int64_t)h * (dh + 2);
  const int G = kCombineThreads / dh;
  const int d = threadIdx.x % dh, g = threadIdx.x / dh;
  const int lane = threadIdx.x & 63;
  const bool active = g < G;
  const int nc = (int)n_chunks;

  float m0 = -INFINITY, l0 = 0.f;
  if ((int)threadIdx.x < nc) {
    m0 = P[(int64_t)threadIdx.x * cstride];
    l0 = P[(int64_t)threadIdx.x * cstride + 1];
  }
  float accv[kCombineRegs];
#pragma unroll
  for (int j = 0; j < kCombineRegs; ++j) {
    const int c = g + G * j;
    accv[j] = (active && c < nc) ? P[(int64_t)c * cstride + 2 + d] : 0.f;
  }
  if ((int)threadIdx.x < nc) {
    mloc[threadIdx.x] = m0;
    lloc[threadIdx.x] = l0;
  }
  for (int c = threadIdx.x + blockDim.x; c < nc; c += blockDim.x) {
    mloc[c] = P[(int64_t)c * cstride];
    lloc[c] = P[(int64_t)c * cstride + 1];
  }
  __syncthreads();
  float mx = -INFINITY;
  for (int c = lane; c < nc; c += 64) mx = fmaxf(mx, mloc[c]);
  const float M = wave_max(mx);
  if (M == -INFINITY) {   // every chunk empty: a sequence without keys
    if ((int)threadIdx.x < dh) stf(reinterpret_cast<T*>(a.out), (b * h + hh) * dh + threadIdx.x, 0.f);
    return;
  }
  float lp = 0.f;
  for (int c = lane; c < nc; c += 64) lp = fmaf(fast_exp2(mloc[c] - M), lloc[c], lp);
  const float L = wave_sum(lp);
  float O = 0.f;
#pragma unroll
  for (int j = 0; j < kCombineRegs; ++j) {
    const int c = g + G * j;
    if (c < nc) O = fmaf(fast_exp2(mloc[c] - M), accv[j], O);
  }
  for (int base = g + G * kCombineRegs; active && base < nc; base += G * kCombineRegs) {
#pragma unroll
    for (int j = 0; j < kCombineRegs; ++j) {
      const int c = base + G * j;
      accv[j] = c < nc ? P[(int64_t)c * cstride + 2 + d] : 0.f;
    }
#pragma unroll
    for (int j = 0; j < kCombineRegs; ++j) {
      const int c = base + G * j;
      if (c < nc) O = fmaf(fast_exp2(mloc[c] - M), accv[j], O);
    }
  }
  part[threadIdx.x] = O;
  __syncthreads();
  if ((int)threadIdx.x < dh) {
    float tot = 0.f;
    for (int gg = 0; gg < G; ++gg) tot += part[gg * dh + d];
    T* out = reinterpret_cast<T*>(a.out);
    stf(out, (b * h + hh) * dh + d, tot * (a.v_scale / L));
  }
}

bool decode_mfma_shape_ok(int dtype, const AttnArgs& a);
bool decode_mfma_supported(int dtype, const AttnArgs& a);
int64_t decode_mfma_wave_tokens(const AttnArgs& a);
int64_t decode_mfma_target_workgroups(const AttnArgs& a);
hipError_t launch_decode_mfma(const AttnArgs& a, int64_t ctx_len, int64_t chunk, int64_t n_chunks, float* ws,
                              hipStream_t st);

static DecodePlan plan_generic(int64_t ctx_len) {
  DecodePlan p;
  p.kernel = 0;
  p.chunk_tokens = 256;
  if ((ctx_len + p.chunk_tokens - 1) / p.chunk_tokens > kCombineMaxChunks)
    p.chunk_tokens = (ctx_len + kCombineMaxChunks - 1) / kCombineMaxChunks;
  p.n_chunks = (ctx_len + p.chunk_tokens - 1) / p.chunk_tokens;
  return p;
}

// Matrix-core plan: chunks are whole multiples of the tokens one workgroup
// covers per step (a value block per wave).  Each sequence gets
// floor(target / B) chunks (at least one; the target is one round of resident
// workgroups, decode_mfma_target_workgroups) and its units are
// spread evenly over them, so no sequence ends in a sliver of a chunk: with
// contexts of 2^k + 1 keys (the new token included) rounding the chunk length
// instead left a one-unit chunk per sequence, whose workgroups ran as a nearly
// empty second round (measured 21.5 -> 19.9 us at 16 x 4097 keys, 169 -> 142
// us at 32 x 16,385 KV-only, unchanged at 8 x 131,073).
static DecodePlan plan_mfma(const AttnArgs& a, int64_t ctx_len) {
  DecodePlan p;
  p.kernel = 1;
  const int64_t vw = decode_mfma_wave_tokens(a);
  const int64_t units = (ctx_len + vw - 1) / vw;
  int64_t per_seq = decode_mfma_target_workgroups(a) / a.n_batch;
  if (per_seq < 1) per_seq = 1;
  int64_t cu = (units + per_seq - 1) / per_seq;
  if ((units + cu - 1) / cu > kCombineMaxChunks) cu = (units + kCombineMaxChunks - 1) / kCombineMaxChunks;
  p.chunk_tokens = cu * vw;
  p.n_chunks = (ctx_len + p.chunk_tokens - 1) / p.chunk_tokens;
  return p;
}

DecodePlan plan_decode(int dtype, const AttnArgs& a, int64_t ctx_len) {
  return decode_mfma_supported(dtype, a) ? plan_mfma(a, ctx_len) : plan_generic(ctx_len);
}

static size_t partial_bytes(const DecodePlan& p, const AttnArgs& a) {
  return (size_t)a.n_batch * (size_t)p.n_chunks * (size_t)a.h * (size_t)(a.d_h + 2) * sizeof(float);
}

size_t decode_plan_bytes(const DecodePlan& p, const AttnArgs& a) { return partial_bytes(p, a); }

// Workspace: partials for either plan the shape allows, so the size does not
// depend on pointer alignment.  (The matrix-core plan exists only for the
// shapes that kernel takes: a workgroup step covers waves * (32 / R_K) tokens.)
size_t decode_workspace_bytes(int dtype, const AttnArgs& a) {
  const int64_t ctx_len = a.start_pos + 1;
  const size_t n = partial_bytes(plan_generic(ctx_len), a);
  const size_t m = decode_mfma_shape_ok(dtype, a) ? partial_bytes(plan_mfma(a, ctx_len), a) : 0;
  return n > m ? n : m;
}

// Scratch of the allocation-free decode entry point: the chunk partials live in
// this file-scope device array instead of a caller's workspace.  Every device
// the library runs on holds its own copy until the process ends.  In host code
// the name only identifies the symbol; the device address comes from
// hipGetSymbolAddress, taken once per device with that device current.
static __device__ __align__(256) unsigned char scratch[kDecodeScratchBytes];

namespace {
constexpr int kScratchDevices = 64;
std::once_flag g_scratch_once[kScratchDevices];
void* g_scratch_ptr[kScratchDevices];
hipError_t g_scratch_err[kScratchDevices];
}  // namespace

hipError_t decode_scratch(void** ptr) {
  *ptr = nullptr;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kScratchDevices) return hipErrorInvalidDevice;
  std::call_once(g_scratch_once[dev], [dev] {
    void* p = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = g_scratch_err[dev] == hipSuccess ? p : nullptr;
  });
  if (g_scratch_err[dev] != hipSuccess) return g_scratch_err[dev];
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_decode(int dtype, const AttnArgs& a, int64_t ctx_len, const DecodePlan& p, void* ws,
                         hipStream_t st) {
  float* wsf = reinterpret_cast<float*>(ws);
  if (p.kernel == 1) {
    hipError_t e = launch_decode_mfma(a, ctx_len, p.chunk_tokens, p.n_chunks, wsf, st);
    if (e != hipSuccess) return e;
  } else {
    const size_t lds = sizeof(float) * ((size_t)a.h * a.d_h + (size_t)kDecodeTile * a.h + 3 * (size_t)a.h);
    dim3 grid((unsigned)p.n_chunks, (unsigned)a.n_batch);
    if (dtype == kF32)
      hipLaunchKernelGGL(decode_generic_kernel<float>, grid, dim3(kDecodeThreads), lds, st, a, ctx_len,
                         p.chunk_tokens, p.n_chunks, wsf);
    else
      hipLaunchKernelGGL(decode_generic_kernel<bf16_t>, grid, dim3(kDecodeThreads), lds, st, a, ctx_len,
                         p.chunk_tokens, p.n_chunks, wsf);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  dim3 cgrid((unsigned)a.h, (unsigned)a.n_batch);
  if (dtype == kF32)
    hipLaunchKernelGGL(decode_combine_kernel<float>, cgrid, dim3(kCombineThreads), 0, st, a, p.n_chunks, wsf);
  else
    hipLaunchKernelGGL(decode_combine_kernel<bf16_t>, cgrid, dim3(kCombineThreads), 0, st, a, p.n_chunks, wsf);
  return hipGetLastError();
}

}  // namespace tpa
