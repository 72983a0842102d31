// Factor-cache append: cache[b, start_pos + s] = factors[b, s] for the four
// key/value factor tensors, as a bit copy ("Tensor Product Attention Is All
// You Need" review on coreui.cn, code walk-through 前向传播: the cache writes
// at [:bsz, start_pos:start_pos+seqlen]).
//
// One launch covers all four tensors (blockIdx.y).  Each sequence's block of
// S tokens is contiguous in the source and in the cache, so the copy runs over
// (sequence, byte-range) with the widest unit that every row, stride and
// pointer allows.  The paged form copies token rows to the pool rows its block
// table names.
#include "kernels.h"

namespace tpa {

// The copy touches each byte once, so both sides carry the non-temporal hint:
// at 32 x 16,384 tokens (738 MB each way) it took the copy from 258 to 237 us
// (the hint on the loads alone gained nothing, on the stores alone 10 us).
template <typename U>
__device__ __forceinline__ U load_once(const U* p) {
  if constexpr (sizeof(U) == 16) {
    typedef unsigned int v4u __attribute__((ext_vector_type(4)));
    const v4u t = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(p));
    return U{t.x, t.y, t.z, t.w};
  } else {
    return __builtin_nontemporal_load(p);
  }
}

template <typename U>
__device__ __forceinline__ void store_once(U* p, const U& v) {
  if constexpr (sizeof(U) == 16) {
    typedef unsigned int v4u __attribute__((ext_vector_type(4)));
    __builtin_nontemporal_store(v4u{v.x, v.y, v.z, v.w}, reinterpret_cast<v4u*>(p));
  } else {
    __builtin_nontemporal_store(v, p);
  }
}

template <typename U>
__global__ void __launch_bounds__(256) append_kernel(AppendArgs a) {
  const int t = blockIdx.y;
  const int64_t units_per_seq = a.width_bytes[t] * a.S / (int64_t)sizeof(U);
  const int64_t total = units_per_seq * a.n_batch;
  const char* src = reinterpret_cast<const char*>(a.src[t]);
  char* dst = reinterpret_cast<char*>(a.dst[t]) + a.start_pos * a.width_bytes[t];
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int64_t b = idx / units_per_seq;
    const int64_t u = idx - b * units_per_seq;
    const U v = load_once(reinterpret_cast<const U*>(src + b * a.src_bstride[t]) + u);
    store_once(reinterpret_cast<U*>(dst + b * a.dst_bstride[t]) + u, v);
  }
}

static bool all_multiple(const AppendArgs& a, int64_t unit) {
  for (int t = 0; t < 4; ++t) {
    if ((a.width_bytes[t] * a.S) % unit || a.src_bstride[t] % unit || a.dst_bstride[t] % unit) return false;
    if (((uintptr_t)a.src[t]) % unit || ((uintptr_t)a.dst[t] + a.start_pos * a.width_bytes[t]) % unit) return false;
  }
  return true;
}

hipError_t launch_append(const AppendArgs& a, hipStream_t st) {
  int64_t max_bytes = 0;
  for (int t = 0; t < 4; ++t) {
    const int64_t v = a.width_bytes[t] * a.S * a.n_batch;
    if (v > max_bytes) max_bytes = v;
  }
  auto grid_for = [&](int64_t unit) {
    int64_t blocks = (max_bytes / unit + 255) / 256;
    if (blocks > 16384) blocks = 16384;
    if (blocks < 1) blocks = 1;
    return dim3((unsigned)blocks, 4);
  };
  if (all_multiple(a, 16))
    hipLaunchKernelGGL(append_kernel<uint4>, grid_for(16), dim3(256), 0, st, a);
  else if (all_multiple(a, 4))
    hipLaunchKernelGGL(append_kernel<uint32_t>, grid_for(4), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(append_kernel<uint16_t>, grid_for(2), dim3(256), 0, st, a);
  return hipGetLastError();
}

// Paged cache: token s of sequence b goes to position start_pos[b] + s, i.e.
// to the pool row the block table gives for it; positions outside
// [0, max_pos) are skipped.  One thread copies one unit of one token's row.
template <typename U>
__global__ void __launch_bounds__(256) append_paged_kernel(PagedAppendArgs a) {
  const int t = blockIdx.y;
  const int64_t units_per_tok = a.width_bytes[t] / (int64_t)sizeof(U);
  const int64_t total = units_per_tok * a.S * a.n_batch;
  const char* src = reinterpret_cast<const char*>(a.src[t]);
  char* dst = reinterpret_cast<char*>(a.dst[t]);
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int64_t tok = idx / units_per_tok;
    const int64_t u = idx - tok * units_per_tok;
    const int64_t b = tok / a.S, s = tok - b * a.S;
    const int64_t pos = (int64_t)a.start_pos[b] + s;
    if (pos < 0 || pos >= a.max_pos) continue;
    const int64_t row = paged_row(a.pm, b, pos);
    const U v = reinterpret_cast<const U*>(src + b * a.src_bstride[t] + s * a.width_bytes[t])[u];
    reinterpret_cast<U*>(dst + row * a.width_bytes[t])[u] = v;
  }
}

static bool paged_multiple(const PagedAppendArgs& a, int64_t unit) {
  for (int t = 0; t < 4; ++t) {
    if (a.width_bytes[t] % unit || a.src_bstride[t] % unit) return false;
    if (((uintptr_t)a.src[t]) % unit || ((uintptr_t)a.dst[t]) % unit) return false;
  }
  return true;
}

hipError_t launch_append_paged(const PagedAppendArgs& a, hipStream_t st) {
  int64_t max_bytes = 0;
  for (int t = 0; t < 4; ++t) {
    const int64_t v = a.width_bytes[t] * a.S * a.n_batch;
    if (v > max_bytes) max_bytes = v;
  }
  auto grid_for = [&](int64_t unit) {
    int64_t blocks = (max_bytes / unit + 255) / 256;
    if (blocks > 16384) blocks = 16384;
    if (blocks < 1) blocks = 1;
    return dim3((unsigned)blocks, 4);
  };
  if (paged_multiple(a, 16))
    hipLaunchKernelGGL(append_paged_kernel<uint4>, grid_for(16), dim3(256), 0, st, a);
  else if (paged_multiple(a, 4))
    hipLaunchKernelGGL(append_paged_kernel<uint32_t>, grid_for(4), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(append_paged_kernel<uint16_t>, grid_for(2), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace tpa
