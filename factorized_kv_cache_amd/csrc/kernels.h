// Internal launch interface between the C ABI layer (tpa_api.cpp) and the HIP
// kernels.  Arguments arrive here already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"

namespace tpa {

enum Dtype { kF32 = 0, kBF16 = 1 };

// ---- factor projection ------------------------------------------------------
// F[M, N] = X[M, K] * W[N, K]^T, column n of F goes to segment e with
// seg_begin[e] <= n < seg_begin[e+1]; row m = b*S + s lands at
// dst[e] + b*bstride[e] + s*width[e] + (n - seg_begin[e]).  Columns below
// rot_cols are rotated (pairs (2i, 2i+1) of each d_h-run) at start_pos + s.
constexpr int kMaxSeg = 6;
struct ProjArgs {
  const void* x;
  const void* w;
  int64_t M, K, N;
  int64_t S;
  int64_t start_pos;
  int32_t head_dim;
  int32_t rot_cols;      // 0 when rotation is off
  int32_t nseg;
  int32_t vec8;          // 1: head_dim, every segment begin, width and batch
                         // stride are multiples of 8 and every destination is
                         // 16-byte aligned, so 8-column pieces store whole
  int32_t seg_begin[kMaxSeg + 1];
  int32_t width[kMaxSeg];
  int64_t bstride[kMaxSeg];  // elements between sequences
  void* dst[kMaxSeg];
  RopeTable rope;
};
hipError_t launch_factor_proj(int dtype, const ProjArgs& a, hipStream_t st);

// ---- standalone rotary embedding --------------------------------------------
struct RopeArgs {
  void* b;
  int64_t n_tok;  // B*S
  int64_t S;
  int64_t start_pos;
  int32_t rows;
  int32_t head_dim;
  RopeTable rope;
};
hipError_t launch_rope(int dtype, const RopeArgs& a, hipStream_t st);

// ---- cache append -------------------------------------------------------------
struct AppendArgs {
  const void* src[4];
  void* dst[4];
  int64_t width_bytes[4];   // bytes per token
  int64_t src_bstride[4];   // bytes between sequences in src
  int64_t dst_bstride[4];   // bytes between sequences in the cache
  int64_t n_batch, S;
  int64_t start_pos;        // destination token offset
};
hipError_t launch_append(const AppendArgs& a, hipStream_t st);

// ---- paged factor cache ------------------------------------------------------
// Sequence b's token t is row block_table[b * max_pages + t / page_tokens] *
// page_tokens + t % page_tokens of the page pools.  Page slots past max_pages
// and page ids outside [0, n_pages) are clamped (bad table contents give wrong
// values, never accesses outside the pools).
struct PageMap {
  const int32_t* block_table;   // nullptr: dense cache
  int32_t page_tokens;
  int32_t max_pages;
  int32_t n_pages;
};

__device__ __forceinline__ int64_t paged_row(const PageMap& pm, int64_t b, int64_t t) {
  int64_t slot = t / pm.page_tokens;
  slot = slot < pm.max_pages ? slot : pm.max_pages - 1;
  int32_t page = pm.block_table[b * pm.max_pages + slot];
  page = page < 0 ? 0 : (page >= pm.n_pages ? pm.n_pages - 1 : page);
  return (int64_t)page * pm.page_tokens + t % pm.page_tokens;
}

struct PagedAppendArgs {
  const void* src[4];
  void* dst[4];               // page pools
  int64_t width_bytes[4];     // bytes per token
  int64_t src_bstride[4];     // bytes between sequences in src
  int64_t n_batch, S;
  const int32_t* start_pos;   // [n_batch] position of each sequence's token 0
  int64_t max_pos;            // positions >= max_pos (or < 0) are not written
  PageMap pm;
};
hipError_t launch_append_paged(const PagedAppendArgs& a, hipStream_t st);

// ---- attention ---------------------------------------------------------------
// Shared description of the query factors and the cache for both attention
// kernels.  Strides are in elements.
struct AttnArgs {
  const void* a_q;       // [B, S, h, R_Q] (unused when rank_q == 0)
  const void* b_q;       // [B, S, R_Q, d_h] or plain Q [B, S, h, d_h]
  int64_t q_bstride_tok; // tokens between sequences of a_q/b_q
  const void* c_ak;      // cache tensors, [max_batch, max_seq, ...]
  const void* c_bk;
  const void* c_av;
  const void* c_bv;
  int64_t max_seq;
  int32_t h, d_h, rq, rk, rv;
  int64_t n_batch;
  int64_t S;             // queries per sequence (1 for decode)
  int64_t start_pos;     // position of query 0
  int32_t causal;
  float q_scale;         // log2(e) / (R_Q * R_K * sqrt(d_h))  (R_Q -> 1 for plain Q)
  float v_scale;         // 1 / R_V
  void* out;
  // decode over a paged cache (pm.block_table != nullptr) and/or ragged
  // lengths (ctx_lens != nullptr: sequence b has ctx_lens[b] keys, clamped to
  // [0, ctx_len]; a sequence with none gets a zero output)
  PageMap pm;
  const int32_t* ctx_lens;
};

// Cache row of token t of sequence b.
__device__ __forceinline__ int64_t cache_row(const AttnArgs& a, int64_t b, int64_t t) {
  return a.pm.block_table ? paged_row(a.pm, b, t) : b * a.max_seq + t;
}

// Keys of sequence b.
__device__ __forceinline__ int64_t seq_keys(const AttnArgs& a, int64_t b, int64_t ctx_len) {
  if (!a.ctx_lens) return ctx_len;
  const int64_t n = a.ctx_lens[b];
  return n < 0 ? 0 : (n > ctx_len ? ctx_len : n);
}

// Decode split: chunk_tokens keys per workgroup; partial results
// (m, l, acc[d_h]) per (b, chunk, head) in float32, then a combine pass.
struct DecodePlan {
  int64_t chunk_tokens;
  int64_t n_chunks;
  int kernel;            // 0 = general VALU kernel, 1 = MFMA kernel
};
DecodePlan plan_decode(int dtype, const AttnArgs& a, int64_t ctx_len);
size_t decode_workspace_bytes(int dtype, const AttnArgs& a);
size_t decode_plan_bytes(const DecodePlan& p, const AttnArgs& a);   // partials of this plan
hipError_t launch_decode(int dtype, const AttnArgs& a, int64_t ctx_len, const DecodePlan& p, void* ws,
                         hipStream_t st);

// The allocation-free decode's scratch: a static device array of this size per
// device; decode_scratch gives the current device's address (looked up once).
constexpr size_t kDecodeScratchBytes = (size_t)16 << 20;
hipError_t decode_scratch(void** ptr);

hipError_t launch_prefill(int dtype, const AttnArgs& a, hipStream_t st);
// Prefill with a workspace for K and V formed once ([B][h][T][d_h], T =
// start_pos + S): prefill_workspace_bytes is 0 where the shape takes no such
// path; launch_prefill_ws with ws == nullptr, or on such a shape, is
// launch_prefill.  ws holds at least prefill_workspace_bytes, 16-byte aligned.
size_t prefill_workspace_bytes(int dtype, const AttnArgs& a);
hipError_t launch_prefill_ws(int dtype, const AttnArgs& a, void* ws, hipStream_t st);
// Prefill over a shared-basis cache: c_bk / c_bv are the bases B_K [R_K, d_h]
// (unrotated) and B_V [R_V, d_h]; key t is rotated at position t with tab.
hipError_t launch_prefill_shared(int dtype, const AttnArgs& a, const RopeTable& tab, hipStream_t st);
// The same with a workspace (sized by prefill_workspace_bytes), as
// launch_prefill_ws: keys formed and rotated once, then attended.
hipError_t launch_prefill_shared_ws(int dtype, const AttnArgs& a, const RopeTable& tab, void* ws, hipStream_t st);

// ---- shared-basis variant: decode over a cache of head factors ------------------
// AttnArgs as for the decode, except c_bk / c_bv are the bases shared by every
// token, B_K [R_K, d_h] (unrotated) and B_V [R_V, d_h]; c_ak / c_av are the
// cache of head factors.  The rotation table gives the keys' angles.
struct SharedPlan {
  int64_t chunk_tokens;
  int64_t n_chunks;
};
bool shared_decode_supported(int dtype, const AttnArgs& a);
SharedPlan plan_shared_decode(int dtype, const AttnArgs& a, int64_t ctx_len);
size_t shared_decode_workspace_bytes(const SharedPlan& p, const AttnArgs& a);
hipError_t launch_shared_decode(int dtype, const AttnArgs& a, const RopeTable& tab, int64_t ctx_len,
                                const SharedPlan& p, void* ws, hipStream_t st);

// ---- prefill backward --------------------------------------------------------
// AttnArgs as for the forward (a.out unused); gradients are float32.
struct BwdArgs {
  const void* dout;      // [B, S, h*d_h], the call's element type
  float* lse;            // [B, S, h]  base-2 log-sum-exp of each query's scores
  float* dvec;           // [B, S, h]  D = sum_d dO * O, O recomputed in fp32
  float* dq;             // [B, S, h, d_h]       dQ  (workspace)
  float* dk;             // [B, n_keys, h, d_h]  dK  (workspace)
  float* dv;             // [B, n_keys, h, d_h]  dV  (workspace)
  bf16_t* q_hi;          // [B, S, h, d_h]       scaled q^ as bf16 hi + lo (workspace, matrix-core path)
  bf16_t* q_lo;
  bf16_t* k_hi;          // [B, n_keys, h, d_h]  k^ as bf16 hi + lo (workspace, matrix-core path)
  bf16_t* k_lo;
  bf16_t* v_hat;         // [B, n_keys, h, d_h]  v^ (workspace, matrix-core path)
  float* d_aq;           // [B, *, h, R_Q]   (unused for KV-only)
  float* d_bq;           // [B, *, R_Q, d_h] (KV-only: dQ [B, *, h, d_h])
  int64_t dq_bstride;    // tokens between sequences of d_aq / d_bq
  float* d_ak;           // cache layout, capacity dkv_max_seq tokens per sequence
  float* d_bk;
  float* d_av;
  float* d_bv;
  int64_t dkv_max_seq;
};
size_t prefill_backward_workspace_bytes(const AttnArgs& a);
void prefill_backward_carve(const AttnArgs& a, void* ws, BwdArgs& g);
hipError_t launch_prefill_backward(int dtype, const AttnArgs& a, const BwdArgs& g, hipStream_t st);

}  // namespace tpa
