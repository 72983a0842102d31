// libtpa C ABI: argument validation and dispatch to the HIP kernels.
//
// Every entry point checks all of its arguments before it enqueues anything;
// on failure it returns a status and records a message for tpa_last_error()
// in thread-local storage (the library's only state).
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "../../include/tpa.h"
#include "kernels.h"

namespace {

thread_local char g_err[320] = "";

tpa_status fail(tpa_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

tpa_status ok() {
  g_err[0] = '\0';
  return TPA_OK;
}

tpa_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(TPA_ERR_HIP, "%s: HIP error %d (%s)", what, (int)e, hipGetErrorString(e));
}

constexpr int64_t kMaxTokens = (int64_t)1 << 31;

// n_batch * seq_len < 2^31 for positive arguments, without overflowing int64
// on the way (each factor is bounded first).
static bool token_count_ok(int64_t n_batch, int64_t seq_len) {
  return n_batch < kMaxTokens && seq_len < kMaxTokens && n_batch * seq_len < kMaxTokens;
}

// 0 <= start_pos and start_pos + seq_len < 2^31 for 0 < seq_len < 2^31,
// without forming a sum that could overflow.
static bool positions_ok(int64_t start_pos, int64_t seq_len) {
  return start_pos >= 0 && start_pos < kMaxTokens - seq_len;
}

tpa_status check_dims(const tpa_dims* d) {
  if (!d) return fail(TPA_ERR_INVALID_ARGUMENT, "dims is NULL");
  if (d->d_model < 1) return fail(TPA_ERR_INVALID_ARGUMENT, "d_model must be >= 1 (got %d)", d->d_model);
  if (d->n_heads < 1 || d->n_heads > 256)
    return fail(TPA_ERR_INVALID_ARGUMENT, "n_heads must be in 1..256 (got %d)", d->n_heads);
  if (d->head_dim < 2 || d->head_dim > 256 || (d->head_dim & 1))
    return fail(TPA_ERR_INVALID_ARGUMENT, "head_dim must be even and in 2..256 (got %d)", d->head_dim);
  if (d->rank_q < 0 || d->rank_q > 64)
    return fail(TPA_ERR_INVALID_ARGUMENT, "rank_q must be in 0..64 (got %d)", d->rank_q);
  if (d->rank_k < 1 || d->rank_k > 64)
    return fail(TPA_ERR_INVALID_ARGUMENT, "rank_k must be in 1..64 (got %d)", d->rank_k);
  if (d->rank_v < 1 || d->rank_v > 64)
    return fail(TPA_ERR_INVALID_ARGUMENT, "rank_v must be in 1..64 (got %d)", d->rank_v);
  if (!(d->rope_base > 0.0) || !isfinite(d->rope_base))
    return fail(TPA_ERR_INVALID_ARGUMENT, "rope_base must be finite and > 0");
  if (d->dtype != TPA_F32 && d->dtype != TPA_BF16)
    return fail(TPA_ERR_INVALID_ARGUMENT, "unknown dtype %d", d->dtype);
  if ((int64_t)d->n_heads * d->head_dim > 8192)
    return fail(TPA_ERR_UNSUPPORTED, "n_heads * head_dim must be <= 8192 (got %lld)",
                (long long)d->n_heads * d->head_dim);
  return TPA_OK;
}

size_t elem_size(const tpa_dims* d) { return d->dtype == TPA_F32 ? 4 : 2; }

tpa::RopeTable rope_table(const tpa_dims* d) {
  tpa::RopeTable t;
  memset(&t, 0, sizeof(t));
  const int half = d->head_dim / 2;
  for (int i = 0; i < half; ++i)
    t.rev[i] = pow(d->rope_base, -2.0 * (double)i / (double)d->head_dim) / (2.0 * M_PI);
  return t;
}

tpa_status check_cache(const tpa_cache* c) {
  if (!c) return fail(TPA_ERR_INVALID_ARGUMENT, "cache is NULL");
  if (!c->a_k || !c->b_k || !c->a_v || !c->b_v) return fail(TPA_ERR_INVALID_ARGUMENT, "a cache tensor is NULL");
  if (c->max_batch < 1 || c->max_seq < 1)
    return fail(TPA_ERR_INVALID_ARGUMENT, "cache capacity must be at least 1 x 1");
  if (c->max_seq >= kMaxTokens) return fail(TPA_ERR_UNSUPPORTED, "max_seq must be < 2^31");
  return TPA_OK;
}

tpa_status check_paged(const tpa_paged_cache* c, int64_t n_batch) {
  if (!c) return fail(TPA_ERR_INVALID_ARGUMENT, "paged cache is NULL");
  if (!c->a_k || !c->b_k || !c->a_v || !c->b_v) return fail(TPA_ERR_INVALID_ARGUMENT, "a page pool is NULL");
  if (!c->block_table) return fail(TPA_ERR_INVALID_ARGUMENT, "block_table is NULL");
  if (c->n_pages < 1 || c->page_tokens < 1 || c->max_pages < 1 || c->max_batch < 1)
    return fail(TPA_ERR_INVALID_ARGUMENT, "n_pages, page_tokens, max_pages and max_batch must be >= 1");
  if (c->n_pages >= kMaxTokens || c->page_tokens >= kMaxTokens || c->max_pages >= kMaxTokens ||
      c->max_pages * c->page_tokens >= kMaxTokens)
    return fail(TPA_ERR_UNSUPPORTED, "a sequence may hold at most 2^31 - 1 positions");
  if (n_batch > c->max_batch)
    return fail(TPA_ERR_CAPACITY, "n_batch %lld exceeds the table's max_batch %lld", (long long)n_batch,
                (long long)c->max_batch);
  return TPA_OK;
}

tpa_status check_shared(const tpa_shared_cache* c) {
  if (!c) return fail(TPA_ERR_INVALID_ARGUMENT, "shared cache is NULL");
  if (!c->a_k || !c->a_v || !c->b_k || !c->b_v)
    return fail(TPA_ERR_INVALID_ARGUMENT, "a shared-cache tensor or basis is NULL");
  if (c->max_batch < 1 || c->max_seq < 1)
    return fail(TPA_ERR_INVALID_ARGUMENT, "cache capacity must be at least 1 x 1");
  if (c->max_seq >= kMaxTokens) return fail(TPA_ERR_UNSUPPORTED, "max_seq must be < 2^31");
  return TPA_OK;
}

// The shared-basis cache seen through the attention arguments: the head
// factors in the cache slots, the shared bases in place of the dim factors.
tpa_cache shared_as_cache(const tpa_shared_cache* c) {
  tpa_cache v;
  v.a_k = c->a_k;
  v.b_k = const_cast<void*>(c->b_k);
  v.a_v = c->a_v;
  v.b_v = const_cast<void*>(c->b_v);
  v.max_batch = c->max_batch;
  v.max_seq = c->max_seq;
  return v;
}

tpa::PageMap page_map(const tpa_paged_cache* c) {
  tpa::PageMap pm;
  pm.block_table = c->block_table;
  pm.page_tokens = (int32_t)c->page_tokens;
  pm.max_pages = (int32_t)c->max_pages;
  pm.n_pages = (int32_t)c->n_pages;
  return pm;
}

tpa_status check_query(const tpa_dims* d, const tpa_factors* q) {
  if (!q) return fail(TPA_ERR_INVALID_ARGUMENT, "query factors are NULL");
  if (!q->b_q) return fail(TPA_ERR_INVALID_ARGUMENT, "b_q (or plain Q) is NULL");
  if (d->rank_q > 0 && !q->a_q) return fail(TPA_ERR_INVALID_ARGUMENT, "a_q is NULL");
  return TPA_OK;
}

tpa_status resolve_stride(int64_t given, int64_t seq_len, const char* name, int64_t* out) {
  if (given == 0) {
    *out = seq_len;
    return TPA_OK;
  }
  if (given < seq_len) return fail(TPA_ERR_INVALID_ARGUMENT, "%s (%lld) is below seq_len (%lld)", name,
                                   (long long)given, (long long)seq_len);
  *out = given;
  return TPA_OK;
}

tpa::AttnArgs attn_args(const tpa_dims* d, const tpa_factors* q, int64_t q_stride, const tpa_cache* c,
                        int64_t n_batch, int64_t seq_len, int64_t start_pos, int causal, void* out) {
  tpa::AttnArgs a;
  memset(&a, 0, sizeof(a));
  a.a_q = q->a_q;
  a.b_q = q->b_q;
  a.q_bstride_tok = q_stride;
  a.c_ak = c->a_k;
  a.c_bk = c->b_k;
  a.c_av = c->a_v;
  a.c_bv = c->b_v;
  a.max_seq = c->max_seq;
  a.h = d->n_heads;
  a.d_h = d->head_dim;
  a.rq = d->rank_q;
  a.rk = d->rank_k;
  a.rv = d->rank_v;
  a.n_batch = n_batch;
  a.S = seq_len;
  a.start_pos = start_pos;
  a.causal = causal ? 1 : 0;
  const double rq = d->rank_q > 0 ? (double)d->rank_q : 1.0;
  a.q_scale = (float)(1.4426950408889634 / (rq * (double)d->rank_k * sqrt((double)d->head_dim)));
  a.v_scale = (float)(1.0 / (double)d->rank_v);
  a.out = out;
  return a;
}

}  // namespace

extern "C" {

int64_t tpa_packed_weight_rows(const tpa_dims* d) {
  if (check_dims(d) != TPA_OK) return -1;
  const int64_t h = d->n_heads, dh = d->head_dim;
  const int64_t q = d->rank_q > 0 ? h * d->rank_q + d->rank_q * dh : h * dh;
  return q + (h + dh) * ((int64_t)d->rank_k + d->rank_v);
}

int64_t tpa_cache_elems_per_token(const tpa_dims* d) {
  if (check_dims(d) != TPA_OK) return -1;
  return ((int64_t)d->n_heads + d->head_dim) * ((int64_t)d->rank_k + d->rank_v);
}

// The projection shared by both cache forms.  shared != 0: the packed weight
// has no dim-factor rows for K and V (their bases are parameters), so the
// outputs are the query factors and the key/value head factors only.
static tpa_status factor_proj(const tpa_dims* d, const void* x, int64_t n_batch, int64_t seq_len, int64_t start_pos,
                              const void* w_packed, int32_t fuse_rope, const tpa_factors* out, void* stream,
                              bool shared, const char* what) {
  tpa_status st = check_dims(d);
  if (st != TPA_OK) return st;
  if (!x || !w_packed) return fail(TPA_ERR_INVALID_ARGUMENT, "x or w_packed is NULL");
  if (!out) return fail(TPA_ERR_INVALID_ARGUMENT, "out factors are NULL");
  if ((st = check_query(d, out)) != TPA_OK) return st;
  if (!out->a_k || !out->a_v || (!shared && (!out->b_k || !out->b_v)))
    return fail(TPA_ERR_INVALID_ARGUMENT, "a key/value output tensor is NULL");
  if (n_batch < 1 || seq_len < 1) return fail(TPA_ERR_INVALID_ARGUMENT, "n_batch and seq_len must be >= 1");
  if (!token_count_ok(n_batch, seq_len)) return fail(TPA_ERR_UNSUPPORTED, "n_batch * seq_len must be < 2^31");
  if (!positions_ok(start_pos, seq_len))
    return fail(TPA_ERR_INVALID_ARGUMENT, "start_pos must be in 0 .. 2^31 - seq_len");
  int64_t qs, kvs;
  if ((st = resolve_stride(out->q_batch_stride, seq_len, "q_batch_stride", &qs)) != TPA_OK) return st;
  if ((st = resolve_stride(out->kv_batch_stride, seq_len, "kv_batch_stride", &kvs)) != TPA_OK) return st;

  tpa::ProjArgs a;
  memset(&a, 0, sizeof(a));
  const int32_t h = d->n_heads, dh = d->head_dim;
  a.x = x;
  a.w = w_packed;
  a.M = n_batch * seq_len;
  a.K = d->d_model;
  a.N = shared ? tpa_shared_packed_weight_rows(d) : tpa_packed_weight_rows(d);
  a.S = seq_len;
  a.start_pos = start_pos;
  a.head_dim = dh;
  struct Seg {
    int32_t width;
    void* p;
    int64_t stride;
  } segs[6];
  int n = 0;
  if (d->rank_q > 0) {
    segs[n++] = {d->rank_q * dh, out->b_q, qs};
  } else {
    segs[n++] = {h * dh, out->b_q, qs};
  }
  if (!shared) {
    segs[n++] = {d->rank_k * dh, out->b_k, kvs};
    segs[n++] = {d->rank_v * dh, out->b_v, kvs};
  }
  if (d->rank_q > 0) segs[n++] = {h * d->rank_q, out->a_q, qs};
  segs[n++] = {h * d->rank_k, out->a_k, kvs};
  segs[n++] = {h * d->rank_v, out->a_v, kvs};
  a.nseg = n;
  int32_t col = 0;
  for (int e = 0; e < n; ++e) {
    a.seg_begin[e] = col;
    a.width[e] = segs[e].width;
    a.dst[e] = segs[e].p;
    a.bstride[e] = segs[e].stride * segs[e].width;
    col += segs[e].width;
  }
  a.seg_begin[n] = col;
  // the rotated columns: the query dim factors, and the key dim factors unless
  // they are the shared basis
  a.rot_cols = fuse_rope ? (shared ? segs[0].width : segs[0].width + segs[1].width) : 0;
  a.vec8 = dh % 8 == 0;
  for (int e = 0; e < n; ++e)
    if (a.seg_begin[e] % 8 || a.width[e] % 8 || a.bstride[e] % 8 || ((uintptr_t)a.dst[e] & 15)) a.vec8 = 0;
  a.rope = rope_table(d);
  return hip_status(tpa::launch_factor_proj(d->dtype, a, (hipStream_t)stream), what);
}

tpa_status tpa_factor_proj(const tpa_dims* d, const void* x, int64_t n_batch, int64_t seq_len, int64_t start_pos,
                           const void* w_packed, int32_t fuse_rope, const tpa_factors* out, void* stream) {
  return factor_proj(d, x, n_batch, seq_len, start_pos, w_packed, fuse_rope, out, stream, false, "tpa_factor_proj");
}

int64_t tpa_shared_packed_weight_rows(const tpa_dims* d) {
  if (check_dims(d) != TPA_OK) return -1;
  const int64_t h = d->n_heads, dh = d->head_dim;
  const int64_t q = d->rank_q > 0 ? h * d->rank_q + d->rank_q * dh : h * dh;
  return q + h * ((int64_t)d->rank_k + d->rank_v);
}

tpa_status tpa_shared_factor_proj(const tpa_dims* d, const void* x, int64_t n_batch, int64_t seq_len,
                                  int64_t start_pos, const void* w_packed, int32_t fuse_rope, const tpa_factors* out,
                                  void* stream) {
  return factor_proj(d, x, n_batch, seq_len, start_pos, w_packed, fuse_rope, out, stream, true,
                     "tpa_shared_factor_proj");
}

tpa_status tpa_rope_b(const tpa_dims* d, void* b, int64_t n_batch, int64_t seq_len, int32_t rows, int64_t start_pos,
                      void* stream) {
  tpa_status st = check_dims(d);
  if (st != TPA_OK) return st;
  if (!b) return fail(TPA_ERR_INVALID_ARGUMENT, "b is NULL");
  if (n_batch < 1 || seq_len < 1 || rows < 1)
    return fail(TPA_ERR_INVALID_ARGUMENT, "n_batch, seq_len and rows must be >= 1");
  if (!token_count_ok(n_batch, seq_len)) return fail(TPA_ERR_UNSUPPORTED, "n_batch * seq_len must be < 2^31");
  if (!positions_ok(start_pos, seq_len))
    return fail(TPA_ERR_INVALID_ARGUMENT, "start_pos must be in 0 .. 2^31 - seq_len");
  tpa::RopeArgs a;
  memset(&a, 0, sizeof(a));
  a.b = b;
  a.n_tok = n_batch * seq_len;
  a.S = seq_len;
  a.start_pos = start_pos;
  a.rows = rows;
  a.head_dim = d->head_dim;
  a.rope = rope_table(d);
  return hip_status(tpa::launch_rope(d->dtype, a, (hipStream_t)stream), "tpa_rope_b");
}

tpa_status tpa_cache_append(const tpa_dims* d, const tpa_cache* c, const tpa_factors* kv, int64_t n_batch,
                            int64_t seq_len, int64_t start_pos, void* stream) {
  tpa_status st = check_dims(d);
  if (st != TPA_OK) return st;
  if ((st = check_cache(c)) != TPA_OK) return st;
  if (!kv || !kv->a_k || !kv->b_k || !kv->a_v || !kv->b_v)
    return fail(TPA_ERR_INVALID_ARGUMENT, "a key/value factor tensor is NULL");
  if (n_batch < 1 || seq_len < 1) return fail(TPA_ERR_INVALID_ARGUMENT, "n_batch and seq_len must be >= 1");
  if (start_pos < 0) return fail(TPA_ERR_INVALID_ARGUMENT, "start_pos must be >= 0");
  if (n_batch > c->max_batch)
    return fail(TPA_ERR_CAPACITY, "n_batch %lld exceeds max_batch %lld", (long long)n_batch,
                (long long)c->max_batch);
  if (seq_len > c->max_seq || start_pos > c->max_seq - seq_len)
    return fail(TPA_ERR_CAPACITY, "start_pos %lld + seq_len %lld exceeds max_seq %lld", (long long)start_pos,
                (long long)seq_len, (long long)c->max_seq);
  int64_t kvs;
  if ((st = resolve_stride(kv->kv_batch_stride, seq_len, "kv_batch_stride", &kvs)) != TPA_OK) return st;
  const int64_t es = (int64_t)elem_size(d);
  const int64_t h = d->n_heads, dh = d->head_dim;
  const int64_t width[4] = {h * d->rank_k * es, d->rank_k * dh * es, h * d->rank_v * es, d->rank_v * dh * es};
  const void* src[4] = {kv->a_k, kv->b_k, kv->a_v, kv->b_v};
  void* dst[4] = {c->a_k, c->b_k, c->a_v, c->b_v};
  tpa::AppendArgs a;
  memset(&a, 0, sizeof(a));
  for (int t = 0; t < 4; ++t) {
    a.src[t] = src[t];
    a.dst[t] = dst[t];
    a.width_bytes[t] = width[t];
    a.src_bstride[t] = kvs * width[t];
    a.dst_bstride[t] = c->max_seq * width[t];
  }
  a.n_batch = n_batch;
  a.S = seq_len;
  a.start_pos = start_pos;
  return hip_status(tpa::launch_append(a, (hipStream_t)stream), "tpa_cache_append");
}

// Checks shared by the two prefill entry points; fills the kernel arguments.
static tpa_status prefill_args(const tpa_dims* d, const tpa_factors* q, const tpa_cache* c, int64_t n_batch,
                               int64_t seq_len, int64_t start_pos, int32_t causal, void* out, tpa::AttnArgs* a) {
  tpa_status st = check_dims(d);
  if (st != TPA_OK) return st;
  if ((st = check_query(d, q)) != TPA_OK) return st;
  if ((st = check_cache(c)) != TPA_OK) return st;
  if (!out) return fail(TPA_ERR_INVALID_ARGUMENT, "out is NULL");
  if (n_batch < 1 || seq_len < 1) return fail(TPA_ERR_INVALID_ARGUMENT, "n_batch and seq_len must be >= 1");
  if (n_batch > 65535) return fail(TPA_ERR_UNSUPPORTED, "n_batch must be <= 65535");
  if (start_pos < 0) return fail(TPA_ERR_INVALID_ARGUMENT, "start_pos must be >= 0");
  if (n_batch > c->max_batch)
    return fail(TPA_ERR_CAPACITY, "n_batch %lld exceeds max_batch %lld", (long long)n_batch,
                (long long)c->max_batch);
  if (seq_len > c->max_seq || start_pos > c->max_seq - seq_len)
    return fail(TPA_ERR_CAPACITY, "start_pos %lld + seq_len %lld exceeds max_seq %lld", (long long)start_pos,
                (long long)seq_len, (long long)c->max_seq);
  int64_t qs;
  if ((st = resolve_stride(q->q_batch_stride, seq_len, "q_batch_stride", &qs)) != TPA_OK) return st;
  *a = attn_args(d, q, qs, c, n_batch, seq_len, start_pos, causal, out);
  return TPA_OK;
}

tpa_status tpa_prefill_attn(const tpa_dims* d, const tpa_factors* q, const tpa_cache* c, int64_t n_batch,
                            int64_t seq_len, int64_t start_pos, int32_t causal, void* out, void* stream) {
  tpa::AttnArgs a;
  const tpa_status st = prefill_args(d, q, c, n_batch, seq_len, start_pos, causal, out, &a);
  if (st != TPA_OK) return st;
  return hip_status(tpa::launch_prefill(d->dtype, a, (hipStream_t)stream), "tpa_prefill_attn");
}

size_t tpa_prefill_workspace_bytes(const tpa_dims* d, int64_t n_batch, int64_t seq_len, int64_t start_pos) {
  if (check_dims(d) != TPA_OK || n_batch < 1 || seq_len < 1 || start_pos < 0) return 0;
  if (n_batch > 65535 || !positions_ok(start_pos, seq_len)) return 0;   // sizes the call rejects
  tpa_factors q;
  memset(&q, 0, sizeof(q));
  tpa_cache c;
  memset(&c, 0, sizeof(c));
  c.max_seq = start_pos + seq_len;
  const tpa::AttnArgs a = attn_args(d, &q, seq_len, &c, n_batch, seq_len, start_pos, 1, nullptr);
  return tpa::prefill_workspace_bytes(d->dtype, a);
}

// A workspace where one is needed: present, large enough, 16-byte aligned.
static tpa_status check_prefill_workspace(size_t need, const void* workspace, size_t workspace_bytes) {
  if (need == 0) return TPA_OK;
  if (!workspace || workspace_bytes < need)
    return fail(TPA_ERR_WORKSPACE, "prefill workspace needs %zu bytes (got %zu%s)", need, workspace_bytes,
                workspace ? "" : ", NULL");
  if ((uintptr_t)workspace % 16) return fail(TPA_ERR_INVALID_ARGUMENT, "workspace must be 16-byte aligned");
  return TPA_OK;
}

tpa_status tpa_prefill_attn_ws(const tpa_dims* d, const tpa_factors* q, const tpa_cache* c, int64_t n_batch,
                               int64_t seq_len, int64_t start_pos, int32_t causal, void* out, void* workspace,
                               size_t workspace_bytes, void* stream) {
  tpa::AttnArgs a;
  tpa_status st = prefill_args(d, q, c, n_batch, seq_len, start_pos, causal, out, &a);
  if (st != TPA_OK) return st;
  const size_t need = tpa::prefill_workspace_bytes(d->dtype, a);
  if ((st = check_prefill_workspace(need, workspace, workspace_bytes)) != TPA_OK) return st;
  return hip_status(tpa::launch_prefill_ws(d->dtype, a, need > 0 ? workspace : nullptr, (hipStream_t)stream),
                    "tpa_prefill_attn_ws");
}

size_t tpa_decode_workspace_bytes(const tpa_dims* d, int64_t n_batch, int64_t ctx_len) {
  if (check_dims(d) != TPA_OK || n_batch < 1 || ctx_len < 1) return 0;
  if (n_batch > 65535 || ctx_len >= kMaxTokens) return 0;   // sizes the decode call rejects
  tpa_factors q;
  memset(&q, 0, sizeof(q));
  tpa_cache c;
  memset(&c, 0, sizeof(c));
  c.max_seq = ctx_len;
  tpa::AttnArgs a = attn_args(d, &q, 1, &c, n_batch, 1, ctx_len - 1, 1, nullptr);
  return tpa::decode_workspace_bytes(d->dtype, a);
}

// Checks shared by the two dense decode entry points; fills the kernel arguments.
static tpa_status decode_args(const tpa_dims* d, const tpa_factors* q, const tpa_cache* c, int64_t n_batch,
                              int64_t ctx_len, void* out, tpa::AttnArgs* a) {
  tpa_status st = check_dims(d);
  if (st != TPA_OK) return st;
  if ((st = check_query(d, q)) != TPA_OK) return st;
  if ((st = check_cache(c)) != TPA_OK) return st;
  if (!out) return fail(TPA_ERR_INVALID_ARGUMENT, "out is NULL");
  if (n_batch < 1 || ctx_len < 1) return fail(TPA_ERR_INVALID_ARGUMENT, "n_batch and ctx_len must be >= 1");
  if (n_batch > 65535) return fail(TPA_ERR_UNSUPPORTED, "n_batch must be <= 65535");
  if (n_batch > c->max_batch)
    return fail(TPA_ERR_CAPACITY, "n_batch %lld exceeds max_batch %lld", (long long)n_batch,
                (long long)c->max_batch);
  if (ctx_len > c->max_seq)
    return fail(TPA_ERR_CAPACITY, "ctx_len %lld exceeds max_seq %lld", (long long)ctx_len, (long long)c->max_seq);
  int64_t qs;
  if ((st = resolve_stride(q->q_batch_stride, 1, "q_batch_stride", &qs)) != TPA_OK) return st;
  *a = attn_args(d, q, qs, c, n_batch, 1, ctx_len - 1, 1, out);
  return TPA_OK;
}

tpa_status tpa_decode_attn(const tpa_dims* d, const tpa_factors* q, const tpa_cache* c, int64_t n_batch,
                           int64_t ctx_len, void* out, void* workspace, size_t ws_bytes, void* stream) {
  tpa::AttnArgs a;
  tpa_status st = decode_args(d, q, c, n_batch, ctx_len, out, &a);
  if (st != TPA_OK) return st;
  const tpa::DecodePlan p = tpa::plan_decode(d->dtype, a, ctx_len);
  const size_t need = tpa::decode_workspace_bytes(d->dtype, a);
  if (need > 0 && (!workspace || ws_bytes < need))
    return fail(TPA_ERR_WORKSPACE, "decode workspace needs %zu bytes (got %zu%s)", need, ws_bytes,
                workspace ? "" : ", NULL");
  return hip_status(tpa::launch_decode(d->dtype, a, ctx_len, p, workspace, (hipStream_t)stream),
                    "tpa_decode_attn");
}

size_t tpa_decode_noalloc_max_bytes(void) { return tpa::kDecodeScratchBytes; }

tpa_status tpa_decode_attn_noalloc(const tpa_dims* d, const tpa_factors* q, const tpa_cache* c, int64_t n_batch,
                                   int64_t ctx_len, void* out, void* stream) {
  tpa::AttnArgs a;
  tpa_status st = decode_args(d, q, c, n_batch, ctx_len, out, &a);
  if (st != TPA_OK) return st;
  const tpa::DecodePlan p = tpa::plan_decode(d->dtype, a, ctx_len);
  const size_t need = tpa::decode_plan_bytes(p, a);
  if (need > tpa::kDecodeScratchBytes)
    return fail(TPA_ERR_WORKSPACE,
                "this decode needs %zu bytes of partials; the built-in scratch holds %zu (use tpa_decode_attn "
                "with a workspace)", need, tpa::kDecodeScratchBytes);
  void* scratch = nullptr;
  const hipError_t e = tpa::decode_scratch(&scratch);
  if (e != hipSuccess) return hip_status(e, "tpa_decode_attn_noalloc (scratch address)");
  return hip_status(tpa::launch_decode(d->dtype, a, ctx_len, p, scratch, (hipStream_t)stream),
                    "tpa_decode_attn_noalloc");
}

size_t tpa_prefill_backward_workspace_bytes(const tpa_dims* d, int64_t n_batch, int64_t seq_len,
                                            int64_t start_pos) {
  if (check_dims(d) != TPA_OK || n_batch < 1 || seq_len < 1 || start_pos < 0) return 0;
  // sizes the backward call rejects
  if (n_batch > 65535 || !token_count_ok(n_batch, seq_len) || !positions_ok(start_pos, seq_len)) return 0;
  tpa_factors q;
  memset(&q, 0, sizeof(q));
  tpa_cache c;
  memset(&c, 0, sizeof(c));
  c.max_seq = start_pos + seq_len;
  tpa::AttnArgs a = attn_args(d, &q, seq_len, &c, n_batch, seq_len, start_pos, 1, nullptr);
  return tpa::prefill_backward_workspace_bytes(a);
}

tpa_status tpa_prefill_attn_backward(const tpa_dims* d, const tpa_factors* q, const tpa_cache* c, int64_t n_batch,
                                     int64_t seq_len, int64_t start_pos, int32_t causal, const void* dout,
                                     const tpa_factors* dq, const tpa_cache* dkv, void* workspace, size_t ws_bytes,
                                     void* stream) {
  tpa_status st = check_dims(d);
  if (st != TPA_OK) return st;
  if ((st = check_query(d, q)) != TPA_OK) return st;
  if ((st = check_cache(c)) != TPA_OK) return st;
  if (!dout) return fail(TPA_ERR_INVALID_ARGUMENT, "dout is NULL");
  if (!dq || !dq->b_q || (d->rank_q > 0 && !dq->a_q))
    return fail(TPA_ERR_INVALID_ARGUMENT, "a query-factor gradient tensor is NULL");
  if ((st = check_cache(dkv)) != TPA_OK) return st;
  if (n_batch < 1 || seq_len < 1) return fail(TPA_ERR_INVALID_ARGUMENT, "n_batch and seq_len must be >= 1");
  if (n_batch > 65535) return fail(TPA_ERR_UNSUPPORTED, "n_batch must be <= 65535");
  if (start_pos < 0) return fail(TPA_ERR_INVALID_ARGUMENT, "start_pos must be >= 0");
  if (n_batch > c->max_batch || n_batch > dkv->max_batch)
    return fail(TPA_ERR_CAPACITY, "n_batch %lld exceeds max_batch", (long long)n_batch);
  if (seq_len > c->max_seq || start_pos > c->max_seq - seq_len || start_pos + seq_len > dkv->max_seq)
    return fail(TPA_ERR_CAPACITY, "start_pos %lld + seq_len %lld exceeds max_seq", (long long)start_pos,
                (long long)seq_len);
  if ((start_pos + seq_len) + seq_len >= kMaxTokens) return fail(TPA_ERR_UNSUPPORTED, "sequence too long");
  int64_t qs, dqs;
  if ((st = resolve_stride(q->q_batch_stride, seq_len, "q_batch_stride", &qs)) != TPA_OK) return st;
  if ((st = resolve_stride(dq->q_batch_stride, seq_len, "dq->q_batch_stride", &dqs)) != TPA_OK) return st;
  tpa::AttnArgs a = attn_args(d, q, qs, c, n_batch, seq_len, start_pos, causal, nullptr);
  const size_t need = tpa::prefill_backward_workspace_bytes(a);
  if (!workspace || ws_bytes < need)
    return fail(TPA_ERR_WORKSPACE, "backward workspace needs %zu bytes (got %zu%s)", need, ws_bytes,
                workspace ? "" : ", NULL");
  tpa::BwdArgs g;
  memset(&g, 0, sizeof(g));
  tpa::prefill_backward_carve(a, workspace, g);
  g.dout = dout;
  g.d_aq = static_cast<float*>(dq->a_q);
  g.d_bq = static_cast<float*>(dq->b_q);
  g.dq_bstride = dqs;
  g.d_ak = static_cast<float*>(dkv->a_k);
  g.d_bk = static_cast<float*>(dkv->b_k);
  g.d_av = static_cast<float*>(dkv->a_v);
  g.d_bv = static_cast<float*>(dkv->b_v);
  g.dkv_max_seq = dkv->max_seq;
  return hip_status(tpa::launch_prefill_backward(d->dtype, a, g, (hipStream_t)stream), "tpa_prefill_attn_backward");
}

tpa_status tpa_rope_b_backward(const tpa_dims* d, float* g, int64_t n_batch, int64_t seq_len, int32_t rows,
                               int64_t start_pos, void* stream) {
  tpa_status st = check_dims(d);
  if (st != TPA_OK) return st;
  if (!g) return fail(TPA_ERR_INVALID_ARGUMENT, "g is NULL");
  if (n_batch < 1 || seq_len < 1 || rows < 1)
    return fail(TPA_ERR_INVALID_ARGUMENT, "n_batch, seq_len and rows must be >= 1");
  if (!token_count_ok(n_batch, seq_len)) return fail(TPA_ERR_UNSUPPORTED, "n_batch * seq_len must be < 2^31");
  if (!positions_ok(start_pos, seq_len))
    return fail(TPA_ERR_INVALID_ARGUMENT, "start_pos must be in 0 .. 2^31 - seq_len");
  tpa::RopeArgs a;
  memset(&a, 0, sizeof(a));
  a.b = g;
  a.n_tok = n_batch * seq_len;
  a.S = seq_len;
  a.start_pos = start_pos;
  a.rows = rows;
  a.head_dim = d->head_dim;
  a.rope = rope_table(d);
  for (int i = 0; i < d->head_dim / 2; ++i) a.rope.rev[i] = -a.rope.rev[i];   // turn back
  return hip_status(tpa::launch_rope(tpa::kF32, a, (hipStream_t)stream), "tpa_rope_b_backward");
}

tpa_status tpa_paged_cache_append(const tpa_dims* d, const tpa_paged_cache* c, const tpa_factors* kv,
                                  int64_t n_batch, int64_t seq_len, const int32_t* start_pos, void* stream) {
  tpa_status st = check_dims(d);
  if (st != TPA_OK) return st;
  if (!kv || !kv->a_k || !kv->b_k || !kv->a_v || !kv->b_v)
    return fail(TPA_ERR_INVALID_ARGUMENT, "a key/value factor tensor is NULL");
  if (!start_pos) return fail(TPA_ERR_INVALID_ARGUMENT, "start_pos is NULL");
  if (n_batch < 1 || seq_len < 1) return fail(TPA_ERR_INVALID_ARGUMENT, "n_batch and seq_len must be >= 1");
  if (!token_count_ok(n_batch, seq_len)) return fail(TPA_ERR_UNSUPPORTED, "n_batch * seq_len must be < 2^31");
  if ((st = check_paged(c, n_batch)) != TPA_OK) return st;
  int64_t kvs;
  if ((st = resolve_stride(kv->kv_batch_stride, seq_len, "kv_batch_stride", &kvs)) != TPA_OK) return st;
  const int64_t es = (int64_t)elem_size(d);
  const int64_t h = d->n_heads, dh = d->head_dim;
  const int64_t width[4] = {h * d->rank_k * es, d->rank_k * dh * es, h * d->rank_v * es, d->rank_v * dh * es};
  const void* src[4] = {kv->a_k, kv->b_k, kv->a_v, kv->b_v};
  void* dst[4] = {c->a_k, c->b_k, c->a_v, c->b_v};
  tpa::PagedAppendArgs a;
  memset(&a, 0, sizeof(a));
  for (int t = 0; t < 4; ++t) {
    a.src[t] = src[t];
    a.dst[t] = dst[t];
    a.width_bytes[t] = width[t];
    a.src_bstride[t] = kvs * width[t];
  }
  a.n_batch = n_batch;
  a.S = seq_len;
  a.start_pos = start_pos;
  a.max_pos = c->max_pages * c->page_tokens;
  a.pm = page_map(c);
  return hip_status(tpa::launch_append_paged(a, (hipStream_t)stream), "tpa_paged_cache_append");
}

size_t tpa_paged_decode_workspace_bytes(const tpa_dims* d, int64_t n_batch, int64_t max_ctx_len) {
  return tpa_decode_workspace_bytes(d, n_batch, max_ctx_len);
}

tpa_status tpa_paged_decode_attn(const tpa_dims* d, const tpa_factors* q, const tpa_paged_cache* c,
                                 int64_t n_batch, const int32_t* ctx_lens, int64_t max_ctx_len, void* out,
                                 void* workspace, size_t ws_bytes, void* stream) {
  tpa_status st = check_dims(d);
  if (st != TPA_OK) return st;
  if ((st = check_query(d, q)) != TPA_OK) return st;
  if (!out) return fail(TPA_ERR_INVALID_ARGUMENT, "out is NULL");
  if (!ctx_lens) return fail(TPA_ERR_INVALID_ARGUMENT, "ctx_lens is NULL");
  if (n_batch < 1 || max_ctx_len < 1) return fail(TPA_ERR_INVALID_ARGUMENT, "n_batch and max_ctx_len must be >= 1");
  if (n_batch > 65535) return fail(TPA_ERR_UNSUPPORTED, "n_batch must be <= 65535");
  if ((st = check_paged(c, n_batch)) != TPA_OK) return st;
  if (max_ctx_len > c->max_pages * c->page_tokens)
    return fail(TPA_ERR_CAPACITY, "max_ctx_len %lld exceeds max_pages * page_tokens = %lld", (long long)max_ctx_len,
                (long long)(c->max_pages * c->page_tokens));
  int64_t qs;
  if ((st = resolve_stride(q->q_batch_stride, 1, "q_batch_stride", &qs)) != TPA_OK) return st;
  tpa_cache view;
  view.a_k = c->a_k;
  view.b_k = c->b_k;
  view.a_v = c->a_v;
  view.b_v = c->b_v;
  view.max_batch = c->max_batch;
  view.max_seq = c->max_pages * c->page_tokens;
  tpa::AttnArgs a = attn_args(d, q, qs, &view, n_batch, 1, max_ctx_len - 1, 1, out);
  a.pm = page_map(c);
  a.ctx_lens = ctx_lens;
  const tpa::DecodePlan p = tpa::plan_decode(d->dtype, a, max_ctx_len);
  const size_t need = tpa::decode_workspace_bytes(d->dtype, a);
  if (need > 0 && (!workspace || ws_bytes < need))
    return fail(TPA_ERR_WORKSPACE, "decode workspace needs %zu bytes (got %zu%s)", need, ws_bytes,
                workspace ? "" : ", NULL");
  return hip_status(tpa::launch_decode(d->dtype, a, max_ctx_len, p, workspace, (hipStream_t)stream),
                    "tpa_paged_decode_attn");
}

tpa_status tpa_shared_cache_append(const tpa_dims* d, const tpa_shared_cache* c, const tpa_factors* kv,
                                   int64_t n_batch, int64_t seq_len, int64_t start_pos, void* stream) {
  tpa_status st = check_dims(d);
  if (st != TPA_OK) return st;
  if ((st = check_shared(c)) != TPA_OK) return st;
  if (!kv || !kv->a_k || !kv->a_v) return fail(TPA_ERR_INVALID_ARGUMENT, "a head-factor tensor is NULL");
  if (n_batch < 1 || seq_len < 1) return fail(TPA_ERR_INVALID_ARGUMENT, "n_batch and seq_len must be >= 1");
  if (start_pos < 0) return fail(TPA_ERR_INVALID_ARGUMENT, "start_pos must be >= 0");
  if (n_batch > c->max_batch)
    return fail(TPA_ERR_CAPACITY, "n_batch %lld exceeds max_batch %lld", (long long)n_batch,
                (long long)c->max_batch);
  if (seq_len > c->max_seq || start_pos > c->max_seq - seq_len)
    return fail(TPA_ERR_CAPACITY, "start_pos %lld + seq_len %lld exceeds max_seq %lld", (long long)start_pos,
                (long long)seq_len, (long long)c->max_seq);
  int64_t kvs;
  if ((st = resolve_stride(kv->kv_batch_stride, seq_len, "kv_batch_stride", &kvs)) != TPA_OK) return st;
  const int64_t es = (int64_t)elem_size(d);
  const int64_t width[2] = {d->n_heads * d->rank_k * es, d->n_heads * d->rank_v * es};
  const void* src[2] = {kv->a_k, kv->a_v};
  void* dst[2] = {c->a_k, c->a_v};
  tpa::AppendArgs a;
  memset(&a, 0, sizeof(a));
  for (int t = 0; t < 4; ++t) {   // slots 2 and 3 copy nothing (width 0)
    a.src[t] = src[t & 1];
    a.dst[t] = dst[t & 1];
    a.width_bytes[t] = t < 2 ? width[t] : 0;
    a.src_bstride[t] = kvs * a.width_bytes[t];
    a.dst_bstride[t] = c->max_seq * a.width_bytes[t];
  }
  a.n_batch = n_batch;
  a.S = seq_len;
  a.start_pos = start_pos;
  return hip_status(tpa::launch_append(a, (hipStream_t)stream), "tpa_shared_cache_append");
}

size_t tpa_shared_decode_workspace_bytes(const tpa_dims* d, int64_t n_batch, int64_t ctx_len) {
  if (check_dims(d) != TPA_OK || n_batch < 1 || ctx_len < 1) return 0;
  if (n_batch > 65535 || ctx_len >= kMaxTokens) return 0;   // sizes the decode call rejects
  tpa_factors q;
  memset(&q, 0, sizeof(q));
  tpa_cache c;
  memset(&c, 0, sizeof(c));
  c.max_seq = ctx_len;
  const tpa::AttnArgs a = attn_args(d, &q, 1, &c, n_batch, 1, ctx_len - 1, 1, nullptr);
  return tpa::shared_decode_workspace_bytes(tpa::plan_shared_decode(d->dtype, a, ctx_len), a);
}

tpa_status tpa_shared_decode_attn(const tpa_dims* d, const tpa_factors* q, const tpa_shared_cache* c,
                                  int64_t n_batch, int64_t ctx_len, void* out, void* workspace, size_t ws_bytes,
                                  void* stream) {
  tpa_status st = check_dims(d);
  if (st != TPA_OK) return st;
  if ((st = check_query(d, q)) != TPA_OK) return st;
  if ((st = check_shared(c)) != TPA_OK) return st;
  if (!out) return fail(TPA_ERR_INVALID_ARGUMENT, "out is NULL");
  if (n_batch < 1 || ctx_len < 1) return fail(TPA_ERR_INVALID_ARGUMENT, "n_batch and ctx_len must be >= 1");
  if (n_batch > 65535) return fail(TPA_ERR_UNSUPPORTED, "n_batch must be <= 65535");
  if (n_batch > c->max_batch)
    return fail(TPA_ERR_CAPACITY, "n_batch %lld exceeds max_batch %lld", (long long)n_batch,
                (long long)c->max_batch);
  if (ctx_len > c->max_seq)
    return fail(TPA_ERR_CAPACITY, "ctx_len %lld exceeds max_seq %lld", (long long)ctx_len, (long long)c->max_seq);
  int64_t qs;
  if ((st = resolve_stride(q->q_batch_stride, 1, "q_batch_stride", &qs)) != TPA_OK) return st;
  const tpa_cache cc = shared_as_cache(c);
  const tpa::AttnArgs a = attn_args(d, q, qs, &cc, n_batch, 1, ctx_len - 1, 1, out);
  if (!tpa::shared_decode_supported(d->dtype, a))
    return fail(TPA_ERR_UNSUPPORTED, "shared-basis decode takes d_h a multiple of 32 up to 128, R_K and R_V "
                                     "up to 4, per-query tables that fit the device's LDS and per-lane state "
                                     "that fits the registers");
  const tpa::SharedPlan p = tpa::plan_shared_decode(d->dtype, a, ctx_len);
  const size_t need = tpa::shared_decode_workspace_bytes(p, a);
  if (!workspace || ws_bytes < need)
    return fail(TPA_ERR_WORKSPACE, "shared decode workspace needs %zu bytes (got %zu%s)", need, ws_bytes,
                workspace ? "" : ", NULL");
  return hip_status(tpa::launch_shared_decode(d->dtype, a, rope_table(d), ctx_len, p, workspace,
                                              (hipStream_t)stream),
                    "tpa_shared_decode_attn");
}

// Checks shared by the two shared-basis prefill entry points.
static tpa_status shared_prefill_args(const tpa_dims* d, const tpa_factors* q, const tpa_shared_cache* c,
                                      int64_t n_batch, int64_t seq_len, int64_t start_pos, int32_t causal, void* out,
                                      tpa::AttnArgs* a) {
  tpa_status st = check_dims(d);
  if (st != TPA_OK) return st;
  if ((st = check_query(d, q)) != TPA_OK) return st;
  if ((st = check_shared(c)) != TPA_OK) return st;
  if (!out) return fail(TPA_ERR_INVALID_ARGUMENT, "out is NULL");
  if (n_batch < 1 || seq_len < 1) return fail(TPA_ERR_INVALID_ARGUMENT, "n_batch and seq_len must be >= 1");
  if (n_batch > 65535) return fail(TPA_ERR_UNSUPPORTED, "n_batch must be <= 65535");
  if (start_pos < 0) return fail(TPA_ERR_INVALID_ARGUMENT, "start_pos must be >= 0");
  if (n_batch > c->max_batch)
    return fail(TPA_ERR_CAPACITY, "n_batch %lld exceeds max_batch %lld", (long long)n_batch,
                (long long)c->max_batch);
  if (seq_len > c->max_seq || start_pos > c->max_seq - seq_len)
    return fail(TPA_ERR_CAPACITY, "start_pos %lld + seq_len %lld exceeds max_seq %lld", (long long)start_pos,
                (long long)seq_len, (long long)c->max_seq);
  int64_t qs;
  if ((st = resolve_stride(q->q_batch_stride, seq_len, "q_batch_stride", &qs)) != TPA_OK) return st;
  const tpa_cache cc = shared_as_cache(c);
  *a = attn_args(d, q, qs, &cc, n_batch, seq_len, start_pos, causal, out);
  return TPA_OK;
}

tpa_status tpa_shared_prefill_attn(const tpa_dims* d, const tpa_factors* q, const tpa_shared_cache* c,
                                   int64_t n_batch, int64_t seq_len, int64_t start_pos, int32_t causal, void* out,
                                   void* stream) {
  tpa::AttnArgs a;
  const tpa_status st = shared_prefill_args(d, q, c, n_batch, seq_len, start_pos, causal, out, &a);
  if (st != TPA_OK) return st;
  return hip_status(tpa::launch_prefill_shared(d->dtype, a, rope_table(d), (hipStream_t)stream),
                    "tpa_shared_prefill_attn");
}

tpa_status tpa_shared_prefill_attn_ws(const tpa_dims* d, const tpa_factors* q, const tpa_shared_cache* c,
                                      int64_t n_batch, int64_t seq_len, int64_t start_pos, int32_t causal, void* out,
                                      void* workspace, size_t workspace_bytes, void* stream) {
  tpa::AttnArgs a;
  tpa_status st = shared_prefill_args(d, q, c, n_batch, seq_len, start_pos, causal, out, &a);
  if (st != TPA_OK) return st;
  const size_t need = tpa::prefill_workspace_bytes(d->dtype, a);
  if ((st = check_prefill_workspace(need, workspace, workspace_bytes)) != TPA_OK) return st;
  return hip_status(tpa::launch_prefill_shared_ws(d->dtype, a, rope_table(d), need > 0 ? workspace : nullptr,
                                                  (hipStream_t)stream),
                    "tpa_shared_prefill_attn_ws");
}

// Takes an int: a C caller may pass any int, and a value outside the enum's
// range must not be loaded as a tpa_status in C++.
const char* tpa_status_string(int s) {
  switch (s) {
    case TPA_OK: return "ok";
    case TPA_ERR_INVALID_ARGUMENT: return "invalid argument";
    case TPA_ERR_UNSUPPORTED: return "unsupported";
    case TPA_ERR_CAPACITY: return "cache capacity exceeded";
    case TPA_ERR_WORKSPACE: return "workspace too small";
    case TPA_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

const char* tpa_last_error(void) { return g_err; }

}  // extern "C"
