/*
 * tpa.h - C ABI of libtpa: Tensor Product Attention (TPA) with a factorised KV
 * cache, for AMD Instinct MI355X (gfx950).
 *
 * TPA writes each token's per-head query, key and value ([h, d_h] each) as a
 * 1/R-scaled sum of R outer products of a head factor a_r(x_t) (length h) and a
 * dim factor b_r(x_t) (length d_h); only the key/value factors are cached, and
 * the key dim factors are rotated (RoPE) before they are cached.
 *   Definitions: "Tensor Product Attention Is All You Need" review on
 *   coreui.cn, section 核心机制总结 item 3 (equations for Q_t, K_t, V_t),
 *   关键问题及回答 question 2 (pre-rotation B~_K <- RoPE_t(B_K)), and its code
 *   walk-through (类定义与初始化: projection layers and cache shapes;
 *   前向传播: projections, cache write/read by start_pos, reconstruction,
 *   softmax attention).
 *
 * Conventions shared by every call
 * --------------------------------
 * - Memory: every data pointer is device memory owned by the caller.  The
 *   library allocates nothing and keeps no state between calls except a
 *   thread-local error message.  Pointers must be aligned to the element size;
 *   16-byte alignment (and the shape limits of each call) selects the fast
 *   kernels, anything else runs a general kernel with the same results
 *   up to rounding order.
 * - Element type: dims->dtype is TPA_F32 (float) or TPA_BF16 (bfloat16, stored
 *   as 16-bit words).  All tensors of a call use it.  Arithmetic is float32
 *   with float32 accumulation; bf16 results are rounded to nearest even.  In
 *   bf16 the matrix-core kernels take bf16 operands: the prefill's query,
 *   rebuilt keys and values and probabilities are rounded to bf16; the
 *   decode's query enters as a bf16 hi + lo pair (fp32-level scores) and its
 *   probability-weighted value factors are rounded to bf16; the backward and
 *   the shared-basis decode split their sensitive operands into hi + lo pairs
 *   as documented with each call.
 * - Streams: `stream` is a hipStream_t passed as void* (NULL = the default
 *   stream).  Every call only enqueues work and returns; ordering between
 *   calls is the caller's, through the stream.
 * - Errors: arguments are checked before anything is enqueued.  A non-zero
 *   status means nothing was launched; tpa_last_error() then describes why.
 *   TPA_ERR_HIP reports a failed launch (the work before it in the same call
 *   may have run).
 * - Positions are zero-based.  Token s of a block that starts at start_pos
 *   sits at position start_pos + s, in every sequence of the batch.
 * - Rotary embedding: element pairs (2i, 2i+1) of a d_h-vector are turned by the
 *   angle pos * rope_base^(-2i/d_h), i < d_h/2; the angle is formed and reduced
 *   in float64.
 *
 * Layouts (all row-major, token-major; "B" is the batch, "S" the block length)
 * --------------------------------------------------------------------------
 *   x         [B, S, d_model]
 *   w_packed  [n_out, d_model]: the six nn.Linear weights stacked by rows in
 *             the order W_B_q, W_B_k, W_B_v, W_A_q, W_A_k, W_A_v
 *             (TPA-KVonly, rank_q == 0: W_Q, W_B_k, W_B_v, W_A_k, W_A_v).
 *             The rotated columns come first, so they are pair-aligned.
 *   a_q [B,S,h,R_Q]  b_q [B,S,R_Q,d_h]   (KV-only: b_q holds Q [B,S,h,d_h], a_q unused)
 *   a_k [B,S,h,R_K]  b_k [B,S,R_K,d_h]  a_v [B,S,h,R_V]  b_v [B,S,R_V,d_h]
 *   cache     a_k [max_batch, max_seq, h, R_K], b_k [max_batch, max_seq, R_K, d_h],
 *             a_v [max_batch, max_seq, h, R_V], b_v [max_batch, max_seq, R_V, d_h]
 *             (the page's cache_kA, cache_kB, cache_vA, cache_vB).
 *   out       prefill [B, S, h*d_h]; decode [B, h*d_h] (head-major per token).
 */
#ifndef TPA_H
#define TPA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  TPA_OK = 0,
  TPA_ERR_INVALID_ARGUMENT = 1, /* null pointer, bad size, odd head_dim, ... */
  TPA_ERR_UNSUPPORTED = 2,      /* valid TPA, but outside what this library runs */
  TPA_ERR_CAPACITY = 3,         /* batch or positions beyond the cache */
  TPA_ERR_WORKSPACE = 4,        /* a needed workspace missing or too small */
  TPA_ERR_HIP = 5               /* a HIP launch failed */
} tpa_status;

typedef enum { TPA_F32 = 0, TPA_BF16 = 1 } tpa_dtype;

/* One layer's dimensions (the page's ModelArgs: dim, n_heads, head_dim, q_rank,
 * rank; key and value ranks are separate, as in its K_t and V_t equations).
 * Limits: d_model >= 1; 1 <= n_heads <= 256; head_dim even, 2..256;
 * rank_k, rank_v in 1..64; rank_q in 0..64, 0 selecting TPA-KVonly (Q is a
 * plain per-head projection, rotated like the key factors).  Dims outside
 * these limits give TPA_ERR_INVALID; n_heads * head_dim above 8192 (one
 * token's heads held by one workgroup) gives TPA_ERR_UNSUPPORTED. */
typedef struct {
  int32_t d_model;
  int32_t n_heads;   /* h */
  int32_t head_dim;  /* d_h */
  int32_t rank_q;    /* R_Q, or 0 for TPA-KVonly */
  int32_t rank_k;    /* R_K */
  int32_t rank_v;    /* R_V */
  double rope_base;  /* finite and > 0, e.g. 10000 */
  int32_t dtype;     /* tpa_dtype */
} tpa_dims;

/* The factor cache: four caller-owned tensors with capacity
 * [max_batch, max_seq] tokens (layouts above). */
typedef struct {
  void* a_k;
  void* b_k;
  void* a_v;
  void* b_v;
  int64_t max_batch;
  int64_t max_seq;
} tpa_cache;

/* A block of factors for B sequences of S tokens (layouts above).
 * q_batch_stride / kv_batch_stride: tokens between consecutive sequences of
 * the query tensors (a_q, b_q) and of the key/value tensors; 0 means S (dense).
 * A kv_batch_stride of max_seq with a_k..b_v pointing at cache slot start_pos
 * lets tpa_factor_proj write straight into the cache. */
typedef struct {
  void* a_q;
  void* b_q;
  void* a_k;
  void* b_k;
  void* a_v;
  void* b_v;
  int64_t q_batch_stride;
  int64_t kv_batch_stride;
} tpa_factors;

/* Number of rows n_out of the packed projection weight:
 * h*R_Q + R_Q*d_h + h*R_K + R_K*d_h + h*R_V + R_V*d_h (KV-only: h*d_h instead of
 * the query terms).  Returns -1 for invalid dims. */
int64_t tpa_packed_weight_rows(const tpa_dims* dims);

/* Cached elements per token, h*(R_K+R_V) + d_h*(R_K+R_V); -1 for invalid dims. */
int64_t tpa_cache_elems_per_token(const tpa_dims* dims);

/* Factor projection: F = x * w_packed^T for all B*S tokens, split into the six
 * factor tensors of `out` (KV-only: five).  With fuse_rope != 0 the query and
 * key dim factors (KV-only: Q) are rotated at positions start_pos + s before
 * they are stored; with fuse_rope == 0 they are stored unrotated and
 * start_pos is ignored.
 *   Passage: the A and B projections of the code walk-through (前向传播),
 *   a^X(x_t) = W_A_X x_t viewed [h, R_X], b^X(x_t) = W_B_X x_t viewed [R_X, d_h];
 *   the pre-rotation of question 2.
 * x [B,S,d_model], w_packed [n_out, d_model]; out->* as in the layouts above
 * (a_q ignored for KV-only).  Errors: any null tensor, B or S < 1 (B*S must fit
 * in 2^31 tokens), start_pos < 0. */
tpa_status tpa_factor_proj(const tpa_dims* dims, const void* x, int64_t n_batch, int64_t seq_len,
                           int64_t start_pos, const void* w_packed, int32_t fuse_rope,
                           const tpa_factors* out, void* stream);

/* In-place rotary embedding of `rows` d_h-vectors per token:
 * b [B, S, rows, d_h], token s at position start_pos + s.  Used standalone for
 * factors projected with fuse_rope == 0 (rows = R_Q, R_K, or h for plain Q).
 *   Passage: question 2's B~_K <- RoPE_t(B_K); the code walk-through rotates
 *   q and k, which equals rotating every query and key dim factor.
 * Errors: null b, B, S or rows < 1, start_pos < 0. */
tpa_status tpa_rope_b(const tpa_dims* dims, void* b, int64_t n_batch, int64_t seq_len, int32_t rows,
                      int64_t start_pos, void* stream);

/* Cache append: cache[b, start_pos + s] = kv[b, s] for the four K/V factor
 * tensors, bit for bit.  kv->a_q / b_q are ignored.
 *   Passage: the cache writes of the code walk-through (前向传播),
 *   cache[:bsz, start_pos:start_pos+seqlen] = factor.
 * Errors: null pointers; n_batch > max_batch or start_pos + S > max_seq
 * (TPA_ERR_CAPACITY). */
tpa_status tpa_cache_append(const tpa_dims* dims, const tpa_cache* cache, const tpa_factors* kv,
                            int64_t n_batch, int64_t seq_len, int64_t start_pos, void* stream);

/* Prefill attention for S query tokens per sequence at positions
 * start_pos .. start_pos+S-1, over the cached keys/values 0 .. start_pos+S-1
 * (the caller appends this block's K/V factors first):
 *   q_{s,h} = (1/R_Q) sum_r a_q[s,h,r] b_q[s,r,:]   (KV-only: b_q[s,h,:])
 *   k_{t,h} = (1/R_K) sum_r a_k[t,h,r] b_k[t,r,:],  v likewise with R_V,
 *   out[s, h*d_h:(h+1)*d_h] = sum_t softmax_t(q.k_t / sqrt(d_h)) v_t,
 * where with causal != 0 key t is visible iff t <= start_pos + s, else every
 * cached key is.  K and V are never written to memory.
 *   Passage: the Q_t/K_t/V_t equations; scaled dot-product attention
 *   (jieyibu.net explainer, section Ⅱ.1; code walk-through, 前向传播).
 * q: factors of this block (q_batch_stride applies); out [B, S, h*d_h].
 * Errors: null pointers, B > max_batch or start_pos + S > max_seq. */
tpa_status tpa_prefill_attn(const tpa_dims* dims, const tpa_factors* q, const tpa_cache* cache,
                            int64_t n_batch, int64_t seq_len, int64_t start_pos, int32_t causal, void* out,
                            void* stream);

/* Bytes of device workspace tpa_prefill_attn_ws (and
 * tpa_shared_prefill_attn_ws) uses for these sizes:
 * 2 * n_batch * h * (start_pos + seq_len) * d_h * 2 where the matrix-core path
 * that forms K and V once applies (bf16, d_h = 64, R_K = R_V in {1, 2, 4}),
 * else 0 (the call then needs no workspace).  0 also for dims or sizes the
 * call rejects.  Host only; depends on the sizes alone. */
size_t tpa_prefill_workspace_bytes(const tpa_dims* dims, int64_t n_batch, int64_t seq_len, int64_t start_pos);

/* tpa_prefill_attn with a caller-owned workspace: the same attention (same
 * passage), computed by first forming k_t and v_t of every key 0 ..
 * start_pos+S-1 and head once, rounded to the compute dtype exactly as
 * tpa_prefill_attn rounds them in on-chip memory, into the workspace
 * ([B][h][start_pos+S][d_h] for K, then V), and then attending over them.
 * Prefill is bound by arithmetic, and forming each key and value once
 * instead of once per 256-query block removes most of that work's vector
 * instructions.  Outputs match tpa_prefill_attn's bit for bit at R_K = R_V
 * in {1, 2}; at rank 4 the keys are taken in 64- rather than 32-key blocks,
 * so only the online softmax's summation order differs.  Where
 * tpa_prefill_workspace_bytes is 0 (or the pointers are not 16-byte
 * aligned) the call runs tpa_prefill_attn and ignores the workspace.
 * workspace: device memory of at least tpa_prefill_workspace_bytes bytes,
 * 16-byte aligned, owned by the caller, overwritten; no contents are kept
 * between calls.  Calls that share a workspace must be ordered on one stream.
 * Errors: as tpa_prefill_attn; where a workspace is needed, a NULL one or one
 * smaller than that (TPA_ERR_WORKSPACE), a misaligned one
 * (TPA_ERR_INVALID_ARGUMENT). */
tpa_status tpa_prefill_attn_ws(const tpa_dims* dims, const tpa_factors* q, const tpa_cache* cache,
                               int64_t n_batch, int64_t seq_len, int64_t start_pos, int32_t causal, void* out,
                               void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of device workspace tpa_decode_attn needs for this batch and context;
 * 0 for dims or sizes that call rejects (n_batch outside 1..65535, ctx_len
 * outside 1 .. 2^31 - 1). */
size_t tpa_decode_workspace_bytes(const tpa_dims* dims, int64_t n_batch, int64_t ctx_len);

/* Decode attention: one new query per sequence at position ctx_len - 1 over the
 * cached keys/values 0 .. ctx_len - 1 (the new token's factors must already be
 * in the cache).  Same arithmetic as tpa_prefill_attn with S = 1, computed as a
 * split over the context with a log-sum-exp combine in a fixed order, so
 * repeated calls give bit-identical results.  Scores use the factored form
 * s_t = (1/R_K) sum_r a_k[t,h,r] (b_k[t,r,:] . q_h) / sqrt(d_h).
 *   Passage: as tpa_prefill_attn; the pre-rotated cache needs no rotation at
 *   decode time (question 2).
 * q: the new token's query factors, a_q [B,h,R_Q], b_q [B,R_Q,d_h]
 * (KV-only: b_q = Q [B,h,d_h]); out [B, h*d_h].
 * workspace: device memory of at least tpa_decode_workspace_bytes(dims, B,
 * ctx_len) bytes; it holds per-chunk partial results during the call only, so
 * its contents on entry do not matter.  Calls that may run at the same time
 * must not share a workspace.
 * Errors: null pointers, ctx_len < 1, B > max_batch or ctx_len > max_seq
 * (TPA_ERR_CAPACITY), workspace too small (TPA_ERR_WORKSPACE). */
tpa_status tpa_decode_attn(const tpa_dims* dims, const tpa_factors* q, const tpa_cache* cache,
                           int64_t n_batch, int64_t ctx_len, void* out, void* workspace, size_t ws_bytes,
                           void* stream);

/* Decode attention without a workspace argument, for callers that cannot
 * allocate device memory at call time (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation).  Same arguments, checks,
 * kernels, split and merge order as tpa_decode_attn, so the same bits; the
 * chunk partials go to a static device array of tpa_decode_noalloc_max_bytes()
 * bytes (16 MiB) that each device holds from the library's first use on it
 * until the process ends.  The call allocates nothing.  Every call on one
 * device shares that device's array and it keeps the last call's contents
 * (nothing in it needs to start at zero): calls that may overlap on one
 * device (several streams, several host threads) race and must be ordered
 * by the caller.
 * Errors: as tpa_decode_attn; TPA_ERR_WORKSPACE when the call's partials,
 * n_batch * chunks * h * (d_h + 2) * 4 bytes for the plan it runs (about
 * 8.5 MB for 8 sequences of 131073 keys at h 32, d_h 128), exceed the array;
 * TPA_ERR_HIP if the array's device address cannot be taken. */
size_t tpa_decode_noalloc_max_bytes(void);
tpa_status tpa_decode_attn_noalloc(const tpa_dims* dims, const tpa_factors* q, const tpa_cache* cache,
                                   int64_t n_batch, int64_t ctx_len, void* out, void* stream);

/* ---------------------------------------------------------------------------
 * Backward (training; the pages train TPA models, the arithmetic is the chain
 * rule through tpa_prefill_attn and tpa_rope_b).  Gradients are float32
 * whatever dims->dtype is.  The projection's own gradients are plain matrix
 * products of the packed factor gradient dF [B*S, n_out]: dX = dF w_packed and
 * dW = dF^T x; the library does not provide them.
 * ------------------------------------------------------------------------- */

/* Bytes of device workspace tpa_prefill_attn_backward needs, with N = B*h*d_h
 * and T = start_pos+S: float32 dQ, dK, dV (N*(S + 2T)*4), the bf16 operands of
 * the matrix-core kernels (N*(2S + 3T)*2) and two float32 statistics per
 * query and head (2*B*S*h*4).  The base address must be 16-byte aligned for
 * the matrix-core path (otherwise the general kernels run).  0 for dims or
 * sizes the backward rejects (n_batch above 65535, B*S or start_pos + S of
 * 2^31 or more). */
size_t tpa_prefill_backward_workspace_bytes(const tpa_dims* dims, int64_t n_batch, int64_t seq_len,
                                            int64_t start_pos);

/* Gradients of the prefill attention: given the forward's inputs (q, cache,
 * start_pos, causal) and the upstream gradient dout [B,S,h*d_h] (the element
 * type of dims->dtype), writes
 *   dq->a_q [B,S,h,R_Q], dq->b_q [B,S,R_Q,d_h]  (KV-only: dq->b_q = dQ [B,S,h,d_h]),
 *     gradients of the query factors as passed (b_q rotated), float32,
 *     dq->q_batch_stride applies (0 = S);
 *   dkv->a_k .. b_v, float32 tensors in the cache layout: positions
 *     0 .. start_pos+S-1 of each sequence are overwritten with the gradients of
 *     the cached factors there (b_k rotated); other positions are untouched.
 * With P the softmax rows and s = q.k/sqrt(d_h): dV = P^T dO, dS = P*(dO V^T -
 * rowsum(dO*O)), dQ = dS K/sqrt(d_h), dK = dS^T Q/sqrt(d_h), then
 * dA[t,h,r] = (1/R) dX[t,h,:].B[t,r,:] and dB[t,r,:] = (1/R) sum_h A[t,h,r] dX[t,h,:].
 * The forward output is not an argument: the row sums rowsum(dO*O) take O as
 * recomputed in fp32 (a stored bf16 output would perturb every dS by its
 * rounding, which the cancelling rows of dS magnify).  In bf16 the matrix-core
 * passes form the scores from q and k as bf16 hi + lo pairs; dS, P, dO, v and
 * the q and k that multiply dS enter their products as plain bf16.
 * Deterministic: repeated calls give the same bits.
 *   Passage: the Q_t/K_t/V_t equations and the attention of the code
 *   walk-through (前向传播), differentiated.
 * Errors: as tpa_prefill_attn; null gradient tensors; dkv smaller than the
 * key range (TPA_ERR_CAPACITY); workspace too small (TPA_ERR_WORKSPACE). */
tpa_status tpa_prefill_attn_backward(const tpa_dims* dims, const tpa_factors* q, const tpa_cache* cache,
                                     int64_t n_batch, int64_t seq_len, int64_t start_pos, int32_t causal,
                                     const void* dout, const tpa_factors* dq, const tpa_cache* dkv,
                                     void* workspace, size_t ws_bytes, void* stream);

/* Gradient through the rotary embedding: in place on g [B,S,rows,d_h]
 * (float32), turns each pair back by the angle tpa_rope_b turned it forward
 * (the rotation is orthogonal), giving the gradient of the unrotated factor.
 * Errors: as tpa_rope_b. */
tpa_status tpa_rope_b_backward(const tpa_dims* dims, float* g, int64_t n_batch, int64_t seq_len, int32_t rows,
                               int64_t start_pos, void* stream);

/* ---------------------------------------------------------------------------
 * Paged factor cache (serving layout: the pages do not describe one; the
 * arithmetic is that of tpa_cache_append and tpa_decode_attn).
 *
 * The four factor tensors are pools of fixed-size pages,
 *   a_k [n_pages, page_tokens, h, R_K]   b_k [n_pages, page_tokens, R_K, d_h]
 *   a_v [n_pages, page_tokens, h, R_V]   b_v [n_pages, page_tokens, R_V, d_h],
 * and block_table [max_batch, max_pages] (int32, device memory) names, for
 * sequence b, the page holding its tokens i*page_tokens .. (i+1)*page_tokens-1
 * in column i.  Pages may appear in any order (and be shared); columns past a
 * sequence's length are never read.  The library does not read the table on
 * the host: page ids outside [0, n_pages) are clamped into the pool, which
 * gives wrong values but never an access outside it.
 * ------------------------------------------------------------------------- */
typedef struct {
  void* a_k;
  void* b_k;
  void* a_v;
  void* b_v;
  const int32_t* block_table;
  int64_t n_pages;
  int64_t page_tokens;
  int64_t max_pages;  /* table columns: a sequence holds up to max_pages*page_tokens tokens */
  int64_t max_batch;  /* table rows */
} tpa_paged_cache;

/* Paged cache append: token s of sequence b of `kv` is written, bit for bit, to
 * position start_pos[b] + s of sequence b (start_pos: int32 device array [B]).
 * Positions outside [0, max_pages*page_tokens) are skipped.  kv->a_q / b_q are
 * ignored.
 *   Passage: the cache writes of the code walk-through (前向传播), with each
 *   sequence's positions mapped through its page list.
 * Errors: null pointers, B or S < 1, B > max_batch, n_pages, page_tokens or
 * max_pages < 1, or more than 2^31 positions per sequence. */
tpa_status tpa_paged_cache_append(const tpa_dims* dims, const tpa_paged_cache* cache, const tpa_factors* kv,
                                  int64_t n_batch, int64_t seq_len, const int32_t* start_pos, void* stream);

/* Bytes of device workspace tpa_paged_decode_attn needs (the same as
 * tpa_decode_workspace_bytes for ctx_len = max_ctx_len). */
size_t tpa_paged_decode_workspace_bytes(const tpa_dims* dims, int64_t n_batch, int64_t max_ctx_len);

/* Decode attention over a paged cache, each sequence with its own key count:
 * sequence b attends over its keys 0 .. ctx_lens[b] - 1 (ctx_lens: int32
 * device array [B]; each value is clamped to [0, max_ctx_len], and a sequence
 * with no keys gets a zero output).  Arithmetic, split and merge order are
 * those of tpa_decode_attn with ctx_len = max_ctx_len, so with an identity
 * table and every length equal to max_ctx_len the two give the same bits
 * (when both run the same kernel: the matrix-core kernel needs page_tokens to
 * be a multiple of 32).
 *   Passage: as tpa_decode_attn.
 * q, out, workspace: as tpa_decode_attn.
 * Errors: null pointers, B or max_ctx_len < 1, B > max_batch, max_ctx_len >
 * max_pages*page_tokens (TPA_ERR_CAPACITY), workspace too small. */
tpa_status tpa_paged_decode_attn(const tpa_dims* dims, const tpa_factors* q, const tpa_paged_cache* cache,
                                 int64_t n_batch, const int32_t* ctx_lens, int64_t max_ctx_len, void* out,
                                 void* workspace, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Shared-basis variant.  The pages list, among TPA's variants, one that shares
 * the basis vectors across tokens (coreui.cn review, 优点与创新 item 5) and give
 * no formula; this library reads it as: the dim factors of K and V are
 * parameters common to every token, B_K [R_K, d_h] (unrotated) and B_V
 * [R_V, d_h], while the head factors stay per token, and key t is rotated at
 * its own position:
 *   K_t[h] = RoPE_t((1/R_K) sum_r A_K[t,h,r] B_K[r]),  V_t[h] = (1/R_V) sum_r A_V[t,h,r] B_V[r].
 * The cache therefore holds only a_k [max_batch, max_seq, h, R_K] and
 * a_v [max_batch, max_seq, h, R_V]: h*(R_K+R_V) elements per token.  The query
 * is the same as for tpa_decode_attn.
 * ------------------------------------------------------------------------- */
typedef struct {
  void* a_k;          /* [max_batch, max_seq, h, R_K], caller-owned device memory */
  void* a_v;          /* [max_batch, max_seq, h, R_V] */
  const void* b_k;    /* [R_K, d_h], shared by every token, unrotated */
  const void* b_v;    /* [R_V, d_h] */
  int64_t max_batch;
  int64_t max_seq;
} tpa_shared_cache;

/* Shared-basis cache append: kv->a_k [B,S,h,R_K] and kv->a_v [B,S,h,R_V] are
 * written, bit for bit, to positions start_pos .. start_pos+S-1 of each
 * sequence (kv->kv_batch_stride applies; the other kv fields are ignored).
 *   Passage: the cache writes of the code walk-through (前向传播), for the
 *   head factors only.
 * Errors: null pointers, B or S < 1, start_pos < 0, B > max_batch,
 * start_pos+S > max_seq (TPA_ERR_CAPACITY). */
tpa_status tpa_shared_cache_append(const tpa_dims* dims, const tpa_shared_cache* cache, const tpa_factors* kv,
                                   int64_t n_batch, int64_t seq_len, int64_t start_pos, void* stream);

/* Number of rows of the packed projection weight for a shared-basis layer:
 * h*R_Q + R_Q*d_h + h*R_K + h*R_V (KV-only: h*d_h instead of the query
 * terms); the key/value dim factors are the shared bases, not projections.
 * Returns -1 for invalid dims. */
int64_t tpa_shared_packed_weight_rows(const tpa_dims* dims);

/* Factor projection of a shared-basis layer: as tpa_factor_proj, with
 * w_packed [n_out, d_model] stacking W_B_q, W_A_q, W_A_k, W_A_v (KV-only: W_Q,
 * W_A_k, W_A_v) and out->b_k / out->b_v ignored; only the query dim factors
 * (KV-only: Q) are rotated.  out->a_k / a_v with kv_batch_stride = max_seq
 * can point at cache slot start_pos of a tpa_shared_cache.
 *   Passage: the A and B projections of the code walk-through (前向传播), with
 *   the dim factors of K and V shared (优点与创新 item 5; the reading above).
 * Errors: as tpa_factor_proj. */
tpa_status tpa_shared_factor_proj(const tpa_dims* dims, const void* x, int64_t n_batch, int64_t seq_len,
                                  int64_t start_pos, const void* w_packed, int32_t fuse_rope,
                                  const tpa_factors* out, void* stream);

/* Prefill attention over a shared-basis cache: S query tokens per sequence at
 * positions start_pos .. start_pos+S-1 (q as for tpa_prefill_attn) over the
 * keys 0 .. start_pos+S-1 (the caller appends this block's head factors
 * first), causal or full as tpa_prefill_attn; out [B, S, h*d_h].  Key t is
 * rebuilt from its head factors and the basis and rotated at position t;
 * keys and values are never written to memory.  bf16 with d_h = 64 and
 * R_K = R_V in {1, 2, 4} runs on the matrix cores (the basis slice each
 * thread rebuilds is loaded once), every other shape on the general kernel.
 *   Passage: the Q_t/K_t/V_t equations (核心机制总结) with the dim factors of
 *   K and V shared, and the masked attention of the code walk-through.
 * Errors: as tpa_prefill_attn. */
tpa_status tpa_shared_prefill_attn(const tpa_dims* dims, const tpa_factors* q, const tpa_shared_cache* cache,
                                   int64_t n_batch, int64_t seq_len, int64_t start_pos, int32_t causal, void* out,
                                   void* stream);

/* tpa_shared_prefill_attn with a caller-owned workspace, as
 * tpa_prefill_attn_ws: every key and value of the call is formed once (each
 * key rotated at its own position, rounded as tpa_shared_prefill_attn rounds
 * it on chip) into the workspace and then attended; outputs equal
 * tpa_shared_prefill_attn's bit for bit at R_K = R_V in {1, 2}.  The
 * workspace is sized by tpa_prefill_workspace_bytes with the same dims and
 * sizes (0: none needed, the call runs tpa_shared_prefill_attn).
 * Errors: as tpa_shared_prefill_attn, and the workspace errors of
 * tpa_prefill_attn_ws. */
tpa_status tpa_shared_prefill_attn_ws(const tpa_dims* dims, const tpa_factors* q, const tpa_shared_cache* cache,
                                      int64_t n_batch, int64_t seq_len, int64_t start_pos, int32_t causal, void* out,
                                      void* workspace, size_t workspace_bytes, void* stream);

/* Device workspace for tpa_shared_decode_attn: float32 partials
 * (max, sum, R_V weights) per sequence, key chunk and head; 0 for dims or
 * sizes as tpa_decode_workspace_bytes. */
size_t tpa_shared_decode_workspace_bytes(const tpa_dims* dims, int64_t n_batch, int64_t ctx_len);

/* Decode attention over a shared-basis cache: each sequence's new query
 * (position ctx_len-1, q as for tpa_decode_attn) attends over its keys
 * 0 .. ctx_len-1; out [B, h*d_h] in dims->dtype.  The score of key t is
 * sum_r A_K[t,h,r] (q . RoPE_t(B_K[r])) / (R_K sqrt(d_h)), formed from per-query
 * products of q with B_K and the key's rotation angles, so only the head
 * factors are read per key; each head accumulates sum_t p_t A_V[t,h,r] and the
 * merge applies B_V.  The score products run on the matrix cores with both
 * operands split into bf16 hi + lo (fp32-level accuracy); angles are reduced
 * in fp64; the rest is fp32.  Deterministic.
 *   Passage: the Q_t/K_t/V_t equations (核心机制总结) with the dim factors of
 *   K and V shared, and the decode of the code walk-through (前向传播).
 * Errors: as tpa_decode_attn; TPA_ERR_UNSUPPORTED unless d_h is a multiple of
 * 32 up to 128 and R_K, R_V are at most 4, for head counts whose per-query
 * alpha/beta rows exceed the device's LDS, and for layers whose per-lane
 * softmax state would not fit the registers (about 64 heads at rank 4). */
tpa_status tpa_shared_decode_attn(const tpa_dims* dims, const tpa_factors* q, const tpa_shared_cache* cache,
                                  int64_t n_batch, int64_t ctx_len, void* out, void* workspace, size_t ws_bytes,
                                  void* stream);

/* Static text for a status code (a tpa_status value; any other int gives
 * "unknown status"). */
const char* tpa_status_string(int status);

/* Description of the last error returned on the calling thread ("" if none). */
const char* tpa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* TPA_H */
