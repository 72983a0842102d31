"""fp64 CPU oracle for Tensor Product Attention (TPA) with a factorised KV cache.

TEST INFRASTRUCTURE.  Only the tests, the smoke check and the benchmark's CPU
baseline may import this module.  The product path (the HIP library and its
Python binding) never calls it, and this module imports nothing from the
product path.

What it computes, and where the pages define it.  Page titles are abbreviated:
  [coreui]  "【拜读】Tensor Product Attention Is All You Need …" (coreui.cn review)
  [jieyibu] "张量积注意力（TPA）：让注意力机制飞得更高、跑得更快的秘密武器" (jieyibu.net)
  [substack] "TPA Paper Explained" (gyanendradas.substack.com)
  [bbzoh]   the MQA/GQA blog post at bbzoh.cn (ChatGLM2 / LLaMA2 sections)

* Factorisation: per token t, Q_t, K_t, V_t (each [h, d_h]) are (1/R) times a sum
  of R outer products a_r(x_t) (length h) x b_r(x_t) (length d_h)
  ([coreui] "核心机制总结", item 3 "公式描述", equations for Q_t, K_t, V_t).
* The factors are linear maps of x_t: six bias-free linear layers W_A_q, W_A_k,
  W_A_v (d_model -> h*R) and W_B_q, W_B_k, W_B_v (d_model -> R*d_h), whose outputs
  are viewed as [h, R] and [R, d_h] ([coreui] "代码", "类定义与初始化" and "前向传播").
* Rotary embedding is applied to the B factors of K (pre-rotation, before
  caching) ([coreui] "关键问题及回答", 问题2, the B~_K <- RoPE_t(B_K) equation;
  [substack] "RoPE Compatibility and Acceleration").  Queries are rotated too
  (the forward code rotates q and k); rotating every b_r^Q equals rotating Q.
* The cache holds only the K/V factors, at slots [start_pos, start_pos + S)
  ([coreui] "前向传播": cache writes and reads by start_pos).
* Scaled dot-product attention softmax(Q K^T / sqrt(d_h)) V per head
  ([jieyibu] section Ⅱ.1, the attention formula; [coreui] "前向传播").

Readings where the pages are silent (each is listed with its reason in the
design notes): rotary pairs are adjacent elements (2i, 2i+1) with angle
pos * base^(-2i/d_h); positions are zero-based, pos = start_pos + s; the mask is
causal with the diagonal visible; the 1/R factors of the equations apply (not
the unscaled sum of [jieyibu] Ⅱ.2); decode attends over the new token too (the
forward code writes the cache before it reads it).

The backward functions (reconstruct_backward, attend_head_backward,
prefill_backward, rope_backward) are the chain rule through the same
definitions, written out; they serve training, which the pages mention as
context.  Paged and ragged decode (paged_gather, decode_paged) serve a layout
the pages do not describe: each sequence's tokens are gathered through its page list and
run through the same decode; a sequence with no keys gets a zero output.
The shared-basis variant (shared_keys_values, decode_shared) takes the dim
factors of K and V as parameters common to every token, so a cache holds only
the head factors; each key is rotated at its own position.

Everything is float64.  Inputs given in bf16 arrive here as their exact values
widened to float64.  Loops run over (batch, head) in Python; numpy's matmul is
the only library primitive used for contractions.  No blocking, no online
softmax, no fusion: Q, K and V are built explicitly as sums of outer products.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional, Sequence

import numpy as np


@dataclasses.dataclass(frozen=True)
class Dims:
    """One TPA layer's dimensions ([coreui] "类定义与初始化": dim, n_heads,
    head_dim, q_rank, rank).  rank_q == 0 selects TPA-KVonly (plain Q)."""

    d_model: int
    n_heads: int
    head_dim: int
    rank_q: int
    rank_k: int
    rank_v: int
    rope_base: float = 10000.0

    @property
    def kv_only(self) -> bool:
        return self.rank_q == 0


# ---------------------------------------------------------------------------
# Step 1: factor projections
# ---------------------------------------------------------------------------

def project(x: np.ndarray, w: Dict[str, np.ndarray], dims: Dims) -> Dict[str, np.ndarray]:
    """Factor projections of x [B, S, d_model] through bias-free linear layers.

    a^X(x_t) = W_A_X x_t viewed as [h, R_X] (head-major), b^X(x_t) = W_B_X x_t
    viewed as [R_X, d_h] ([coreui] "前向传播", the six projections and their views).
    TPA-KVonly: q(x_t) = W_Q x_t viewed as [h, d_h].
    Weights use the nn.Linear layout [out_features, d_model].
    """
    x = np.asarray(x, dtype=np.float64)
    B, S, _ = x.shape
    h, dh = dims.n_heads, dims.head_dim

    def lin(name):
        return x @ np.asarray(w[name], dtype=np.float64).T

    out = {}
    if dims.kv_only:
        out["q"] = lin("w_q").reshape(B, S, h, dh)
    else:
        out["a_q"] = lin("w_a_q").reshape(B, S, h, dims.rank_q)
        out["b_q"] = lin("w_b_q").reshape(B, S, dims.rank_q, dh)
    out["a_k"] = lin("w_a_k").reshape(B, S, h, dims.rank_k)
    out["b_k"] = lin("w_b_k").reshape(B, S, dims.rank_k, dh)
    out["a_v"] = lin("w_a_v").reshape(B, S, h, dims.rank_v)
    out["b_v"] = lin("w_b_v").reshape(B, S, dims.rank_v, dh)
    return out


# ---------------------------------------------------------------------------
# Step 2: rotary position embedding
# ---------------------------------------------------------------------------

def rope_angles(pos: np.ndarray, head_dim: int, base: float) -> np.ndarray:
    """angle[p, i] = pos[p] * base^(-2i/d_h), i < d_h/2, in float64."""
    if head_dim % 2:
        raise ValueError("rotary embedding needs an even head_dim")
    i = np.arange(head_dim // 2, dtype=np.float64)
    theta = np.power(float(base), -2.0 * i / head_dim)
    return np.asarray(pos, dtype=np.float64)[:, None] * theta[None, :]


def rope(v: np.ndarray, pos: np.ndarray, base: float) -> np.ndarray:
    """Rotate v [B, S, rows, d_h] at positions pos [S] (all rows of a token share them).

    Element pairs (2i, 2i+1) turn by angle pos * theta_i:
        y_2i = x_2i cos - x_2i+1 sin,   y_2i+1 = x_2i sin + x_2i+1 cos.
    ([coreui] "关键问题及回答" 问题2: RoPE_t applied to a token's B_K factor.)
    """
    v = np.asarray(v, dtype=np.float64)
    ang = rope_angles(pos, v.shape[-1], base)          # [S, d_h/2]
    c = np.cos(ang)[None, :, None, :]
    s = np.sin(ang)[None, :, None, :]
    x0 = v[..., 0::2]
    x1 = v[..., 1::2]
    out = np.empty_like(v)
    out[..., 0::2] = x0 * c - x1 * s
    out[..., 1::2] = x0 * s + x1 * c
    return out


def positions(start_pos: int, seq: int) -> np.ndarray:
    """Zero-based absolute positions start_pos + s of a block of seq tokens."""
    return np.arange(start_pos, start_pos + seq, dtype=np.int64)


def rotate_factors(f: Dict[str, np.ndarray], start_pos: int, dims: Dims) -> Dict[str, np.ndarray]:
    """Pre-rotate the query B factors and the key B factors (KV-only: the plain Q).

    B~_K(x_t) <- RoPE_t(B_K(x_t)) ([coreui] 问题2); B_Q likewise; A factors and
    B_V are not rotated.
    """
    out = dict(f)
    S = f["b_k"].shape[1]
    pos = positions(start_pos, S)
    out["b_k"] = rope(f["b_k"], pos, dims.rope_base)
    if dims.kv_only:
        out["q"] = rope(f["q"], pos, dims.rope_base)
    else:
        out["b_q"] = rope(f["b_q"], pos, dims.rope_base)
    return out


# ---------------------------------------------------------------------------
# Step 3: factor cache
# ---------------------------------------------------------------------------

def cache_new(dims: Dims, max_batch: int, max_seq: int) -> Dict[str, np.ndarray]:
    """The four factor-cache tensors ([coreui] "类定义与初始化": cache_kA, cache_vA
    [max_batch, max_seq, h, R]; cache_kB, cache_vB [max_batch, max_seq, R, d_h])."""
    h, dh = dims.n_heads, dims.head_dim
    return {
        "a_k": np.zeros((max_batch, max_seq, h, dims.rank_k)),
        "b_k": np.zeros((max_batch, max_seq, dims.rank_k, dh)),
        "a_v": np.zeros((max_batch, max_seq, h, dims.rank_v)),
        "b_v": np.zeros((max_batch, max_seq, dims.rank_v, dh)),
    }


def cache_append(cache: Dict[str, np.ndarray], f: Dict[str, np.ndarray], start_pos: int) -> None:
    """cache[:B, start_pos:start_pos+S] = factors ([coreui] "前向传播", cache writes)."""
    B, S = f["b_k"].shape[:2]
    for k in ("a_k", "b_k", "a_v", "b_v"):
        cache[k][:B, start_pos:start_pos + S] = f[k]


# ---------------------------------------------------------------------------
# Step 4: reconstruction of Q, K, V from their factors
# ---------------------------------------------------------------------------

def reconstruct(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """X = (1/R) sum_r a_r (x) b_r for a [..., h, R], b [..., R, d_h] -> [..., h, d_h].

    Written as an explicit sum of R outer products ([coreui] "公式描述").
    """
    R = a.shape[-1]
    if b.shape[-2] != R:
        raise ValueError("rank mismatch between head and dim factors")
    out = np.zeros(a.shape[:-1] + (b.shape[-1],), dtype=np.float64)
    for r in range(R):
        out += a[..., :, r, None] * b[..., None, r, :]
    return out / R


def queries(f: Dict[str, np.ndarray], dims: Dims) -> np.ndarray:
    """Q [B, S, h, d_h] from the (rotated) query factors, or the plain rotated Q."""
    if dims.kv_only:
        return np.asarray(f["q"], dtype=np.float64)
    return reconstruct(np.asarray(f["a_q"], np.float64), np.asarray(f["b_q"], np.float64))


# ---------------------------------------------------------------------------
# Steps 5-7: scaled dot-product attention
# ---------------------------------------------------------------------------

def attend_head(q: np.ndarray, k: np.ndarray, v: np.ndarray, q_pos: np.ndarray, causal: bool,
                return_probs: bool = False):
    """One head: q [Sq, d_h] at absolute positions q_pos, keys/values k, v [T, d_h] at 0..T-1.

    scores = q k^T / sqrt(d_h) ([jieyibu] Ⅱ.1; [coreui] "前向传播"); with the causal
    mask, key t is visible to a query at position p iff t <= p.  Softmax over the
    visible keys: subtract the row maximum, exponentiate, divide by the sum.
    """
    d_h = q.shape[-1]
    out = np.empty((q.shape[0], v.shape[-1]), dtype=np.float64)
    probs = []
    for i in range(q.shape[0]):
        n = int(q_pos[i]) + 1 if causal else k.shape[0]
        scores = (k[:n] @ q[i]) / math.sqrt(d_h)
        e = np.exp(scores - scores.max())
        p = e / e.sum()
        out[i] = p @ v[:n]
        if return_probs:
            probs.append(p)
    if return_probs:
        return out, probs
    return out


def prefill(fq: Dict[str, np.ndarray], cache: Dict[str, np.ndarray], dims: Dims, batch: int, seq: int,
            start_pos: int, causal: bool = True, rows: Optional[Sequence[int]] = None) -> np.ndarray:
    """Attention of seq queries (positions start_pos..start_pos+seq-1) over the cached
    keys/values 0..start_pos+seq-1.  Returns out [B, S, h*d_h] (head-major, as the
    forward code's transpose/view lays it out).  With `rows` given, only those query
    rows s are computed (the others stay NaN): each row is its own definition.
    """
    h, dh = dims.n_heads, dims.head_dim
    T = start_pos + seq
    Q = queries(fq, dims)                                           # [B, S, h, d_h]
    out = np.full((batch, seq, h * dh), np.nan)
    sel = np.arange(seq) if rows is None else np.asarray(rows, dtype=np.int64)
    q_pos = positions(start_pos, seq)[sel]
    for b in range(batch):
        for hh in range(h):
            k = reconstruct(cache["a_k"][b, :T, hh:hh + 1, :], cache["b_k"][b, :T])[:, 0, :]
            v = reconstruct(cache["a_v"][b, :T, hh:hh + 1, :], cache["b_v"][b, :T])[:, 0, :]
            o = attend_head(Q[b, sel, hh, :], k, v, q_pos, causal)
            out[b, sel, hh * dh:(hh + 1) * dh] = o
    return out


def decode(fq: Dict[str, np.ndarray], cache: Dict[str, np.ndarray], dims: Dims, batch: int,
           ctx_len: int) -> np.ndarray:
    """One new query per sequence, at position ctx_len-1, over keys 0..ctx_len-1.

    The new token's factors must already be in the cache (the forward code writes
    before it reads).  fq holds the query factors with a sequence axis of length 1.
    Returns out [B, h*d_h].
    """
    return prefill(fq, cache, dims, batch, 1, ctx_len - 1, causal=True)[:, 0, :]


# --------------------------------------------------------------------------
# Backward (training): gradients of prefill() by the chain rule, written out
# --------------------------------------------------------------------------

def reconstruct_backward(a: np.ndarray, b: np.ndarray, dx: np.ndarray):
    """Gradients of X = (1/R) sum_r a_r (x) b_r given dX [..., h, d_h]:
    dA[..., h, r] = (1/R) dX[..., h, :] . b[..., r, :] and
    dB[..., r, :] = (1/R) sum_h a[..., h, r] dX[..., h, :].
    """
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    R = a.shape[-1]
    da = np.zeros(a.shape, dtype=np.float64)
    db = np.zeros(b.shape, dtype=np.float64)
    for r in range(R):
        da[..., :, r] = (dx * b[..., None, r, :]).sum(-1) / R
        db[..., r, :] = (a[..., :, r, None] * dx).sum(-2) / R
    return da, db


def attend_head_backward(q: np.ndarray, k: np.ndarray, v: np.ndarray, q_pos: np.ndarray, causal: bool,
                         dout: np.ndarray):
    """Gradients of attend_head given dO [Sq, d_h]: returns dq [Sq, d_h], dk, dv [T, d_h].

    Per query row with visible keys n, scores s = k q / sqrt(d_h), p = softmax(s):
    dv += p (x) dO, dp = v dO, ds = p * (dp - p . dp), dq = ds k / sqrt(d_h),
    dk += ds (x) q / sqrt(d_h).
    """
    d_h = q.shape[-1]
    rs = 1.0 / math.sqrt(d_h)
    dq = np.zeros(q.shape, dtype=np.float64)
    dk = np.zeros(k.shape, dtype=np.float64)
    dv = np.zeros(v.shape, dtype=np.float64)
    for i in range(q.shape[0]):
        n = int(q_pos[i]) + 1 if causal else k.shape[0]
        scores = (k[:n] @ q[i]) * rs
        e = np.exp(scores - scores.max())
        p = e / e.sum()
        dv[:n] += p[:, None] * dout[i][None, :]
        dp = v[:n] @ dout[i]
        ds = p * (dp - p @ dp)
        dq[i] = (ds @ k[:n]) * rs
        dk[:n] += ds[:, None] * q[i][None, :] * rs
    return dq, dk, dv


def prefill_backward(fq: Dict[str, np.ndarray], cache: Dict[str, np.ndarray], dims: Dims, batch: int, seq: int,
                     start_pos: int, causal: bool, dout: np.ndarray, heads=None):
    """Gradients of sum(prefill(...) * dout) with respect to the query factors
    (as passed: b_q rotated; KV-only: the rotated Q) and to the cached key/value
    factors at positions 0..start_pos+seq-1.

    Returns (dfq, dkv): dfq has the keys of fq; dkv has a_k, b_k, a_v, b_v
    shaped [B, start_pos+seq, ...].

    heads: if given, only these heads' attention gradients are formed (the rest
    stay zero), so only those heads' entries of the head-factor gradients
    (a_q, a_k, a_v) are complete; the dim-factor gradients, which sum over the
    heads, are then partial.
    """
    h, dh = dims.n_heads, dims.head_dim
    T = start_pos + seq
    Q = queries(fq, dims)
    dQ = np.zeros((batch, seq, h, dh))
    dK = np.zeros((batch, T, h, dh))
    dV = np.zeros((batch, T, h, dh))
    q_pos = positions(start_pos, seq)
    dout = np.asarray(dout, np.float64).reshape(batch, seq, h, dh)
    for b in range(batch):
        for hh in (range(h) if heads is None else heads):
            k = reconstruct(cache["a_k"][b, :T, hh:hh + 1, :], cache["b_k"][b, :T])[:, 0, :]
            v = reconstruct(cache["a_v"][b, :T, hh:hh + 1, :], cache["b_v"][b, :T])[:, 0, :]
            dq, dk, dv = attend_head_backward(Q[b, :, hh, :], k, v, q_pos, causal, dout[b, :, hh, :])
            dQ[b, :, hh] = dq
            dK[b, :, hh] = dk
            dV[b, :, hh] = dv
    if dims.kv_only:
        dfq = {"q": dQ}
    else:
        da, db = reconstruct_backward(fq["a_q"], fq["b_q"], dQ)
        dfq = {"a_q": da, "b_q": db}
    da_k, db_k = reconstruct_backward(cache["a_k"][:batch, :T], cache["b_k"][:batch, :T], dK)
    da_v, db_v = reconstruct_backward(cache["a_v"][:batch, :T], cache["b_v"][:batch, :T], dV)
    return dfq, {"a_k": da_k, "b_k": db_k, "a_v": da_v, "b_v": db_v}


def rope_backward(g: np.ndarray, pos: np.ndarray, base: float) -> np.ndarray:
    """Gradient with respect to the unrotated vectors of rope(v, pos, base), given
    the gradient g of the rotated ones: each pair's rotation is orthogonal, so
    the gradient is turned back by the same angle, rope(g, -pos)."""
    return rope(g, -np.asarray(pos, dtype=np.float64), base)


def paged_gather(pools: Dict[str, np.ndarray], block_table: np.ndarray, b: int, n: int) -> Dict[str, np.ndarray]:
    """Cache rows of tokens 0..n-1 of sequence b from page pools [n_pages, P, ...].

    Serving layout, not on the pages: token t of sequence b lives in page
    block_table[b, t // P] at row t % P.
    """
    P = pools["a_k"].shape[1]
    t = np.arange(n, dtype=np.int64)
    pages = np.asarray(block_table, dtype=np.int64)[b, t // P]
    rows = t % P
    return {k: np.asarray(pools[k], dtype=np.float64)[pages, rows] for k in ("a_k", "b_k", "a_v", "b_v")}


def decode_paged(fq: Dict[str, np.ndarray], pools: Dict[str, np.ndarray], block_table: np.ndarray,
                 ctx_lens, dims: Dims) -> np.ndarray:
    """Decode with a key count per sequence over a paged cache: sequence b's new
    query (position ctx_lens[b]-1) attends over its keys 0..ctx_lens[b]-1, exactly
    as decode() does for one sequence.  A sequence with no keys gets zeros
    (a convention: the pages never call attention over nothing).
    Returns out [B, h*d_h].
    """
    B = len(ctx_lens)
    out = np.zeros((B, dims.n_heads * dims.head_dim), dtype=np.float64)
    for b in range(B):
        L = int(ctx_lens[b])
        if L == 0:
            continue
        rows = paged_gather(pools, block_table, b, L)
        cache_b = {k: v[None] for k, v in rows.items()}
        fq_b = {k: (None if v is None else np.asarray(v)[b:b + 1]) for k, v in fq.items()}
        out[b] = decode(fq_b, cache_b, dims, 1, L)[0]
    return out


# ---------------------------------------------------------------------------
# Shared-basis variant: dim factors shared by every token
# ---------------------------------------------------------------------------

def shared_keys_values(a_k: np.ndarray, a_v: np.ndarray, b_k: np.ndarray, b_v: np.ndarray, base: float,
                       n: int):
    """Keys and values 0..n-1 of one sequence in the shared-basis variant ([coreui]
    "优点与创新", item 5, names a variant that shares the basis vectors across
    tokens; it gives no formula, the reading is in the design notes): the dim
    factors b_k [R_K, d_h] and b_v [R_V, d_h] are parameters common to all tokens,
    the head factors a_k [n, h, R_K] and a_v [n, h, R_V] stay per token, and each
    key is rotated at its own position:
        k[t, h] = rope((1/R_K) sum_r a_k[t, h, r] b_k[r], t),
        v[t, h] = (1/R_V) sum_r a_v[t, h, r] b_v[r].
    Returns k, v [n, h, d_h]."""
    a_k = np.asarray(a_k, np.float64)[:n]
    a_v = np.asarray(a_v, np.float64)[:n]
    b_k = np.asarray(b_k, np.float64)
    b_v = np.asarray(b_v, np.float64)
    k = reconstruct(a_k, np.broadcast_to(b_k, (n,) + b_k.shape))
    k = rope(k[None], positions(0, n), base)[0]
    v = reconstruct(a_v, np.broadcast_to(b_v, (n,) + b_v.shape))
    return k, v


def decode_shared(fq: Dict[str, np.ndarray], cache_a: Dict[str, np.ndarray], basis: Dict[str, np.ndarray],
                  dims: Dims, batch: int, ctx_len: int) -> np.ndarray:
    """One new query per sequence, at position ctx_len-1, over keys 0..ctx_len-1 of
    a shared-basis cache (cache_a: a_k [B, max_seq, h, R_K], a_v [B, max_seq, h, R_V];
    basis: b_k [R_K, d_h], b_v [R_V, d_h], b_k unrotated).  fq as for decode().
    Returns out [B, h*d_h]."""
    h, dh = dims.n_heads, dims.head_dim
    Q = queries(fq, dims)                                           # [B, 1, h, d_h]
    out = np.empty((batch, h * dh), dtype=np.float64)
    q_pos = np.array([ctx_len - 1], dtype=np.int64)
    for b in range(batch):
        k, v = shared_keys_values(cache_a["a_k"][b], cache_a["a_v"][b], basis["b_k"], basis["b_v"],
                                  dims.rope_base, ctx_len)
        for hh in range(h):
            out[b, hh * dh:(hh + 1) * dh] = attend_head(Q[b, :, hh, :], k[:, hh, :], v[:, hh, :], q_pos, True)[0]
    return out


def prefill_shared(fq: Dict[str, np.ndarray], cache_a: Dict[str, np.ndarray], basis: Dict[str, np.ndarray],
                   dims: Dims, batch: int, seq: int, start_pos: int, causal: bool = True,
                   rows: Optional[Sequence[int]] = None) -> np.ndarray:
    """Attention of seq queries (positions start_pos..start_pos+seq-1) over keys
    0..start_pos+seq-1 of a shared-basis cache (cache_a and basis as for
    decode_shared; the block's own head factors already appended).  Keys and
    values are those of shared_keys_values; the attention is the standard
    masked softmax of prefill().  Returns out [B, S, h*d_h]; with `rows` given,
    only those query rows are computed (the others stay NaN)."""
    h, dh = dims.n_heads, dims.head_dim
    T = start_pos + seq
    Q = queries(fq, dims)                                           # [B, S, h, d_h]
    out = np.full((batch, seq, h * dh), np.nan)
    sel = np.arange(seq) if rows is None else np.asarray(rows, dtype=np.int64)
    q_pos = positions(start_pos, seq)[sel]
    for b in range(batch):
        k, v = shared_keys_values(cache_a["a_k"][b], cache_a["a_v"][b], basis["b_k"], basis["b_v"],
                                  dims.rope_base, T)
        for hh in range(h):
            out[b, sel, hh * dh:(hh + 1) * dh] = attend_head(Q[b, sel, hh, :], k[:, hh, :], v[:, hh, :], q_pos,
                                                             causal)
    return out


def layer_forward(x: np.ndarray, w: Dict[str, np.ndarray], dims: Dims, cache: Dict[str, np.ndarray],
                  start_pos: int, causal: bool = True, rows: Optional[Sequence[int]] = None) -> np.ndarray:
    """The whole TPA attention path for one block of tokens, without the output
    projection: project, pre-rotate, append to the cache, attend over the cache
    ([coreui] "前向传播": the cache is written before it is read).  With `rows`
    given, only those query rows are attended (the others stay NaN), as in
    prefill."""
    B, S, _ = x.shape
    f = rotate_factors(project(x, w, dims), start_pos, dims)
    cache_append(cache, f, start_pos)
    return prefill(f, cache, dims, B, S, start_pos, causal, rows=rows)
