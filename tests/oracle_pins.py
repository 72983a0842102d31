"""Pins of the fp64 oracle to facts it does not compute itself.

Each pin is a plain function that raises AssertionError on failure, so that the
mutation tests can run the whole set against deliberately broken copies of the
oracle and check that every planted mistake is caught by at least one pin.

What pins what:
  brute_force_*        everything (pure-Python scalar loops, complex-number RoPE)
  textbook_*           MHA / MQA / GQA as TPA with constant head factors, against
                       torch's scaled_dot_product_attention with textbook RoPE
  rope_*               rotary embedding identities (identity at 0, isometry,
                       composition, relative-position invariance of scores)
  commute_*            rotating each b_r equals rotating the reconstructed tensor,
                       so pre-rotating the cached factor matches the forward code's order
  softmax_rows         attention rows sum to 1, outputs lie in the hull of the values
  closed_form_*        hand-derived values and exact special cases
  incremental_*        chunked prefill and decode against one long prefill
  paged_*              decode with a key count per sequence over a paged cache,
                       against the brute force run on each sequence's own prefix
  backward_*           the written-out gradients against central finite
                       differences of the forward oracle; the inverse rotation
                       against the adjoint identity
  shared_*             the shared-basis decode and prefill against their scalar
                       brute force, against the standard decode / prefill over
                       per-token rotated copies of the basis, and with constant
                       values
"""
import math

import numpy as np
import torch

import oracle.tpa_oracle as O
import brute_force
import textbook

TOL = 1e-12


def _close(a, b, tol=TOL, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    err = np.max(np.abs(a - b)) if a.size else 0.0
    scale = max(1.0, float(np.max(np.abs(b)))) if b.size else 1.0
    assert err <= tol * scale, f"{what}: max abs err {err:.3e} > {tol * scale:.3e}"


def _weights(rng, dims, std=0.5):
    h, d, dm = dims.n_heads, dims.head_dim, dims.d_model
    w = {}
    if dims.kv_only:
        w["w_q"] = rng.normal(0, std, (h * d, dm))
    else:
        w["w_a_q"] = rng.normal(0, std, (h * dims.rank_q, dm))
        w["w_b_q"] = rng.normal(0, std, (dims.rank_q * d, dm))
    w["w_a_k"] = rng.normal(0, std, (h * dims.rank_k, dm))
    w["w_b_k"] = rng.normal(0, std, (dims.rank_k * d, dm))
    w["w_a_v"] = rng.normal(0, std, (h * dims.rank_v, dm))
    w["w_b_v"] = rng.normal(0, std, (dims.rank_v * d, dm))
    return w


def _factors(rng, dims, B, S, std=0.7):
    h, d = dims.n_heads, dims.head_dim
    f = {}
    if dims.kv_only:
        f["q"] = rng.normal(0, std, (B, S, h, d))
    else:
        f["a_q"] = rng.normal(0, std, (B, S, h, dims.rank_q))
        f["b_q"] = rng.normal(0, std, (B, S, dims.rank_q, d))
    f["a_k"] = rng.normal(0, std, (B, S, h, dims.rank_k))
    f["b_k"] = rng.normal(0, std, (B, S, dims.rank_k, d))
    f["a_v"] = rng.normal(0, std, (B, S, h, dims.rank_v))
    f["b_v"] = rng.normal(0, std, (B, S, dims.rank_v, d))
    return f


def _oracle_chunked(x, w, dims, split, causal=True):
    """Run the oracle's layer in two chunks [0, split) and [split, T); return all rows."""
    B, T, _ = x.shape
    cache = O.cache_new(dims, B, T)
    outs = []
    if split > 0:
        outs.append(O.layer_forward(x[:, :split], w, dims, cache, 0, causal))
    outs.append(O.layer_forward(x[:, split:], w, dims, cache, split, causal))
    return np.concatenate(outs, axis=1)


# --------------------------------------------------------------------------
# Brute force
# --------------------------------------------------------------------------

BRUTE_CASES = [
    # d_model, h, d_h, R_Q, R_K, R_V, base, B, T, split
    (6, 3, 4, 2, 3, 1, 10000.0, 2, 5, 0),
    (5, 2, 6, 3, 2, 2, 3.0, 1, 6, 2),
    (4, 3, 2, 1, 1, 3, 1.7, 2, 4, 3),
    (6, 2, 4, 0, 2, 3, 2.5, 2, 5, 1),     # TPA-KVonly
]


def brute_force_causal():
    for ci, (dm, h, d, rq, rk, rv, base, B, T, split) in enumerate(BRUTE_CASES):
        rng = np.random.default_rng(100 + ci)
        dims = O.Dims(dm, h, d, rq, rk, rv, base)
        x = rng.normal(0, 1, (B, T, dm))
        w = _weights(rng, dims)
        got = _oracle_chunked(x, w, dims, split, causal=True)
        ref = brute_force.layer(x.tolist(), {k: v.tolist() for k, v in w.items()}, dm, h, d, rq, rk, rv, base,
                                causal=True)
        _close(got, ref, what=f"brute causal case {ci}")


def brute_force_noncausal():
    for ci, (dm, h, d, rq, rk, rv, base, B, T, _) in enumerate(BRUTE_CASES):
        rng = np.random.default_rng(200 + ci)
        dims = O.Dims(dm, h, d, rq, rk, rv, base)
        x = rng.normal(0, 1, (B, T, dm))
        w = _weights(rng, dims)
        got = _oracle_chunked(x, w, dims, 0, causal=False)
        ref = brute_force.layer(x.tolist(), {k: v.tolist() for k, v in w.items()}, dm, h, d, rq, rk, rv, base,
                                causal=False)
        _close(got, ref, what=f"brute non-causal case {ci}")


# --------------------------------------------------------------------------
# Textbook MHA / MQA / GQA as non-contextual TPA
# --------------------------------------------------------------------------

def _noncontextual_a(B, S, h, groups):
    """Head factor with R = groups: a_r[h] = groups * [h belongs to group r]."""
    a = np.zeros((B, S, h, groups))
    per = h // groups
    for hh in range(h):
        a[:, :, hh, hh // per] = groups
    return a


def _textbook_case(h, d, groups, q_mode, B, S, start_pos, base, causal, seed):
    rng = np.random.default_rng(seed)
    T = start_pos + S
    rq = 0 if q_mode == "plain" else h
    dims = O.Dims(8, h, d, rq, groups, groups, base)
    # unrotated dim factors for all T tokens (history + this chunk)
    bk = rng.normal(0, 1, (B, T, groups, d))
    bv = rng.normal(0, 1, (B, T, groups, d))
    qraw = rng.normal(0, 1, (B, S, h, d))
    cache = O.cache_new(dims, B, T)
    chunks = [(0, start_pos), (start_pos, T)] if start_pos > 0 else [(0, T)]
    out = None
    for lo, hi in chunks:
        f = {"a_k": _noncontextual_a(B, hi - lo, h, groups), "b_k": bk[:, lo:hi],
             "a_v": _noncontextual_a(B, hi - lo, h, groups), "b_v": bv[:, lo:hi]}
        if hi == T:
            if q_mode == "plain":
                f["q"] = qraw
            else:   # MHA-style query factors: R_Q = h, a_r = h e_r, b_r = per-head query
                f["a_q"] = _noncontextual_a(B, S, h, h)
                f["b_q"] = qraw
        else:
            if q_mode == "plain":
                f["q"] = np.zeros((B, hi - lo, h, d))
            else:
                f["a_q"] = np.zeros((B, hi - lo, h, h))
                f["b_q"] = np.zeros((B, hi - lo, h, d))
        f = O.rotate_factors(f, lo, dims)
        O.cache_append(cache, f, lo)
        if hi == T:
            out = O.prefill(f, cache, dims, B, hi - lo, lo, causal)
    pos_q = torch.arange(start_pos, T)
    pos_k = torch.arange(T)
    q_t = textbook.rope_complex(torch.from_numpy(qraw), pos_q, base)
    k_t = textbook.rope_complex(torch.from_numpy(bk), pos_k, base)
    ref = textbook.attention(q_t, k_t, torch.from_numpy(bv), start_pos, causal)
    _close(out, ref.numpy(), tol=1e-11, what=f"textbook h={h} groups={groups} q={q_mode} sp={start_pos}")


def textbook_mha():
    _textbook_case(h=4, d=8, groups=4, q_mode="factored", B=2, S=7, start_pos=0, base=10000.0, causal=True, seed=1)
    _textbook_case(h=3, d=6, groups=3, q_mode="plain", B=1, S=5, start_pos=4, base=50.0, causal=True, seed=2)


def textbook_mqa():
    _textbook_case(h=4, d=8, groups=1, q_mode="factored", B=2, S=9, start_pos=0, base=100.0, causal=True, seed=3)
    _textbook_case(h=5, d=4, groups=1, q_mode="plain", B=2, S=6, start_pos=0, base=10000.0, causal=False, seed=4)


def textbook_gqa():
    _textbook_case(h=8, d=8, groups=4, q_mode="factored", B=1, S=8, start_pos=0, base=10000.0, causal=True, seed=5)
    _textbook_case(h=6, d=4, groups=2, q_mode="plain", B=2, S=5, start_pos=3, base=7.0, causal=True, seed=6)


# --------------------------------------------------------------------------
# Rotary embedding identities
# --------------------------------------------------------------------------

def rope_identities():
    rng = np.random.default_rng(7)
    for d, base in ((2, 3.0), (8, 10000.0), (64, 10000.0), (128, 500000.0)):
        v = rng.normal(0, 1, (2, 5, 3, d))
        # position 0 is the identity
        _close(O.rope(v[:, :1], np.array([0]), base), v[:, :1], what="rope at position 0")
        # each (2i, 2i+1) pair keeps its length
        pos = np.array([1, 7, 100, 4095, 131072])
        r = O.rope(v, pos, base)
        _close(r[..., 0::2] ** 2 + r[..., 1::2] ** 2, v[..., 0::2] ** 2 + v[..., 1::2] ** 2, tol=1e-12,
               what="rope pair norms")
        # rotations compose: R_q R_p = R_{p+q}
        p2 = np.array([3, 11, 9, 1, 65536])
        _close(O.rope(O.rope(v, pos, base), p2, base), O.rope(v, pos + p2, base), tol=1e-10,
               what="rope composition")
        # scores depend only on the position difference
        u = rng.normal(0, 1, (1, 5, 1, d))
        w = rng.normal(0, 1, (1, 5, 1, d))
        sh = 1234
        a = np.sum(O.rope(u, pos, base) * O.rope(w, pos[::-1].copy(), base), axis=-1)
        b = np.sum(O.rope(u, pos + sh, base) * O.rope(w, pos[::-1] + sh, base), axis=-1)
        _close(a, b, tol=1e-9, what="rope relative position")


def rope_textbook():
    """The oracle's rotary embedding equals the complex-product formulation."""
    rng = np.random.default_rng(8)
    for d, base in ((2, 2.0), (6, 10.0), (64, 10000.0)):
        v = rng.normal(0, 1, (2, 6, 4, d))
        pos = np.array([0, 1, 2, 17, 1000, 131072])
        ref = textbook.rope_complex(torch.from_numpy(v), torch.from_numpy(pos), base).numpy()
        _close(O.rope(v, pos, base), ref, tol=1e-10, what=f"rope vs complex d={d}")


# --------------------------------------------------------------------------
# Rotating the factors commutes with the factor sum
# --------------------------------------------------------------------------

def commute_rope_factor_sum():
    rng = np.random.default_rng(9)
    for h, R, d in ((4, 2, 8), (3, 6, 64), (5, 1, 4)):
        a = rng.normal(0, 1, (2, 5, h, R))
        b = rng.normal(0, 1, (2, 5, R, d))
        pos = np.array([0, 3, 9, 70, 4000])
        lhs = O.rope(O.reconstruct(a, b), pos, 10000.0)        # rotate the reconstructed tensor
        rhs = O.reconstruct(a, O.rope(b, pos, 10000.0))        # rotate each b_r (pre-rotation)
        _close(lhs, rhs, what="RoPE commutes with the factor sum")


def commute_code_order_attention():
    """Attention in the forward code's order (cache unrotated factors, rotate the
    reconstructed q and k) equals the pre-rotated cache order."""
    rng = np.random.default_rng(10)
    dims = O.Dims(8, 3, 8, 2, 2, 3, 10000.0)
    B, S = 2, 7
    f = _factors(rng, dims, B, S)
    # prose order: pre-rotate, cache, attend
    fr = O.rotate_factors(f, 0, dims)
    cache = O.cache_new(dims, B, S)
    O.cache_append(cache, fr, 0)
    got = O.prefill(fr, cache, dims, B, S, 0, True)
    # code order: reconstruct unrotated, then rotate q and k per head row
    pos = O.positions(0, S)
    q = O.rope(O.reconstruct(f["a_q"], f["b_q"]), pos, dims.rope_base)
    k = O.rope(O.reconstruct(f["a_k"], f["b_k"]), pos, dims.rope_base)
    v = O.reconstruct(f["a_v"], f["b_v"])
    ref = np.empty_like(got)
    for b in range(B):
        for hh in range(dims.n_heads):
            ref[b, :, hh * 8:(hh + 1) * 8] = O.attend_head(q[b, :, hh], k[b, :, hh], v[b, :, hh], pos, True)
    _close(got, ref, what="code order vs pre-rotated order")


# --------------------------------------------------------------------------
# Softmax rows
# --------------------------------------------------------------------------

def softmax_rows():
    rng = np.random.default_rng(11)
    T, d = 40, 16
    q = rng.normal(0, 3, (T, d))
    k = rng.normal(0, 3, (T, d))
    v = rng.normal(0, 1, (T, d))
    pos = np.arange(T)
    for causal in (True, False):
        out, probs = O.attend_head(q, k, v, pos, causal, return_probs=True)
        for i, p in enumerate(probs):
            n = i + 1 if causal else T
            assert len(p) == n, "row covers the visible keys"
            assert abs(p.sum() - 1.0) < 1e-14, "row sums to 1"
            assert np.all(p >= 0)
            assert np.all(out[i] <= v[:n].max(axis=0) + 1e-12)
            assert np.all(out[i] >= v[:n].min(axis=0) - 1e-12)


# --------------------------------------------------------------------------
# Closed forms and exact special cases
# --------------------------------------------------------------------------

def closed_form_two_tokens():
    """h = 1, d_h = 2, every rank 1 and every head factor 1, theta_0 = 1:
    key 0 = (0, 1) at position 0, key 1 = (1, 0) at position 1, query (1, 0) at
    position 1.  After rotation q = k1 = (cos 1, sin 1), so the scores are
    sin(1)/sqrt(2) and 1/sqrt(2), and the output is their softmax applied to v0, v1.
    The sign of sin(1) fixes the direction of the rotation."""
    dims = O.Dims(4, 1, 2, 1, 1, 1, 10000.0)
    one = np.ones((1, 2, 1, 1))
    f = {"a_q": one, "b_q": np.array([[[[0.0, 0.0]], [[1.0, 0.0]]]]),
         "a_k": one, "b_k": np.array([[[[0.0, 1.0]], [[1.0, 0.0]]]]),
         "a_v": one, "b_v": np.array([[[[2.0, -1.0]], [[0.5, 3.0]]]])}
    fr = O.rotate_factors(f, 0, dims)
    cache = O.cache_new(dims, 1, 2)
    O.cache_append(cache, fr, 0)
    out = O.prefill(fr, cache, dims, 1, 2, 0, True)
    s0, s1 = math.sin(1.0) / math.sqrt(2.0), 1.0 / math.sqrt(2.0)
    p1 = 1.0 / (1.0 + math.exp(s0 - s1))
    p0 = 1.0 - p1
    exp_row1 = [p0 * 2.0 + p1 * 0.5, p0 * -1.0 + p1 * 3.0]
    _close(out[0, 1], exp_row1, tol=1e-14, what="two-token closed form")
    _close(out[0, 0], [2.0, -1.0], tol=1e-15, what="first row sees only itself")


def closed_form_special_cases():
    rng = np.random.default_rng(12)
    dims = O.Dims(8, 3, 8, 2, 2, 2, 10000.0)
    B, S = 2, 6

    def run(f, dd=dims):
        fr = O.rotate_factors(f, 0, dd)
        c = O.cache_new(dd, B, S)
        O.cache_append(c, fr, 0)
        return O.prefill(fr, c, dd, B, S, 0, True)

    f = _factors(rng, dims, B, S)
    base = run(f)
    v = O.reconstruct(f["a_v"], f["b_v"])                                  # [B,S,h,d]
    # the first token sees only itself: its output is V[0] exactly
    _close(base[:, 0], v[:, 0].reshape(B, -1), tol=1e-15, what="row 0 = V[0]")
    # zero key dim-factors: uniform attention, output = running mean of V
    g = dict(f)
    g["b_k"] = np.zeros_like(f["b_k"])
    out = run(g)
    mean = np.cumsum(v, axis=1) / np.arange(1, S + 1)[None, :, None, None]
    _close(out, mean.reshape(B, S, -1), what="B_K = 0 gives the running mean")
    # rank 2 with two identical terms equals rank 1 (pins the 1/R scale)
    d1 = O.Dims(8, 3, 8, 1, 1, 1, 10000.0)
    f1 = {k: val[..., :1] if k.startswith("a_") else val[..., :1, :] for k, val in f.items()}
    f2 = {k: np.concatenate([val, val], axis=-1) if k.startswith("a_") else np.concatenate([val, val], axis=-2)
          for k, val in f1.items()}
    _close(run(f2), run(f1, d1), what="rank-2 duplicate terms = rank 1")
    # (c a, b / c) leaves every product unchanged
    g = dict(f)
    g["a_k"] = f["a_k"] * 3.0
    g["b_k"] = f["b_k"] / 3.0
    g["a_q"] = f["a_q"] * -0.5
    g["b_q"] = f["b_q"] / -0.5
    _close(run(g), base, what="(c a, b/c) invariance")
    # scaling the value head factor scales the output
    g = dict(f)
    g["a_v"] = f["a_v"] * 2.5
    _close(run(g), base * 2.5, what="A_V scaling")


# --------------------------------------------------------------------------
# Incremental consistency (chunked prefill, decode)
# --------------------------------------------------------------------------

def incremental_decode():
    """Prefill of S tokens then k decode steps equals rows S..S+k-1 of one prefill
    of S+k tokens; each decode step equals the last row of that prefill."""
    rng = np.random.default_rng(13)
    for dims in (O.Dims(16, 4, 8, 3, 2, 2, 10000.0), O.Dims(12, 3, 6, 0, 2, 1, 500.0)):
        B, S, k = 2, 5, 4
        x = rng.normal(0, 1, (B, S + k, dims.d_model))
        w = _weights(rng, dims, std=0.4)
        full = O.layer_forward(x, w, dims, O.cache_new(dims, B, S + k), 0, True)
        cache = O.cache_new(dims, B, S + k)
        O.layer_forward(x[:, :S], w, dims, cache, 0, True)
        for j in range(k):
            pos = S + j
            f = O.rotate_factors(O.project(x[:, pos:pos + 1], w, dims), pos, dims)
            O.cache_append(cache, f, pos)
            out = O.decode(f, cache, dims, B, pos + 1)
            _close(out, full[:, pos], what=f"decode step {j}")


def incremental_chunked_prefill():
    rng = np.random.default_rng(14)
    dims = O.Dims(10, 2, 4, 2, 3, 2, 10000.0)
    B, T = 2, 11
    x = rng.normal(0, 1, (B, T, dims.d_model))
    w = _weights(rng, dims, std=0.4)
    full = O.layer_forward(x, w, dims, O.cache_new(dims, B, T), 0, True)
    cache = O.cache_new(dims, B, T)
    outs = []
    for lo, hi in ((0, 3), (3, 4), (4, 9), (9, 11)):
        outs.append(O.layer_forward(x[:, lo:hi], w, dims, cache, lo, True))
    _close(np.concatenate(outs, axis=1), full, what="chunked prefill")


# --------------------------------------------------------------------------
# Paged cache, key count per sequence
# --------------------------------------------------------------------------

def _scatter_pages(f, table, P, n_pages):
    """Inverse of a gather through the table: token t of sequence b goes to page
    table[b, t // P], row t % P (unused rows hold a value no sequence reads)."""
    pools = {}
    for k in ("a_k", "b_k", "a_v", "b_v"):
        B, T = f[k].shape[:2]
        pool = np.full((n_pages, P) + f[k].shape[2:], 7.0e3)
        for b in range(B):
            for t in range(T):
                pool[table[b, t // P], t % P] = f[k][b, t]
        pools[k] = pool
    return pools


PAGED_CASES = [
    # d_model, h, d_h, R_Q, R_K, R_V, base, page, lengths
    (6, 3, 4, 2, 3, 1, 10000.0, 2, (5, 1, 0, 3)),
    (5, 2, 6, 0, 2, 2, 7.0, 3, (4, 6)),
]


def _paged_case(ci, seed):
    dm, h, d, rq, rk, rv, base, P, lens = PAGED_CASES[ci]
    rng = np.random.default_rng(seed)
    dims = O.Dims(dm, h, d, rq, rk, rv, base)
    B, T = len(lens), max(lens)
    x = rng.normal(0, 1, (B, T, dm))
    w = _weights(rng, dims)
    f = O.rotate_factors(O.project(x, w, dims), 0, dims)
    pages_per_seq = (T + P - 1) // P
    n_pages = B * pages_per_seq + 2
    table = rng.permutation(n_pages)[:B * pages_per_seq].reshape(B, pages_per_seq)
    # each sequence's query factors at its own last position
    qkeys = ("q",) if dims.kv_only else ("a_q", "b_q")
    fq = {k: np.stack([f[k][b, max(lens[b] - 1, 0)] for b in range(B)])[:, None] for k in qkeys}
    return dims, x, w, f, fq, table, n_pages, P, lens


def paged_ragged_brute_force():
    """Decode with ctx_lens[b] keys for sequence b, through a shuffled page table,
    equals the brute force's last row on that sequence's own prefix; a sequence
    without keys gives zeros."""
    for ci in range(len(PAGED_CASES)):
        dims, x, w, f, fq, table, n_pages, P, lens = _paged_case(ci, 300 + ci)
        pools = _scatter_pages(f, table, P, n_pages)
        got = O.decode_paged(fq, pools, table, lens, dims)
        for b, L in enumerate(lens):
            if L == 0:
                _close(got[b], np.zeros_like(got[b]), what=f"paged case {ci} empty sequence {b}")
                continue
            ref = brute_force.layer(x[b:b + 1, :L].tolist(), {k: v.tolist() for k, v in w.items()},
                                    dims.d_model, dims.n_heads, dims.head_dim, dims.rank_q, dims.rank_k,
                                    dims.rank_v, dims.rope_base, causal=True)
            _close(got[b], ref[0][L - 1], what=f"paged case {ci} sequence {b}")


def paged_permutation_invariance():
    """Moving pages to other pool slots (with the table updated) changes nothing."""
    dims, x, w, f, fq, table, n_pages, P, lens = _paged_case(0, 400)
    a = O.decode_paged(fq, _scatter_pages(f, table, P, n_pages), table, lens, dims)
    perm = np.random.default_rng(401).permutation(n_pages)
    table2 = perm[table]
    b = O.decode_paged(fq, _scatter_pages(f, table2, P, n_pages), table2, lens, dims)
    assert np.array_equal(a, b), "paged decode depends on where the pages sit"


# --------------------------------------------------------------------------
# Backward
# --------------------------------------------------------------------------

def _fd_grad(f, x, eps=1e-6):
    """Central differences of the scalar f() with respect to every element of x
    (perturbed in place and restored)."""
    g = np.zeros_like(x)
    for idx in np.ndindex(x.shape):
        old = x[idx]
        x[idx] = old + eps
        fp = f()
        x[idx] = old - eps
        fm = f()
        x[idx] = old
        g[idx] = (fp - fm) / (2 * eps)
    return g


BACKWARD_CASES = [
    # h, d_h, R_Q, R_K, R_V, base, B, S, start_pos, causal
    (2, 4, 2, 2, 3, 10000.0, 2, 3, 2, True),     # chunked: earlier keys get gradients too
    (3, 2, 0, 1, 2, 5.0, 1, 4, 0, False),        # KV-only, every key visible
    (2, 6, 3, 3, 1, 100.0, 1, 3, 0, True),
]


def backward_finite_differences():
    for ci, (h, d, rq, rk, rv, base, B, S, sp, causal) in enumerate(BACKWARD_CASES):
        rng = np.random.default_rng(500 + ci)
        dims = O.Dims(8, h, d, rq, rk, rv, base)
        T = sp + S
        fq = {"q": rng.normal(0, 0.8, (B, S, h, d))} if dims.kv_only else \
            {"a_q": rng.normal(0, 0.8, (B, S, h, rq)), "b_q": rng.normal(0, 0.8, (B, S, rq, d))}
        cache = O.cache_new(dims, B, T)
        for k, shape in (("a_k", (h, rk)), ("b_k", (rk, d)), ("a_v", (h, rv)), ("b_v", (rv, d))):
            cache[k][:] = rng.normal(0, 0.8, (B, T) + shape)
        dout = rng.normal(0, 1, (B, S, h * d))
        loss = lambda: float(np.sum(O.prefill(fq, cache, dims, B, S, sp, causal) * dout))
        dfq, dkv = O.prefill_backward(fq, cache, dims, B, S, sp, causal, dout)
        for k in fq:
            _close(dfq[k], _fd_grad(loss, fq[k]), tol=1e-6, what=f"backward case {ci} d{k}")
        for k in ("a_k", "b_k", "a_v", "b_v"):
            _close(dkv[k], _fd_grad(loss, cache[k]), tol=1e-6, what=f"backward case {ci} d{k}")


def backward_rope_adjoint():
    """<rope(v), g> = <v, rope_backward(g)> at positions up to 131,072."""
    rng = np.random.default_rng(600)
    for d, base in ((8, 10000.0), (64, 500000.0)):
        pos = np.array([0, 3, 4095, 131071])
        v = rng.normal(0, 1, (2, 4, 3, d))
        g = rng.normal(0, 1, (2, 4, 3, d))
        lhs = np.sum(O.rope(v, pos, base) * g)
        rhs = np.sum(v * O.rope_backward(g, pos, base))
        _close(lhs, rhs, tol=1e-12, what=f"rope adjoint d={d}")


# ---------------------------------------------------------------------------
# Shared-basis variant
# ---------------------------------------------------------------------------

SHARED_CASES = [
    # h, d, rq, rk, rv, base, B, ctx
    (2, 4, 2, 2, 1, 10000.0, 2, 5),
    (3, 6, 0, 1, 3, 100.0, 1, 7),      # KV-only query
    (1, 8, 1, 3, 2, 10.0, 2, 9),       # large angles
]


def _shared_case(ci, seed, std=0.8):
    h, d, rq, rk, rv, base, B, ctx = SHARED_CASES[ci]
    rng = np.random.default_rng(seed)
    dims = O.Dims(8, h, d, rq, rk, rv, base)
    fq = {"q": rng.normal(0, std, (B, 1, h, d))} if dims.kv_only else \
        {"a_q": rng.normal(0, std, (B, 1, h, rq)), "b_q": rng.normal(0, std, (B, 1, rq, d))}
    cache_a = {"a_k": rng.normal(0, std, (B, ctx + 2, h, rk)), "a_v": rng.normal(0, std, (B, ctx + 2, h, rv))}
    basis = {"b_k": rng.normal(0, std, (rk, d)), "b_v": rng.normal(0, std, (rv, d))}
    return dims, fq, cache_a, basis, B, ctx


def shared_brute_force():
    """Shared-basis decode against the scalar brute force (complex rotation)."""
    for ci in range(len(SHARED_CASES)):
        dims, fq, cache_a, basis, B, ctx = _shared_case(ci, 700 + ci)
        got = O.decode_shared(fq, cache_a, basis, dims, B, ctx)
        Q = O.queries(fq, dims)
        for b in range(B):
            want = brute_force.shared_decode(Q[b, 0].tolist(), cache_a["a_k"][b, :ctx].tolist(),
                                             cache_a["a_v"][b, :ctx].tolist(), basis["b_k"].tolist(),
                                             basis["b_v"].tolist(), dims.rope_base)
            _close(got[b], np.array(want), what=f"shared case {ci} seq {b}")


def shared_equals_standard_with_rotated_copies():
    """A standard factor cache holding, for every token t, the shared basis
    pre-rotated at t (b_k[t] = rope(b_k, t)) and b_v itself gives the same decode."""
    for ci in range(len(SHARED_CASES)):
        dims, fq, cache_a, basis, B, ctx = _shared_case(ci, 720 + ci)
        n = ctx + 2
        cache = O.cache_new(dims, B, n)
        cache["a_k"][:] = cache_a["a_k"]
        cache["a_v"][:] = cache_a["a_v"]
        bk = np.broadcast_to(basis["b_k"], (B, n) + basis["b_k"].shape)
        cache["b_k"][:] = O.rope(bk, O.positions(0, n), dims.rope_base)
        cache["b_v"][:] = basis["b_v"]
        _close(O.decode_shared(fq, cache_a, basis, dims, B, ctx), O.decode(fq, cache, dims, B, ctx),
               what=f"shared vs standard case {ci}")


def shared_constant_values():
    """With R_V = 1 and a constant value head factor c, every value is c * b_v,
    so every head returns exactly c * b_v whatever the scores."""
    dims, fq, cache_a, basis, B, ctx = _shared_case(0, 740)
    cache_a["a_v"][:] = 0.6
    out = O.decode_shared(fq, cache_a, basis, dims, B, ctx)
    want = np.tile(0.6 * basis["b_v"][0], dims.n_heads)
    for b in range(B):
        _close(out[b], want, what="constant shared values")


SHARED_PREFILL_CASES = [
    # h, d, rq, rk, rv, base, B, S, start_pos, causal
    (2, 4, 2, 2, 1, 10000.0, 2, 4, 3, True),
    (3, 6, 0, 1, 3, 100.0, 1, 5, 0, True),     # KV-only query
    (1, 8, 1, 3, 2, 10.0, 2, 3, 4, False),     # large angles, every key visible
]


def _shared_prefill_case(ci, seed, std=0.8):
    h, d, rq, rk, rv, base, B, S, sp, causal = SHARED_PREFILL_CASES[ci]
    rng = np.random.default_rng(seed)
    dims = O.Dims(8, h, d, rq, rk, rv, base)
    fq = {"q": rng.normal(0, std, (B, S, h, d))} if dims.kv_only else \
        {"a_q": rng.normal(0, std, (B, S, h, rq)), "b_q": rng.normal(0, std, (B, S, rq, d))}
    n = sp + S + 2
    cache_a = {"a_k": rng.normal(0, std, (B, n, h, rk)), "a_v": rng.normal(0, std, (B, n, h, rv))}
    basis = {"b_k": rng.normal(0, std, (rk, d)), "b_v": rng.normal(0, std, (rv, d))}
    return dims, fq, cache_a, basis, B, S, sp, causal


def shared_prefill_brute_force():
    """Shared-basis prefill, row by row, against the scalar brute force: row s
    (position start_pos + s) attends over keys 0 .. start_pos + s (causal) or
    over every key."""
    for ci in range(len(SHARED_PREFILL_CASES)):
        dims, fq, cache_a, basis, B, S, sp, causal = _shared_prefill_case(ci, 760 + ci)
        got = O.prefill_shared(fq, cache_a, basis, dims, B, S, sp, causal)
        Q = O.queries(fq, dims)
        for b in range(B):
            for s_ in range(S):
                n = sp + s_ + 1 if causal else sp + S
                want = brute_force.shared_decode(Q[b, s_].tolist(), cache_a["a_k"][b, :n].tolist(),
                                                 cache_a["a_v"][b, :n].tolist(), basis["b_k"].tolist(),
                                                 basis["b_v"].tolist(), dims.rope_base)
                _close(got[b, s_], np.array(want), what=f"shared prefill case {ci} seq {b} row {s_}")


def shared_prefill_equals_standard_with_rotated_copies():
    """The standard prefill over a factor cache holding, for every token t, the
    shared basis rotated at t gives the same rows as the shared-basis prefill."""
    for ci in range(len(SHARED_PREFILL_CASES)):
        dims, fq, cache_a, basis, B, S, sp, causal = _shared_prefill_case(ci, 780 + ci)
        n = cache_a["a_k"].shape[1]
        cache = O.cache_new(dims, B, n)
        cache["a_k"][:] = cache_a["a_k"]
        cache["a_v"][:] = cache_a["a_v"]
        bk = np.broadcast_to(basis["b_k"], (B, n) + basis["b_k"].shape)
        cache["b_k"][:] = O.rope(bk, O.positions(0, n), dims.rope_base)
        cache["b_v"][:] = basis["b_v"]
        _close(O.prefill_shared(fq, cache_a, basis, dims, B, S, sp, causal),
               O.prefill(fq, cache, dims, B, S, sp, causal), what=f"shared prefill vs standard case {ci}")


ALL_PINS = [
    brute_force_causal, brute_force_noncausal, textbook_mha, textbook_mqa, textbook_gqa,
    rope_identities, rope_textbook, commute_rope_factor_sum, commute_code_order_attention,
    softmax_rows, closed_form_two_tokens, closed_form_special_cases, incremental_decode,
    incremental_chunked_prefill, paged_ragged_brute_force, paged_permutation_invariance,
    backward_finite_differences, backward_rope_adjoint, shared_brute_force,
    shared_equals_standard_with_rotated_copies, shared_constant_values, shared_prefill_brute_force,
    shared_prefill_equals_standard_with_rotated_copies,
]
