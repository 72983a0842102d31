"""CPU tests: the fp64 oracle against its pins, and the pins against planted mistakes.

The second half plants plausible mistakes in the oracle (on the CPU, by
monkeypatching its module) and checks that each one makes at least one pin fail.
"""
import math

import numpy as np
import pytest

import oracle.tpa_oracle as O
import oracle_pins as P


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=[p.__name__ for p in P.ALL_PINS])
def test_pin(pin):
    pin()


# --------------------------------------------------------------------------
# Planted mistakes
# --------------------------------------------------------------------------

_orig = {name: getattr(O, name) for name in
         ("rope", "rope_angles", "reconstruct", "project", "attend_head", "cache_append", "rotate_factors",
          "prefill", "positions", "paged_gather", "decode_paged", "attend_head_backward",
          "reconstruct_backward", "rope_backward")}


def _rope_sign(v, pos, base):
    return _orig["rope"](v, -np.asarray(pos), base)


def _rope_half_split(v, pos, base):
    v = np.asarray(v, dtype=np.float64)
    d = v.shape[-1]
    ang = _orig["rope_angles"](pos, d, base)
    c = np.cos(ang)[None, :, None, :]
    s = np.sin(ang)[None, :, None, :]
    x0, x1 = v[..., : d // 2], v[..., d // 2:]
    return np.concatenate([x0 * c - x1 * s, x0 * s + x1 * c], axis=-1)


def _angles_theta(pos, head_dim, base):
    i = np.arange(head_dim // 2, dtype=np.float64)
    return np.asarray(pos, dtype=np.float64)[:, None] * np.power(float(base), -i / head_dim)[None, :]


def _reconstruct_no_scale(a, b):
    return _orig["reconstruct"](a, b) * a.shape[-1]


def _project_a_transposed(x, w, dims):
    out = _orig["project"](x, w, dims)
    for k in ("a_q", "a_k", "a_v"):
        if k in out:
            B, S, h, R = out[k].shape
            out[k] = out[k].reshape(B, S, R, h).swapaxes(-1, -2).copy()
    return out


def _project_b_transposed(x, w, dims):
    out = _orig["project"](x, w, dims)
    for k in ("b_q", "b_k", "b_v"):
        if k in out:
            B, S, R, d = out[k].shape
            out[k] = out[k].reshape(B, S, d, R).swapaxes(-1, -2).copy()
    return out


def _attend_sees_next(q, k, v, q_pos, causal, return_probs=False):
    if not causal:
        return _orig["attend_head"](q, k, v, q_pos, causal, return_probs)
    T = k.shape[0]
    outs = []
    for i in range(q.shape[0]):
        n = min(int(q_pos[i]) + 2, T)
        s = (k[:n] @ q[i]) / math.sqrt(q.shape[-1])
        e = np.exp(s - s.max())
        outs.append((e / e.sum()) @ v[:n])
    out = np.array(outs).reshape(q.shape[0], v.shape[-1])
    if return_probs:
        return out, []
    return out


def _attend_scale_d(q, k, v, q_pos, causal, return_probs=False):
    return _orig["attend_head"](q * math.sqrt(q.shape[-1]) / q.shape[-1], k, v, q_pos, causal, return_probs)


def _append_at_zero(cache, f, start_pos):
    return _orig["cache_append"](cache, f, 0)


def _rotate_queries_shifted(f, start_pos, dims):
    """Queries rotated one position ahead of the keys.  (A shift of every position
    together is not a mistake: scores depend only on position differences.)"""
    out = _orig["rotate_factors"](f, start_pos, dims)
    ahead = _orig["rotate_factors"](f, start_pos + 1, dims)
    for k in ("b_q", "q"):
        if k in f:
            out[k] = ahead[k]
    return out


def _rotate_keys_only(f, start_pos, dims):
    out = _orig["rotate_factors"](f, start_pos, dims)
    for k in ("b_q", "q"):
        if k in f:
            out[k] = f[k]
    return out


def _prefill_v_from_k(fq, cache, dims, batch, seq, start_pos, causal=True, rows=None):
    c = dict(cache)
    if dims.rank_k == dims.rank_v:
        c["a_v"], c["b_v"] = cache["a_k"], cache["b_k"]
    else:
        c["b_v"] = cache["b_v"][..., ::-1, :].copy()
    return _orig["prefill"](fq, c, dims, batch, seq, start_pos, causal, rows)


def _gather_next_row(pools, block_table, b, n):
    """Rows shifted by one within each page."""
    P = pools["a_k"].shape[1]
    t = np.arange(n, dtype=np.int64)
    pages = np.asarray(block_table, dtype=np.int64)[b, t // P]
    return {k: np.asarray(pools[k], dtype=np.float64)[pages, (t + 1) % P] for k in ("a_k", "b_k", "a_v", "b_v")}


def _gather_first_table_row(pools, block_table, b, n):
    return _orig["paged_gather"](pools, block_table, 0, n)


def _decode_paged_max_len(fq, pools, block_table, ctx_lens, dims):
    """Every sequence attends over the longest sequence's key count."""
    m = max(int(v) for v in ctx_lens)
    return _orig["decode_paged"](fq, pools, block_table, [m if int(v) else 0 for v in ctx_lens], dims)


def _attend_backward_no_d(q, k, v, q_pos, causal, dout):
    """dS = P dP (the softmax Jacobian's -p (p . dp) term dropped)."""
    d_h = q.shape[-1]
    rs = 1.0 / math.sqrt(d_h)
    dq, dk, dv = (np.zeros(x.shape) for x in (q, k, v))
    for i in range(q.shape[0]):
        n = int(q_pos[i]) + 1 if causal else k.shape[0]
        sc = (k[:n] @ q[i]) * rs
        p = np.exp(sc - sc.max())
        p /= p.sum()
        dv[:n] += p[:, None] * dout[i][None, :]
        ds = p * (v[:n] @ dout[i])
        dq[i] = (ds @ k[:n]) * rs
        dk[:n] += ds[:, None] * q[i][None, :] * rs
    return dq, dk, dv


def _reconstruct_backward_no_scale(a, b, dx):
    da, db = _orig["reconstruct_backward"](a, b, dx)
    return da, db * a.shape[-1]


def _rope_backward_forward_turn(g, pos, base):
    return O.rope(g, pos, base)


def _shared_unrotated(a_k, a_v, b_k, b_v, base, n):
    k = O.reconstruct(np.asarray(a_k, np.float64)[:n], np.broadcast_to(np.asarray(b_k, np.float64), (n,) + b_k.shape))
    v = O.reconstruct(np.asarray(a_v, np.float64)[:n], np.broadcast_to(np.asarray(b_v, np.float64), (n,) + b_v.shape))
    return k, v


def _shared_rotated_at_last(a_k, a_v, b_k, b_v, base, n):
    k, v = _shared_unrotated(a_k, a_v, b_k, b_v, base, n)
    return O.rope(k[None], np.full(n, n - 1), base)[0], v


MUTATIONS = {
    "rope rotates the wrong way": ("rope", _rope_sign),
    "rope pairs (i, i+d/2)": ("rope", _rope_half_split),
    "rope theta base^(-i/d)": ("rope_angles", _angles_theta),
    "1/R dropped": ("reconstruct", _reconstruct_no_scale),
    "head factor viewed [R, h]": ("project", _project_a_transposed),
    "dim factor viewed [d_h, R]": ("project", _project_b_transposed),
    "causal mask admits the next key": ("attend_head", _attend_sees_next),
    "score scale 1/d_h": ("attend_head", _attend_scale_d),
    "cache append ignores start_pos": ("cache_append", _append_at_zero),
    "query positions off by one": ("rotate_factors", _rotate_queries_shifted),
    "queries left unrotated": ("rotate_factors", _rotate_keys_only),
    "values built from the wrong factors": ("prefill", _prefill_v_from_k),
    "paged rows shifted within a page": ("paged_gather", _gather_next_row),
    "every sequence read through the first table row": ("paged_gather", _gather_first_table_row),
    "ragged lengths ignored": ("decode_paged", _decode_paged_max_len),
    "backward drops the softmax row term": ("attend_head_backward", _attend_backward_no_d),
    "dim-factor gradient without 1/R": ("reconstruct_backward", _reconstruct_backward_no_scale),
    "rope gradient turned the forward way": ("rope_backward", _rope_backward_forward_turn),
    "shared keys left unrotated": ("shared_keys_values", _shared_unrotated),
    "shared keys rotated at the query's position": ("shared_keys_values", _shared_rotated_at_last),
}


@pytest.mark.parametrize("name", list(MUTATIONS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(O, attr, fn)
    caught = []
    for pin in P.ALL_PINS:
        try:
            pin()
        except Exception as e:     # an AssertionError, or the mistake breaking a shape
            caught.append((pin.__name__, type(e).__name__))
    assert caught, f"no pin catches the planted mistake: {name}"
