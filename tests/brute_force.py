"""Pure-Python scalar brute force of one TPA attention layer, for tiny inputs.

Written independently of the fp64 oracle: nested lists, scalar loops, and the
rotary embedding as multiplication by the unit complex number exp(i*pos*theta)
on the pair (x_2i + i x_2i+1).  It shares no code with the oracle or the HIP
path.  Every token sits at its absolute position 0..T-1 and every row is
returned; chunked use (start_pos > 0) is compared against the matching rows.

Definitions followed: the factorisation with its 1/R scale ([coreui] "公式描述"),
the views of the linear outputs as [h, R] and [R, d_h] and the score scale
1/sqrt(d_h) ([coreui] "前向传播"), softmax attention ([jieyibu] Ⅱ.1).
"""
import cmath
import math


def _matvec_rows(x_tok, w_rows):
    return [sum(xi * wi for xi, wi in zip(x_tok, row)) for row in w_rows]


def _rotate(vec, pos, base):
    d = len(vec)
    out = [0.0] * d
    for i in range(d // 2):
        theta = base ** (-(2.0 * i) / d)
        z = complex(vec[2 * i], vec[2 * i + 1]) * cmath.exp(1j * pos * theta)
        out[2 * i], out[2 * i + 1] = z.real, z.imag
    return out


def _head_tensor(a_flat, b_flat, h, R, d, rotate_pos=None, base=None):
    """a_flat: h*R values (head-major), b_flat: R*d values; returns [h][d]."""
    b_rows = [b_flat[r * d:(r + 1) * d] for r in range(R)]
    if rotate_pos is not None:
        b_rows = [_rotate(row, rotate_pos, base) for row in b_rows]
    out = []
    for hh in range(h):
        row = [0.0] * d
        for r in range(R):
            a = a_flat[hh * R + r]
            for j in range(d):
                row[j] += a * b_rows[r][j]
        out.append([v / R for v in row])
    return out


def layer(x, w, d_model, h, d, rq, rk, rv, base, causal=True):
    """x: [B][T][d_model] lists; w: dict of weight row lists (nn.Linear layout).

    Returns out[B][T][h*d] for queries at positions 0..T-1 over keys 0..T-1.
    """
    B = len(x)
    T = len(x[0])
    out = []
    for b in range(B):
        Q, K, V = [], [], []
        for t in range(T):
            xt = x[b][t]
            if rq == 0:
                qf = _matvec_rows(xt, w["w_q"])
                Q.append([_rotate(qf[hh * d:(hh + 1) * d], t, base) for hh in range(h)])
            else:
                Q.append(_head_tensor(_matvec_rows(xt, w["w_a_q"]), _matvec_rows(xt, w["w_b_q"]),
                                      h, rq, d, rotate_pos=t, base=base))
            K.append(_head_tensor(_matvec_rows(xt, w["w_a_k"]), _matvec_rows(xt, w["w_b_k"]),
                                  h, rk, d, rotate_pos=t, base=base))
            V.append(_head_tensor(_matvec_rows(xt, w["w_a_v"]), _matvec_rows(xt, w["w_b_v"]), h, rv, d))
        rows = []
        for s in range(T):
            row = []
            for hh in range(h):
                n = s + 1 if causal else T
                sc = [sum(Q[s][hh][j] * K[t][hh][j] for j in range(d)) / math.sqrt(d) for t in range(n)]
                mx = max(sc)
                e = [math.exp(v - mx) for v in sc]
                z = sum(e)
                for j in range(d):
                    row.append(sum(e[t] / z * V[t][hh][j] for t in range(n)))
            rows.append(row)
        out.append(rows)
    return out


def shared_decode(q, a_k, a_v, b_k, b_v, base):
    """Shared-basis decode of one sequence: q [h][d] (already rotated at its
    position), a_k [T][h][R_K], a_v [T][h][R_V] per token, b_k [R_K][d] and
    b_v [R_V][d] common to all tokens.  Key t is (1/R_K) sum_r a_k[t][h][r] b_k[r]
    turned by exp(i t theta) pairwise; value t is (1/R_V) sum_r a_v[t][h][r] b_v[r].
    Returns [h*d] for the query attending over all T keys."""
    T, h, d = len(a_k), len(q), len(q[0])
    rk, rv = len(b_k), len(b_v)
    out = []
    for hh in range(h):
        keys, vals = [], []
        for t in range(T):
            k = [sum(a_k[t][hh][r] * b_k[r][j] for r in range(rk)) / rk for j in range(d)]
            keys.append(_rotate(k, t, base))
            vals.append([sum(a_v[t][hh][r] * b_v[r][j] for r in range(rv)) / rv for j in range(d)])
        sc = [sum(q[hh][j] * keys[t][j] for j in range(d)) / math.sqrt(d) for t in range(T)]
        mx = max(sc)
        e = [math.exp(v - mx) for v in sc]
        z = sum(e)
        for j in range(d):
            out.append(sum(e[t] / z * vals[t][j] for t in range(T)))
    return out
