"""GPU parity of the backward: gradients of the prefill attention with respect to
the query factors and the cached key/value factors, and the gradient through
the rotary embedding, against the fp64 oracle's written-out gradients (which
are pinned to finite differences of the forward).

Bounds.  fp32 mode: max |err| <= 1e-4 as for the forward.  bf16 mode: the
gradients are float32 sums whose scale is set by the upstream gradient dO (they
are linear in it) and grows with the number of keys and queries summed, so the
bf16 bounds apply to them normalised by their largest magnitude:
max |err| <= 2e-2 * max(1, max |ref|) and relative L2 <= 5e-3 (assert_grad).
"""
import numpy as np
import pytest
import torch

import oracle.tpa_oracle as O
import tpa_inputs as I
from factorized_kv_cache_amd import tpa as T
from gpu_util import (BF16_MAX_ABS, announce, assert_close, fill_cache, oracle_cache, oracle_dims, oracle_query,
                      query_factors_gpu, require_gpu, shape_of)

pytestmark = pytest.mark.gpu

KV = ("a_k", "b_k", "a_v", "b_v")


def assert_grad(got, ref, dtype, what):
    if dtype == "f32":
        return assert_close(got, ref, dtype, what)
    scale = max(1.0, float(np.max(np.abs(np.asarray(ref, dtype=np.float64))))) if np.size(ref) else 1.0
    assert_close(got, ref, dtype, what, max_abs=BF16_MAX_ABS * scale)


def D(d_model, h, dh, rq, rk, rv, dtype, base=10000.0):
    return T.Dims(d_model, h, dh, rq, rk, rv, base, dtype)


def f32_cache(dims, B, max_seq):
    h, d = dims.n_heads, dims.head_dim
    z = lambda *s: torch.zeros(*s, dtype=torch.float32, device="cuda")
    return T.Cache(z(B, max_seq, h, dims.rank_k), z(B, max_seq, dims.rank_k, d), z(B, max_seq, h, dims.rank_v),
                   z(B, max_seq, dims.rank_v, d))


BACKWARD_CASES = [
    # name, dtype, B, S, start_pos, causal, d_model, h, dh, rq, rk, rv, std
    ("f32_chunked", "f32", 1, 40, 7, True, 64, 3, 32, 2, 3, 1, 1.0),
    ("bf16_chunked", "bf16", 2, 70, 9, True, 256, 4, 64, 3, 2, 2, 1.0),
    ("bf16_kvonly_full", "bf16", 2, 50, 0, False, 384, 6, 64, 0, 4, 4, 1.0),
    ("bf16_dh128", "bf16", 1, 45, 5, True, 512, 2, 128, 2, 2, 2, 1.0),
    ("f32_dh256", "f32", 1, 20, 0, True, 64, 2, 256, 2, 2, 2, 0.7),
    # several key blocks, query tiles and query blocks of the matrix-core
    # kernels, each with a ragged tail
    ("bf16_mfma_chunked_ragged", "bf16", 2, 300, 37, True, 256, 4, 64, 3, 2, 2, 1.0),
    ("bf16_mfma_kvonly_full_rv3", "bf16", 1, 200, 0, False, 384, 6, 64, 0, 4, 3, 1.0),
    ("bf16_mfma_dh128_r1", "bf16", 1, 150, 70, True, 512, 2, 128, 2, 1, 2, 1.0),
    ("bf16_mfma_mqa_r1", "bf16", 2, 129, 0, True, 256, 8, 64, 2, 1, 1, 1.2),
    # a query block that ends exactly on a tile edge
    ("bf16_mfma_aligned", "bf16", 1, 256, 128, True, 128, 2, 64, 2, 2, 2, 1.0),
    # the dims limits: d_h 256 with every rank at 64; 256 heads (n_heads * d_h
    # = 8192); the smallest dims
    ("limit_f32_dh256_r64", "f32", 1, 12, 3, True, 128, 32, 256, 64, 64, 64, 3.0),
    ("limit_bf16_h256", "bf16", 1, 20, 2, True, 512, 256, 32, 2, 2, 2, 1.5),
    ("limit_f32_min_dims", "f32", 2, 9, 1, True, 4, 1, 2, 1, 1, 1, 1.5),
]


def grad_buffers(dims, B, S, n_keys):
    h, dh = dims.n_heads, dims.head_dim
    z = lambda *s: torch.zeros(*s, dtype=torch.float32, device="cuda")
    dq = T.Factors(None if dims.kv_only else z(B, S, h, dims.rank_q),
                   z(B, S, h, dh) if dims.kv_only else z(B, S, dims.rank_q, dh), None, None, None, None)
    return dq, f32_cache(dims, B, n_keys + 3)


@pytest.mark.parametrize("case", BACKWARD_CASES, ids=[c[0] for c in BACKWARD_CASES])
def test_prefill_backward(case):
    require_gpu()
    name, dtype, B, S, sp, causal, dm, h, dh, rq, rk, rv, std = case
    dims = D(dm, h, dh, rq, rk, rv, dtype)
    n_keys = sp + S
    announce(f"prefill backward {name} B={B} S={S} sp={sp} causal={causal}")
    sh = shape_of(dims)
    kv = I.factors(sh, B, n_keys, seed=111, dtype=dtype, std=std, with_query=False)
    fq = I.factors(sh, B, S, seed=112, dtype=dtype, std=std)
    g = torch.Generator().manual_seed(113)
    dout = torch.randn(B, S, h * dh, generator=g).to(dims.torch_dtype)
    cache = T.new_cache(dims, B, n_keys + 3)
    fill_cache(cache, kv)
    q = query_factors_gpu(T, dims, fq)
    dq, dkv = grad_buffers(dims, B, S, n_keys)
    ws = torch.empty(T.tpa_prefill_backward_workspace_bytes(dims, B, S, sp), dtype=torch.uint8, device="cuda")
    T.tpa_prefill_attn_backward(dims, q, cache, sp, causal, dout.cuda(), dq, dkv, ws)
    first = [t.clone() for t in (dq.a_q, dq.b_q) if t is not None] + [getattr(dkv, k).clone() for k in KV]
    T.tpa_prefill_attn_backward(dims, q, cache, sp, causal, dout.cuda(), dq, dkv, ws)
    torch.cuda.synchronize()
    second = [t for t in (dq.a_q, dq.b_q) if t is not None] + [getattr(dkv, k) for k in KV]
    assert all(torch.equal(x, y) for x, y in zip(first, second)), "repeated backward calls are not bit-identical"

    od = oracle_dims(dims)
    dfq, ddkv = O.prefill_backward(oracle_query(fq, dims), oracle_cache(kv, od, B, n_keys), od, B, S, sp, causal,
                                   I.to_f64(dout))
    if dims.kv_only:
        assert_grad(dq.b_q, dfq["q"], dtype, f"{name} dQ")
    else:
        assert_grad(dq.a_q, dfq["a_q"], dtype, f"{name} dA_q")
        assert_grad(dq.b_q, dfq["b_q"], dtype, f"{name} dB_q")
    for k in KV:
        assert_grad(getattr(dkv, k)[:, :n_keys], ddkv[k], dtype, f"{name} d{k}")
        assert torch.all(getattr(dkv, k)[:, n_keys:] == 0), f"{k}: positions past the keys were written"


def factor_pairing(a, b, da, db):
    """Per token: sum_{h,r} A dA and sum_{r,d} B dB.  Both equal (1/R) sum_h X_h . dX_h
    for X = (1/R) sum_r a_r (x) b_r, so they agree whatever dX is."""
    lhs = (a.double() * da.double()).sum(dim=(-2, -1))
    rhs = (b.double() * db.double()).sum(dim=(-2, -1))
    return lhs, rhs


def test_prefill_backward_full_size_sampled_heads():
    """The backward at the prefill workload (4 x 4096, d_model 1024, h 16, d_h 64,
    R_Q 6, R 2) in the launch configuration the benchmark times.  The oracle
    forms two heads of sequence 0 in full (their head-factor gradients for every
    token); for every token of every sequence the dim-factor gradients must pair
    with the head-factor gradients: sum A dA = sum B dB."""
    require_gpu()
    wl = I.WORKLOADS["prefill_b4_s4k"]
    sh = wl.shape
    dims = D(sh.d_model, sh.n_heads, sh.head_dim, sh.rank_q, sh.rank_k, sh.rank_v, "bf16", sh.rope_base)
    B, S = wl.batch, wl.seq
    h, dh = dims.n_heads, dims.head_dim
    announce(f"prefill backward full size B={B} S={S}")
    kv = I.factors(sh, B, S, seed=131, dtype="bf16", with_query=False)
    fq = I.factors(sh, B, S, seed=132, dtype="bf16")
    dout = torch.randn(B, S, h * dh, generator=torch.Generator().manual_seed(133)).to(torch.bfloat16)
    cache = T.new_cache(dims, B, S)
    fill_cache(cache, kv)
    q = query_factors_gpu(T, dims, fq)
    dq, dkv = grad_buffers(dims, B, S, S)
    ws = torch.empty(T.tpa_prefill_backward_workspace_bytes(dims, B, S, 0), dtype=torch.uint8, device="cuda")
    T.tpa_prefill_attn_backward(dims, q, cache, 0, True, dout.cuda(), dq, dkv, ws)
    torch.cuda.synchronize()

    heads = [0, 11]
    od = oracle_dims(dims)
    one = lambda d: {k: v[:1] for k, v in d.items()}
    dfq, ddkv = O.prefill_backward(oracle_query(one(fq), dims), oracle_cache(one(kv), od, 1, S), od, 1, S, 0, True,
                                   I.to_f64(dout[:1]), heads=heads)
    for hh in heads:
        assert_grad(dq.a_q[0, :, hh], dfq["a_q"][0, :, hh], "bf16", f"full size dA_q head {hh}")
        assert_grad(dkv.a_k[0, :S, hh], ddkv["a_k"][0, :, hh], "bf16", f"full size dA_k head {hh}")
        assert_grad(dkv.a_v[0, :S, hh], ddkv["a_v"][0, :, hh], "bf16", f"full size dA_v head {hh}")
    fqc = {k: v.cuda() for k, v in fq.items()}
    kvc = {k: v.cuda() for k, v in kv.items()}
    for name, a, b, da, db in (("q", fqc["a_q"], fqc["b_q"], dq.a_q, dq.b_q),
                               ("k", kvc["a_k"], kvc["b_k"], dkv.a_k[:, :S], dkv.b_k[:, :S]),
                               ("v", kvc["a_v"], kvc["b_v"], dkv.a_v[:, :S], dkv.b_v[:, :S])):
        lhs, rhs = factor_pairing(a, b, da, db)
        scale = float(torch.max(torch.abs(lhs)))
        err = float(torch.max(torch.abs(lhs - rhs)))
        print(f"  pairing {name}: max |sum A dA - sum B dB| = {err:.3e} (scale {scale:.3e})", flush=True)
        assert err <= 1e-4 * max(scale, 1e-6), f"{name}: dim-factor gradients do not pair with head-factor ones"


@pytest.mark.parametrize("dh,rows,sp", [(8, 3, 0), (64, 6, 4093), (128, 2, 131060)])
def test_rope_b_backward(dh, rows, sp):
    require_gpu()
    dims = D(64, 4, dh, 2, 2, 2, "f32")
    announce(f"rope backward dh={dh} rows={rows} sp={sp}")
    g = torch.Generator().manual_seed(121)
    grad = torch.randn(2, 5, rows, dh, generator=g)
    got = T.tpa_rope_b_backward(dims, grad.clone().cuda(), start_pos=sp)
    torch.cuda.synchronize()
    ref = O.rope_backward(grad.double().numpy(), O.positions(sp, 5), dims.rope_base)
    assert_close(got, ref, "f32", f"rope backward dh={dh}")
