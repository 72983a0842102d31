"""GPU parity of the shared-basis variant (dim factors of K and V common to
every token, only the head factors cached): the cache append bit for bit, and
the decode against the fp64 oracle's decode_shared on the same seeded inputs;
the decode also against the standard GPU decode over a cache that holds the
basis rotated at every token."""
import numpy as np
import pytest
import torch

import oracle.tpa_oracle as O
import tpa_inputs as I
from factorized_kv_cache_amd import tpa as T
from gpu_util import (announce, assert_close, oracle_dims, oracle_query, query_factors_gpu, require_gpu, shape_of,
                      value_std)

pytestmark = pytest.mark.gpu


def D(d_model, h, dh, rq, rk, rv, dtype, base=10000.0):
    return T.Dims(d_model, h, dh, rq, rk, rv, base, dtype)


def shared_setup(dims, B, ctx, seed, std=None, extra=3):
    sh = shape_of(dims)
    f = I.factors(sh, B, ctx, seed=seed, dtype=dims.dtype, std=std, with_query=False, v_std=value_std(std))
    basis = I.shared_basis(sh, seed=seed + 1, dtype=dims.dtype, std=std, v_std=value_std(std))
    fq = I.factors(sh, B, 1, seed=seed + 2, dtype=dims.dtype, std=std)
    cache = T.new_shared_cache(dims, B, ctx + extra, basis["b_k"], basis["b_v"])
    cache.a_k[:, :ctx].copy_(f["a_k"].cuda())
    cache.a_v[:, :ctx].copy_(f["a_v"].cuda())
    return f, basis, fq, cache


def oracle_shared(fq, f, basis, dims, B, ctx):
    cache_a = {"a_k": I.to_f64(f["a_k"]), "a_v": I.to_f64(f["a_v"])}
    return O.decode_shared(oracle_query(fq, dims), cache_a, {k: I.to_f64(v) for k, v in basis.items()},
                           oracle_dims(dims), B, ctx)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_shared_append_bitwise(dtype):
    require_gpu()
    dims = D(128, 6, 32, 2, 3, 2, dtype)
    B, S, sp, max_seq = 3, 7, 5, 16
    announce(f"shared append {dtype}")
    f = I.factors(shape_of(dims), B, S, seed=61, dtype=dtype, with_query=False)
    basis = I.shared_basis(shape_of(dims), seed=62, dtype=dtype)
    cache = T.new_shared_cache(dims, B + 1, max_seq, basis["b_k"], basis["b_v"])
    cache.a_k.fill_(5.0)
    cache.a_v.fill_(5.0)
    kv = T.Factors(None, None, f["a_k"].cuda(), None, f["a_v"].cuda(), None)
    T.tpa_shared_cache_append(dims, cache, kv, sp)
    torch.cuda.synchronize()
    for k in ("a_k", "a_v"):
        want = torch.full_like(getattr(cache, k).cpu(), 5.0)
        want[:B, sp:sp + S] = f[k]
        assert torch.equal(getattr(cache, k).cpu(), want), k


SHARED_CASES = [
    # name, dtype, B, ctx, d_model, h, dh, rq, rk, rv, std
    ("bf16_h16_r2", "bf16", 3, 1000, 1024, 16, 64, 6, 2, 2, None),
    ("bf16_h32_dh128", "bf16", 2, 777, 4096, 32, 128, 6, 2, 2, None),
    ("bf16_kvonly_h24_r4", "bf16", 2, 300, 1536, 24, 64, 0, 4, 4, None),
    ("f32_h5_rk3_rv1", "f32", 3, 45, 64, 5, 32, 3, 3, 1, 1.0),
    ("f32_h64_wide", "f32", 1, 70, 256, 64, 32, 2, 1, 4, 1.0),
    ("bf16_h40_r2", "bf16", 2, 200, 640, 40, 64, 2, 2, 1, None),
    ("bf16_one_key", "bf16", 2, 1, 256, 8, 64, 2, 2, 2, None),
    ("bf16_33_keys_sharp", "bf16", 2, 33, 256, 8, 64, 2, 2, 2, 1.5),
    ("f32_long_131072", "f32", 1, 131072, 256, 4, 64, 2, 2, 2, 1.0),
]


@pytest.mark.parametrize("case", SHARED_CASES, ids=[c[0] for c in SHARED_CASES])
def test_shared_decode(case):
    require_gpu()
    name, dtype, B, ctx, dm, h, dh, rq, rk, rv, std = case
    dims = D(dm, h, dh, rq, rk, rv, dtype)
    announce(f"shared decode {name} B={B} ctx={ctx}")
    f, basis, fq, cache = shared_setup(dims, B, ctx, seed=71, std=std)
    q = query_factors_gpu(T, dims, fq, squeeze=True)
    ws = torch.empty(T.tpa_shared_decode_workspace_bytes(dims, B, ctx), dtype=torch.uint8, device="cuda")
    out = T.tpa_shared_decode_attn(dims, q, cache, ctx, ws)
    out2 = T.tpa_shared_decode_attn(dims, q, cache, ctx, ws)
    torch.cuda.synchronize()
    assert torch.equal(out, out2), "repeated shared decode calls are not bit-identical"
    assert_close(out, oracle_shared(fq, f, basis, dims, B, ctx), dtype, f"shared decode {name}")


def test_shared_decode_full_size():
    """The decode workload's shapes (16 sequences, 4097 keys, d_model 1024, h 16,
    d_h 64, R_Q 6, R 2) with a shared basis; every output against the oracle."""
    require_gpu()
    wl = I.WORKLOADS["decode_b16_ctx4k"]
    s = wl.shape
    dims = D(s.d_model, s.n_heads, s.head_dim, s.rank_q, s.rank_k, s.rank_v, "bf16", s.rope_base)
    B, ctx = wl.batch, wl.seq + 1
    announce(f"shared decode full size B={B} ctx={ctx}")
    f, basis, fq, cache = shared_setup(dims, B, ctx, seed=81)
    q = query_factors_gpu(T, dims, fq, squeeze=True)
    ws = torch.empty(T.tpa_shared_decode_workspace_bytes(dims, B, ctx), dtype=torch.uint8, device="cuda")
    out = T.tpa_shared_decode_attn(dims, q, cache, ctx, ws)
    torch.cuda.synchronize()
    assert_close(out, oracle_shared(fq, f, basis, dims, B, ctx), "bf16", "shared decode full size")


def test_shared_decode_long_context_sampled_heads():
    """The long-context decode shape the benchmark times (8 sequences of
    131,072 cached keys + the new one, d_model 4096, h 32, d_h 128, R_Q 6, R 2)
    with a shared basis, in one call; the oracle checks two seeded heads per
    sequence (and the first and last), rebuilding each sampled head's keys and
    values in fp64 on its own."""
    require_gpu()
    wl = I.WORKLOADS["decode_b8_ctx128k"]
    s = wl.shape
    dims = D(s.d_model, s.n_heads, s.head_dim, s.rank_q, s.rank_k, s.rank_v, "bf16", s.rope_base)
    B, ctx = wl.batch, wl.seq + 1
    announce(f"shared decode long context B={B} ctx={ctx}")
    f, basis, fq, cache = shared_setup(dims, B, ctx, seed=91, extra=0)
    q = query_factors_gpu(T, dims, fq, squeeze=True)
    ws = torch.empty(T.tpa_shared_decode_workspace_bytes(dims, B, ctx), dtype=torch.uint8, device="cuda")
    out = T.tpa_shared_decode_attn(dims, q, cache, ctx, ws)
    torch.cuda.synchronize()
    del cache
    rng = np.random.default_rng(92)
    h, dh = s.n_heads, s.head_dim
    pairs = sorted({(0, 0), (B - 1, h - 1)} | {(b, int(x)) for b in range(B) for x in rng.choice(h, 2, replace=False)})
    od = oracle_dims(dims)
    Q = O.queries(oracle_query(fq, dims), od)                               # [B, 1, h, d_h]
    bk, bv = I.to_f64(basis["b_k"]), I.to_f64(basis["b_v"])
    got, want = [], []
    for b, hh in pairs:
        k, v = O.shared_keys_values(I.to_f64(f["a_k"][b, :, hh:hh + 1]), I.to_f64(f["a_v"][b, :, hh:hh + 1]),
                                    bk, bv, od.rope_base, ctx)              # [ctx, 1, d_h]
        want.append(O.attend_head(Q[b, :, hh], k[:, 0], v[:, 0], np.array([ctx - 1]), True)[0])
        got.append(out[b, hh * dh:(hh + 1) * dh])
    assert_close(torch.stack(got), np.stack(want), "bf16", f"shared decode long context, {len(pairs)} heads")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_shared_equals_standard_decode(dtype):
    """A standard cache holding, for every token t, RoPE_t(B_K) (rotated by the
    library's own tpa_rope_b) and B_V decodes to the same outputs as the
    shared-basis cache, up to the two kernels' rounding."""
    require_gpu()
    dims = D(1024, 16, 64, 6, 2, 2, dtype)
    B, ctx = 2, 600
    announce(f"shared vs standard decode {dtype}")
    f, basis, fq, cache = shared_setup(dims, B, ctx, seed=91, extra=0)
    std_cache = T.new_cache(dims, B, ctx)
    std_cache.a_k.copy_(cache.a_k)
    std_cache.a_v.copy_(cache.a_v)
    std_cache.b_k.copy_(cache.b_k.expand(B, ctx, *cache.b_k.shape))
    std_cache.b_v.copy_(cache.b_v.expand(B, ctx, *cache.b_v.shape))
    T.tpa_rope_b(dims, std_cache.b_k, start_pos=0)   # every token's copy of B_K turned to its position
    q = query_factors_gpu(T, dims, fq, squeeze=True)
    ws = torch.empty(max(T.tpa_shared_decode_workspace_bytes(dims, B, ctx),
                         T.tpa_decode_workspace_bytes(dims, B, ctx)), dtype=torch.uint8, device="cuda")
    shared = T.tpa_shared_decode_attn(dims, q, cache, ctx, ws).float().cpu()
    standard = T.tpa_decode_attn(dims, q, std_cache, ctx, ws).float().cpu()
    assert_close(shared, standard.double().numpy(), dtype, "shared vs standard decode")
