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


def shared_setup(dims, B, ctx, seed, std=None, extra=3, vstd=None):
    sh = shape_of(dims)
    vs = value_std(std) if vstd is None else vstd
    f = I.factors(sh, B, ctx, seed=seed, dtype=dims.dtype, std=std, with_query=False, v_std=vs)
    basis = I.shared_basis(sh, seed=seed + 1, dtype=dims.dtype, std=std, v_std=vs)
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


# --------------------------------------------------------------------------
# Shared-basis prefill and the head-factor-only projection
# --------------------------------------------------------------------------

SHARED_PREFILL_CASES = [
    # name, dtype, B, S, start_pos, causal, d_model, h, dh, rq, rk, rv, std, value std (None: the capped std)
    ("bf16_h16_r2", "bf16", 2, 300, 0, True, 1024, 16, 64, 6, 2, 2, None, None),   # 32x32 matrix-core path
    ("bf16_kvonly_r4", "bf16", 2, 257, 0, True, 1536, 24, 64, 0, 4, 4, None, None),
    # rank 1 with one shared B_V: every output of a head is one scalar times
    # B_V, so the outputs (and the bf16 rounding of the operands) grow with the
    # value spread; 0.5 keeps them inside the bf16 bound while the scores stay sharp
    ("bf16_r1", "bf16", 2, 200, 0, True, 256, 8, 64, 2, 1, 1, 1.0, 0.5),
    ("bf16_chunk", "bf16", 2, 100, 333, True, 1024, 16, 64, 6, 2, 2, None, None),  # queries after a cached prefix
    ("bf16_noncausal", "bf16", 2, 70, 50, False, 1024, 16, 64, 6, 2, 2, None, None),
    ("bf16_one_token", "bf16", 3, 1, 40, True, 256, 8, 64, 2, 2, 2, None, None),
    ("bf16_mixed_ranks", "bf16", 2, 90, 11, True, 512, 8, 64, 3, 2, 1, 1.0, None),  # generic kernel (R_K != R_V)
    ("bf16_dh128", "bf16", 2, 150, 20, True, 1024, 8, 128, 6, 2, 2, None, None),    # generic kernel (d_h 128)
    ("f32_h5_rk3_rv1", "f32", 3, 45, 7, True, 64, 5, 32, 3, 3, 1, 1.0, None),
    ("f32_r1_sharp", "f32", 2, 120, 9, True, 256, 8, 64, 2, 1, 1, 1.5, None),
    ("f32_noncausal", "f32", 2, 33, 0, False, 256, 4, 64, 2, 2, 2, 1.0, None),
]


def shared_prefill(dims, q, cache, sp, causal, path):
    """tpa_shared_prefill_attn, or (path "ws") tpa_shared_prefill_attn_ws with a
    workspace of the size the library asks for (none where it asks for none)."""
    if path == "fused":
        return T.tpa_shared_prefill_attn(dims, q, cache, sp, causal)
    B, S = q.b_q.shape[0], q.b_q.shape[1]
    n = T.tpa_prefill_workspace_bytes(dims, B, S, sp)
    ws = torch.empty(n, dtype=torch.uint8, device="cuda") if n else None
    return T.tpa_shared_prefill_attn_ws(dims, q, cache, sp, ws, causal)


@pytest.mark.parametrize("path", ["fused", "ws"])
@pytest.mark.parametrize("case", SHARED_PREFILL_CASES, ids=[c[0] for c in SHARED_PREFILL_CASES])
def test_shared_prefill(case, path):
    require_gpu()
    name, dtype, B, S, sp, causal, dm, h, dh, rq, rk, rv, std, vstd = case
    dims = D(dm, h, dh, rq, rk, rv, dtype)
    Tn = sp + S
    announce(f"shared prefill {name} B={B} S={S} sp={sp} causal={causal} path={path}")
    f, basis, _, cache = shared_setup(dims, B, Tn, seed=171, std=std, vstd=vstd)
    fq = I.factors(shape_of(dims), B, S, seed=172, dtype=dtype, std=std)
    out = shared_prefill(dims, query_factors_gpu(T, dims, fq), cache, sp, causal, path)
    out2 = shared_prefill(dims, query_factors_gpu(T, dims, fq), cache, sp, causal, path)
    torch.cuda.synchronize()
    assert torch.equal(out, out2), "repeated shared prefill calls are not bit-identical"
    cache_a = {"a_k": I.to_f64(f["a_k"]), "a_v": I.to_f64(f["a_v"])}
    ref = O.prefill_shared(oracle_query(fq, dims), cache_a, {k: I.to_f64(v) for k, v in basis.items()},
                           oracle_dims(dims), B, S, sp, causal)
    assert_close(out, ref, dtype, f"shared prefill {name} ({path})")


@pytest.mark.parametrize("case", [(2, 300, 0, True, 1024, 16, 6, 2, 2), (3, 130, 41, True, 256, 8, 2, 1, 1),
                                  (2, 90, 30, False, 1024, 16, 6, 2, 2)])
def test_shared_prefill_ws_matches_fused_bitwise(case):
    """At ranks 1 and 2 the workspace path forms the same rotated bf16 keys and
    values as the shared rebuild in LDS and attends in the same order: equal
    outputs bit for bit, also after a stale workspace."""
    require_gpu()
    B, S, sp, causal, dm, h, rq, rk, rv = case
    dims = D(dm, h, 64, rq, rk, rv, "bf16")
    announce(f"shared prefill ws vs fused bitwise case={case}")
    f, basis, _, cache = shared_setup(dims, B, sp + S, seed=173, std=1.0, vstd=0.5)
    fq = I.factors(shape_of(dims), B, S, seed=174, dtype="bf16", std=1.0)
    q = query_factors_gpu(T, dims, fq)
    n = T.tpa_prefill_workspace_bytes(dims, B, S, sp)
    assert n == 2 * B * h * (sp + S) * 64 * 2
    ws = torch.full((n,), 0x7f, dtype=torch.uint8, device="cuda")
    fused = T.tpa_shared_prefill_attn(dims, q, cache, sp, causal)
    staged = T.tpa_shared_prefill_attn_ws(dims, q, cache, sp, ws, causal)
    torch.cuda.synchronize()
    assert torch.equal(fused, staged)


@pytest.mark.parametrize("path", ["fused", "ws"])
def test_shared_prefill_full_size_sampled_rows(path):
    """The prefill workload's shapes (4 sequences of 4096 tokens, d_model 1024,
    h 16, d_h 64, R_Q 6, R 2) with a shared basis, in one call; the oracle
    attends 40 sampled query rows per sequence."""
    require_gpu()
    wl = I.WORKLOADS["prefill_b4_s4k"]
    s = wl.shape
    dims = D(s.d_model, s.n_heads, s.head_dim, s.rank_q, s.rank_k, s.rank_v, "bf16", s.rope_base)
    B, S = wl.batch, wl.seq
    announce(f"shared prefill full size B={B} S={S} path={path}")
    f, basis, _, cache = shared_setup(dims, B, S, seed=181, extra=0)
    fq = I.factors(shape_of(dims), B, S, seed=182, dtype="bf16")
    out = shared_prefill(dims, query_factors_gpu(T, dims, fq), cache, 0, True, path)
    torch.cuda.synchronize()
    rng = np.random.default_rng(183)
    rows = np.unique(np.concatenate([[0, 1, 63, 64, S - 1], rng.integers(0, S, 35)]))
    cache_a = {"a_k": I.to_f64(f["a_k"]), "a_v": I.to_f64(f["a_v"])}
    ref = O.prefill_shared(oracle_query(fq, dims), cache_a, {k: I.to_f64(v) for k, v in basis.items()},
                           oracle_dims(dims), B, S, 0, True, rows=rows)
    assert_close(out[:, rows], ref[:, rows], "bf16", "shared prefill full size, sampled rows")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_shared_prefill_equals_standard(dtype):
    """A standard cache holding RoPE_t(B_K) and B_V at every token t prefills to
    the same outputs as the shared-basis cache, up to the kernels' rounding."""
    require_gpu()
    dims = D(1024, 16, 64, 6, 2, 2, dtype)
    B, S, sp = 2, 200, 77
    Tn = sp + S
    announce(f"shared vs standard prefill {dtype}")
    f, basis, _, cache = shared_setup(dims, B, Tn, seed=191, extra=0)
    std_cache = T.new_cache(dims, B, Tn)
    std_cache.a_k.copy_(cache.a_k)
    std_cache.a_v.copy_(cache.a_v)
    std_cache.b_k.copy_(cache.b_k.expand(B, Tn, *cache.b_k.shape))
    std_cache.b_v.copy_(cache.b_v.expand(B, Tn, *cache.b_v.shape))
    T.tpa_rope_b(dims, std_cache.b_k, start_pos=0)
    fq = I.factors(shape_of(dims), B, S, seed=192, dtype=dtype)
    q = query_factors_gpu(T, dims, fq)
    shared = T.tpa_shared_prefill_attn(dims, q, cache, sp, True).float().cpu()
    standard = T.tpa_prefill_attn(dims, q, std_cache, sp, True).float().cpu()
    assert_close(shared, standard.double().numpy(), dtype, "shared vs standard prefill")


SHARED_PROJ_CASES = [
    # B, S, d_model, h, dh, rq, rk, rv, start_pos
    (2, 37, 200, 3, 16, 5, 3, 2, 0),
    (3, 70, 1024, 16, 64, 6, 2, 2, 11),
    (2, 33, 192, 24, 64, 0, 4, 4, 100),
    (4, 4096, 1024, 16, 64, 6, 2, 2, 0),         # the prefill workload's projection
    (16, 1, 1024, 16, 64, 6, 2, 2, 4096),        # a decode batch
    (1, 1, 4096, 32, 128, 6, 2, 2, 131072),
]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("case", SHARED_PROJ_CASES)
@pytest.mark.parametrize("fuse", [True, False])
def test_shared_factor_proj(dtype, case, fuse):
    """Query factors and the key/value head factors of a shared-basis layer
    against the oracle's projection (the bases are not projected)."""
    require_gpu()
    B, S, dm, h, dh, rq, rk, rv, sp = case
    dims = D(dm, h, dh, rq, rk, rv, dtype)
    announce(f"shared factor_proj {dtype} fuse={fuse} case={case}")
    x = I.activations(B, S, dm, seed=201, dtype=dtype)
    w = I.weights(shape_of(dims), seed=201, dtype=dtype)
    wp = T.pack_shared_weights({k: v.cuda() for k, v in w.items()}, dims.kv_only)
    assert wp.shape[0] == T.tpa_shared_packed_weight_rows(dims)
    out = T.new_factors(dims, B, S)
    out = T.Factors(out.a_q, out.b_q, out.a_k, None, out.a_v, None)
    T.tpa_shared_factor_proj(dims, x.cuda(), wp, out, start_pos=sp, fuse_rope=fuse)
    torch.cuda.synchronize()
    od = oracle_dims(dims)
    ref = O.project(I.to_f64(x), {k: I.to_f64(v) for k, v in w.items()}, od)
    if fuse:
        ref = O.rotate_factors(ref, sp, od)
    names = ["a_k", "a_v"] + ([] if dims.kv_only else ["a_q", "b_q"])
    for k in names:
        assert_close(getattr(out, k), ref[k], dtype, f"shared proj {k}")
    if dims.kv_only:
        assert_close(out.b_q, ref["q"], dtype, "shared proj q")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_shared_layer_path(dtype):
    """Project a block straight into the shared cache's head-factor slots, then
    prefill over the cache: the fused path against the oracle's projection
    followed by its shared-basis prefill."""
    require_gpu()
    dims = D(512, 8, 64, 4, 2, 2, dtype)
    B, S, sp, max_s = 2, 96, 40, 160
    announce(f"shared layer path {dtype}")
    sh = shape_of(dims)
    prefix = I.factors(sh, B, sp, seed=211, dtype=dtype, with_query=False)
    basis = I.shared_basis(sh, seed=212, dtype=dtype)
    cache = T.new_shared_cache(dims, B, max_s, basis["b_k"], basis["b_v"])
    cache.a_k[:, :sp].copy_(prefix["a_k"].cuda())
    cache.a_v[:, :sp].copy_(prefix["a_v"].cuda())
    x = I.activations(B, S, dims.d_model, seed=213, dtype=dtype)
    w = I.weights(sh, seed=213, dtype=dtype)
    wp = T.pack_shared_weights({k: v.cuda() for k, v in w.items()}, False)
    q = T.new_factors(dims, B, S)
    f = T.Factors(q.a_q, q.b_q, cache.a_k[:, sp:], None, cache.a_v[:, sp:], None, 0, max_s)
    T.tpa_shared_factor_proj(dims, x.cuda(), wp, f, start_pos=sp)
    out = T.tpa_shared_prefill_attn(dims, T.Factors(q.a_q, q.b_q, None, None, None, None), cache, sp, True)
    torch.cuda.synchronize()
    od = oracle_dims(dims)
    p = O.rotate_factors(O.project(I.to_f64(x), {k: I.to_f64(v) for k, v in w.items()}, od), sp, od)
    # the oracle reads what the kernel wrote into the cache, so that the
    # projection's rounding of the head factors is not counted twice
    got_a = {k: I.to_f64(getattr(cache, k)[:, :sp + S].cpu()) for k in ("a_k", "a_v")}
    for k in ("a_k", "a_v"):
        assert_close(getattr(cache, k)[:, sp:sp + S], p[k], dtype, f"shared layer {k}")
        assert torch.equal(getattr(cache, k)[:, :sp].cpu(), prefix[k]), f"prefix of {k} overwritten"
    fq = {"a_q": q.a_q.cpu(), "b_q": q.b_q.cpu()}
    ref = O.prefill_shared(oracle_query(fq, dims), got_a, {k: I.to_f64(v) for k, v in basis.items()}, od, B, S, sp,
                           True)
    assert_close(out, ref, dtype, "shared layer prefill")
