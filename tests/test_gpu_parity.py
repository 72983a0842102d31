"""GPU parity: every entry point of libtpa against the fp64 oracle, element by
element, on the same seeded inputs (small and ragged shapes that span several
tiles, plus the decode workload at its full size)."""
import numpy as np
import pytest
import torch

import oracle.tpa_oracle as O
import tpa_inputs as I
from factorized_kv_cache_amd import tpa as T
from gpu_util import (announce, assert_close, fill_cache, oracle_cache, oracle_dims, oracle_factors,
                      oracle_query, query_factors_gpu, require_gpu, shape_of, value_std)

pytestmark = pytest.mark.gpu


def D(d_model, h, dh, rq, rk, rv, dtype, base=10000.0):
    return T.Dims(d_model, h, dh, rq, rk, rv, base, dtype)


# --------------------------------------------------------------------------
# Cache append: a bit copy
# --------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("B,S,sp,max_b,max_s,dims_args", [
    (2, 5, 3, 3, 11, (64, 3, 6, 2, 3, 1)),        # odd row widths (2-byte copies)
    (4, 17, 0, 4, 17, (128, 16, 64, 6, 2, 2)),
    (3, 1, 40, 5, 41, (64, 24, 64, 0, 4, 4)),
])
def test_cache_append_bitwise(dtype, B, S, sp, max_b, max_s, dims_args):
    require_gpu()
    dims = D(*dims_args, dtype)
    announce(f"cache_append {dtype} B={B} S={S} sp={sp} dims={dims_args}")
    f = I.factors(shape_of(dims), B, S, seed=31, dtype=dtype, with_query=False)
    cache = T.new_cache(dims, max_b, max_s)
    for k in ("a_k", "b_k", "a_v", "b_v"):
        getattr(cache, k).fill_(7.0)
    kv = T.Factors(None, None, *(f[k].cuda() for k in ("a_k", "b_k", "a_v", "b_v")))
    T.tpa_cache_append(dims, cache, kv, sp)
    torch.cuda.synchronize()
    for k in ("a_k", "b_k", "a_v", "b_v"):
        c = getattr(cache, k).cpu()
        assert torch.equal(c[:B, sp:sp + S], f[k]), k
        mask = torch.ones(c.shape[:2], dtype=torch.bool)
        mask[:B, sp:sp + S] = False
        assert torch.all(c[mask] == 7.0), f"{k}: slots outside the block changed"


# --------------------------------------------------------------------------
# Standalone rotary embedding
# --------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("B,S,rows,dh,sp,base", [
    (2, 7, 3, 8, 0, 10000.0),
    (3, 33, 6, 64, 5, 10000.0),
    (1, 4, 2, 128, 131069, 10000.0),     # positions near 128K
    (2, 5, 24, 64, 16380, 500000.0),
    (2, 9, 3, 6, 7, 10000.0),            # d_h 6: no whole 16-byte pieces, the element kernel
])
def test_rope_b(dtype, B, S, rows, dh, sp, base):
    require_gpu()
    dims = D(16, 2, dh, 1, 1, 1, dtype, base)
    announce(f"rope_b {dtype} B={B} S={S} rows={rows} dh={dh} sp={sp}")
    b = I.normal((B, S, rows, dh), 1.0, seed=41, stream="f_b_k", dtype=dtype)
    ref = O.rope(I.to_f64(b), O.positions(sp, S), base)
    g = b.cuda()
    T.tpa_rope_b(dims, g, sp)
    torch.cuda.synchronize()
    assert_close(g, ref, dtype, "rope_b", max_abs=(2e-6 if dtype == "f32" else None))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_rope_b_piece_and_element_kernels_agree(dtype):
    """The same rotation through the 16-byte-piece kernel (aligned b) and the
    element kernel (b two bytes past a 16-byte boundary): bit for bit, and both
    within the oracle bound."""
    require_gpu()
    B, S, rows, dh, sp, base = 3, 41, 5, 64, 1000, 10000.0
    dims = D(16, 2, dh, 1, 1, 1, dtype, base)
    announce(f"rope_b piece vs element {dtype}")
    b = I.normal((B, S, rows, dh), 1.0, seed=43, stream="f_b_k", dtype=dtype)
    ref = O.rope(I.to_f64(b), O.positions(sp, S), base)
    g_piece = b.cuda()
    g_elem = _misaligned(b.cuda())
    T.tpa_rope_b(dims, g_piece, sp)
    T.tpa_rope_b(dims, g_elem, sp)
    torch.cuda.synchronize()
    assert torch.equal(g_piece.cpu(), g_elem.cpu())
    assert_close(g_piece, ref, dtype, "rope_b piece", max_abs=(2e-6 if dtype == "f32" else None))


# --------------------------------------------------------------------------
# Factor projection (+ fused rotary embedding)
# --------------------------------------------------------------------------

PROJ_CASES = [
    # B, S, d_model, h, dh, rq, rk, rv, start_pos
    (2, 37, 200, 3, 16, 5, 3, 2, 0),
    (3, 70, 1024, 16, 64, 6, 2, 2, 11),
    (2, 33, 192, 24, 64, 0, 4, 4, 100),
    (1, 1, 4096, 32, 128, 6, 2, 2, 131072),
    (16, 1, 1024, 16, 64, 6, 2, 2, 4096),       # decode batch: few-token kernel
    (40, 1, 1536, 24, 64, 0, 4, 4, 16384),
    (3, 150, 1536, 24, 64, 0, 4, 4, 0),          # KV-only, many tokens
    (2, 4500, 1536, 24, 64, 0, 4, 4, 7),         # 256 x 128 matrix-core tiles, ragged in M and N
    (4, 4096, 1024, 16, 64, 6, 2, 2, 0),         # the prefill workload's projection (128 x 128 tiles)
    # the dims limits: every rank and head_dim at their maximum; the most heads
    # (n_heads * head_dim = 8192); the smallest dims
    (1, 5, 64, 32, 256, 64, 64, 64, 7),
    (2, 9, 512, 256, 32, 2, 2, 2, 3),
    (3, 4, 4, 1, 2, 1, 1, 1, 0),
]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("case", PROJ_CASES)
@pytest.mark.parametrize("fuse", [True, False])
def test_factor_proj(dtype, case, fuse):
    require_gpu()
    B, S, dm, h, dh, rq, rk, rv, sp = case
    dims = D(dm, h, dh, rq, rk, rv, dtype)
    announce(f"factor_proj {dtype} fuse={fuse} case={case}")
    x = I.activations(B, S, dm, seed=51, dtype=dtype)
    w = I.weights(shape_of(dims), seed=51, dtype=dtype)
    wp = T.pack_weights({k: v.cuda() for k, v in w.items()}, dims.kv_only)
    assert wp.shape[0] == T.tpa_packed_weight_rows(dims)
    out = T.new_factors(dims, B, S)
    T.tpa_factor_proj(dims, x.cuda(), wp, out, start_pos=sp, fuse_rope=fuse)
    torch.cuda.synchronize()
    od = oracle_dims(dims)
    ref = O.project(I.to_f64(x), {k: I.to_f64(v) for k, v in w.items()}, od)
    if fuse:
        ref = O.rotate_factors(ref, sp, od)
    names = (["b_q"] if not dims.kv_only else []) + ["a_k", "b_k", "a_v", "b_v"] + ([] if dims.kv_only else ["a_q"])
    for k in names:
        assert_close(getattr(out, k), ref[k], dtype, f"proj {k}")
    if dims.kv_only:
        assert_close(out.b_q, ref["q"], dtype, "proj q")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_factor_proj_into_cache(dtype):
    """Key/value factors written straight into cache slots (kv_batch_stride = max_seq)."""
    require_gpu()
    B, S, sp, max_s = 3, 9, 20, 40
    dims = D(96, 4, 32, 3, 2, 3, dtype)
    announce(f"factor_proj into cache {dtype}")
    x = I.activations(B, S, 96, seed=52, dtype=dtype)
    w = I.weights(shape_of(dims), seed=52, dtype=dtype)
    wp = T.pack_weights({k: v.cuda() for k, v in w.items()}, False)
    cache = T.new_cache(dims, B, max_s)
    dense = T.new_factors(dims, B, S)
    slot = cache.slot_factors(sp)
    fused = T.Factors(dense.a_q, dense.b_q, slot.a_k, slot.b_k, slot.a_v, slot.b_v, 0, max_s)
    T.tpa_factor_proj(dims, x.cuda(), wp, fused, start_pos=sp)
    T.tpa_factor_proj(dims, x.cuda(), wp, dense, start_pos=sp)
    torch.cuda.synchronize()
    for k in ("a_k", "b_k", "a_v", "b_v"):
        assert torch.equal(getattr(cache, k)[:, sp:sp + S], getattr(dense, k)), k
        assert torch.count_nonzero(getattr(cache, k)[:, :sp]) == 0


# --------------------------------------------------------------------------
# Decode attention
# --------------------------------------------------------------------------

DECODE_CASES = [
    # name, dtype, B, ctx, d_model, h, dh, rq, rk, rv, std
    ("tiny_fp32", "f32", 1, 80, 256, 4, 64, 6, 2, 2, None),
    ("ragged_fp32", "f32", 3, 1000, 64, 5, 32, 3, 1, 2, 1.0),
    ("ragged_bf16", "bf16", 3, 1000, 64, 5, 32, 3, 1, 2, 1.0),
    ("decode_b16_ctx4k_full", "bf16", 16, 4097, 1024, 16, 64, 6, 2, 2, None),
    ("decode_b16_sharp", "bf16", 16, 777, 1024, 16, 64, 6, 2, 2, 1.6),
    ("kvonly_bf16", "bf16", 4, 3000, 1536, 24, 64, 0, 4, 4, None),
    ("kvonly_sharp", "bf16", 2, 517, 1536, 24, 64, 0, 4, 4, 1.4),
    ("dh128_h32_bf16", "bf16", 2, 1500, 4096, 32, 128, 6, 2, 2, None),
    ("single_token", "bf16", 5, 1, 1024, 16, 64, 6, 2, 2, None),
    ("r1_bf16", "bf16", 3, 300, 256, 8, 64, 2, 1, 1, 1.5),
    ("h24_r1_bf16", "bf16", 2, 500, 768, 24, 64, 3, 1, 1, 1.0),      # two head tiles at rank 1
    ("h40_r2_bf16", "bf16", 2, 700, 640, 40, 64, 4, 2, 2, 1.0),      # three head tiles
    ("h64_r4_bf16", "bf16", 2, 333, 1024, 64, 64, 2, 4, 4, 1.0),     # four head tiles
    ("h20_dh128_bf16", "bf16", 1, 999, 2560, 20, 128, 2, 2, 2, 1.0),
    ("h10_r2_bf16", "bf16", 2, 400, 640, 10, 64, 3, 2, 2, 1.0),
    # the dims limits (see the projection cases); std chosen so the scores are O(1)
    ("limit_dh256_r64_fp32", "f32", 1, 21, 128, 32, 256, 64, 64, 64, 3.0),
    ("limit_dh256_r64_bf16", "bf16", 1, 21, 128, 32, 256, 64, 64, 64, 3.0),
    ("limit_h256_fp32", "f32", 2, 37, 512, 256, 32, 2, 2, 2, 1.5),
    ("limit_h256_bf16", "bf16", 2, 37, 512, 256, 32, 2, 2, 2, 1.5),
    ("limit_min_dims_fp32", "f32", 3, 9, 4, 1, 2, 1, 1, 1, 1.5),
    ("limit_min_dims_bf16", "bf16", 3, 9, 4, 1, 2, 1, 1, 1, 1.5),
]


@pytest.mark.parametrize("case", DECODE_CASES, ids=[c[0] for c in DECODE_CASES])
def test_decode(case):
    require_gpu()
    name, dtype, B, ctx, dm, h, dh, rq, rk, rv, std = case
    dims = D(dm, h, dh, rq, rk, rv, dtype)
    announce(f"decode {name} B={B} ctx={ctx}")
    sh = shape_of(dims)
    kv = I.factors(sh, B, ctx, seed=61, dtype=dtype, std=std, with_query=False, v_std=value_std(std))
    fq = I.factors(sh, B, 1, seed=62, dtype=dtype, std=std)
    cache = T.new_cache(dims, B, ctx + 3)
    fill_cache(cache, kv)
    q = query_factors_gpu(T, dims, fq, squeeze=True)
    ws = T.new_workspace(dims, B, ctx)
    out = T.tpa_decode_attn(dims, q, cache, ctx, ws)
    out2 = T.tpa_decode_attn(dims, q, cache, ctx, ws)
    torch.cuda.synchronize()
    od = oracle_dims(dims)
    ref = O.decode(oracle_query(fq, dims), oracle_cache(kv, od, B, ctx + 3), od, B, ctx)
    assert_close(out, ref, dtype, f"decode {name}")
    assert torch.equal(out, out2), "repeated decode calls are not bit-identical"


# --------------------------------------------------------------------------
# Prefill attention
# --------------------------------------------------------------------------

PREFILL_CASES = [
    # name, dtype, B, S, start_pos, causal, d_model, h, dh, rq, rk, rv, std
    ("tiny_fp32", "f32", 1, 64, 0, True, 256, 4, 64, 6, 2, 2, None),
    ("ragged_fp32_chunk", "f32", 2, 45, 19, True, 64, 3, 32, 2, 3, 1, 1.0),
    ("ragged_bf16", "bf16", 2, 133, 0, True, 1024, 16, 64, 6, 2, 2, 1.2),
    ("noncausal_bf16", "bf16", 2, 70, 10, False, 1024, 16, 64, 6, 2, 2, 1.2),
    ("kvonly_bf16", "bf16", 2, 150, 0, True, 1536, 24, 64, 0, 4, 4, 1.0),
    ("dh128_bf16", "bf16", 1, 97, 30, True, 4096, 32, 128, 6, 2, 2, 1.0),
    ("dh256_f32", "f32", 1, 40, 0, True, 64, 2, 256, 2, 2, 2, 0.5),
    ("odd_heads_r1_bf16", "bf16", 2, 200, 7, True, 320, 5, 64, 3, 1, 1, 1.0),
    ("odd_heads_dh128_bf16", "bf16", 1, 150, 0, True, 384, 3, 128, 2, 2, 2, 1.0),
    ("kvonly_chunk_bf16", "bf16", 2, 100, 150, True, 1536, 24, 64, 0, 4, 4, 1.0),
    ("r1_noncausal_bf16", "bf16", 2, 77, 20, False, 256, 8, 64, 2, 1, 1, 1.0),
    # the dims limits
    ("limit_dh256_r64_fp32", "f32", 1, 24, 3, True, 128, 32, 256, 64, 64, 64, 3.0),
    ("limit_dh256_r64_bf16", "bf16", 1, 24, 3, True, 128, 32, 256, 64, 64, 64, 3.0),
    ("limit_h256_bf16", "bf16", 1, 40, 5, True, 512, 256, 32, 2, 2, 2, 1.5),
    ("limit_min_dims_fp32", "f32", 2, 17, 2, True, 4, 1, 2, 1, 1, 1, 1.5),
]


def prefill(dims, q, cache, sp, causal, path):
    """tpa_prefill_attn, or (path "ws") tpa_prefill_attn_ws with a workspace of
    the size the library asks for (none where it asks for none)."""
    if path == "fused":
        return T.tpa_prefill_attn(dims, q, cache, sp, causal)
    B, S = q.b_q.shape[0], q.b_q.shape[1]
    n = T.tpa_prefill_workspace_bytes(dims, B, S, sp)
    ws = torch.empty(n, dtype=torch.uint8, device="cuda") if n else None
    return T.tpa_prefill_attn_ws(dims, q, cache, sp, ws, causal)


@pytest.mark.parametrize("path", ["fused", "ws"])
@pytest.mark.parametrize("case", PREFILL_CASES, ids=[c[0] for c in PREFILL_CASES])
def test_prefill(case, path):
    require_gpu()
    name, dtype, B, S, sp, causal, dm, h, dh, rq, rk, rv, std = case
    dims = D(dm, h, dh, rq, rk, rv, dtype)
    announce(f"prefill {name} B={B} S={S} sp={sp} causal={causal} path={path}")
    sh = shape_of(dims)
    Tn = sp + S
    kv = I.factors(sh, B, Tn, seed=71, dtype=dtype, std=std, with_query=False, v_std=value_std(std))
    fq = I.factors(sh, B, S, seed=72, dtype=dtype, std=std)
    cache = T.new_cache(dims, B, Tn + 5)
    fill_cache(cache, kv)
    q = query_factors_gpu(T, dims, fq)
    out = prefill(dims, q, cache, sp, causal, path)
    torch.cuda.synchronize()
    od = oracle_dims(dims)
    ref = O.prefill(oracle_query(fq, dims), oracle_cache(kv, od, B, Tn + 5), od, B, S, sp, causal)
    assert_close(out, ref, dtype, f"prefill {name} ({path})")


WS_BITWISE_CASES = [
    # dtype bf16, d_h 64: B, S, start_pos, causal, d_model, h, rq, rk, rv
    (2, 300, 0, True, 1024, 16, 6, 2, 2),
    (3, 257, 41, True, 320, 5, 3, 1, 1),
    (2, 90, 30, False, 1024, 16, 6, 2, 2),
    (1, 1, 0, True, 256, 8, 2, 1, 1),
]


@pytest.mark.parametrize("case", WS_BITWISE_CASES)
def test_prefill_ws_matches_fused_bitwise(case):
    """At ranks 1 and 2 the workspace path forms the same bf16 K and V as the
    rebuild in LDS and attends in the same 64-key blocks and order: the outputs
    are equal bit for bit.  Workspace contents from an earlier, larger call do
    not leak into a later one."""
    require_gpu()
    B, S, sp, causal, dm, h, rq, rk, rv = case
    dims = D(dm, h, 64, rq, rk, rv, "bf16")
    announce(f"prefill ws vs fused bitwise case={case}")
    sh = shape_of(dims)
    kv = I.factors(sh, B, sp + S, seed=75, dtype="bf16", std=1.0, with_query=False, v_std=value_std(1.0))
    fq = I.factors(sh, B, S, seed=76, dtype="bf16", std=1.0)
    cache = T.new_cache(dims, B, sp + S)
    fill_cache(cache, kv)
    q = query_factors_gpu(T, dims, fq)
    n = T.tpa_prefill_workspace_bytes(dims, B, S, sp)
    assert n == 2 * B * h * (sp + S) * 64 * 2
    ws = torch.full((n + 4096,), 0x7f, dtype=torch.uint8, device="cuda")   # stale bytes: huge bf16 values
    fused = T.tpa_prefill_attn(dims, q, cache, sp, causal)
    staged = T.tpa_prefill_attn_ws(dims, q, cache, sp, ws, causal)
    torch.cuda.synchronize()
    assert torch.equal(fused, staged)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decode_equals_prefill_last_row(dtype):
    require_gpu()
    dims = D(128, 8, 64, 3, 2, 2, dtype)
    B, Tn = 2, 300
    announce(f"decode vs prefill last row {dtype}")
    sh = shape_of(dims)
    kv = I.factors(sh, B, Tn, seed=81, dtype=dtype, std=1.0, with_query=False)
    fq = I.factors(sh, B, 1, seed=82, dtype=dtype, std=1.0)
    cache = T.new_cache(dims, B, Tn)
    fill_cache(cache, kv)
    pre = T.tpa_prefill_attn(dims, query_factors_gpu(T, dims, fq), cache, Tn - 1, True)
    dec = T.tpa_decode_attn(dims, query_factors_gpu(T, dims, fq, squeeze=True), cache, Tn,
                            T.new_workspace(dims, B, Tn))
    torch.cuda.synchronize()
    assert_close(dec, pre[:, 0].double().cpu().numpy(), dtype, "decode vs prefill",
                 max_abs=(1e-5 if dtype == "f32" else 1e-2))


# --------------------------------------------------------------------------
# End to end: the tiny fp32 workload (64-token prefill, then 16 decode steps)
# --------------------------------------------------------------------------

def test_tiny_fp32_end_to_end():
    require_gpu()
    wl = I.WORKLOADS["tiny_fp32"]
    sh = wl.shape
    dims = D(sh.d_model, sh.n_heads, sh.head_dim, sh.rank_q, sh.rank_k, sh.rank_v, "f32", sh.rope_base)
    B, S, steps = wl.batch, wl.seq, wl.decode_steps
    announce(f"end to end tiny_fp32 B={B} S={S} steps={steps}")
    x = I.activations(B, S + steps, sh.d_model, seed=1001, dtype="f32")
    w = I.weights(sh, seed=1001, dtype="f32")
    wp = T.pack_weights({k: v.cuda() for k, v in w.items()}, False)
    cache = T.new_cache(dims, B, S + steps)
    xg = x.cuda()
    f = T.new_factors(dims, B, S)
    T.tpa_factor_proj(dims, xg[:, :S].contiguous(), wp, f, start_pos=0)
    T.tpa_cache_append(dims, cache, f, 0)
    outs = [T.tpa_prefill_attn(dims, f, cache, 0, True)]
    ws = T.new_workspace(dims, B, S + steps)
    for j in range(steps):
        pos = S + j
        fj = T.new_factors(dims, B, 1)
        T.tpa_factor_proj(dims, xg[:, pos:pos + 1].contiguous(), wp, fj, start_pos=pos)
        T.tpa_cache_append(dims, cache, fj, pos)
        qj = T.Factors(fj.a_q[:, 0], fj.b_q[:, 0], None, None, None, None)
        outs.append(T.tpa_decode_attn(dims, qj, cache, pos + 1, ws)[:, None, :])
    got = torch.cat(outs, dim=1)
    torch.cuda.synchronize()
    od = oracle_dims(dims)
    ref = O.layer_forward(I.to_f64(x), {k: I.to_f64(v) for k, v in w.items()}, od, O.cache_new(od, B, S + steps),
                          0, True)
    assert_close(got, ref, "f32", "tiny fp32 end to end")


def _misaligned(t: torch.Tensor) -> torch.Tensor:
    """Same values at an address 2 bytes past a 16-byte boundary."""
    flat = torch.empty(t.numel() + 8, dtype=t.dtype, device=t.device)
    v = flat[1:1 + t.numel()].view(t.shape)
    v.copy_(t)
    return v


def test_decode_general_path_matches_fast_path():
    """An MFMA-eligible shape with misaligned cache pointers runs the general
    kernel; both must meet the oracle bound."""
    require_gpu()
    dims = D(1024, 16, 64, 6, 2, 2, "bf16")
    B, ctx = 4, 700
    announce("decode general vs fast path")
    sh = shape_of(dims)
    kv = I.factors(sh, B, ctx, seed=91, dtype="bf16", with_query=False)
    fq = I.factors(sh, B, 1, seed=92, dtype="bf16")
    cache = T.new_cache(dims, B, ctx)
    fill_cache(cache, kv)
    q = query_factors_gpu(T, dims, fq, squeeze=True)
    ws = T.new_workspace(dims, B, ctx)
    fast = T.tpa_decode_attn(dims, q, cache, ctx, ws)
    mis = T.Cache(*(_misaligned(getattr(cache, k)) for k in ("a_k", "b_k", "a_v", "b_v")))
    slow = T.tpa_decode_attn(dims, q, mis, ctx, ws)
    torch.cuda.synchronize()
    od = oracle_dims(dims)
    ref = O.decode(oracle_query(fq, dims), oracle_cache(kv, od, B, ctx), od, B, ctx)
    assert_close(fast, ref, "bf16", "decode fast path")
    assert_close(slow, ref, "bf16", "decode general path")


@pytest.mark.parametrize("path", ["fused", "ws"])
@pytest.mark.parametrize("kv_only", [False, True])
def test_prefill_strided_queries(path, kv_only):
    """Query factors that are the first S tokens of longer per-sequence buffers
    (q_batch_stride = S + 7 tokens): the same outputs as contiguous ones."""
    require_gpu()
    dims = D(1536, 24, 64, 0, 4, 4, "bf16") if kv_only else D(1024, 16, 64, 6, 2, 2, "bf16")
    B, S, sp = 3, 100, 20
    announce(f"prefill strided queries kv_only={kv_only} path={path}")
    sh = shape_of(dims)
    kv = I.factors(sh, B, sp + S, seed=79, dtype="bf16", std=1.0, with_query=False, v_std=value_std(1.0))
    fq = I.factors(sh, B, S + 7, seed=80, dtype="bf16", std=1.0)
    cache = T.new_cache(dims, B, sp + S)
    fill_cache(cache, kv)
    full = query_factors_gpu(T, dims, fq)
    strided = T.Factors(None if full.a_q is None else full.a_q[:, :S], full.b_q[:, :S], None, None, None, None,
                        S + 7, 0)
    dense = T.Factors(None if full.a_q is None else full.a_q[:, :S].contiguous(), full.b_q[:, :S].contiguous(),
                      None, None, None, None)
    got = prefill(dims, strided, cache, sp, True, path)
    want = prefill(dims, dense, cache, sp, True, path)
    torch.cuda.synchronize()
    assert torch.equal(got, want)
    od = oracle_dims(dims)
    q_ref = {k: v[:, :S] for k, v in fq.items() if k in ("a_q", "b_q", "q")}
    ref = O.prefill(oracle_query(q_ref, dims), oracle_cache(kv, od, B, sp + S), od, B, S, sp, True)
    assert_close(got, ref, "bf16", f"prefill strided queries ({path})")


@pytest.mark.parametrize("kv_only", [False, True])
def test_decode_strided_queries(kv_only):
    """The new tokens' query factors read from the last row of longer
    per-sequence buffers (q_batch_stride = 5 tokens): the same outputs as
    contiguous ones, on the matrix-core decode."""
    require_gpu()
    dims = D(1536, 24, 64, 0, 4, 4, "bf16") if kv_only else D(1024, 16, 64, 6, 2, 2, "bf16")
    B, ctx = 4, 900
    announce(f"decode strided queries kv_only={kv_only}")
    sh = shape_of(dims)
    kv = I.factors(sh, B, ctx, seed=83, dtype="bf16", std=1.0, with_query=False, v_std=value_std(1.0))
    fq = I.factors(sh, B, 5, seed=84, dtype="bf16", std=1.0)
    cache = T.new_cache(dims, B, ctx)
    fill_cache(cache, kv)
    full = query_factors_gpu(T, dims, fq)
    strided = T.Factors(None if full.a_q is None else full.a_q[:, 4], full.b_q[:, 4], None, None, None, None, 5, 0)
    dense = T.Factors(None if full.a_q is None else full.a_q[:, 4].contiguous(), full.b_q[:, 4].contiguous(),
                      None, None, None, None)
    ws = T.new_workspace(dims, B, ctx)
    got = T.tpa_decode_attn(dims, strided, cache, ctx, ws)
    want = T.tpa_decode_attn(dims, dense, cache, ctx, ws)
    torch.cuda.synchronize()
    assert torch.equal(got, want)
    od = oracle_dims(dims)
    q_ref = {k: v[:, 4:5] for k, v in fq.items() if k in ("a_q", "b_q", "q")}
    ref = O.decode(oracle_query(q_ref, dims), oracle_cache(kv, od, B, ctx), od, B, ctx)
    assert_close(got, ref, "bf16", "decode strided queries")


def test_prefill_ws_misaligned_output_takes_the_rebuild_path():
    """An output 2 bytes past a 16-byte boundary: the workspace call runs the
    kernels that take any alignment, leaves the workspace untouched and still
    matches the oracle."""
    require_gpu()
    dims = D(1024, 16, 64, 6, 2, 2, "bf16")
    B, S, sp = 2, 150, 10
    announce("prefill ws misaligned output")
    sh = shape_of(dims)
    kv = I.factors(sh, B, sp + S, seed=77, dtype="bf16", std=1.0, with_query=False, v_std=value_std(1.0))
    fq = I.factors(sh, B, S, seed=78, dtype="bf16", std=1.0)
    cache = T.new_cache(dims, B, sp + S)
    fill_cache(cache, kv)
    n = T.tpa_prefill_workspace_bytes(dims, B, S, sp)
    ws = torch.full((n,), 0x5a, dtype=torch.uint8, device="cuda")
    out = _misaligned(torch.zeros(B, S, dims.n_heads * dims.head_dim, dtype=torch.bfloat16, device="cuda"))
    T.tpa_prefill_attn_ws(dims, query_factors_gpu(T, dims, fq), cache, sp, ws, True, out=out)
    torch.cuda.synchronize()
    assert bool((ws == 0x5a).all()), "the workspace was written on the fallback path"
    od = oracle_dims(dims)
    ref = O.prefill(oracle_query(fq, dims), oracle_cache(kv, od, B, sp + S), od, B, S, sp, True)
    assert_close(out, ref, "bf16", "prefill ws, misaligned output")


@pytest.mark.parametrize("path", ["fused", "ws"])
@pytest.mark.parametrize("wl_name,B,S,n_rows", [
    ("prefill_b4_s4k", 4, 4096, 48),       # the causal prefill workload at full size
    ("kvonly_b32_ctx16k", 2, 2048, 32),    # the KV-only shape, two sequences of 2048
])
def test_prefill_full_size_sampled_rows(wl_name, B, S, n_rows, path):
    """Prefill in the launch configuration the benchmark times; the oracle computes
    sampled query rows one by one (each row is its own definition)."""
    require_gpu()
    wl = I.WORKLOADS[wl_name]
    sh = wl.shape
    dims = D(sh.d_model, sh.n_heads, sh.head_dim, sh.rank_q, sh.rank_k, sh.rank_v, "bf16")
    announce(f"prefill full size {wl_name} B={B} S={S} path={path}")
    kv = I.factors(sh, B, S, seed=101, dtype="bf16", with_query=False)
    fq = I.factors(sh, B, S, seed=102, dtype="bf16")
    cache = T.new_cache(dims, B, S)
    fill_cache(cache, kv)
    out = prefill(dims, query_factors_gpu(T, dims, fq), cache, 0, True, path)
    torch.cuda.synchronize()
    rng = np.random.default_rng(7)
    rows = np.unique(np.concatenate([[0, 1, S - 1], rng.integers(0, S, n_rows)]))
    od = oracle_dims(dims)
    ref = O.prefill(oracle_query(fq, dims), oracle_cache(kv, od, B, S), od, B, S, 0, True, rows=rows)
    assert_close(out[:, rows], ref[:, rows], "bf16", f"prefill {wl_name} sampled rows")


@pytest.mark.parametrize("path", ["fused", "ws"])
def test_prefill_kvonly_full_size_sampled_rows(path):
    """The KV-only prefill at its full size (32 sequences of 16,384 tokens, 24
    heads of 64, plain Q, R 4) in one call; the oracle checks 256 sampled query
    rows (16 per sequence, 16 sequences, every head), rebuilding each sampled
    sequence's K and V in fp64 once and attending those rows alone."""
    require_gpu()
    wl = I.WORKLOADS["kvonly_b32_ctx16k"]
    sh = wl.shape
    dims = D(sh.d_model, sh.n_heads, sh.head_dim, sh.rank_q, sh.rank_k, sh.rank_v, "bf16")
    B, S = wl.batch, wl.seq
    announce(f"prefill full size kvonly_b32_ctx16k B={B} S={S} path={path}")
    kv = I.factors(sh, B, S, seed=141, dtype="bf16", with_query=False)
    fq = I.factors(sh, B, S, seed=142, dtype="bf16")
    cache = T.new_cache(dims, B, S)
    fill_cache(cache, kv)
    out = prefill(dims, query_factors_gpu(T, dims, fq), cache, 0, True, path)
    torch.cuda.synchronize()
    del cache
    rng = np.random.default_rng(143)
    seqs = np.sort(rng.choice(B, 16, replace=False))
    dh, h = sh.head_dim, sh.n_heads
    got, want = [], []
    for b in seqs:
        rows = np.unique(np.concatenate([[0, S - 1], rng.integers(0, S, 14)])) if b == seqs[0] else \
            np.unique(rng.integers(0, S, 16))
        T_b = int(rows.max()) + 1
        k = O.reconstruct(I.to_f64(kv["a_k"][b, :T_b]), I.to_f64(kv["b_k"][b, :T_b]))   # [T_b, h, d_h]
        v = O.reconstruct(I.to_f64(kv["a_v"][b, :T_b]), I.to_f64(kv["b_v"][b, :T_b]))
        q = I.to_f64(fq["q"][b, rows])                                                 # [rows, h, d_h]
        ref = np.empty((len(rows), h * dh))
        for hh in range(h):
            ref[:, hh * dh:(hh + 1) * dh] = O.attend_head(q[:, hh], k[:, hh], v[:, hh], rows, True)
        got.append(out[b, torch.as_tensor(rows, device=out.device)])
        want.append(ref)
    assert_close(torch.cat(got), np.concatenate(want), "bf16", "prefill kvonly_b32_ctx16k sampled rows")


def test_decode_step_graph_replay_matches_eager():
    """The decode step (projection into the cache slot, decode attention) captured
    as a HIP graph and replayed several times, with eager work and synchronisation
    between replays, gives the eager result bit for bit every time."""
    require_gpu()
    dims = D(1024, 16, 64, 6, 2, 2, "bf16")
    B, ctx = 8, 1500
    announce("decode step graph replay")
    sh = shape_of(dims)
    kv = I.factors(sh, B, ctx - 1, seed=111, dtype="bf16", with_query=False)
    w = I.weights(sh, seed=111, dtype="bf16")
    wp = T.pack_weights({k: v.cuda() for k, v in w.items()}, False)
    x_new = I.activations(B, 1, 1024, seed=112, dtype="bf16").cuda()
    cache = T.new_cache(dims, B, ctx)
    fill_cache(cache, kv)
    qf = T.new_factors(dims, B, 1)
    slot = cache.slot_factors(ctx - 1)
    into = T.Factors(qf.a_q, qf.b_q, slot.a_k, slot.b_k, slot.a_v, slot.b_v, 0, ctx)
    q = T.Factors(qf.a_q[:, 0], qf.b_q[:, 0], None, None, None, None)
    ws = T.new_workspace(dims, B, ctx)
    out = torch.empty(B, 16 * 64, dtype=torch.bfloat16, device="cuda")

    def step():
        T.tpa_factor_proj(dims, x_new, wp, into, start_pos=ctx - 1)
        T.tpa_decode_attn(dims, q, cache, ctx, ws, out=out)

    step()
    torch.cuda.synchronize()
    eager = out.clone()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            step()
    torch.cuda.current_stream().wait_stream(side)
    for rep in range(4):
        out.zero_()
        slot.a_k.zero_()                      # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {rep} differs from the eager step"


def _oracle_decode_heads(fq: dict, kv: dict, dims, pairs, ctx):
    """fp64 oracle decode output of the sampled (sequence, head) pairs only: each
    sequence's sampled heads are reconstructed together and attended one by one
    (each output is its own definition)."""
    od = oracle_dims(dims)
    Q = O.queries(oracle_query(fq, dims), od)                   # [B, 1, h, d_h]
    out = {}
    for b in sorted({p[0] for p in pairs}):
        heads = sorted({hh for bb, hh in pairs if bb == b})
        k = O.reconstruct(I.to_f64(kv["a_k"][b, :ctx, heads]), I.to_f64(kv["b_k"][b, :ctx]))   # [ctx, n, d_h]
        v = O.reconstruct(I.to_f64(kv["a_v"][b, :ctx, heads]), I.to_f64(kv["b_v"][b, :ctx]))
        for j, hh in enumerate(heads):
            out[(b, hh)] = O.attend_head(Q[b, :, hh], k[:, j], v[:, j], np.array([ctx - 1]), True)[0]
    return out


def _decode_pairs(wl_name):
    """The sampled (sequence, head) pairs: every pair of the KV-only workload; two
    seeded heads per sequence (incl. the first and last) of the long-context one,
    whose per-sequence fp64 rebuild of every head would take 4.3 GB."""
    wl = I.WORKLOADS[wl_name]
    B, h = wl.batch, wl.shape.n_heads
    if wl_name == "kvonly_b32_ctx16k":
        return [(b, hh) for b in range(B) for hh in range(h)]
    rng = np.random.default_rng(144)
    pairs = [(0, 0), (B - 1, h - 1)]
    for b in range(B):
        pairs += [(b, int(x)) for x in rng.choice(h, 2, replace=False)]
    return sorted(set(pairs))


@pytest.mark.parametrize("wl_name", ["decode_b8_ctx128k", "kvonly_b32_ctx16k"])
def test_decode_full_size_sampled(wl_name):
    """Decode at the workload's full size, in the launch configuration of a real
    call; the oracle computes sampled (sequence, head) outputs one by one."""
    require_gpu()
    wl = I.WORKLOADS[wl_name]
    sh = wl.shape
    dims = D(sh.d_model, sh.n_heads, sh.head_dim, sh.rank_q, sh.rank_k, sh.rank_v, "bf16")
    B, ctx = wl.batch, wl.seq + 1
    pairs = _decode_pairs(wl_name)
    announce(f"decode full size {wl_name} B={B} ctx={ctx}, {len(pairs)} (sequence, head) pairs")
    kv = I.factors(sh, B, ctx, seed=121, dtype="bf16", with_query=False)
    fq = I.factors(sh, B, 1, seed=122, dtype="bf16")
    cache = T.new_cache(dims, B, ctx)
    fill_cache(cache, kv)
    out = T.tpa_decode_attn(dims, query_factors_gpu(T, dims, fq, squeeze=True), cache, ctx,
                            T.new_workspace(dims, B, ctx))
    torch.cuda.synchronize()
    ref = _oracle_decode_heads(fq, kv, dims, pairs, ctx)
    dh = sh.head_dim
    got = torch.stack([out[b, hh * dh:(hh + 1) * dh] for b, hh in pairs])
    assert_close(got, np.stack([ref[p] for p in pairs]), "bf16", f"decode {wl_name} sampled heads")
    del cache, kv


@pytest.mark.parametrize("name,rank,n_kv", [("MQA", 1, 1), ("GQA", 4, 4), ("MHA", 24, 24)])
def test_textbook_equivalence_kvonly_shape(name, rank, n_kv):
    """Non-contextual head factors reduce TPA to the textbook forms: R = 1 with
    a = 1 is multi-query attention; R = g groups with a_r[h] = g for h in group r
    (0 otherwise) is grouped-query attention with g K/V heads; R = h with
    a_r[h] = h for r = h is multi-head attention (the factor cancels the 1/R).
    Decode and prefill at the KV-only shape (24 heads of 64, plain Q) against
    the textbook forms through torch's scaled dot-product attention in fp64,
    written without the factor machinery.  R = 4 runs the matrix-core kernels,
    R = 24 the general ones."""
    require_gpu()
    import textbook
    B, S, ctx, h = 4, 257, 2048, 24
    dims = D(1536, h, 64, 0, rank, rank, "bf16")
    announce(f"{name} equivalence at the KV-only shape (R = {rank})")
    sh = shape_of(dims)
    kv = I.factors(sh, B, ctx, seed=131, dtype="bf16", std=1.0, with_query=False)
    group = torch.arange(h) // (h // n_kv)                              # K/V head of each query head
    a = torch.zeros(h, rank, dtype=torch.bfloat16)
    a[torch.arange(h), group] = float(rank)
    for k in ("a_k", "a_v"):
        kv[k] = a.expand(B, ctx, h, rank).contiguous()
    fq = I.factors(sh, B, S, seed=132, dtype="bf16", std=1.0)
    cache = T.new_cache(dims, B, ctx)
    fill_cache(cache, kv)
    # prefill of the last S positions (queries at ctx-S .. ctx-1), and a decode at ctx-1
    pre = T.tpa_prefill_attn(dims, query_factors_gpu(T, dims, fq), cache, ctx - S, True)
    dq = {"q": fq["q"][:, -1:]}
    dec = T.tpa_decode_attn(dims, query_factors_gpu(T, dims, dq, squeeze=True), cache, ctx,
                            T.new_workspace(dims, B, ctx))
    torch.cuda.synchronize()
    q = I.to_f64(fq["q"])                                     # [B, S, 24, 64]
    k = I.to_f64(kv["b_k"])                                   # [B, ctx, n_kv, 64]: the K/V heads
    v = I.to_f64(kv["b_v"])
    ref = textbook.attention(torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), ctx - S, True).numpy()
    assert_close(pre, ref, "bf16", f"prefill vs textbook {name}")
    assert_close(dec, ref[:, -1], "bf16", f"decode vs textbook {name}")
