"""GPU parity of the paged factor cache: the paged append (a bit copy through the
block table) and decode with a key count per sequence, against the fp64
oracle's decode_paged on the same seeded inputs; the paged decode with an
identity table against the dense decode, bit for bit."""
import numpy as np
import pytest
import torch

import oracle.tpa_oracle as O
import tpa_inputs as I
from factorized_kv_cache_amd import tpa as T
from gpu_util import (announce, assert_close, oracle_dims, oracle_query, query_factors_gpu, require_gpu, shape_of,
                      value_std)

pytestmark = pytest.mark.gpu

KV = ("a_k", "b_k", "a_v", "b_v")


def D(d_model, h, dh, rq, rk, rv, dtype, base=10000.0):
    return T.Dims(d_model, h, dh, rq, rk, rv, base, dtype)


def random_table(B, pages_per_seq, n_pages, seed):
    """Distinct pages in a seeded random order (CPU, int32)."""
    g = torch.Generator().manual_seed(seed)
    perm = torch.randperm(n_pages, generator=g)[:B * pages_per_seq]
    return perm.reshape(B, pages_per_seq).to(torch.int32).contiguous()


def fill_pages(pc, kv: dict, table: torch.Tensor, lens):
    """Test setup: token t of sequence b to page table[b, t // P], row t % P."""
    P = pc.page_tokens
    for k in KV:
        pool = getattr(pc, k)
        for b, L in enumerate(lens):
            if L == 0:
                continue
            t = torch.arange(L)
            pool[table[b, t // P].long().cuda(), (t % P).cuda()] = kv[k][b, :L].to(pool.device, pool.dtype)


def oracle_pools(pc) -> dict:
    return {k: I.to_f64(getattr(pc, k).cpu()) for k in KV}


# --------------------------------------------------------------------------
# Paged append
# --------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("B,S,page,dims_args", [
    (3, 5, 4, (64, 3, 6, 2, 3, 1)),        # odd row widths (2-byte copies)
    (4, 17, 16, (128, 16, 64, 6, 2, 2)),
    (2, 1, 64, (64, 24, 64, 0, 4, 4)),
])
def test_paged_append_bitwise(dtype, B, S, page, dims_args):
    require_gpu()
    dims = D(*dims_args, dtype)
    announce(f"paged append {dtype} B={B} S={S} page={page} dims={dims_args}")
    f = I.factors(shape_of(dims), B, S, seed=71, dtype=dtype, with_query=False)
    max_pages = 4
    n_pages = B * max_pages + 3
    table = random_table(B, max_pages, n_pages, seed=72)
    pc = T.new_paged_cache(dims, n_pages, page, table)
    for k in KV:
        getattr(pc, k).fill_(7.0)
    cap = max_pages * page
    # per-sequence start positions; the last sequence's block runs past the
    # capacity, so its tail must be skipped
    starts = [(3 * b + 1) % max(1, cap - S) for b in range(B)]
    starts[-1] = cap - 1
    kv = T.Factors(None, None, *(f[k].cuda() for k in KV))
    T.tpa_paged_cache_append(dims, pc, kv, torch.tensor(starts, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    for k in KV:
        want = torch.full_like(getattr(pc, k).cpu(), 7.0)
        for b in range(B):
            for s in range(S):
                pos = starts[b] + s
                if pos < cap:
                    want[table[b, pos // page], pos % page] = f[k][b, s]
        assert torch.equal(getattr(pc, k).cpu(), want), k


# --------------------------------------------------------------------------
# Paged decode, key count per sequence
# --------------------------------------------------------------------------

PAGED_DECODE_CASES = [
    # name, dtype, lengths, page, extra max_ctx_len, d_model, h, dh, rq, rk, rv, std
    ("bf16_p64", "bf16", (1, 64, 65, 1000, 0, 333), 64, 0, 1024, 16, 64, 6, 2, 2, 1.2),
    ("bf16_dh128_p128", "bf16", (3000, 17), 128, 40, 4096, 32, 128, 6, 2, 2, 1.0),
    ("bf16_kvonly_p32", "bf16", (700, 1, 90), 32, 0, 1536, 24, 64, 0, 4, 4, 1.0),
    ("bf16_r1_p96", "bf16", (500, 96, 97), 96, 0, 256, 8, 64, 2, 1, 1, 1.4),
    ("bf16_p16_general", "bf16", (300, 45, 2), 16, 0, 256, 8, 64, 2, 2, 2, 1.2),   # page 16: general kernel
    ("f32_p8", "f32", (50, 7, 0, 129), 8, 3, 64, 5, 32, 3, 1, 2, 1.0),
]


@pytest.mark.parametrize("case", PAGED_DECODE_CASES, ids=[c[0] for c in PAGED_DECODE_CASES])
def test_paged_decode(case):
    require_gpu()
    name, dtype, lens, page, extra, dm, h, dh, rq, rk, rv, std = case
    dims = D(dm, h, dh, rq, rk, rv, dtype)
    B, Tmax = len(lens), max(lens)
    max_ctx = Tmax + extra
    announce(f"paged decode {name} lens={lens} page={page} max_ctx={max_ctx}")
    sh = shape_of(dims)
    kv = I.factors(sh, B, Tmax, seed=81, dtype=dtype, std=std, with_query=False, v_std=value_std(std))
    fq = I.factors(sh, B, 1, seed=82, dtype=dtype, std=std)
    pps = (max_ctx + page - 1) // page
    n_pages = B * pps + 5
    table = random_table(B, pps, n_pages, seed=83)
    pc = T.new_paged_cache(dims, n_pages, page, table)
    fill_pages(pc, kv, table, lens)
    q = query_factors_gpu(T, dims, fq, squeeze=True)
    ws = torch.zeros(max(T.tpa_paged_decode_workspace_bytes(dims, B, max_ctx), 16), dtype=torch.uint8,
                     device="cuda")
    ctx_lens = torch.tensor(lens, dtype=torch.int32, device="cuda")
    out = T.tpa_paged_decode_attn(dims, q, pc, ctx_lens, max_ctx, ws)
    out2 = T.tpa_paged_decode_attn(dims, q, pc, ctx_lens, max_ctx, ws)
    torch.cuda.synchronize()
    ref = O.decode_paged(oracle_query(fq, dims), oracle_pools(pc), table.numpy(), lens, oracle_dims(dims))
    assert_close(out, ref, dtype, f"paged decode {name}")
    assert torch.equal(out, out2), "repeated paged decode calls are not bit-identical"


@pytest.mark.parametrize("dtype,page,dims_args", [
    ("bf16", 64, (1024, 16, 64, 6, 2, 2)),     # matrix-core kernel
    ("f32", 8, (64, 5, 32, 3, 1, 2)),          # general kernel
])
def test_paged_identity_equals_dense(dtype, page, dims_args):
    """Identity table, every sequence at full length: the same rows, chunks and
    merge order as the dense decode, so the same bits."""
    require_gpu()
    dims = D(*dims_args, dtype)
    B, ctx = 3, 1000
    pps = (ctx + page - 1) // page
    announce(f"paged identity vs dense {dtype} page={page}")
    sh = shape_of(dims)
    kv = I.factors(sh, B, ctx, seed=91, dtype=dtype, with_query=False)
    fq = I.factors(sh, B, 1, seed=92, dtype=dtype)
    cache = T.new_cache(dims, B, pps * page)
    for k in KV:
        getattr(cache, k)[:, :ctx].copy_(kv[k].cuda())
    table = torch.arange(B * pps, dtype=torch.int32).reshape(B, pps).contiguous()
    # the pools are the dense cache's memory viewed as pages
    pools = [getattr(cache, k).view(B * pps, page, *getattr(cache, k).shape[2:]) for k in KV]
    pc = T.PagedCache(*pools, table.cuda())
    q = query_factors_gpu(T, dims, fq, squeeze=True)
    ws = T.new_workspace(dims, B, ctx)
    dense = T.tpa_decode_attn(dims, q, cache, ctx, ws)
    paged = T.tpa_paged_decode_attn(dims, q, pc, torch.full((B,), ctx, dtype=torch.int32, device="cuda"), ctx, ws)
    torch.cuda.synchronize()
    assert torch.equal(dense, paged), "paged decode with an identity table differs from the dense decode"


def test_paged_decode_full_size():
    """The decode workload (16 sequences, 4097 keys, d_model 1024, h 16, d_h 64,
    R_Q 6, R 2) through a shuffled table of 64-token pages, with some shorter
    sequences; every output against the oracle."""
    require_gpu()
    wl = I.WORKLOADS["decode_b16_ctx4k"]
    s = wl.shape
    dims = D(s.d_model, s.n_heads, s.head_dim, s.rank_q, s.rank_k, s.rank_v, "bf16", s.rope_base)
    B, ctx, page = wl.batch, wl.seq + 1, 64
    lens = [ctx] * B
    lens[3], lens[7], lens[11] = 1, 2048, 4000
    announce(f"paged decode full size B={B} ctx={ctx} page={page}")
    kv = I.factors(s, B, ctx, seed=93, dtype="bf16", with_query=False)
    fq = I.factors(s, B, 1, seed=94, dtype="bf16")
    pps = (ctx + page - 1) // page
    table = random_table(B, pps, B * pps, seed=95)
    pc = T.new_paged_cache(dims, B * pps, page, table)
    fill_pages(pc, kv, table, lens)
    q = query_factors_gpu(T, dims, fq, squeeze=True)
    ws = T.new_workspace(dims, B, ctx)
    out = T.tpa_paged_decode_attn(dims, q, pc, torch.tensor(lens, dtype=torch.int32, device="cuda"), ctx, ws)
    torch.cuda.synchronize()
    ref = O.decode_paged(oracle_query(fq, dims), oracle_pools(pc), table.numpy(), lens, oracle_dims(dims))
    assert_close(out, ref, "bf16", "paged decode full size")
