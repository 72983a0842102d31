"""GPU test of the allocation-free decode entry point (tpa_decode_attn_noalloc):
through the C ABI, its output equals tpa_decode_attn's (same kernels, plan and
merge order, so the same bits) and meets the fp64 oracle's bound, on two calls
in a row, the second with a smaller input, so the second call runs on the
scratch the first one left behind."""
import pytest
import torch

import oracle.tpa_oracle as O
import tpa_inputs as I
from factorized_kv_cache_amd import tpa as T
from gpu_util import (announce, assert_close, fill_cache, oracle_cache, oracle_dims, oracle_query,
                      query_factors_gpu, require_gpu, shape_of)

pytestmark = pytest.mark.gpu

CASES = [
    # name, B, ctx, d_model, h, dh, rq, rk, rv: the batch-16 decode at its full
    # size (matrix-core kernel, 32 chunks per sequence), then a smaller,
    # ragged one
    ("b16_ctx4097", 16, 4097, 1024, 16, 64, 6, 2, 2),
    ("b3_ctx777_kvonly", 3, 777, 1536, 24, 64, 0, 4, 4),
]


def test_decode_noalloc_matches_workspace_entry_point():
    require_gpu()
    assert T.tpa_decode_noalloc_max_bytes() == 16 << 20
    for seed, (name, B, ctx, dm, h, dh, rq, rk, rv) in enumerate(CASES):
        dims = T.Dims(dm, h, dh, rq, rk, rv, 10000.0, "bf16")
        announce(f"decode noalloc {name} B={B} ctx={ctx}")
        sh = shape_of(dims)
        kv = I.factors(sh, B, ctx, seed=171 + seed, dtype="bf16", with_query=False)
        fq = I.factors(sh, B, 1, seed=181 + seed, dtype="bf16")
        cache = T.new_cache(dims, B, ctx + 2)
        fill_cache(cache, kv)
        q = query_factors_gpu(T, dims, fq, squeeze=True)
        ref = T.tpa_decode_attn(dims, q, cache, ctx, T.new_workspace(dims, B, ctx))
        got = T.tpa_decode_attn_noalloc(dims, q, cache, ctx)
        torch.cuda.synchronize()
        assert torch.equal(got, ref), f"{name}: the allocation-free decode differs from tpa_decode_attn"
        od = oracle_dims(dims)
        want = O.decode(oracle_query(fq, dims), oracle_cache(kv, od, B, ctx + 2), od, B, ctx)
        assert_close(got, want, "bf16", f"decode noalloc {name}")
