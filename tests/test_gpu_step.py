"""GPU parity of the whole decode step against the fp64 oracle's layer forward.

The step is the library's fused form: the projection writes the new token's
key/value factors straight into cache slot ctx (kv_batch_stride = max_seq) and
its query factors into a small buffer, then the decode attends over ctx + 1
keys.  The context itself goes through the same projection into the cache.
The oracle runs its whole layer (projection, rotation, cache write, attention;
"Tensor Product Attention Is All You Need" review on coreui.cn, 前向传播) on the
same bf16 inputs and attends the last row only.  The step runs eagerly, then as
a captured HIP graph replayed three times with eager work and synchronisation
between replays; every replay must equal the eager result bit for bit and the
oracle to the bf16 tolerance.
"""
import numpy as np
import pytest
import torch

import oracle.tpa_oracle as O
import tpa_inputs as I
from factorized_kv_cache_amd import tpa as T
from gpu_util import announce, assert_close, oracle_dims, require_gpu

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("wl_name,oracle_seqs", [
    ("decode_b16_ctx4k", None),              # every sequence and head
    ("kvonly_b32_ctx16k", (0, 17, 31)),      # three of the 32 sequences, every head
])
def test_fused_decode_step_against_oracle(wl_name, oracle_seqs):
    require_gpu()
    wl = I.WORKLOADS[wl_name]
    sh = wl.shape
    dims = T.Dims(sh.d_model, sh.n_heads, sh.head_dim, sh.rank_q, sh.rank_k, sh.rank_v, sh.rope_base, "bf16")
    B, ctx = wl.batch, wl.seq                 # ctx cached tokens; the new token sits at position ctx
    n = ctx + 1
    h, dh = sh.n_heads, sh.head_dim
    announce(f"fused decode step {wl_name} B={B} ctx={ctx}")
    # each sequence's activations from its own generator stream (salt = b), so
    # the oracle can draw just the sequences it checks
    x = torch.cat([I.activations(1, n, sh.d_model, seed=151, dtype="bf16", salt=b) for b in range(B)])
    w = I.weights(sh, seed=151, dtype="bf16")
    wp = T.pack_weights({k: v.cuda() for k, v in w.items()}, dims.kv_only)
    xg = x.cuda()
    cache = T.new_cache(dims, B, n)

    # the context, projected (with rotation) straight into cache slots 0 .. ctx-1
    qctx = T.new_factors(dims, B, ctx)
    s0 = cache.slot_factors(0)
    T.tpa_factor_proj(dims, xg[:, :ctx].contiguous(), wp,
                      T.Factors(qctx.a_q, qctx.b_q, s0.a_k, s0.b_k, s0.a_v, s0.b_v, 0, n), start_pos=0)
    del qctx

    # the step
    qf = T.new_factors(dims, B, 1)
    slot = cache.slot_factors(ctx)
    into = T.Factors(qf.a_q, qf.b_q, slot.a_k, slot.b_k, slot.a_v, slot.b_v, 0, n)
    q = T.Factors(None if dims.kv_only else qf.a_q[:, 0], qf.b_q[:, 0], None, None, None, None)
    ws = T.new_workspace(dims, B, n)
    out = torch.empty(B, h * dh, dtype=torch.bfloat16, device="cuda")
    x_new = xg[:, ctx:ctx + 1].contiguous()

    def step():
        T.tpa_factor_proj(dims, x_new, wp, into, start_pos=ctx)
        T.tpa_decode_attn(dims, q, cache, n, ws, out=out)

    step()
    torch.cuda.synchronize()
    eager = out.clone()
    del xg

    seqs = list(range(B)) if oracle_seqs is None else list(oracle_seqs)
    od = oracle_dims(dims)
    xs = I.to_f64(x[seqs])
    ref = O.layer_forward(xs, {k: I.to_f64(v) for k, v in w.items()}, od, O.cache_new(od, len(seqs), n), 0, True,
                          rows=[ctx])[:, ctx]
    sel = torch.as_tensor(seqs, device="cuda")
    assert_close(eager[sel], ref, "bf16", f"fused step {wl_name} (eager)")

    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            step()
    torch.cuda.current_stream().wait_stream(side)
    for rep in range(3):
        out.zero_()
        slot.a_k.zero_()                      # the replay must rewrite the slot
        slot.b_v.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {rep} differs from the eager step"
        assert_close(out[sel], ref, "bf16", f"fused step {wl_name} (replay {rep})")
