"""Benchmark of the TPA hot path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline] [--no-prefill]

A step is one decode step of one TPA attention layer for the whole batch of
the decode workload (batch 16, 4096 cached tokens plus the new one, d_model
1024, 16 heads of 64, R_Q 6, R_K = R_V 2, bf16): factor projection of the new
tokens with fused RoPE, whose epilogue appends their K/V factors straight into
cache slot 4096, then decode attention over the 4097 keys (main pass +
combine).  Eight independent layers (weights and factor caches,
336 MB of cache) are visited in turn, so each step reads its cache cold from
HBM, as in a multi-layer model; the caches are built through the same
projection and append kernels from synthetic N(0,1) activations and
N(0,0.02) weights.

Prints one JSON line.  `value` is decode throughput in tokens/s (batch /
step time), with the eight-layer step captured once as a HIP graph and
replayed (K steps = K/8 replays).  `roofline` covers the decode attention call
(the dominant kernel): algorithmic factor-cache bytes per call over its
average duration, timed with HIP events on the stream it runs on in an eager
pass over the same steps.  `cpu_baseline` is the fp64
oracle timed on a bounded sample of the same decode step.  `prefill` reports
the causal prefill workload (batch 4, 4096 tokens) in TFLOP/s.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import tpa_inputs as I  # noqa: E402
from factorized_kv_cache_amd import tpa as T  # noqa: E402

HBM_PEAK_GBPS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
LAYERS = 8
METRIC = "TPA decode tok/s + factor-cache HBM GB/s; prefill attention TFLOP/s"


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def dims_of(wl: I.Workload) -> T.Dims:
    s = wl.shape
    return T.Dims(s.d_model, s.n_heads, s.head_dim, s.rank_q, s.rank_k, s.rank_v, s.rope_base, wl.dtype)


def source_digest(*names) -> str:
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "factorized_kv_cache_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(kernel_sources, per_launch_bytes_key="bytes_per_launch"):
    """HBM bytes per launch measured with rocprofv3 counters, if they were taken
    on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "decode_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("source_digest") != source_digest(*kernel_sources):
        return None
    return d.get(per_launch_bytes_key)


# ---------------------------------------------------------------------------
# Decode workload
# ---------------------------------------------------------------------------

class DecodeBench:
    def __init__(self, wl: I.Workload, seed: int = 1002):
        self.wl = wl
        self.dims = dims_of(wl)
        d = self.dims
        self.B = wl.batch
        self.ctx = wl.seq + 1                # cached context plus the new token
        dev = "cuda"
        g = torch.Generator(device=dev)
        g.manual_seed(seed)
        self.layers = []
        x_ctx = (torch.randn(self.B, wl.seq, d.d_model, generator=g, device=dev)).to(torch.bfloat16)
        for layer in range(LAYERS):
            w = I.weights(wl.shape, seed=seed + 17 * layer, dtype="bf16")
            wp = T.pack_weights({k: v.to(dev) for k, v in w.items()}, d.kv_only)
            cache = T.new_cache(d, self.B, self.ctx)
            f = T.new_factors(d, self.B, wl.seq)
            T.tpa_factor_proj(d, x_ctx, wp, f, start_pos=0)
            T.tpa_cache_append(d, cache, f, 0)
            del f
            x_new = torch.randn(self.B, 1, d.d_model, generator=g, device=dev).to(torch.bfloat16)
            qf = T.new_factors(d, self.B, 1)
            slot = cache.slot_factors(self.ctx - 1)
            # the new token's K/V factors are written straight into their cache slot
            into = T.Factors(qf.a_q, qf.b_q, slot.a_k, slot.b_k, slot.a_v, slot.b_v, 0, self.ctx)
            self.layers.append(dict(wp=wp, cache=cache, x_new=x_new, qf=qf, into=into,
                                    q=T.Factors(qf.a_q[:, 0] if qf.a_q is not None else None, qf.b_q[:, 0],
                                                None, None, None, None),
                                    ws=T.new_workspace(d, self.B, self.ctx),
                                    out=torch.empty(self.B, d.n_heads * d.head_dim, dtype=torch.bfloat16,
                                                    device=dev)))
        del x_ctx
        torch.cuda.synchronize()

    def step(self, k: int, ev=None):
        d = self.dims
        L = self.layers[k % LAYERS]
        T.tpa_factor_proj(d, L["x_new"], L["wp"], L["into"], start_pos=self.ctx - 1)
        if ev is not None:
            ev[0].record()
        T.tpa_decode_attn(d, L["q"], L["cache"], self.ctx, L["ws"], out=L["out"])
        if ev is not None:
            ev[1].record()

    def cache_bytes(self) -> int:
        return self.B * self.ctx * T.tpa_cache_elems_per_token(self.dims) * 2


def run_decode(args):
    """Returns (bench, workload, graph ms/step, eager ms/step, decode-call ms, eager per-call
    median ms, steps timed).

    Three timed regions over the same caches: an eager pass with events around
    every decode call (per-call medians, which include launch gaps); the
    eight-layer step captured once as a HIP graph and replayed (the throughput);
    and the eight layers' decode calls alone captured as a HIP graph and
    replayed between two events on their stream, back to back (the per-call
    duration of the roofline: the kernels' time with the short gaps of a
    graph, comparable to the profiler's kernel durations)."""
    wl = I.WORKLOADS["decode_b16_ctx4k"]
    log(f"[bench] building {LAYERS} layer caches for {wl.name}")
    db = DecodeBench(wl)
    for k in range(args.warmup):
        db.step(k)
    torch.cuda.synchronize()
    n = args.steps
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for k in range(n):
        db.step(k, evs[k])
    stop.record()
    torch.cuda.synchronize()
    eager_ms = start.elapsed_time(stop) / n
    dec_ms = sorted(a.elapsed_time(b) for a, b in evs)
    dec_med_ms = dec_ms[len(dec_ms) // 2]

    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            for k in range(LAYERS):
                db.step(k)
    torch.cuda.current_stream().wait_stream(side)
    for _ in range(max(1, args.warmup // LAYERS)):
        graph.replay()
    torch.cuda.synchronize()
    reps = max(1, (n + LAYERS - 1) // LAYERS)
    start.record()
    for _ in range(reps):
        graph.replay()
    stop.record()
    torch.cuda.synchronize()
    graph_ms = start.elapsed_time(stop) / (reps * LAYERS)

    d = db.dims
    dgraph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(dgraph, stream=side):
            for L in db.layers:
                T.tpa_decode_attn(d, L["q"], L["cache"], db.ctx, L["ws"], out=L["out"])
    torch.cuda.current_stream().wait_stream(side)
    dgraph.replay()
    torch.cuda.synchronize()
    start.record()
    for _ in range(reps):
        dgraph.replay()
    stop.record()
    torch.cuda.synchronize()
    dec_graph_ms = start.elapsed_time(stop) / (reps * LAYERS)
    return db, wl, graph_ms, eager_ms, dec_graph_ms, dec_med_ms, reps * LAYERS


# ---------------------------------------------------------------------------
# Paged decode (reported alongside): the same caches moved into shuffled pages
# ---------------------------------------------------------------------------

PAGE_TOKENS = 64


def run_paged(db, reps: int = 64):
    """Decode-call time over paged copies of the benchmark's caches (64-token
    pages in a seeded random order), once with every sequence at full length
    and once with seeded random lengths in [1, ctx]; layers visited in turn so
    each call reads its pages cold."""
    d, B, ctx = db.dims, db.B, db.ctx
    pps = (ctx + PAGE_TOKENS - 1) // PAGE_TOKENS
    g = torch.Generator().manual_seed(4242)
    layers = []
    for L in db.layers:
        table = torch.randperm(B * pps, generator=g).to(torch.int32).reshape(B, pps).contiguous()
        pc = T.new_paged_cache(d, B * pps, PAGE_TOKENS, table)
        t = torch.arange(ctx)
        for k in ("a_k", "b_k", "a_v", "b_v"):
            pool, dense = getattr(pc, k), getattr(L["cache"], k)
            for b in range(B):
                pool[table[b, t // PAGE_TOKENS].long().cuda(), (t % PAGE_TOKENS).cuda()] = dense[b, :ctx]
        layers.append(pc)
    full = torch.full((B,), ctx, dtype=torch.int32, device="cuda")
    ragged_cpu = torch.randint(1, ctx + 1, (B,), generator=g, dtype=torch.int32)
    ragged = ragged_cpu.cuda()
    e_tok = T.tpa_cache_elems_per_token(d)

    def timed(lens):
        for i in range(2 * LAYERS):
            L = db.layers[i % LAYERS]
            T.tpa_paged_decode_attn(d, L["q"], layers[i % LAYERS], lens, ctx, L["ws"], out=L["out"])
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for i in range(reps):
            L = db.layers[i % LAYERS]
            evs[i][0].record()
            T.tpa_paged_decode_attn(d, L["q"], layers[i % LAYERS], lens, ctx, L["ws"], out=L["out"])
            evs[i][1].record()
        torch.cuda.synchronize()
        return sum(a.elapsed_time(b) for a, b in evs) / reps

    full_ms = timed(full)
    ragged_ms = timed(ragged)
    full_bytes = B * ctx * e_tok * 2
    ragged_bytes = int(ragged_cpu.sum()) * e_tok * 2
    return {"page_tokens": PAGE_TOKENS, "pages": B * pps, "table": "seeded random permutation",
            "full_call_us": round(full_ms * 1e3, 2), "full_GBps": round(full_bytes / (full_ms * 1e-3) / 1e9, 1),
            "ragged_keys": int(ragged_cpu.sum()), "ragged_call_us": round(ragged_ms * 1e3, 2),
            "ragged_GBps": round(ragged_bytes / (ragged_ms * 1e-3) / 1e9, 1)}


def run_shared(db, reps: int = 64):
    """Decode-call time of the shared-basis variant on the benchmark's shapes:
    each layer's head factors (A_K, A_V of its dense cache) with seeded bases
    B_K, B_V common to every token; layers visited in turn.  Bytes per call:
    only the head factors, B*ctx*h*(R_K+R_V)*2; work: the per-key rotated
    products, h*R_K*d_h multiply-adds per key (run on the matrix cores as
    three bf16 products of hi/lo splits)."""
    d, B, ctx = db.dims, db.B, db.ctx
    s = db.wl.shape
    g = torch.Generator(device="cuda")
    g.manual_seed(4343)
    std = I.factor_std(s)
    layers = []
    for L in db.layers:
        b_k = (torch.randn(s.rank_k, s.head_dim, generator=g, device="cuda") * std).to(torch.bfloat16)
        b_v = (torch.randn(s.rank_v, s.head_dim, generator=g, device="cuda") * std).to(torch.bfloat16)
        sc = T.SharedCache(L["cache"].a_k, L["cache"].a_v, b_k, b_v)
        layers.append(sc)
    ws = torch.empty(T.tpa_shared_decode_workspace_bytes(d, B, ctx), dtype=torch.uint8, device="cuda")
    for i in range(2 * LAYERS):
        L = db.layers[i % LAYERS]
        T.tpa_shared_decode_attn(d, L["q"], layers[i % LAYERS], ctx, ws, out=L["out"])
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for i in range(reps):
        L = db.layers[i % LAYERS]
        evs[i][0].record()
        T.tpa_shared_decode_attn(d, L["q"], layers[i % LAYERS], ctx, ws, out=L["out"])
        evs[i][1].record()
    torch.cuda.synchronize()
    ms = sum(a.elapsed_time(b) for a, b in evs) / reps
    nbytes = B * ctx * s.n_heads * (s.rank_k + s.rank_v) * 2
    flop = 2.0 * B * ctx * s.n_heads * s.rank_k * s.head_dim
    return {"call_us": round(ms * 1e3, 2), "bytes_per_call": nbytes,
            "GBps": round(nbytes / (ms * 1e-3) / 1e9, 1), "hbm_frac": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
            "products_TFLOPs": round(flop / (ms * 1e-3) / 1e12, 2),
            "cache_bytes_per_token": s.n_heads * (s.rank_k + s.rank_v) * 2,
            "standard_cache_bytes_per_token": T.tpa_cache_elems_per_token(d) * 2}


def run_shared_long(reps: int = 20):
    """The shared-basis decode at the long-context decode workload's shape
    (8 sequences x 131072 cached keys + the new one, h 32, d_h 128, R 2): the
    head factors are seeded draws with the factors' spread, bases likewise."""
    wl = I.WORKLOADS["decode_b8_ctx128k"]
    d = dims_of(wl)
    s = wl.shape
    B, ctx = wl.batch, wl.seq + 1
    g = torch.Generator(device="cuda")
    g.manual_seed(4747)
    std = I.factor_std(s)
    rnd = lambda *shape: (torch.randn(*shape, generator=g, device="cuda") * std).to(torch.bfloat16)
    sc = T.SharedCache(rnd(B, ctx, s.n_heads, s.rank_k), rnd(B, ctx, s.n_heads, s.rank_v),
                       rnd(s.rank_k, s.head_dim), rnd(s.rank_v, s.head_dim))
    q = T.Factors(rnd(B, s.n_heads, s.rank_q), rnd(B, s.rank_q, s.head_dim), None, None, None, None)
    ws = torch.empty(T.tpa_shared_decode_workspace_bytes(d, B, ctx), dtype=torch.uint8, device="cuda")
    out = torch.empty(B, s.n_heads * s.head_dim, dtype=torch.bfloat16, device="cuda")
    for _ in range(3):
        T.tpa_shared_decode_attn(d, q, sc, ctx, ws, out=out)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for i in range(reps):
        evs[i][0].record()
        T.tpa_shared_decode_attn(d, q, sc, ctx, ws, out=out)
        evs[i][1].record()
    torch.cuda.synchronize()
    ms = sum(a.elapsed_time(b) for a, b in evs) / reps
    nbytes = B * ctx * s.n_heads * (s.rank_k + s.rank_v) * 2
    flop = 2.0 * B * ctx * s.n_heads * s.rank_k * s.head_dim
    return {"workload": wl.name, "batch": B, "context": ctx, "call_us": round(ms * 1e3, 2),
            "bytes_per_call": nbytes, "GBps": round(nbytes / (ms * 1e-3) / 1e9, 1),
            "hbm_frac": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
            "products_TFLOPs": round(flop / (ms * 1e-3) / 1e12, 2)}


# ---------------------------------------------------------------------------
# Prefill workload (reported alongside)
# ---------------------------------------------------------------------------

def run_prefill(reps: int = 5):
    wl = I.WORKLOADS["prefill_b4_s4k"]
    d = dims_of(wl)
    B, S = wl.batch, wl.seq
    g = torch.Generator(device="cuda")
    g.manual_seed(1003)
    x = torch.randn(B, S, d.d_model, generator=g, device="cuda").to(torch.bfloat16)
    w = I.weights(wl.shape, seed=1003, dtype="bf16")
    wp = T.pack_weights({k: v.cuda() for k, v in w.items()}, d.kv_only)
    cache = T.new_cache(d, B, S)
    f = T.new_factors(d, B, S)
    out = torch.empty(B, S, d.n_heads * d.head_dim, dtype=torch.bfloat16, device="cuda")
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    times = {"proj": [], "append": [], "attn": []}
    for r in range(reps + 1):
        ev[0].record()
        T.tpa_factor_proj(d, x, wp, f, start_pos=0)
        ev[1].record()
        T.tpa_cache_append(d, cache, f, 0)
        ev[2].record()
        T.tpa_prefill_attn(d, f, cache, 0, True, out=out)
        ev[3].record()
        torch.cuda.synchronize()
        if r:
            times["proj"].append(ev[0].elapsed_time(ev[1]))
            times["append"].append(ev[1].elapsed_time(ev[2]))
            times["attn"].append(ev[2].elapsed_time(ev[3]))
    med = {k: sorted(v)[len(v) // 2] for k, v in times.items()}
    n_out = T.tpa_packed_weight_rows(d)
    attn_flop = 4.0 * B * d.n_heads * d.head_dim * S * (S + 1) / 2
    proj_flop = 2.0 * B * S * d.d_model * n_out
    return {
        "workload": wl.name, "batch": B, "seq": S,
        "attn_ms": round(med["attn"], 4), "attn_tflops": round(attn_flop / med["attn"] / 1e9, 2),
        "attn_frac_bf16_peak": round(attn_flop / med["attn"] / 1e9 / BF16_PEAK_TFLOPS, 4),
        "proj_ms": round(med["proj"], 4), "proj_tflops": round(proj_flop / med["proj"] / 1e9, 2),
        "append_ms": round(med["append"], 4),
        "step_ms": round(med["proj"] + med["append"] + med["attn"], 4),
    }


def run_prefill_backward(reps: int = 3):
    """Backward of the prefill attention at prefill_b4_s4k: gradients of all six
    factor tensors from a seeded dO.  Algorithmic work: the usual 2.5x the
    forward's matrix-product flops (dV, dP, dQ, dK and the score recomputation)."""
    wl = I.WORKLOADS["prefill_b4_s4k"]
    d = dims_of(wl)
    B, S = wl.batch, wl.seq
    h, dh = d.n_heads, d.head_dim
    g = torch.Generator(device="cuda")
    g.manual_seed(1004)
    x = torch.randn(B, S, d.d_model, generator=g, device="cuda").to(torch.bfloat16)
    w = I.weights(wl.shape, seed=1004, dtype="bf16")
    wp = T.pack_weights({k: v.cuda() for k, v in w.items()}, d.kv_only)
    cache = T.new_cache(d, B, S)
    f = T.new_factors(d, B, S)
    T.tpa_factor_proj(d, x, wp, f, start_pos=0)
    T.tpa_cache_append(d, cache, f, 0)
    dout = torch.randn(B, S, h * dh, generator=g, device="cuda").to(torch.bfloat16)
    f32 = lambda *s: torch.zeros(*s, dtype=torch.float32, device="cuda")
    dq = T.Factors(f32(B, S, h, d.rank_q), f32(B, S, d.rank_q, dh), None, None, None, None)
    dkv = T.Cache(f32(B, S, h, d.rank_k), f32(B, S, d.rank_k, dh), f32(B, S, h, d.rank_v), f32(B, S, d.rank_v, dh))
    ws = torch.empty(T.tpa_prefill_backward_workspace_bytes(d, B, S, 0), dtype=torch.uint8, device="cuda")
    T.tpa_prefill_attn_backward(d, f, cache, 0, True, dout, dq, dkv, ws)
    torch.cuda.synchronize()
    times = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        T.tpa_prefill_attn_backward(d, f, cache, 0, True, dout, dq, dkv, ws)
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    ms = sorted(times)[len(times) // 2]
    flop = 2.5 * 4.0 * B * h * dh * S * (S + 1) / 2
    return {"workload": wl.name, "ms": round(ms, 3), "tflops": round(flop / ms / 1e9, 2),
            "frac_bf16_peak": round(flop / ms / 1e9 / BF16_PEAK_TFLOPS, 4),
            "kernels": "matrix cores (bf16 MFMA): statistics, k^/v^ rebuild, dK/dV, dQ; factor gradients"}


# ---------------------------------------------------------------------------
# CPU baseline: the fp64 oracle on a bounded sample of the decode step
# ---------------------------------------------------------------------------

def cpu_baseline(wl: I.Workload, budget_s: float = 12.0):
    import numpy as np
    from threadpoolctl import threadpool_limits

    import oracle.tpa_oracle as O
    s = wl.shape
    od = O.Dims(s.d_model, s.n_heads, s.head_dim, s.rank_q, s.rank_k, s.rank_v, s.rope_base)
    B, ctx = wl.batch, wl.seq + 1
    kv = I.factors(s, B, wl.seq, seed=2002, dtype="bf16", with_query=False)
    cache = O.cache_new(od, B, ctx)
    for k in ("a_k", "b_k", "a_v", "b_v"):
        cache[k][:, :wl.seq] = I.to_f64(kv[k])
    w = {k: I.to_f64(v) for k, v in I.weights(s, seed=2002, dtype="bf16").items()}
    x_new = I.to_f64(I.activations(B, 1, s.d_model, seed=2002, dtype="bf16", stream="x_new"))
    steps, t_used = 0, 0.0
    with threadpool_limits(limits=1):
        while t_used < budget_s and steps < 100:
            t0 = time.perf_counter()
            f = O.rotate_factors(O.project(x_new, w, od), ctx - 1, od)
            O.cache_append(cache, f, ctx - 1)
            O.decode(f, cache, od, B, ctx)
            t_used += time.perf_counter() - t0
            steps += 1
    return {"value": round(B * steps / t_used, 2), "unit": "tok/s", "cores": 1, "kind": "oracle",
            "sample": f"{steps} full decode steps of the same workload (batch {B}, {ctx} keys), fp64 numpy, "
                      f"{t_used:.1f} s, BLAS limited to one thread"}


def calibrate_copy(tokens: int = 26214, batch: int = 16):
    """A plain copy of known size through the cache-append kernel (a bit copy):
    batch * tokens * 640 bytes read and the same written.  Used to scale the
    HBM byte counters of the profiler."""
    wl = I.WORKLOADS["decode_b16_ctx4k"]
    d = dims_of(wl)
    src = T.new_factors(d, batch, tokens)
    for t in (src.a_k, src.b_k, src.a_v, src.b_v):
        t.fill_(1.0)
    cache = T.new_cache(d, batch, tokens)
    for _ in range(5):
        T.tpa_cache_append(d, cache, src, 0)
    torch.cuda.synchronize()
    nbytes = batch * tokens * T.tpa_cache_elems_per_token(d) * 2
    print(json.dumps({"calibration": "tpa_cache_append bit copy", "bytes_read": nbytes, "bytes_written": nbytes,
                      "launches": 5}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain copy of known size (for profiler byte counters)")
    ap.add_argument("--shared-long-only", action="store_true",
                    help="only time the shared-basis decode at the long-context shape (for a kernel trace of it)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the multi-GPU layout is a design "
              f"note, not a measured path.", file=sys.stderr)
        sys.exit(2)
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.shared_long_only:
        print(json.dumps({"shared_decode_long": run_shared_long()}), flush=True)
        return

    db, wl, ms_per_step, eager_ms, dec_call_ms, dec_med_ms, graph_steps = run_decode(args)
    bytes_per_call = db.cache_bytes()
    achieved = bytes_per_call / (dec_call_ms * 1e-3) / 1e9
    traffic = load_traffic(["decode_mfma.hip", "decode.hip"])
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic,
                "kernel": "tpa_decode_attn (main pass + combine)", "bytes_per_launch": bytes_per_call,
                "avg_us": round(dec_call_ms * 1e3, 2), "timing": "HIP graph of back-to-back decode calls, events",
                "eager_call_median_us": round(dec_med_ms * 1e3, 2)}
    result = {
        "metric": METRIC,
        "value": round(db.B / (ms_per_step * 1e-3), 1),
        "unit": "tok/s",
        "n_gpus": 1, "steps": graph_steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": wl.name, "batch": db.B, "context": db.ctx, "d_model": wl.shape.d_model,
                   "heads": wl.shape.n_heads, "head_dim": wl.shape.head_dim, "rank_q": wl.shape.rank_q,
                   "rank_k": wl.shape.rank_k, "rank_v": wl.shape.rank_v, "layers_cycled": LAYERS},
        "roofline": roofline,
        "launch": {"hip_graph_ms_per_step": round(ms_per_step, 5), "eager_ms_per_step": round(eager_ms, 5)},
    }
    log("[bench] paged decode")
    result["paged_decode"] = run_paged(db)
    log("[bench] shared-basis decode")
    result["shared_decode"] = run_shared(db)
    log("[bench] shared-basis decode, long context")
    result["shared_decode_long"] = run_shared_long()
    if not args.no_prefill:
        log("[bench] prefill workload")
        result["prefill"] = run_prefill()
        log("[bench] prefill backward")
        result["prefill_backward"] = run_prefill_backward()
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle)")
        result["cpu_baseline"] = cpu_baseline(wl)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
