"""Benchmark of the TPA hot path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline] [--only PART]

Headline: the long-context decode workload (batch 8, 131072 cached tokens plus
the new one, d_model 4096, 32 heads of 128, R_Q 6, R_K = R_V 2, bf16; a 1.34 GB
factor cache).  A step is one decode step of one TPA attention layer for the
whole batch: the factor projection of the new tokens with fused RoPE, whose
epilogue writes their K/V factors straight into cache slot 131072, then decode
attention over the 131073 keys (main pass + combine).  The cache is built
through the same projection from synthetic N(0,1) activations and N(0,0.02)
weights; at 1.34 GB it is five times the last-level cache, so every step reads
it from HBM.

Prints one JSON line.  `value` is decode throughput in tokens/s (batch / mean
step time over exactly K timed steps, HIP events on the launch stream, eager
launches: at ~0.27 ms a step the host stays ahead of the GPU).  `roofline`
covers the decode attention call, the dominant kernel pair: algorithmic
factor-cache bytes per call over its mean duration, timed with events around
each call on its stream over at least 100 calls.  `cpu_baseline` is the fp64
oracle on the host's cores (one thread per head) on a bounded sample of the same
decode step, plus a prefill sample.  Secondary keys: the KV-only workload at
full size (prefill of 32 x 16384 tokens: projection, append, attention; then
its decode step over 16385 keys), the batch-16 decode over 4097 keys, the
batch-4 prefill over 4096 tokens, the paged and shared-basis decodes, and the
prefill backward.
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
METRIC = "TPA decode tok/s + factor-cache HBM GB/s; prefill attention TFLOP/s"
ROOFLINE_REPS = 100
CPU_THREADS_MAX = 16


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


DECODE_SOURCES = ("decode_mfma.hip", "decode.hip")


def load_traffic(workload: str, sources=DECODE_SOURCES):
    """HBM bytes per decode call measured with rocprofv3 counters for this
    workload, if they were taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", "decode_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    entry = d.get("workloads", {}).get(workload)
    if not entry or d.get("source_digest") != source_digest(*sources):
        return None
    return entry.get("bytes_per_call")


def stats_ms(times_ms):
    """mean / median / p10 / p90 of a list of durations (ms)."""
    v = sorted(times_ms)
    n = len(v)

    def q(p):
        return v[min(n - 1, max(0, int(round(p * (n - 1)))))]

    return {"mean": sum(v) / n, "median": q(0.5), "p10": q(0.1), "p90": q(0.9), "n": n}


def us(st):
    return {k: (round(v * 1e3, 2) if k != "n" else v) for k, v in st.items()}


def time_calls(fn, reps: int, warm: int = 3):
    """Durations (ms) of `reps` calls of fn, each between two events on the
    current stream."""
    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    ev[0].record()
    for i in range(reps):
        fn()
        ev[i + 1].record()
    torch.cuda.synchronize()
    return [ev[i].elapsed_time(ev[i + 1]) for i in range(reps)]


# ---------------------------------------------------------------------------
# A decode layer: factor cache built through the projection, the new token's
# step (projection into slot ctx-1, decode over ctx keys)
# ---------------------------------------------------------------------------

class DecodeLayer:
    def __init__(self, wl: I.Workload, seed: int, chunk: int = 8192, x_ctx=None):
        self.wl, self.dims = wl, dims_of(wl)
        d = self.dims
        self.B, self.ctx = wl.batch, wl.seq + 1          # cached context plus the new token
        g = torch.Generator(device="cuda")
        g.manual_seed(seed)
        w = I.weights(wl.shape, seed=seed, dtype="bf16")
        self.wp = T.pack_weights({k: v.cuda() for k, v in w.items()}, d.kv_only)
        self.cache = T.new_cache(d, self.B, self.ctx)
        if x_ctx is None:
            for t0 in range(0, wl.seq, chunk):
                n = min(chunk, wl.seq - t0)
                x = torch.randn(self.B, n, d.d_model, generator=g, device="cuda").to(torch.bfloat16)
                self._project_into(x, t0)
                del x
        else:
            self._project_into(x_ctx, 0)
        self.x_new = torch.randn(self.B, 1, d.d_model, generator=g, device="cuda").to(torch.bfloat16)
        qf = T.new_factors(d, self.B, 1)
        slot = self.cache.slot_factors(self.ctx - 1)
        self.into = T.Factors(qf.a_q, qf.b_q, slot.a_k, slot.b_k, slot.a_v, slot.b_v, 0, self.ctx)
        self.q = T.Factors(qf.a_q[:, 0] if qf.a_q is not None else None, qf.b_q[:, 0], None, None, None, None)
        self.ws = T.new_workspace(d, self.B, self.ctx)
        self.out = torch.empty(self.B, d.n_heads * d.head_dim, dtype=torch.bfloat16, device="cuda")
        torch.cuda.synchronize()

    def _project_into(self, x, t0):
        d = self.dims
        qd = T.new_factors(d, self.B, x.shape[1])
        s = self.cache.slot_factors(t0)
        T.tpa_factor_proj(d, x, self.wp, T.Factors(qd.a_q, qd.b_q, s.a_k, s.b_k, s.a_v, s.b_v, 0, self.ctx),
                          start_pos=t0)
        del qd

    def proj(self):
        T.tpa_factor_proj(self.dims, self.x_new, self.wp, self.into, start_pos=self.ctx - 1)

    def attend(self):
        T.tpa_decode_attn(self.dims, self.q, self.cache, self.ctx, self.ws, out=self.out)

    def cache_bytes(self) -> int:
        return self.B * self.ctx * T.tpa_cache_elems_per_token(self.dims) * 2


def back_to_back_ms(fn, reps: int, warm: int = 3) -> float:
    """Mean duration (ms) of `reps` calls of fn issued back to back between two
    events on the current stream."""
    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(reps):
        fn()
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / reps


def call_stats(fn, reps: int):
    """Spread (ms) of single calls with an event around each (stats_ms), plus
    "avg": the mean over back-to-back calls between two events, which the
    rates use (an event between calls costs a few microseconds)."""
    st = stats_ms(time_calls(fn, reps))
    st["avg"] = back_to_back_ms(fn, reps)
    return st


def decode_roofline(layer: DecodeLayer, reps: int = ROOFLINE_REPS):
    """The decode call's average duration over `reps` back-to-back calls (the
    roofline's time), and the spread of single calls from a second pass with
    events around each call."""
    avg = back_to_back_ms(layer.attend, reps)
    st = stats_ms(time_calls(layer.attend, reps))
    nbytes = layer.cache_bytes()
    achieved = nbytes / (avg * 1e-3) / 1e9
    return achieved, st, nbytes, avg


def run_headline(args):
    """The long-context decode step, timed for exactly args.steps steps."""
    wl = I.WORKLOADS["decode_b8_ctx128k"]
    log(f"[bench] building the {wl.name} factor cache (8 x 131072 tokens through the projection)")
    L = DecodeLayer(wl, seed=1002)
    for _ in range(args.warmup):
        L.proj()
        L.attend()
    torch.cuda.synchronize()
    K = args.steps
    # the timed region: K whole steps between two events, nothing else on the
    # stream (an event recorded between kernels costs a few microseconds)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for k in range(K):
        L.proj()
        L.attend()
    end.record()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    log(f"[bench] {wl.name}: {K} steps in {total_ms:.3f} ms")
    # a second pass of K steps with events around each kernel group, for the
    # spread of the step and its split into projection and attention call
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    end2 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    for k in range(K):
        ev[k][0].record()
        L.proj()
        ev[k][1].record()
        L.attend()
    end2.record()
    torch.cuda.synchronize()
    step_ms = [ev[k][0].elapsed_time(ev[k + 1][0] if k + 1 < K else end2) for k in range(K)]
    call_ms = [ev[k][1].elapsed_time(ev[k + 1][0] if k + 1 < K else end2) for k in range(K)]
    proj_ms = [ev[k][0].elapsed_time(ev[k][1]) for k in range(K)]
    achieved, rst, nbytes, avg = decode_roofline(L)
    return L, wl, total_ms / K, stats_ms(step_ms), stats_ms(call_ms), stats_ms(proj_ms), achieved, rst, nbytes, avg


def rope_standalone(d, f, reps: int = 20) -> dict:
    """The standalone rotation (tpa_rope_b, in place) of the query dim factors
    (the plain queries in KV-only mode) and the key dim factors of a projection
    output: HBM-bound, each element read and written once.  The rotations
    change the values in f, which nothing times afterwards."""
    t_q = back_to_back_ms(lambda: T.tpa_rope_b(d, f.b_q, 0), reps)
    t_k = back_to_back_ms(lambda: T.tpa_rope_b(d, f.b_k, 0), reps)
    nbytes = 2 * (f.b_q.numel() + f.b_k.numel()) * f.b_k.element_size()
    gbps = nbytes / ((t_q + t_k) * 1e-3) / 1e9
    return {"rope_b_q_us": round(t_q * 1e3, 2), "rope_b_k_us": round(t_k * 1e3, 2),
            "rope_bytes": nbytes, "rope_GBps": round(gbps, 1), "rope_frac_hbm": round(gbps / HBM_PEAK_GBPS, 4),
            "rope_timing": "tpa_rope_b on the query and on the key dim factors, each averaged over back-to-back calls"}


# ---------------------------------------------------------------------------
# KV-only workload at full size: prefill of 32 x 16384 tokens, then a decode step
# ---------------------------------------------------------------------------

def run_kvonly(reps: int = 8, dec_reps: int = 100):
    wl = I.WORKLOADS["kvonly_b32_ctx16k"]
    d = dims_of(wl)
    B, S = wl.batch, wl.seq
    g = torch.Generator(device="cuda")
    g.manual_seed(1005)
    x = torch.randn(B, S, d.d_model, generator=g, device="cuda").to(torch.bfloat16)
    w = I.weights(wl.shape, seed=1005, dtype="bf16")
    wp = T.pack_weights({k: v.cuda() for k, v in w.items()}, d.kv_only)
    cache = T.new_cache(d, B, S + 1)
    f = T.new_factors(d, B, S)
    out = torch.empty(B, S, d.n_heads * d.head_dim, dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(T.tpa_prefill_workspace_bytes(d, B, S, 0), dtype=torch.uint8, device="cuda")
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(5)]
    times = {"proj": [], "append": [], "attn": [], "attn_no_ws": []}
    for r in range(reps + 1):
        ev[0].record()
        T.tpa_factor_proj(d, x, wp, f, start_pos=0)
        ev[1].record()
        T.tpa_cache_append(d, cache, f, 0)
        ev[2].record()
        T.tpa_prefill_attn_ws(d, f, cache, 0, ws, True, out=out)
        ev[3].record()
        T.tpa_prefill_attn(d, f, cache, 0, True, out=out)
        ev[4].record()
        torch.cuda.synchronize()
        if r:
            times["proj"].append(ev[0].elapsed_time(ev[1]))
            times["append"].append(ev[1].elapsed_time(ev[2]))
            times["attn"].append(ev[2].elapsed_time(ev[3]))
            times["attn_no_ws"].append(ev[3].elapsed_time(ev[4]))
    n_out = T.tpa_packed_weight_rows(d)
    attn_flop = 4.0 * B * d.n_heads * d.head_dim * S * (S + 1) / 2
    proj_flop = 2.0 * B * S * d.d_model * n_out
    app_bytes = 2.0 * B * S * T.tpa_cache_elems_per_token(d) * 2
    st = {k: stats_ms(v) for k, v in times.items()}
    pre = {
        "workload": wl.name, "batch": B, "seq": S, "reps": reps,
        "attn_ms": round(st["attn"]["mean"], 3), "attn_ms_p10_p90": [round(st["attn"]["p10"], 3), round(st["attn"]["p90"], 3)],
        "attn_tflops": round(attn_flop / st["attn"]["mean"] / 1e9, 1),
        "attn_frac_bf16_peak": round(attn_flop / st["attn"]["mean"] / 1e9 / BF16_PEAK_TFLOPS, 4),
        "attn_path": "tpa_prefill_attn_ws (K and V formed once into a workspace, then attended)",
        "workspace_bytes": ws.numel(),
        "attn_no_workspace_ms": round(st["attn_no_ws"]["mean"], 3),
        "attn_no_workspace_frac_bf16_peak": round(attn_flop / st["attn_no_ws"]["mean"] / 1e9 / BF16_PEAK_TFLOPS, 4),
        "proj_ms": round(st["proj"]["mean"], 4), "proj_tflops": round(proj_flop / st["proj"]["mean"] / 1e9, 1),
        "proj_frac_bf16_peak": round(proj_flop / st["proj"]["mean"] / 1e9 / BF16_PEAK_TFLOPS, 4),
        "append_ms": round(st["append"]["mean"], 4),
        "append_GBps": round(app_bytes / (st["append"]["mean"] * 1e-3) / 1e9, 1),
        "append_frac_hbm": round(app_bytes / (st["append"]["mean"] * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "attn_flop": attn_flop, "proj_flop": proj_flop, "append_bytes": app_bytes,
    }
    pre.update(rope_standalone(d, f))
    del f, out, ws
    torch.cuda.synchronize()
    # the decode step over the 16385 keys: the prefilled cache plus the new token
    L = DecodeLayer(wl, seed=1005, x_ctx=x)
    del x
    step_avg = back_to_back_ms(lambda: (L.proj(), L.attend()), dec_reps)
    step = stats_ms(time_calls(lambda: (L.proj(), L.attend()), dec_reps))
    achieved, rst, nbytes, avg = decode_roofline(L)
    dec = {"workload": wl.name, "batch": B, "context": L.ctx, "step_avg_us": round(step_avg * 1e3, 2),
           "tok_per_s": round(B / (step_avg * 1e-3), 1), "step_us": us(step),
           "call_avg_us": round(avg * 1e3, 2), "call_us": us(rst), "bytes_per_call": nbytes,
           "GBps": round(achieved, 1), "frac_hbm": round(achieved / HBM_PEAK_GBPS, 4),
           "traffic": load_traffic(wl.name),
           "timing": "averages of back-to-back steps / calls between two events; step_us and call_us: events "
                     "around each one (a second pass)"}
    return pre, dec


# ---------------------------------------------------------------------------
# The batch-16 decode over 4097 keys: eight layers visited in turn (336 MB of
# caches), the eight-layer step captured once as a HIP graph and replayed
# ---------------------------------------------------------------------------

LAYERS_B16 = 8


def run_decode_b16(reps: int = 50):
    wl = I.WORKLOADS["decode_b16_ctx4k"]
    g = torch.Generator(device="cuda")
    g.manual_seed(1002)
    d = dims_of(wl)
    x_ctx = torch.randn(wl.batch, wl.seq, d.d_model, generator=g, device="cuda").to(torch.bfloat16)
    layers = [DecodeLayer(wl, seed=1002 + 17 * k, x_ctx=x_ctx) for k in range(LAYERS_B16)]
    del x_ctx

    def capture(fn):
        graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            with torch.cuda.graph(graph, stream=side):
                fn()
        torch.cuda.current_stream().wait_stream(side)
        return graph

    step_graph = capture(lambda: [(L.proj(), L.attend()) for L in layers])
    call_graph = capture(lambda: [L.attend() for L in layers])
    step_avg = back_to_back_ms(step_graph.replay, reps) / LAYERS_B16
    call_avg = back_to_back_ms(call_graph.replay, reps) / LAYERS_B16
    step = stats_ms([t / LAYERS_B16 for t in time_calls(step_graph.replay, reps)])
    call = stats_ms([t / LAYERS_B16 for t in time_calls(call_graph.replay, reps)])
    eager = stats_ms(time_calls(layers[0].attend, reps))
    nbytes = layers[0].cache_bytes()
    gbps = nbytes / (call_avg * 1e-3) / 1e9
    return {"workload": wl.name, "batch": wl.batch, "context": wl.seq + 1, "layers_cycled": LAYERS_B16,
            "tok_per_s": round(wl.batch / (step_avg * 1e-3), 1), "step_avg_us": round(step_avg * 1e3, 2),
            "step_us": us(step), "call_avg_us": round(call_avg * 1e3, 2), "call_us": us(call),
            "timing": ("HIP graph of the eight layers' steps / calls: averages over back-to-back replays between "
                       "two events; step_us and call_us from a second pass with events around each replay"),
            "eager_call_us": us(eager), "bytes_per_call": nbytes, "GBps": round(gbps, 1),
            "frac_hbm": round(gbps / HBM_PEAK_GBPS, 4), "traffic": load_traffic(wl.name)}, layers


# ---------------------------------------------------------------------------
# Paged decode: the batch-16 caches moved into shuffled pages
# ---------------------------------------------------------------------------

PAGE_TOKENS = 64


def run_paged(layers, reps: int = 64):
    """Decode-call time over paged copies of the batch-16 caches (64-token pages
    in a seeded random order), once with every sequence at full length and once
    with seeded random lengths in [1, ctx]; layers visited in turn so each call
    reads its pages cold."""
    L0 = layers[0]
    d, B, ctx = L0.dims, L0.B, L0.ctx
    pps = (ctx + PAGE_TOKENS - 1) // PAGE_TOKENS
    g = torch.Generator().manual_seed(4242)
    pcs = []
    for L in layers:
        table = torch.randperm(B * pps, generator=g).to(torch.int32).reshape(B, pps).contiguous()
        pc = T.new_paged_cache(d, B * pps, PAGE_TOKENS, table)
        t = torch.arange(ctx)
        for k in ("a_k", "b_k", "a_v", "b_v"):
            pool, dense = getattr(pc, k), getattr(L.cache, k)
            for b in range(B):
                pool[table[b, t // PAGE_TOKENS].long().cuda(), (t % PAGE_TOKENS).cuda()] = dense[b, :ctx]
        pcs.append(pc)
    full = torch.full((B,), ctx, dtype=torch.int32, device="cuda")
    ragged_cpu = torch.randint(1, ctx + 1, (B,), generator=g, dtype=torch.int32)
    ragged = ragged_cpu.cuda()
    e_tok = T.tpa_cache_elems_per_token(d)

    def timed(lens):
        it = [0]

        def call():
            i = it[0] % len(layers)
            it[0] += 1
            L = layers[i]
            T.tpa_paged_decode_attn(d, L.q, pcs[i], lens, ctx, L.ws, out=L.out)
        for _ in range(2 * len(layers)):
            call()
        return call_stats(call, reps)

    full_st, ragged_st = timed(full), timed(ragged)
    full_bytes = B * ctx * e_tok * 2
    ragged_bytes = int(ragged_cpu.sum()) * e_tok * 2
    return {"page_tokens": PAGE_TOKENS, "pages": B * pps, "table": "seeded random permutation",
            "full_call_us": us(full_st), "full_GBps": round(full_bytes / (full_st["avg"] * 1e-3) / 1e9, 1),
            "ragged_keys": int(ragged_cpu.sum()), "ragged_call_us": us(ragged_st),
            "ragged_GBps": round(ragged_bytes / (ragged_st["avg"] * 1e-3) / 1e9, 1),
            "timing": "rates from avg: eager calls back to back between two events; the spread: an event around each"}


def run_shared(layers, reps: int = 64):
    """Decode-call time of the shared-basis variant on the batch-16 shapes: each
    layer's head factors (A_K, A_V of its dense cache) with seeded bases B_K, B_V
    common to every token.  Bytes per call: only the head factors,
    B*ctx*h*(R_K+R_V)*2; work: the per-key rotated products, h*R_K*d_h
    multiply-adds per key."""
    L0 = layers[0]
    d, B, ctx = L0.dims, L0.B, L0.ctx
    s = L0.wl.shape
    g = torch.Generator(device="cuda")
    g.manual_seed(4343)
    std = I.factor_std(s)
    scs = []
    for L in layers:
        b_k = (torch.randn(s.rank_k, s.head_dim, generator=g, device="cuda") * std).to(torch.bfloat16)
        b_v = (torch.randn(s.rank_v, s.head_dim, generator=g, device="cuda") * std).to(torch.bfloat16)
        scs.append(T.SharedCache(L.cache.a_k, L.cache.a_v, b_k, b_v))
    ws = torch.empty(T.tpa_shared_decode_workspace_bytes(d, B, ctx), dtype=torch.uint8, device="cuda")
    it = [0]

    def call():
        i = it[0] % len(layers)
        it[0] += 1
        T.tpa_shared_decode_attn(d, layers[i].q, scs[i], ctx, ws, out=layers[i].out)

    for _ in range(2 * len(layers)):
        call()
    st = call_stats(call, reps)
    nbytes = B * ctx * s.n_heads * (s.rank_k + s.rank_v) * 2
    flop = 2.0 * B * ctx * s.n_heads * s.rank_k * s.head_dim
    ms = st["avg"]
    return {"call_us": us(st), "bytes_per_call": nbytes,
            "GBps": round(nbytes / (ms * 1e-3) / 1e9, 1), "hbm_frac": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
            "products_TFLOPs": round(flop / (ms * 1e-3) / 1e12, 2),
            "cache_bytes_per_token": s.n_heads * (s.rank_k + s.rank_v) * 2,
            "standard_cache_bytes_per_token": T.tpa_cache_elems_per_token(d) * 2}


def run_shared_long(reps: int = 50):
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
    st = call_stats(lambda: T.tpa_shared_decode_attn(d, q, sc, ctx, ws, out=out), reps)
    ms = st["avg"]
    nbytes = B * ctx * s.n_heads * (s.rank_k + s.rank_v) * 2
    flop = 2.0 * B * ctx * s.n_heads * s.rank_k * s.head_dim
    return {"workload": wl.name, "batch": B, "context": ctx, "call_us": us(st),
            "bytes_per_call": nbytes, "GBps": round(nbytes / (ms * 1e-3) / 1e9, 1),
            "hbm_frac": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
            "products_TFLOPs": round(flop / (ms * 1e-3) / 1e12, 2)}


# ---------------------------------------------------------------------------
# The batch-4 prefill over 4096 tokens
# ---------------------------------------------------------------------------

def run_prefill(reps: int = 50):
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
    ws = torch.empty(T.tpa_prefill_workspace_bytes(d, B, S, 0), dtype=torch.uint8, device="cuda")
    st = {
        "proj": call_stats(lambda: T.tpa_factor_proj(d, x, wp, f, start_pos=0), reps),
        "append": call_stats(lambda: T.tpa_cache_append(d, cache, f, 0), reps),
        "attn": call_stats(lambda: T.tpa_prefill_attn_ws(d, f, cache, 0, ws, True, out=out), reps),
        "attn_no_ws": call_stats(lambda: T.tpa_prefill_attn(d, f, cache, 0, True, out=out), reps),
    }
    # the same projection writing the key/value factors straight into the cache
    # slots (kv_batch_stride = max_seq), so the step needs no separate append
    slot = cache.slot_factors(0)
    into = T.Factors(f.a_q, f.b_q, slot.a_k, slot.b_k, slot.a_v, slot.b_v, 0, slot.kv_batch_stride)
    st["proj_into_cache"] = call_stats(lambda: T.tpa_factor_proj(d, x, wp, into, start_pos=0), reps)
    n_out = T.tpa_packed_weight_rows(d)
    attn_flop = 4.0 * B * d.n_heads * d.head_dim * S * (S + 1) / 2
    proj_flop = 2.0 * B * S * d.d_model * n_out
    a, p, a0 = st["attn"]["avg"], st["proj"]["avg"], st["attn_no_ws"]["avg"]
    return {
        "workload": wl.name, "batch": B, "seq": S,
        "attn_us": us(st["attn"]), "attn_tflops": round(attn_flop / a / 1e9, 1),
        "attn_frac_bf16_peak": round(attn_flop / a / 1e9 / BF16_PEAK_TFLOPS, 4),
        "attn_path": "tpa_prefill_attn_ws (K and V formed once into a workspace, then attended)",
        "workspace_bytes": ws.numel(),
        "attn_no_workspace_us": us(st["attn_no_ws"]),
        "attn_no_workspace_frac_bf16_peak": round(attn_flop / a0 / 1e9 / BF16_PEAK_TFLOPS, 4),
        "proj_us": us(st["proj"]), "proj_tflops": round(proj_flop / p / 1e9, 1),
        "proj_frac_bf16_peak": round(proj_flop / p / 1e9 / BF16_PEAK_TFLOPS, 4),
        "append_us": us(st["append"]),
        "step_ms": round((a + p + st["append"]["avg"]), 4),
        "proj_into_cache_us": us(st["proj_into_cache"]),
        "step_fused_ms": round(a + st["proj_into_cache"]["avg"], 4),
        "step_fused": "projection into the cache slots, then the attention (no append launch)",
        **rope_standalone(d, f),
    }


def run_shared_prefill(reps: int = 50):
    """The prefill workload's shapes (4 x 4096 tokens, d_model 1024, h 16, d_h 64,
    R_Q 6, R 2) with a shared basis: the head-factor-only projection, the
    head-factor append and the attention over the shared-basis cache."""
    wl = I.WORKLOADS["prefill_b4_s4k"]
    d = dims_of(wl)
    s = wl.shape
    B, S = wl.batch, wl.seq
    g = torch.Generator(device="cuda")
    g.manual_seed(1013)
    x = torch.randn(B, S, d.d_model, generator=g, device="cuda").to(torch.bfloat16)
    w = I.weights(s, seed=1013, dtype="bf16")
    wp = T.pack_shared_weights({k: v.cuda() for k, v in w.items()}, d.kv_only)
    std = I.factor_std(s)
    rnd = lambda *shape: (torch.randn(*shape, generator=g, device="cuda") * std).to(torch.bfloat16)
    cache = T.new_shared_cache(d, B, S, rnd(s.rank_k, s.head_dim), rnd(s.rank_v, s.head_dim))
    f = T.new_factors(d, B, S)
    f = T.Factors(f.a_q, f.b_q, f.a_k, None, f.a_v, None)
    out = torch.empty(B, S, d.n_heads * d.head_dim, dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(T.tpa_prefill_workspace_bytes(d, B, S, 0), dtype=torch.uint8, device="cuda")
    T.tpa_shared_factor_proj(d, x, wp, f, start_pos=0)
    st = {
        "proj": call_stats(lambda: T.tpa_shared_factor_proj(d, x, wp, f, start_pos=0), reps),
        "append": call_stats(lambda: T.tpa_shared_cache_append(d, cache, f, 0), reps),
        "attn": call_stats(lambda: T.tpa_shared_prefill_attn_ws(d, f, cache, 0, ws, True, out=out), reps),
        "attn_no_ws": call_stats(lambda: T.tpa_shared_prefill_attn(d, f, cache, 0, True, out=out), reps),
    }
    attn_flop = 4.0 * B * d.n_heads * d.head_dim * S * (S + 1) / 2
    proj_flop = 2.0 * B * S * d.d_model * T.tpa_shared_packed_weight_rows(d)
    a, p = st["attn"]["avg"], st["proj"]["avg"]
    return {
        "workload": wl.name + " (shared basis)", "batch": B, "seq": S,
        "attn_us": us(st["attn"]), "attn_tflops": round(attn_flop / a / 1e9, 1),
        "attn_frac_bf16_peak": round(attn_flop / a / 1e9 / BF16_PEAK_TFLOPS, 4),
        "attn_path": "tpa_shared_prefill_attn_ws (keys rotated and formed once into a workspace, then attended)",
        "attn_no_workspace_us": us(st["attn_no_ws"]),
        "attn_no_workspace_frac_bf16_peak": round(attn_flop / st["attn_no_ws"]["avg"] / 1e9 / BF16_PEAK_TFLOPS, 4),
        "proj_us": us(st["proj"]), "proj_tflops": round(proj_flop / p / 1e9, 1),
        "proj_frac_bf16_peak": round(proj_flop / p / 1e9 / BF16_PEAK_TFLOPS, 4),
        "append_us": us(st["append"]),
        "step_ms": round((a + p + st["append"]["avg"]), 4),
    }


def run_prefill_backward(reps: int = 5):
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
    st = stats_ms(time_calls(lambda: T.tpa_prefill_attn_backward(d, f, cache, 0, True, dout, dq, dkv, ws), reps,
                             warm=1))
    ms = st["mean"]
    flop = 2.5 * 4.0 * B * h * dh * S * (S + 1) / 2
    return {"workload": wl.name, "ms": round(ms, 3), "tflops": round(flop / ms / 1e9, 1),
            "frac_bf16_peak": round(flop / ms / 1e9 / BF16_PEAK_TFLOPS, 4),
            "kernels": "matrix cores (bf16 MFMA): statistics, k^/v^ rebuild, dK/dV, dQ; factor gradients"}


# ---------------------------------------------------------------------------
# CPU baseline: the fp64 oracle on the host's cores, one head per thread
# ---------------------------------------------------------------------------

def cpu_threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(CPU_THREADS_MAX, n))


def _one_head(od, fq, cache, hh):
    """The oracle's own inputs restricted to head hh (heads are independent):
    a one-head problem with the same dim factors."""
    import oracle.tpa_oracle as O
    od1 = O.Dims(od.d_model, 1, od.head_dim, od.rank_q, od.rank_k, od.rank_v, od.rope_base)
    if od.kv_only:
        q1 = {"q": fq["q"][:, :, hh:hh + 1]}
    else:
        q1 = {"a_q": fq["a_q"][:, :, hh:hh + 1], "b_q": fq["b_q"]}
    c1 = {"a_k": cache["a_k"][:, :, hh:hh + 1], "b_k": cache["b_k"],
          "a_v": cache["a_v"][:, :, hh:hh + 1], "b_v": cache["b_v"]}
    return od1, q1, c1


def cpu_baseline():
    """The oracle, unchanged, on bounded samples of two workloads, run as
    one-head sub-problems on a thread pool (numpy releases the interpreter lock
    in its array operations; BLAS is held to one thread per worker).

    decode: the long-context decode step for all 8 sequences (the new token's
    projection, rotation and cache write, then attention over 131073 keys,
    every head), one sequence after another, so tok/s = 8 / time.  prefill:
    2048 seeded query rows of one of the 32
    sequences of the KV-only prefill (16384 keys, every head), rated by the
    algorithmic flops of those rows (4 * d_h * (p + 1) per row and head)."""
    import concurrent.futures as cf

    import numpy as np
    from threadpoolctl import threadpool_limits

    import oracle.tpa_oracle as O
    n_thr = cpu_threads()
    res = {}
    with threadpool_limits(limits=1):
        # ---- decode: the whole step of the batch, one sequence after another
        wl = I.WORKLOADS["decode_b8_ctx128k"]
        s = wl.shape
        od = O.Dims(s.d_model, s.n_heads, s.head_dim, s.rank_q, s.rank_k, s.rank_v, s.rope_base)
        ctx = wl.seq + 1
        w = {k: I.to_f64(v) for k, v in I.weights(s, seed=2002, dtype="bf16").items()}
        t_dec = 0.0
        for b in range(wl.batch):
            kv = I.factors(s, 1, wl.seq, seed=2002, dtype="bf16", with_query=False, salt=b)
            cache = O.cache_new(od, 1, ctx)
            for k in ("a_k", "b_k", "a_v", "b_v"):
                cache[k][:, :wl.seq] = I.to_f64(kv[k])
            del kv
            x_new = I.to_f64(I.activations(1, 1, s.d_model, seed=2002, dtype="bf16", stream="x_new", salt=b))
            t0 = time.perf_counter()
            f = O.rotate_factors(O.project(x_new, w, od), ctx - 1, od)
            O.cache_append(cache, f, ctx - 1)

            def dec_head(hh):
                od1, q1, c1 = _one_head(od, f, cache, hh)
                return O.decode(q1, c1, od1, 1, ctx)

            with cf.ThreadPoolExecutor(n_thr) as ex:
                outs = list(ex.map(dec_head, range(s.n_heads)))
            t_dec += time.perf_counter() - t0
            assert all(np.all(np.isfinite(o)) for o in outs)
            del cache, outs
        nbytes = wl.batch * ctx * (s.n_heads + s.head_dim) * (s.rank_k + s.rank_v) * 2
        res["value"] = round(wl.batch / t_dec, 3)
        res["unit"] = "tok/s"
        res["cores"] = n_thr
        res["kind"] = "oracle"
        res["GBps_equivalent"] = round(nbytes / t_dec / 1e9, 4)
        res["sample"] = (f"decode_b8_ctx128k: one whole decode step of the 8 sequences (projection of the new "
                         f"token, rotation, cache write, attention over {ctx} keys, all {s.n_heads} heads), fp64 "
                         f"numpy, one head per thread on {n_thr} threads, {t_dec:.1f} s of timed work (cache "
                         f"draws excluded)")
        # ---- prefill sample
        wl = I.WORKLOADS["kvonly_b32_ctx16k"]
        s = wl.shape
        od = O.Dims(s.d_model, s.n_heads, s.head_dim, s.rank_q, s.rank_k, s.rank_v, s.rope_base)
        S = wl.seq
        kv = I.factors(s, 1, S, seed=2003, dtype="bf16")
        cache = O.cache_new(od, 1, S)
        for k in ("a_k", "b_k", "a_v", "b_v"):
            cache[k][:, :S] = I.to_f64(kv[k])
        fq = {"q": I.to_f64(kv["q"])}
        rows = np.sort(np.random.default_rng(2003).choice(S, 2048, replace=False))
        t0 = time.perf_counter()

        def pre_head(hh):
            od1, q1, c1 = _one_head(od, fq, cache, hh)
            return O.prefill(q1, c1, od1, 1, S, 0, True, rows=rows)

        with cf.ThreadPoolExecutor(n_thr) as ex:
            outs = list(ex.map(pre_head, range(s.n_heads)))
        t_pre = time.perf_counter() - t0
        assert all(np.all(np.isfinite(o[:, rows])) for o in outs)
        flop = float(sum(4.0 * s.head_dim * (int(p) + 1) for p in rows)) * s.n_heads
        res["prefill"] = {"tflops": round(flop / t_pre / 1e12, 6), "unit": "TFLOP/s", "seconds": round(t_pre, 2),
                          "sample": f"kvonly_b32_ctx16k: 2048 seeded query rows of 1 of 32 sequences, all "
                                    f"{s.n_heads} heads, causal over up to {S} keys; rate of those rows' "
                                    f"algorithmic flops"}
        del cache, kv, outs
    # ---- projection sample: the oracle's six products are matrix products, so
    #      here the BLAS library takes all the threads
    wl = I.WORKLOADS["kvonly_b32_ctx16k"]
    s = wl.shape
    od = O.Dims(s.d_model, s.n_heads, s.head_dim, s.rank_q, s.rank_k, s.rank_v, s.rope_base)
    n_tok = 32768
    x = I.to_f64(I.activations(1, n_tok, s.d_model, seed=2004, dtype="bf16"))
    w = {k: I.to_f64(v) for k, v in I.weights(s, seed=2004, dtype="bf16").items()}
    n_out = sum(v.shape[0] for v in w.values())
    with threadpool_limits(limits=n_thr):
        O.project(x[:, :64], w, od)   # (warm the library)
        t0 = time.perf_counter()
        f = O.project(x, w, od)
        t_proj = time.perf_counter() - t0
    assert all(np.all(np.isfinite(v)) for v in f.values())
    res["projection"] = {"tflops": round(2.0 * n_tok * s.d_model * n_out / t_proj / 1e12, 5), "unit": "TFLOP/s",
                         "seconds": round(t_proj, 3),
                         "sample": f"kvonly_b32_ctx16k: {n_tok} of the 524288 tokens through the {n_out} x "
                                   f"{s.d_model} packed projection (fp64 matrix products, BLAS on {n_thr} threads)"}
    return res


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


PARTS = ("headline", "kvonly", "b16", "prefill", "backward", "shared_long", "shared_prefill")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", choices=PARTS, default=None,
                    help="run one part alone and print its JSON (for profiler runs)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain copy of known size (for profiler byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the multi-GPU layout is a design "
              f"note, not a measured path.", file=sys.stderr)
        sys.exit(2)
    if args.steps < 1 or args.warmup < 0:
        print("--steps must be >= 1 and --warmup >= 0", file=sys.stderr)
        sys.exit(2)
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.only and args.only != "headline":
        fn = {"kvonly": lambda: dict(zip(("prefill", "decode"), run_kvonly())),
              "b16": lambda: run_decode_b16()[0], "prefill": run_prefill,
              "backward": run_prefill_backward, "shared_long": run_shared_long,
              "shared_prefill": run_shared_prefill}[args.only]
        print(json.dumps({args.only: fn()}), flush=True)
        return

    L, wl, ms_per_step, step_st, call_st, proj_st, achieved, rst, nbytes, avg = run_headline(args)
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": load_traffic(wl.name),
                "kernel": "tpa_decode_attn (decode_mfma_kernel main pass + decode_combine_kernel)",
                "bytes_per_launch": nbytes, "avg_us": round(avg * 1e3, 2), "call_us": us(rst),
                "timing": (f"avg_us: {rst['n']} eager decode calls back to back between two events on the launch "
                           f"stream; call_us: a second pass with events around each call"),
                "second_pass_call_us": us(call_st)}
    result = {
        "metric": METRIC,
        "value": round(L.B / (ms_per_step * 1e-3), 1),
        "unit": "tok/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": wl.name, "batch": L.B, "context": L.ctx, "d_model": wl.shape.d_model,
                   "heads": wl.shape.n_heads, "head_dim": wl.shape.head_dim, "rank_q": wl.shape.rank_q,
                   "rank_k": wl.shape.rank_k, "rank_v": wl.shape.rank_v,
                   "cache_bytes": nbytes},
        "roofline": roofline,
        "step_us": us(step_st), "proj_us": us(proj_st),
        "step_timing": ("value and ms_per_step: two events around the K timed steps; step_us, proj_us and "
                        "roofline.second_pass_call_us: a second pass of K steps with events around each kernel "
                        "group (each such event adds a few microseconds)"),
    }
    del L
    torch.cuda.synchronize()
    if args.only == "headline":
        print(json.dumps(result), flush=True)
        return
    log("[bench] KV-only workload at full size: prefill, then decode")
    result["kvonly_b32_ctx16k"] = dict(zip(("prefill", "decode"), run_kvonly()))
    log("[bench] batch-16 decode over 4097 keys")
    result["decode_b16_ctx4k"], layers = run_decode_b16()
    log("[bench] paged decode")
    result["paged_decode"] = run_paged(layers)
    log("[bench] shared-basis decode")
    result["shared_decode"] = run_shared(layers)
    del layers
    log("[bench] shared-basis decode, long context")
    result["shared_decode_long"] = run_shared_long()
    log("[bench] prefill workload")
    result["prefill"] = run_prefill()
    log("[bench] shared-basis prefill")
    result["shared_prefill"] = run_shared_prefill()
    log("[bench] prefill backward")
    result["prefill_backward"] = run_prefill_backward()
    if not args.no_cpu_baseline:
        log(f"[bench] cpu baseline (oracle, {cpu_threads()} threads)")
        result["cpu_baseline"] = cpu_baseline()
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
