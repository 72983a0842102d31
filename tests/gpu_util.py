"""Helpers for the GPU parity tests: tolerances, comparisons, input plumbing.

Tolerances: float32 mode max |err| <= 1e-4; bf16 mode max |err| <= 2e-2 and
relative L2 error <= 5e-3, both against the fp64 oracle on the same inputs, as
absolute bounds with no scaling.

A bf16 output of magnitude m is stored with an error of up to half its unit in
the last place: 2^-8 * 2^floor(log2 m), which is 7.8e-3 for m in [2, 4),
1.6e-2 for m in [4, 8) and 3.1e-2 from 8 on, where the 2e-2 bound can no longer
be met by any bf16 result.  assert_close refuses bf16 output cases whose
reference reaches 8.  The attention cases keep their outputs below 4, so
storage costs at most 7.8e-3 of the bound: the sharp cases keep their large
query and key factors (sharp scores exercise the online softmax's rescaling)
and draw the value factors at VALUE_STD_CAP at most.
"""
import sys

import numpy as np
import pytest
import torch

import oracle.tpa_oracle as O
import tpa_inputs as I

F32_MAX_ABS = 1e-4
BF16_MAX_ABS = 2e-2
BF16_REL_L2 = 5e-3
BF16_OUT_LIMIT = 8.0      # bf16 outputs below this: storage error <= 2^-6
VALUE_STD_CAP = 0.8


def value_std(std):
    """Spread of the value factors for a case drawn with factor spread std (None:
    the workload's own spread, whose outputs are small)."""
    return None if std is None else min(std, VALUE_STD_CAP)


def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


def announce(msg: str):
    """Name the case before any GPU work, flushed, so a failing run says where it was."""
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def errors(got, ref):
    g = got.detach().float().cpu().double().numpy() if isinstance(got, torch.Tensor) else np.asarray(got)
    r = np.asarray(ref, dtype=np.float64)
    assert g.shape == r.shape, f"shape {g.shape} vs {r.shape}"
    assert np.all(np.isfinite(g)), "non-finite output"
    diff = g - r
    max_abs = float(np.max(np.abs(diff))) if diff.size else 0.0
    denom = float(np.linalg.norm(r))
    rel = float(np.linalg.norm(diff)) / denom if denom > 0 else float(np.linalg.norm(diff))
    return max_abs, rel


def assert_close(got, ref, dtype: str, what: str, max_abs=None, rel_l2=None):
    max_abs_err, rel = errors(got, ref)
    ref_max = float(np.max(np.abs(np.asarray(ref, dtype=np.float64)))) if np.size(ref) else 0.0
    print(f"  {what}: max_abs={max_abs_err:.3e} rel_l2={rel:.3e} max|ref|={ref_max:.3g}", flush=True)
    if dtype == "f32":
        lim = F32_MAX_ABS if max_abs is None else max_abs
        assert max_abs_err <= lim, f"{what}: max abs err {max_abs_err:.3e} > {lim:.1e}"
    else:
        if isinstance(got, torch.Tensor) and got.dtype == torch.bfloat16:
            assert ref_max < BF16_OUT_LIMIT, (
                f"{what}: outputs reach {ref_max:.3g}; bf16 storage alone could exceed the 2e-2 bound")
        lim_a = BF16_MAX_ABS if max_abs is None else max_abs
        lim_r = BF16_REL_L2 if rel_l2 is None else rel_l2
        assert max_abs_err <= lim_a, f"{what}: max abs err {max_abs_err:.3e} > {lim_a:.1e}"
        assert rel <= lim_r, f"{what}: rel L2 err {rel:.3e} > {lim_r:.1e}"


def oracle_dims(d) -> O.Dims:
    return O.Dims(d.d_model, d.n_heads, d.head_dim, d.rank_q, d.rank_k, d.rank_v, d.rope_base)


def shape_of(d) -> I.Shape:
    return I.Shape(d.d_model, d.n_heads, d.head_dim, d.rank_q, d.rank_k, d.rank_v, d.rope_base)


def oracle_factors(f: dict) -> dict:
    return {k: I.to_f64(v) for k, v in f.items()}


def fill_cache(cache, kv: dict, lo: int = 0):
    """Copy drawn key/value factors [B, T, ...] into cache slots lo..lo+T-1 (test setup)."""
    B, T = kv["a_k"].shape[:2]
    for k in ("a_k", "b_k", "a_v", "b_v"):
        getattr(cache, k)[:B, lo:lo + T].copy_(kv[k].to(getattr(cache, k).device))


def oracle_cache(kv: dict, dims: O.Dims, max_batch: int, max_seq: int) -> dict:
    c = O.cache_new(dims, max_batch, max_seq)
    B, T = kv["a_k"].shape[:2]
    for k in ("a_k", "b_k", "a_v", "b_v"):
        c[k][:B, :T] = I.to_f64(kv[k])
    return c


def query_factors_gpu(T, dims, f: dict, squeeze: bool = False):
    """Build binding Factors for the query part of drawn factors (on the GPU)."""
    sq = (lambda t: t[:, 0]) if squeeze else (lambda t: t)
    if dims.kv_only:
        return T.Factors(None, sq(f["q"]).cuda().contiguous(), None, None, None, None)
    return T.Factors(sq(f["a_q"]).cuda().contiguous(), sq(f["b_q"]).cuda().contiguous(), None, None, None, None)


def oracle_query(f: dict, dims) -> dict:
    if dims.kv_only:
        return {"q": I.to_f64(f["q"])}
    return {"a_q": I.to_f64(f["a_q"]), "b_q": I.to_f64(f["b_q"])}
