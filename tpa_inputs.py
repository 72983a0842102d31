"""Seeded synthetic inputs for Tensor Product Attention (TPA) workloads.

This module only draws random numbers and names the workload shapes.  It holds
none of the method's arithmetic: no projection, no rotary embedding, no
attention.  Both the fp64 oracle and the HIP path are fed from here, so the
two sides see bit-identical inputs.

Every tensor is drawn in float32 from its own torch CPU generator, seeded from
``(seed, stream id)``, and is rounded to bfloat16 (round-to-nearest-even, the
torch cast) when the workload runs in bf16.  The oracle receives the rounded
values widened to float64.

The distributions follow the workload definitions: activations x ~ N(0, 1),
every factor weight matrix ~ N(0, 0.02^2).  Tests that feed the attention
kernels factors directly draw them from N(0, sigma^2) with
sigma = 0.02 * sqrt(d_model), the spread a factor has when it is produced from
such x through such weights.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional

import torch


@dataclasses.dataclass(frozen=True)
class Shape:
    """Model-side dimensions of one TPA layer (the page's ModelArgs fields).

    rank_q == 0 selects the TPA-KVonly variant: Q is a plain per-head linear
    projection and only K and V are factorised.
    """

    d_model: int
    n_heads: int
    head_dim: int
    rank_q: int
    rank_k: int
    rank_v: int
    rope_base: float = 10000.0

    @property
    def kv_only(self) -> bool:
        return self.rank_q == 0


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    shape: Shape
    dtype: str            # "f32" or "bf16"
    batch: int
    seq: int              # prefill length, or cached context before the new token
    decode_steps: int = 0
    kind: str = "decode"  # "decode", "prefill" or "prefill+decode"


# The five workloads (their shapes, ranks and dtypes); the first is small
# enough for the oracle to finish in seconds.
WORKLOADS: Dict[str, Workload] = {
    "tiny_fp32": Workload("tiny_fp32", Shape(256, 4, 64, 6, 2, 2), "f32", 1, 64, 16, "prefill+decode"),
    "decode_b16_ctx4k": Workload("decode_b16_ctx4k", Shape(1024, 16, 64, 6, 2, 2), "bf16", 16, 4096, 1, "decode"),
    "prefill_b4_s4k": Workload("prefill_b4_s4k", Shape(1024, 16, 64, 6, 2, 2), "bf16", 4, 4096, 0, "prefill"),
    "decode_b8_ctx128k": Workload("decode_b8_ctx128k", Shape(4096, 32, 128, 6, 2, 2), "bf16", 8, 131072, 1, "decode"),
    "kvonly_b32_ctx16k": Workload("kvonly_b32_ctx16k", Shape(1536, 24, 64, 0, 4, 4), "bf16", 32, 16384, 1, "prefill+decode"),
}

WEIGHT_STD = 0.02

# Generator stream ids: one stream per tensor, in a fixed order.
_STREAMS = {
    "x": 0, "w_a_q": 1, "w_b_q": 2, "w_a_k": 3, "w_b_k": 4, "w_a_v": 5, "w_b_v": 6,
    "w_q": 7, "x_new": 8,
    "f_a_q": 10, "f_b_q": 11, "f_a_k": 12, "f_b_k": 13, "f_a_v": 14, "f_b_v": 15, "f_q": 16,
    "basis_k": 20, "basis_v": 21,
}


def _gen(seed: int, stream: str, salt: int = 0) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed((int(seed) * 1_000_003 + _STREAMS[stream] * 7919 + salt) & 0x7FFF_FFFF_FFFF_FFFF)
    return g


def to_dtype(t: torch.Tensor, dtype: str) -> torch.Tensor:
    """Round a float32 tensor to the workload dtype (bf16: torch's RNE cast)."""
    if dtype == "f32":
        return t.float().contiguous()
    if dtype == "bf16":
        return t.to(torch.bfloat16).contiguous()
    raise ValueError(f"unknown dtype {dtype!r}")


def normal(shape, std: float, seed: int, stream: str, dtype: str = "f32", salt: int = 0) -> torch.Tensor:
    t = torch.randn(*shape, generator=_gen(seed, stream, salt), dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return to_dtype(t, dtype)


def activations(batch: int, seq: int, d_model: int, seed: int, dtype: str, stream: str = "x", salt: int = 0):
    """x ~ N(0, 1), shape [batch, seq, d_model]."""
    return normal((batch, seq, d_model), 1.0, seed, stream, dtype, salt)


def weights(shape: Shape, seed: int, dtype: str, std: float = WEIGHT_STD) -> Dict[str, torch.Tensor]:
    """The per-layer projection weights, nn.Linear layout [out_features, d_model].

    Keys: w_a_q [h*R_Q, d], w_b_q [R_Q*d_h, d] (or w_q [h*d_h, d] when rank_q == 0),
    w_a_k [h*R_K, d], w_b_k [R_K*d_h, d], w_a_v [h*R_V, d], w_b_v [R_V*d_h, d].
    """
    h, dh, d = shape.n_heads, shape.head_dim, shape.d_model
    out = {}
    if shape.kv_only:
        out["w_q"] = normal((h * dh, d), std, seed, "w_q", dtype)
    else:
        out["w_a_q"] = normal((h * shape.rank_q, d), std, seed, "w_a_q", dtype)
        out["w_b_q"] = normal((shape.rank_q * dh, d), std, seed, "w_b_q", dtype)
    out["w_a_k"] = normal((h * shape.rank_k, d), std, seed, "w_a_k", dtype)
    out["w_b_k"] = normal((shape.rank_k * dh, d), std, seed, "w_b_k", dtype)
    out["w_a_v"] = normal((h * shape.rank_v, d), std, seed, "w_a_v", dtype)
    out["w_b_v"] = normal((shape.rank_v * dh, d), std, seed, "w_b_v", dtype)
    return out


def factor_std(shape: Shape) -> float:
    return WEIGHT_STD * math.sqrt(shape.d_model)


def factors(shape: Shape, batch: int, seq: int, seed: int, dtype: str, std: Optional[float] = None,
            salt: int = 0, with_query: bool = True, v_std: Optional[float] = None) -> Dict[str, torch.Tensor]:
    """Directly drawn factor tensors, token-major, as a projection would lay them out.

    a_q [B,S,h,R_Q], b_q [B,S,R_Q,d_h] (KV-only: q [B,S,h,d_h]),
    a_k [B,S,h,R_K], b_k [B,S,R_K,d_h], a_v [B,S,h,R_V], b_v [B,S,R_V,d_h].
    The values are i.i.d. normal; "already rotated" is a statement about how they
    are used, and an i.i.d. isotropic draw has the same law before and after a rotation.
    v_std, when given, is the spread of the value factors alone (a_v, b_v): the
    query and key factors set how sharp the scores are, the value factors how
    large the outputs are, and the two can be chosen apart.
    """
    s = factor_std(shape) if std is None else std
    sv = s if v_std is None else v_std
    h, dh = shape.n_heads, shape.head_dim
    out = {}
    if with_query:
        if shape.kv_only:
            out["q"] = normal((batch, seq, h, dh), s, seed, "f_q", dtype, salt)
        else:
            out["a_q"] = normal((batch, seq, h, shape.rank_q), s, seed, "f_a_q", dtype, salt)
            out["b_q"] = normal((batch, seq, shape.rank_q, dh), s, seed, "f_b_q", dtype, salt)
    out["a_k"] = normal((batch, seq, h, shape.rank_k), s, seed, "f_a_k", dtype, salt)
    out["b_k"] = normal((batch, seq, shape.rank_k, dh), s, seed, "f_b_k", dtype, salt)
    out["a_v"] = normal((batch, seq, h, shape.rank_v), sv, seed, "f_a_v", dtype, salt)
    out["b_v"] = normal((batch, seq, shape.rank_v, dh), sv, seed, "f_b_v", dtype, salt)
    return out


def shared_basis(shape: Shape, seed: int, dtype: str, std: Optional[float] = None,
                 v_std: Optional[float] = None) -> Dict[str, torch.Tensor]:
    """Bases of the shared-basis variant, common to every token: b_k [R_K, d_h]
    (unrotated) and b_v [R_V, d_h], i.i.d. normal with the factors' spread
    (v_std, when given, for b_v alone, as in factors)."""
    s = factor_std(shape) if std is None else std
    sv = s if v_std is None else v_std
    return {"b_k": normal((shape.rank_k, shape.head_dim), s, seed, "basis_k", dtype),
            "b_v": normal((shape.rank_v, shape.head_dim), sv, seed, "basis_v", dtype)}


def to_f64(t: torch.Tensor):
    """Widen a (possibly bf16) torch tensor to a float64 numpy array, exactly."""
    return t.detach().to("cpu").double().numpy()
