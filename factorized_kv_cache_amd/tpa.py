"""Python binding of libtpa (ctypes): argument marshalling only.

Every function has the name of the C entry point it calls and passes torch
tensors' device pointers and the current HIP stream; all arithmetic runs in
the library's HIP kernels.  The library must have been built
(``python -m factorized_kv_cache_amd.build``); importing this module without it
raises, there is no fallback.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Optional

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libtpa.so")

TPA_F32, TPA_BF16 = 0, 1
_STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported", 3: "cache capacity exceeded",
           4: "workspace too small", 5: "HIP error"}


class TPAError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{_STATUS.get(status, status)}: {msg}")
        self.status = status


class tpa_dims(ctypes.Structure):
    _fields_ = [("d_model", ctypes.c_int32), ("n_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("rank_q", ctypes.c_int32), ("rank_k", ctypes.c_int32), ("rank_v", ctypes.c_int32),
                ("rope_base", ctypes.c_double), ("dtype", ctypes.c_int32)]


class tpa_cache(ctypes.Structure):
    _fields_ = [("a_k", ctypes.c_void_p), ("b_k", ctypes.c_void_p), ("a_v", ctypes.c_void_p),
                ("b_v", ctypes.c_void_p), ("max_batch", ctypes.c_int64), ("max_seq", ctypes.c_int64)]


class tpa_paged_cache(ctypes.Structure):
    _fields_ = [("a_k", ctypes.c_void_p), ("b_k", ctypes.c_void_p), ("a_v", ctypes.c_void_p),
                ("b_v", ctypes.c_void_p), ("block_table", ctypes.c_void_p), ("n_pages", ctypes.c_int64),
                ("page_tokens", ctypes.c_int64), ("max_pages", ctypes.c_int64), ("max_batch", ctypes.c_int64)]


class tpa_shared_cache(ctypes.Structure):
    _fields_ = [("a_k", ctypes.c_void_p), ("a_v", ctypes.c_void_p), ("b_k", ctypes.c_void_p),
                ("b_v", ctypes.c_void_p), ("max_batch", ctypes.c_int64), ("max_seq", ctypes.c_int64)]


class tpa_factors(ctypes.Structure):
    _fields_ = [("a_q", ctypes.c_void_p), ("b_q", ctypes.c_void_p), ("a_k", ctypes.c_void_p),
                ("b_k", ctypes.c_void_p), ("a_v", ctypes.c_void_p), ("b_v", ctypes.c_void_p),
                ("q_batch_stride", ctypes.c_int64), ("kv_batch_stride", ctypes.c_int64)]


def _load():
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is not built; run `python -m factorized_kv_cache_amd.build`")
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.POINTER
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    sig = {
        "tpa_packed_weight_rows": (i64, [P(tpa_dims)]),
        "tpa_cache_elems_per_token": (i64, [P(tpa_dims)]),
        "tpa_factor_proj": (ctypes.c_int, [P(tpa_dims), vp, i64, i64, i64, vp, i32, P(tpa_factors), vp]),
        "tpa_rope_b": (ctypes.c_int, [P(tpa_dims), vp, i64, i64, i32, i64, vp]),
        "tpa_cache_append": (ctypes.c_int, [P(tpa_dims), P(tpa_cache), P(tpa_factors), i64, i64, i64, vp]),
        "tpa_prefill_attn": (ctypes.c_int, [P(tpa_dims), P(tpa_factors), P(tpa_cache), i64, i64, i64, i32, vp, vp]),
        "tpa_prefill_workspace_bytes": (ctypes.c_size_t, [P(tpa_dims), i64, i64, i64]),
        "tpa_prefill_attn_ws": (ctypes.c_int, [P(tpa_dims), P(tpa_factors), P(tpa_cache), i64, i64, i64, i32, vp,
                                               vp, ctypes.c_size_t, vp]),
        "tpa_decode_workspace_bytes": (ctypes.c_size_t, [P(tpa_dims), i64, i64]),
        "tpa_decode_attn": (ctypes.c_int, [P(tpa_dims), P(tpa_factors), P(tpa_cache), i64, i64, vp, vp,
                                           ctypes.c_size_t, vp]),
        "tpa_decode_noalloc_max_bytes": (ctypes.c_size_t, []),
        "tpa_decode_attn_noalloc": (ctypes.c_int, [P(tpa_dims), P(tpa_factors), P(tpa_cache), i64, i64, vp, vp]),
        "tpa_prefill_backward_workspace_bytes": (ctypes.c_size_t, [P(tpa_dims), i64, i64, i64]),
        "tpa_prefill_attn_backward": (ctypes.c_int, [P(tpa_dims), P(tpa_factors), P(tpa_cache), i64, i64, i64, i32,
                                                     vp, P(tpa_factors), P(tpa_cache), vp, ctypes.c_size_t, vp]),
        "tpa_rope_b_backward": (ctypes.c_int, [P(tpa_dims), vp, i64, i64, i32, i64, vp]),
        "tpa_paged_cache_append": (ctypes.c_int, [P(tpa_dims), P(tpa_paged_cache), P(tpa_factors), i64, i64, vp,
                                                  vp]),
        "tpa_paged_decode_workspace_bytes": (ctypes.c_size_t, [P(tpa_dims), i64, i64]),
        "tpa_paged_decode_attn": (ctypes.c_int, [P(tpa_dims), P(tpa_factors), P(tpa_paged_cache), i64, vp, i64,
                                                 vp, vp, ctypes.c_size_t, vp]),
        "tpa_shared_cache_append": (ctypes.c_int, [P(tpa_dims), P(tpa_shared_cache), P(tpa_factors), i64, i64, i64,
                                                   vp]),
        "tpa_shared_packed_weight_rows": (i64, [P(tpa_dims)]),
        "tpa_shared_factor_proj": (ctypes.c_int, [P(tpa_dims), vp, i64, i64, i64, vp, i32, P(tpa_factors), vp]),
        "tpa_shared_prefill_attn": (ctypes.c_int, [P(tpa_dims), P(tpa_factors), P(tpa_shared_cache), i64, i64, i64,
                                                   i32, vp, vp]),
        "tpa_shared_prefill_attn_ws": (ctypes.c_int, [P(tpa_dims), P(tpa_factors), P(tpa_shared_cache), i64, i64,
                                                      i64, i32, vp, vp, ctypes.c_size_t, vp]),
        "tpa_shared_decode_workspace_bytes": (ctypes.c_size_t, [P(tpa_dims), i64, i64]),
        "tpa_shared_decode_attn": (ctypes.c_int, [P(tpa_dims), P(tpa_factors), P(tpa_shared_cache), i64, i64, vp, vp,
                                                  ctypes.c_size_t, vp]),
        "tpa_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        "tpa_last_error": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    return lib


_lib = _load()
EXPORTED = ("tpa_packed_weight_rows", "tpa_cache_elems_per_token", "tpa_factor_proj", "tpa_rope_b",
            "tpa_cache_append", "tpa_prefill_attn", "tpa_prefill_workspace_bytes", "tpa_prefill_attn_ws",
            "tpa_decode_workspace_bytes", "tpa_decode_attn",
            "tpa_decode_noalloc_max_bytes", "tpa_decode_attn_noalloc",
            "tpa_prefill_backward_workspace_bytes", "tpa_prefill_attn_backward", "tpa_rope_b_backward",
            "tpa_paged_cache_append", "tpa_paged_decode_workspace_bytes", "tpa_paged_decode_attn",
            "tpa_shared_cache_append", "tpa_shared_packed_weight_rows", "tpa_shared_factor_proj",
            "tpa_shared_prefill_attn", "tpa_shared_prefill_attn_ws", "tpa_shared_decode_workspace_bytes",
            "tpa_shared_decode_attn",
            "tpa_status_string", "tpa_last_error")


def library():
    """The loaded ctypes library (for tests that call entry points directly)."""
    return _lib


def library_path() -> str:
    return _LIB_PATH


# ---------------------------------------------------------------------------
# Python-side descriptions
# ---------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class Dims:
    d_model: int
    n_heads: int
    head_dim: int
    rank_q: int
    rank_k: int
    rank_v: int
    rope_base: float = 10000.0
    dtype: str = "bf16"

    @property
    def kv_only(self) -> bool:
        return self.rank_q == 0

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    def c(self) -> tpa_dims:
        return tpa_dims(self.d_model, self.n_heads, self.head_dim, self.rank_q, self.rank_k, self.rank_v,
                        float(self.rope_base), TPA_F32 if self.dtype == "f32" else TPA_BF16)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    return t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _check(status: int):
    if status != 0:
        raise TPAError(status, _lib.tpa_last_error().decode())


@dataclasses.dataclass
class Factors:
    """Factor tensors of a block of tokens (see the layouts in include/tpa.h).
    For TPA-KVonly, b_q holds the plain Q and a_q is None."""
    a_q: Optional[torch.Tensor]
    b_q: Optional[torch.Tensor]
    a_k: Optional[torch.Tensor]
    b_k: Optional[torch.Tensor]
    a_v: Optional[torch.Tensor]
    b_v: Optional[torch.Tensor]
    q_batch_stride: int = 0
    kv_batch_stride: int = 0

    def c(self) -> tpa_factors:
        return tpa_factors(_ptr(self.a_q), _ptr(self.b_q), _ptr(self.a_k), _ptr(self.b_k), _ptr(self.a_v),
                           _ptr(self.b_v), self.q_batch_stride, self.kv_batch_stride)


@dataclasses.dataclass
class Cache:
    a_k: torch.Tensor
    b_k: torch.Tensor
    a_v: torch.Tensor
    b_v: torch.Tensor

    @property
    def max_batch(self) -> int:
        return self.a_k.shape[0]

    @property
    def max_seq(self) -> int:
        return self.a_k.shape[1]

    def c(self) -> tpa_cache:
        return tpa_cache(_ptr(self.a_k), _ptr(self.b_k), _ptr(self.a_v), _ptr(self.b_v), self.max_batch, self.max_seq)

    def slot_factors(self, start_pos: int) -> Factors:
        """Key/value factor views at cache slot start_pos, for writing a projection
        straight into the cache (kv_batch_stride = max_seq)."""
        return Factors(None, None, self.a_k[:, start_pos], self.b_k[:, start_pos], self.a_v[:, start_pos],
                       self.b_v[:, start_pos], 0, self.max_seq)


@dataclasses.dataclass
class PagedCache:
    """Page pools [n_pages, page_tokens, ...] and an int32 block table
    [max_batch, max_pages] on the device (see include/tpa.h)."""
    a_k: torch.Tensor
    b_k: torch.Tensor
    a_v: torch.Tensor
    b_v: torch.Tensor
    block_table: torch.Tensor

    @property
    def n_pages(self) -> int:
        return self.a_k.shape[0]

    @property
    def page_tokens(self) -> int:
        return self.a_k.shape[1]

    def c(self) -> tpa_paged_cache:
        mb, mp = self.block_table.shape
        return tpa_paged_cache(_ptr(self.a_k), _ptr(self.b_k), _ptr(self.a_v), _ptr(self.b_v),
                               _ptr(self.block_table), self.n_pages, self.page_tokens, mp, mb)


@dataclasses.dataclass
class SharedCache:
    """Shared-basis cache: head factors a_k [max_batch, max_seq, h, R_K], a_v
    [.., h, R_V], and the bases b_k [R_K, d_h] (unrotated), b_v [R_V, d_h]
    common to every token (see include/tpa.h)."""
    a_k: torch.Tensor
    a_v: torch.Tensor
    b_k: torch.Tensor
    b_v: torch.Tensor

    @property
    def max_batch(self) -> int:
        return self.a_k.shape[0]

    @property
    def max_seq(self) -> int:
        return self.a_k.shape[1]

    def c(self) -> tpa_shared_cache:
        return tpa_shared_cache(_ptr(self.a_k), _ptr(self.a_v), _ptr(self.b_k), _ptr(self.b_v), self.max_batch,
                                self.max_seq)


def new_shared_cache(dims: Dims, max_batch: int, max_seq: int, b_k: torch.Tensor, b_v: torch.Tensor,
                     device="cuda") -> SharedCache:
    dt = dims.torch_dtype
    h = dims.n_heads
    assert b_k.shape == (dims.rank_k, dims.head_dim) and b_v.shape == (dims.rank_v, dims.head_dim)
    return SharedCache(torch.zeros(max_batch, max_seq, h, dims.rank_k, dtype=dt, device=device),
                       torch.zeros(max_batch, max_seq, h, dims.rank_v, dtype=dt, device=device),
                       b_k.to(device=device, dtype=dt).contiguous(), b_v.to(device=device, dtype=dt).contiguous())


def new_paged_cache(dims: Dims, n_pages: int, page_tokens: int, block_table: torch.Tensor,
                    device="cuda") -> PagedCache:
    dt = dims.torch_dtype
    h, d = dims.n_heads, dims.head_dim
    assert block_table.dtype == torch.int32 and block_table.dim() == 2 and block_table.is_contiguous()
    return PagedCache(torch.zeros(n_pages, page_tokens, h, dims.rank_k, dtype=dt, device=device),
                      torch.zeros(n_pages, page_tokens, dims.rank_k, d, dtype=dt, device=device),
                      torch.zeros(n_pages, page_tokens, h, dims.rank_v, dtype=dt, device=device),
                      torch.zeros(n_pages, page_tokens, dims.rank_v, d, dtype=dt, device=device),
                      block_table.to(device))


def new_cache(dims: Dims, max_batch: int, max_seq: int, device="cuda") -> Cache:
    dt = dims.torch_dtype
    h, d = dims.n_heads, dims.head_dim
    return Cache(torch.zeros(max_batch, max_seq, h, dims.rank_k, dtype=dt, device=device),
                 torch.zeros(max_batch, max_seq, dims.rank_k, d, dtype=dt, device=device),
                 torch.zeros(max_batch, max_seq, h, dims.rank_v, dtype=dt, device=device),
                 torch.zeros(max_batch, max_seq, dims.rank_v, d, dtype=dt, device=device))


def new_factors(dims: Dims, batch: int, seq: int, device="cuda", squeeze_seq: bool = False) -> Factors:
    dt = dims.torch_dtype
    h, d = dims.n_heads, dims.head_dim
    lead = (batch,) if squeeze_seq else (batch, seq)

    def z(*shape):
        return torch.empty(*lead, *shape, dtype=dt, device=device)

    if dims.kv_only:
        a_q, b_q = None, z(h, d)
    else:
        a_q, b_q = z(h, dims.rank_q), z(dims.rank_q, d)
    return Factors(a_q, b_q, z(h, dims.rank_k), z(dims.rank_k, d), z(h, dims.rank_v), z(dims.rank_v, d))


def pack_weights(w: dict, kv_only: bool) -> torch.Tensor:
    """Stack the per-factor nn.Linear weights in the library's row order:
    W_B_q, W_B_k, W_B_v, W_A_q, W_A_k, W_A_v (KV-only: W_Q first, no W_A_q)."""
    order = (["w_q"] if kv_only else ["w_b_q"]) + ["w_b_k", "w_b_v"] + ([] if kv_only else ["w_a_q"]) + \
        ["w_a_k", "w_a_v"]
    return torch.cat([w[k] for k in order], dim=0).contiguous()


# ---------------------------------------------------------------------------
# Entry points (same names as the C ABI)
# ---------------------------------------------------------------------------

def tpa_packed_weight_rows(dims: Dims) -> int:
    return int(_lib.tpa_packed_weight_rows(ctypes.byref(dims.c())))


def tpa_cache_elems_per_token(dims: Dims) -> int:
    return int(_lib.tpa_cache_elems_per_token(ctypes.byref(dims.c())))


def tpa_factor_proj(dims: Dims, x: torch.Tensor, w_packed: torch.Tensor, out: Factors, start_pos: int = 0,
                    fuse_rope: bool = True, stream=None) -> Factors:
    B, S = x.shape[0], x.shape[1]
    _check(_lib.tpa_factor_proj(ctypes.byref(dims.c()), _ptr(x), B, S, start_pos, _ptr(w_packed),
                                1 if fuse_rope else 0, ctypes.byref(out.c()), _stream(stream)))
    return out


def tpa_rope_b(dims: Dims, b: torch.Tensor, start_pos: int = 0, stream=None) -> torch.Tensor:
    """In place on b [B, S, rows, d_h]."""
    B, S, rows = b.shape[0], b.shape[1], b.shape[2]
    _check(_lib.tpa_rope_b(ctypes.byref(dims.c()), _ptr(b), B, S, rows, start_pos, _stream(stream)))
    return b


def tpa_cache_append(dims: Dims, cache: Cache, kv: Factors, start_pos: int, stream=None):
    B, S = kv.a_k.shape[0], kv.a_k.shape[1]
    _check(_lib.tpa_cache_append(ctypes.byref(dims.c()), ctypes.byref(cache.c()), ctypes.byref(kv.c()), B, S,
                                 start_pos, _stream(stream)))


def tpa_prefill_attn(dims: Dims, q: Factors, cache: Cache, start_pos: int, causal: bool = True,
                     out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    B, S = q.b_q.shape[0], q.b_q.shape[1]
    if out is None:
        out = torch.empty(B, S, dims.n_heads * dims.head_dim, dtype=dims.torch_dtype, device=q.b_q.device)
    _check(_lib.tpa_prefill_attn(ctypes.byref(dims.c()), ctypes.byref(q.c()), ctypes.byref(cache.c()), B, S,
                                 start_pos, 1 if causal else 0, _ptr(out), _stream(stream)))
    return out


def tpa_prefill_workspace_bytes(dims: Dims, batch: int, seq: int, start_pos: int) -> int:
    return int(_lib.tpa_prefill_workspace_bytes(ctypes.byref(dims.c()), batch, seq, start_pos))


def tpa_prefill_attn_ws(dims: Dims, q: Factors, cache: Cache, start_pos: int, workspace: Optional[torch.Tensor],
                        causal: bool = True, out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    B, S = q.b_q.shape[0], q.b_q.shape[1]
    if out is None:
        out = torch.empty(B, S, dims.n_heads * dims.head_dim, dtype=dims.torch_dtype, device=q.b_q.device)
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_lib.tpa_prefill_attn_ws(ctypes.byref(dims.c()), ctypes.byref(q.c()), ctypes.byref(cache.c()), B, S,
                                    start_pos, 1 if causal else 0, _ptr(out), _ptr(workspace), nbytes,
                                    _stream(stream)))
    return out


def tpa_decode_workspace_bytes(dims: Dims, batch: int, ctx_len: int) -> int:
    return int(_lib.tpa_decode_workspace_bytes(ctypes.byref(dims.c()), batch, ctx_len))


def new_workspace(dims: Dims, batch: int, ctx_len: int, device="cuda") -> torch.Tensor:
    n = max(tpa_decode_workspace_bytes(dims, batch, ctx_len), 16)
    return torch.zeros(n, dtype=torch.uint8, device=device)


def tpa_decode_attn(dims: Dims, q: Factors, cache: Cache, ctx_len: int, workspace: torch.Tensor,
                    out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """q holds the new token's factors without a sequence axis: a_q [B,h,R_Q], b_q [B,R_Q,d_h]."""
    B = q.b_q.shape[0]
    if out is None:
        out = torch.empty(B, dims.n_heads * dims.head_dim, dtype=dims.torch_dtype, device=q.b_q.device)
    _check(_lib.tpa_decode_attn(ctypes.byref(dims.c()), ctypes.byref(q.c()), ctypes.byref(cache.c()), B, ctx_len,
                                _ptr(out), _ptr(workspace), workspace.numel() * workspace.element_size(),
                                _stream(stream)))
    return out


def tpa_decode_noalloc_max_bytes() -> int:
    return int(_lib.tpa_decode_noalloc_max_bytes())


def tpa_decode_attn_noalloc(dims: Dims, q: Factors, cache: Cache, ctx_len: int, out: Optional[torch.Tensor] = None,
                            stream=None) -> torch.Tensor:
    """tpa_decode_attn with the chunk partials in the library's static device
    scratch (no workspace argument).  Overlapping calls on one device race."""
    B = q.b_q.shape[0]
    if out is None:
        out = torch.empty(B, dims.n_heads * dims.head_dim, dtype=dims.torch_dtype, device=q.b_q.device)
    _check(_lib.tpa_decode_attn_noalloc(ctypes.byref(dims.c()), ctypes.byref(q.c()), ctypes.byref(cache.c()), B,
                                        ctx_len, _ptr(out), _stream(stream)))
    return out


def tpa_paged_cache_append(dims: Dims, cache: PagedCache, kv: Factors, start_pos: torch.Tensor, stream=None):
    """start_pos: int32 [B] on the device (position of each sequence's token 0)."""
    B, S = kv.a_k.shape[0], kv.a_k.shape[1]
    assert start_pos.dtype == torch.int32 and start_pos.numel() >= B
    _check(_lib.tpa_paged_cache_append(ctypes.byref(dims.c()), ctypes.byref(cache.c()), ctypes.byref(kv.c()), B, S,
                                       _ptr(start_pos), _stream(stream)))


def tpa_paged_decode_workspace_bytes(dims: Dims, batch: int, max_ctx_len: int) -> int:
    return int(_lib.tpa_paged_decode_workspace_bytes(ctypes.byref(dims.c()), batch, max_ctx_len))


def tpa_paged_decode_attn(dims: Dims, q: Factors, cache: PagedCache, ctx_lens: torch.Tensor, max_ctx_len: int,
                          workspace: torch.Tensor, out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """ctx_lens: int32 [B] on the device, each in [0, max_ctx_len]."""
    B = q.b_q.shape[0]
    assert ctx_lens.dtype == torch.int32 and ctx_lens.numel() >= B
    if out is None:
        out = torch.empty(B, dims.n_heads * dims.head_dim, dtype=dims.torch_dtype, device=q.b_q.device)
    _check(_lib.tpa_paged_decode_attn(ctypes.byref(dims.c()), ctypes.byref(q.c()), ctypes.byref(cache.c()), B,
                                      _ptr(ctx_lens), max_ctx_len, _ptr(out), _ptr(workspace),
                                      workspace.numel() * workspace.element_size(), _stream(stream)))
    return out


def tpa_shared_cache_append(dims: Dims, cache: SharedCache, kv: Factors, start_pos: int, stream=None):
    """Writes kv.a_k, kv.a_v (the head factors) at positions start_pos.. of each sequence."""
    B, S = kv.a_k.shape[0], kv.a_k.shape[1]
    _check(_lib.tpa_shared_cache_append(ctypes.byref(dims.c()), ctypes.byref(cache.c()), ctypes.byref(kv.c()), B, S,
                                        start_pos, _stream(stream)))


def pack_shared_weights(w: dict, kv_only: bool) -> torch.Tensor:
    """Stack the per-factor weights of a shared-basis layer in the library's row
    order: W_B_q, W_A_q, W_A_k, W_A_v (KV-only: W_Q, W_A_k, W_A_v)."""
    order = (["w_q"] if kv_only else ["w_b_q", "w_a_q"]) + ["w_a_k", "w_a_v"]
    return torch.cat([w[k] for k in order], dim=0).contiguous()


def tpa_shared_packed_weight_rows(dims: Dims) -> int:
    return int(_lib.tpa_shared_packed_weight_rows(ctypes.byref(dims.c())))


def tpa_shared_factor_proj(dims: Dims, x: torch.Tensor, w_packed: torch.Tensor, out: Factors, start_pos: int = 0,
                           fuse_rope: bool = True, stream=None) -> Factors:
    """Query factors and key/value head factors (out.b_k, out.b_v are ignored)."""
    B, S = x.shape[0], x.shape[1]
    _check(_lib.tpa_shared_factor_proj(ctypes.byref(dims.c()), _ptr(x), B, S, start_pos, _ptr(w_packed),
                                       1 if fuse_rope else 0, ctypes.byref(out.c()), _stream(stream)))
    return out


def tpa_shared_prefill_attn(dims: Dims, q: Factors, cache: SharedCache, start_pos: int, causal: bool = True,
                            out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    B, S = q.b_q.shape[0], q.b_q.shape[1]
    if out is None:
        out = torch.empty(B, S, dims.n_heads * dims.head_dim, dtype=dims.torch_dtype, device=q.b_q.device)
    _check(_lib.tpa_shared_prefill_attn(ctypes.byref(dims.c()), ctypes.byref(q.c()), ctypes.byref(cache.c()), B, S,
                                        start_pos, 1 if causal else 0, _ptr(out), _stream(stream)))
    return out


def tpa_shared_prefill_attn_ws(dims: Dims, q: Factors, cache: SharedCache, start_pos: int,
                               workspace: Optional[torch.Tensor], causal: bool = True,
                               out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Workspace sized by tpa_prefill_workspace_bytes (None where it is 0)."""
    B, S = q.b_q.shape[0], q.b_q.shape[1]
    if out is None:
        out = torch.empty(B, S, dims.n_heads * dims.head_dim, dtype=dims.torch_dtype, device=q.b_q.device)
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_lib.tpa_shared_prefill_attn_ws(ctypes.byref(dims.c()), ctypes.byref(q.c()), ctypes.byref(cache.c()), B,
                                           S, start_pos, 1 if causal else 0, _ptr(out), _ptr(workspace), nbytes,
                                           _stream(stream)))
    return out


def tpa_shared_decode_workspace_bytes(dims: Dims, batch: int, ctx_len: int) -> int:
    return int(_lib.tpa_shared_decode_workspace_bytes(ctypes.byref(dims.c()), batch, ctx_len))


def tpa_shared_decode_attn(dims: Dims, q: Factors, cache: SharedCache, ctx_len: int, workspace: torch.Tensor,
                           out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    B = q.b_q.shape[0]
    if out is None:
        out = torch.empty(B, dims.n_heads * dims.head_dim, dtype=dims.torch_dtype, device=q.b_q.device)
    _check(_lib.tpa_shared_decode_attn(ctypes.byref(dims.c()), ctypes.byref(q.c()), ctypes.byref(cache.c()), B,
                                       ctx_len, _ptr(out), _ptr(workspace),
                                       workspace.numel() * workspace.element_size(), _stream(stream)))
    return out


def tpa_prefill_backward_workspace_bytes(dims: Dims, batch: int, seq: int, start_pos: int) -> int:
    return int(_lib.tpa_prefill_backward_workspace_bytes(ctypes.byref(dims.c()), batch, seq, start_pos))


def tpa_prefill_attn_backward(dims: Dims, q: Factors, cache: Cache, start_pos: int, causal: bool,
                              dout: torch.Tensor, dq: Factors, dkv: Cache, workspace: torch.Tensor, stream=None):
    """Gradients into dq (a_q, b_q; KV-only b_q = dQ) and dkv (cache layout), all float32."""
    B, S = q.b_q.shape[0], q.b_q.shape[1]
    _check(_lib.tpa_prefill_attn_backward(ctypes.byref(dims.c()), ctypes.byref(q.c()), ctypes.byref(cache.c()), B,
                                          S, start_pos, 1 if causal else 0, _ptr(dout),
                                          ctypes.byref(dq.c()), ctypes.byref(dkv.c()), _ptr(workspace),
                                          workspace.numel() * workspace.element_size(), _stream(stream)))


def tpa_rope_b_backward(dims: Dims, g: torch.Tensor, start_pos: int = 0, stream=None) -> torch.Tensor:
    """In place on g [B, S, rows, d_h], float32."""
    assert g.dtype == torch.float32
    B, S, rows = g.shape[0], g.shape[1], g.shape[2]
    _check(_lib.tpa_rope_b_backward(ctypes.byref(dims.c()), _ptr(g), B, S, rows, start_pos, _stream(stream)))
    return g
