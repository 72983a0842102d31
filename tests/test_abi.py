"""CPU tests of the C ABI: the library loads, exports every function that
include/tpa.h declares, and rejects bad arguments before it launches anything.

No call here reaches a kernel launch: every call is built to fail validation.
Device pointers are dummy non-null addresses that are never dereferenced.
"""
import ctypes
import os
import re

import pytest

from factorized_kv_cache_amd import tpa as T

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tpa.h")
FAKE = 0x10000  # never dereferenced: every call below fails validation first

OK, INVALID, UNSUPPORTED, CAPACITY, WORKSPACE = 0, 1, 2, 3, 4


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tpa_[a-z_]+)\s*\(", text)))


def test_header_functions_are_exported():
    lib = ctypes.CDLL(T.library_path())
    names = declared_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(lib, n), f"{n} declared in tpa.h but not exported"
    assert sorted(T.EXPORTED) == names


def dims(**kw):
    base = dict(d_model=1024, n_heads=16, head_dim=64, rank_q=6, rank_k=2, rank_v=2, rope_base=10000.0, dtype=1)
    base.update(kw)
    return T.tpa_dims(**base)


@pytest.mark.parametrize("kw,n_out,elems", [
    (dict(d_model=256, n_heads=4, head_dim=64, rank_q=6, rank_k=2, rank_v=2, dtype=0), 680, 272),
    (dict(), 800, 320),
    (dict(d_model=4096, n_heads=32, head_dim=128), 1600, 640),
    (dict(d_model=1536, n_heads=24, head_dim=64, rank_q=0, rank_k=4, rank_v=4), 2240, 704),
])
def test_sizes(kw, n_out, elems):
    lib = T.library()
    d = dims(**kw)
    assert lib.tpa_packed_weight_rows(ctypes.byref(d)) == n_out
    assert lib.tpa_cache_elems_per_token(ctypes.byref(d)) == elems


@pytest.mark.parametrize("kw", [
    dict(head_dim=63), dict(head_dim=0), dict(head_dim=258), dict(n_heads=0), dict(rank_k=0), dict(rank_v=65),
    dict(rank_q=-1), dict(d_model=0), dict(rope_base=0.0), dict(rope_base=float("inf")), dict(dtype=7),
])
def test_invalid_dims(kw):
    lib = T.library()
    d = dims(**kw)
    assert lib.tpa_packed_weight_rows(ctypes.byref(d)) == -1
    f = T.tpa_factors(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, 0)
    st = lib.tpa_factor_proj(ctypes.byref(d), FAKE, 1, 1, 0, FAKE, 1, ctypes.byref(f), None)
    assert st == INVALID
    assert lib.tpa_last_error().decode()


def test_unsupported_head_elems():
    lib = T.library()
    d = dims(n_heads=128, head_dim=128)
    f = T.tpa_factors(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, 0)
    assert lib.tpa_factor_proj(ctypes.byref(d), FAKE, 1, 1, 0, FAKE, 1, ctypes.byref(f), None) == UNSUPPORTED


def test_factor_proj_validation():
    lib = T.library()
    d = dims()
    f = T.tpa_factors(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, 0)
    call = lambda **k: lib.tpa_factor_proj(ctypes.byref(d), k.get("x", FAKE), k.get("B", 2), k.get("S", 3),
                                           k.get("sp", 0), k.get("w", FAKE), 1, ctypes.byref(k.get("f", f)), None)
    assert call(x=None) == INVALID
    assert call(w=None) == INVALID
    assert call(B=0) == INVALID
    assert call(S=-1) == INVALID
    assert call(sp=-1) == INVALID
    assert call(f=T.tpa_factors(None, FAKE, FAKE, FAKE, FAKE, FAKE, 0, 0)) == INVALID   # a_q needed
    assert call(f=T.tpa_factors(FAKE, FAKE, FAKE, None, FAKE, FAKE, 0, 0)) == INVALID
    assert call(f=T.tpa_factors(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2, 0)) == INVALID   # stride < S
    assert call(B=1 << 20, S=1 << 12) == UNSUPPORTED
    assert call(f=T.tpa_factors(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, 1)) == INVALID   # kv stride < S
    assert "kv_batch_stride" in lib.tpa_last_error().decode()


def test_rope_validation():
    lib = T.library()
    d = dims()
    assert lib.tpa_rope_b(ctypes.byref(d), None, 1, 1, 2, 0, None) == INVALID
    assert lib.tpa_rope_b(ctypes.byref(d), FAKE, 1, 1, 0, 0, None) == INVALID
    assert lib.tpa_rope_b(ctypes.byref(d), FAKE, 1, 1, 2, -5, None) == INVALID
    assert lib.tpa_rope_b(ctypes.byref(dims(head_dim=7)), FAKE, 1, 1, 2, 0, None) == INVALID


def test_cache_append_validation():
    lib = T.library()
    d = dims()
    c = T.tpa_cache(FAKE, FAKE, FAKE, FAKE, 4, 100)
    kv = T.tpa_factors(None, None, FAKE, FAKE, FAKE, FAKE, 0, 0)
    app = lambda B, S, sp, cc=c, kk=kv: lib.tpa_cache_append(ctypes.byref(d), ctypes.byref(cc), ctypes.byref(kk),
                                                             B, S, sp, None)
    assert app(5, 1, 0) == CAPACITY
    assert app(4, 101, 0) == CAPACITY
    assert app(4, 10, 91) == CAPACITY
    assert app(1, 1, -1) == INVALID
    assert app(1, 1, 0, cc=T.tpa_cache(FAKE, None, FAKE, FAKE, 4, 100)) == INVALID
    assert app(1, 1, 0, cc=T.tpa_cache(FAKE, FAKE, FAKE, FAKE, 0, 100)) == INVALID
    assert app(1, 1, 0, kk=T.tpa_factors(None, None, FAKE, FAKE, None, FAKE, 0, 0)) == INVALID
    assert "max_seq" in lib.tpa_last_error().decode() or "NULL" in lib.tpa_last_error().decode()


def test_prefill_validation():
    lib = T.library()
    d = dims()
    c = T.tpa_cache(FAKE, FAKE, FAKE, FAKE, 2, 64)
    q = T.tpa_factors(FAKE, FAKE, None, None, None, None, 0, 0)
    pf = lambda B, S, sp, qq=q, out=FAKE: lib.tpa_prefill_attn(ctypes.byref(d), ctypes.byref(qq), ctypes.byref(c),
                                                               B, S, sp, 1, out, None)
    assert pf(3, 4, 0) == CAPACITY
    assert pf(2, 65, 0) == CAPACITY
    assert pf(2, 8, 57) == CAPACITY
    assert pf(2, 8, 0, out=None) == INVALID
    assert pf(2, 8, 0, qq=T.tpa_factors(None, FAKE, None, None, None, None, 0, 0)) == INVALID
    kvonly = dims(rank_q=0)
    assert lib.tpa_prefill_attn(ctypes.byref(kvonly), ctypes.byref(T.tpa_factors(None, None, None, None, None, None,
                                                                                 0, 0)),
                                ctypes.byref(c), 1, 1, 0, 1, FAKE, None) == INVALID


def test_prefill_workspace_sizes_and_validation():
    """The workspace prefill needs 2 * B * h * (start_pos + S) * d_h * 2 bytes
    where K and V are formed once (bf16, d_h 64, R_K = R_V in {1, 2, 4}), none
    elsewhere; a missing, misaligned or short workspace is rejected before
    anything is enqueued, after the checks the plain prefill makes."""
    lib = T.library()
    ws = lambda dd, B, S, sp: lib.tpa_prefill_workspace_bytes(ctypes.byref(dd), B, S, sp)
    d = dims()
    assert ws(d, 2, 40, 24) == 2 * 2 * 16 * 64 * 64 * 2
    assert ws(dims(rank_k=4, rank_v=4), 1, 1, 0) == 2 * 16 * 64 * 2
    assert ws(dims(rank_k=1, rank_v=1, n_heads=5, d_model=320), 3, 7, 0) == 2 * 3 * 5 * 7 * 64 * 2
    for other in (dims(dtype=0), dims(head_dim=128, d_model=2048), dims(rank_k=2, rank_v=1), dims(rank_k=3, rank_v=3)):
        assert ws(other, 2, 40, 24) == 0
    for B, S, sp in ((0, 1, 0), (1, 0, 0), (1, 1, -1), (65536, 1, 0), (1, 2**31, 0), (1, 1, 2**31), (1, 2**62, 2**62)):
        assert ws(d, B, S, sp) == 0, (B, S, sp)
    need = ws(d, 2, 8, 0)
    c = T.tpa_cache(FAKE, FAKE, FAKE, FAKE, 2, 64)
    q = T.tpa_factors(FAKE, FAKE, None, None, None, None, 0, 0)
    pf = lambda B, S, sp, w=FAKE, n=need: lib.tpa_prefill_attn_ws(ctypes.byref(d), ctypes.byref(q), ctypes.byref(c),
                                                                  B, S, sp, 1, FAKE, w, n, None)
    assert pf(3, 4, 0) == CAPACITY
    assert pf(2, 65, 0) == CAPACITY
    assert pf(2, 8, 0, w=None) == WORKSPACE
    assert pf(2, 8, 0, w=FAKE + 8) == INVALID
    assert pf(2, 8, 0, n=need - 1) == WORKSPACE
    assert pf(2, 8, 2, n=need) == WORKSPACE   # two more keys than sized for
    # the shared-basis prefill takes the same sizes and checks
    sc = T.tpa_shared_cache(FAKE, FAKE, FAKE, FAKE, 2, 64)
    sf = lambda B, S, sp, w=FAKE, n=need: lib.tpa_shared_prefill_attn_ws(ctypes.byref(d), ctypes.byref(q),
                                                                         ctypes.byref(sc), B, S, sp, 1, FAKE, w, n, None)
    assert sf(3, 4, 0) == CAPACITY
    assert sf(2, 8, 0, w=None) == WORKSPACE
    assert sf(2, 8, 0, w=FAKE + 8) == INVALID
    assert sf(2, 8, 0, n=need - 1) == WORKSPACE
    fp32 = dims(dtype=0)
    assert lib.tpa_shared_prefill_attn_ws(ctypes.byref(fp32), ctypes.byref(q), ctypes.byref(sc), 2, 8, 0, 1, None,
                                          None, 0, None) == INVALID   # out NULL, before any workspace check


def test_decode_validation():
    lib = T.library()
    d = dims()
    c = T.tpa_cache(FAKE, FAKE, FAKE, FAKE, 16, 4097)
    q = T.tpa_factors(FAKE, FAKE, None, None, None, None, 0, 0)
    need = lib.tpa_decode_workspace_bytes(ctypes.byref(d), 16, 4097)
    assert need > 0
    dec = lambda B, L, ws, n: lib.tpa_decode_attn(ctypes.byref(d), ctypes.byref(q), ctypes.byref(c), B, L, FAKE,
                                                  ws, n, None)
    assert dec(16, 4097, FAKE, need - 1) == WORKSPACE
    assert dec(16, 4097, None, need) == WORKSPACE
    assert dec(17, 4097, FAKE, need) == CAPACITY
    assert dec(16, 4098, FAKE, need * 2) == CAPACITY
    assert dec(16, 0, FAKE, need) == INVALID
    assert lib.tpa_decode_workspace_bytes(ctypes.byref(dims(head_dim=5)), 16, 4097) == 0


def test_paged_validation():
    lib = T.library()
    d = dims()
    pc = T.tpa_paged_cache(FAKE, FAKE, FAKE, FAKE, FAKE, 100, 64, 65, 16)   # 65 pages of 64 = 4160 positions
    q = T.tpa_factors(FAKE, FAKE, None, None, None, None, 0, 0)
    kv = T.tpa_factors(None, None, FAKE, FAKE, FAKE, FAKE, 0, 0)
    need = lib.tpa_paged_decode_workspace_bytes(ctypes.byref(d), 16, 4097)
    assert need == lib.tpa_decode_workspace_bytes(ctypes.byref(d), 16, 4097) > 0
    dec = lambda B, L, ws, n, c=pc, lens=FAKE: lib.tpa_paged_decode_attn(
        ctypes.byref(d), ctypes.byref(q), ctypes.byref(c), B, lens, L, FAKE, ws, n, None)
    assert dec(16, 4097, FAKE, need - 1) == WORKSPACE
    assert dec(16, 4097, None, need) == WORKSPACE
    assert dec(17, 4097, FAKE, need) == CAPACITY                     # more sequences than table rows
    assert dec(16, 4161, FAKE, need * 2) == CAPACITY                 # past max_pages * page_tokens
    assert dec(16, 0, FAKE, need) == INVALID
    assert dec(16, 4097, FAKE, need, lens=None) == INVALID           # no lengths
    assert dec(16, 4097, FAKE, need, c=T.tpa_paged_cache(FAKE, FAKE, FAKE, FAKE, None, 100, 64, 65, 16)) == INVALID
    assert dec(16, 4097, FAKE, need, c=T.tpa_paged_cache(FAKE, FAKE, FAKE, FAKE, FAKE, 0, 64, 65, 16)) == INVALID
    assert dec(16, 4097, FAKE, need, c=T.tpa_paged_cache(FAKE, FAKE, FAKE, FAKE, FAKE, 100, 1 << 20, 1 << 12,
                                                         16)) == UNSUPPORTED   # 2^32 positions
    app = lambda B, S, sp=FAKE, c=pc, k=kv: lib.tpa_paged_cache_append(ctypes.byref(d), ctypes.byref(c),
                                                                        ctypes.byref(k), B, S, sp, None)
    assert app(17, 1) == CAPACITY
    assert app(1, 0) == INVALID
    assert app(1, 1, sp=None) == INVALID
    assert app(1, 1, k=T.tpa_factors(None, None, FAKE, None, FAKE, FAKE, 0, 0)) == INVALID
    assert app(1, 1, c=T.tpa_paged_cache(None, FAKE, FAKE, FAKE, FAKE, 100, 64, 65, 16)) == INVALID


def test_shared_validation():
    lib = T.library()
    d = dims()
    sc = T.tpa_shared_cache(FAKE, FAKE, FAKE, FAKE, 16, 4097)
    q = T.tpa_factors(FAKE, FAKE, None, None, None, None, 0, 0)
    kv = T.tpa_factors(None, None, FAKE, None, FAKE, None, 0, 0)
    need = lib.tpa_shared_decode_workspace_bytes(ctypes.byref(d), 16, 4097)
    assert need > 0 and need % (4 * 16 * 16 * (2 + 2)) == 0      # (max, sum, R_V weights) per chunk and head
    assert lib.tpa_shared_decode_workspace_bytes(ctypes.byref(d), 0, 4097) == 0
    dec = lambda B, L, c=sc, qq=q: lib.tpa_shared_decode_attn(ctypes.byref(d), ctypes.byref(qq), ctypes.byref(c), B,
                                                               L, FAKE, FAKE, need, None)
    assert dec(17, 4097) == CAPACITY
    assert dec(16, 4098) == CAPACITY
    assert dec(16, 0) == INVALID
    assert dec(16, 4097, c=T.tpa_shared_cache(FAKE, FAKE, None, FAKE, 16, 4097)) == INVALID    # no basis
    assert dec(16, 4097, c=T.tpa_shared_cache(FAKE, None, FAKE, FAKE, 16, 4097)) == INVALID    # no a_v
    assert dec(16, 4097, qq=T.tpa_factors(None, FAKE, None, None, None, None, 0, 0)) == INVALID   # a_q missing
    app = lambda B, S, sp, c=sc, k=kv: lib.tpa_shared_cache_append(ctypes.byref(d), ctypes.byref(c), ctypes.byref(k),
                                                                   B, S, sp, None)
    assert app(17, 1, 0) == CAPACITY
    assert app(1, 1, 4097) == CAPACITY
    assert app(1, 0, 0) == INVALID
    assert app(1, 1, -1) == INVALID
    assert app(1, 1, 0, k=T.tpa_factors(None, None, None, None, FAKE, None, 0, 0)) == INVALID


@pytest.mark.parametrize("kw,n_out", [
    (dict(), 16 * 6 + 6 * 64 + 16 * (2 + 2)),                       # W_B_q, W_A_q, W_A_k, W_A_v
    (dict(d_model=1536, n_heads=24, head_dim=64, rank_q=0, rank_k=4, rank_v=4), 24 * 64 + 24 * 8),
])
def test_shared_projection_and_prefill_validation(kw, n_out):
    lib = T.library()
    d = dims(**kw)
    assert lib.tpa_shared_packed_weight_rows(ctypes.byref(d)) == n_out
    assert lib.tpa_shared_packed_weight_rows(ctypes.byref(dims(head_dim=63))) == -1
    # the projection needs the query factors and the key/value head factors only
    f = T.tpa_factors(FAKE, FAKE, FAKE, None, FAKE, None, 0, 0)
    proj = lambda B, S, sp, x=FAKE, ff=f: lib.tpa_shared_factor_proj(ctypes.byref(d), x, B, S, sp, FAKE, 1,
                                                                       ctypes.byref(ff), None)
    assert proj(1, 0, 0) == INVALID
    assert proj(1, 1, -1) == INVALID
    assert proj(1, 1, 0, x=None) == INVALID
    assert proj(1, 1, 0, ff=T.tpa_factors(FAKE, FAKE, None, None, FAKE, None, 0, 0)) == INVALID   # no a_k
    sc = T.tpa_shared_cache(FAKE, FAKE, FAKE, FAKE, 4, 4096)
    q = T.tpa_factors(FAKE, FAKE, None, None, None, None, 0, 0)
    pre = lambda B, S, sp, c=sc: lib.tpa_shared_prefill_attn(ctypes.byref(d), ctypes.byref(q), ctypes.byref(c), B, S,
                                                             sp, 1, FAKE, None)
    assert pre(5, 1, 0) == CAPACITY
    assert pre(1, 4096, 1) == CAPACITY
    assert pre(1, 0, 0) == INVALID
    assert pre(1, 1, -1) == INVALID
    assert pre(1, 1, 0, c=T.tpa_shared_cache(FAKE, FAKE, FAKE, None, 4, 4096)) == INVALID   # no value basis


def test_status_strings():
    lib = T.library()
    for s in range(6):
        assert lib.tpa_status_string(s).decode() == T._STATUS[s]
    assert lib.tpa_status_string(99).decode() == "unknown status"


@pytest.mark.parametrize("dtype", [0, 1])
@pytest.mark.parametrize("kw", [
    dict(n_heads=32, head_dim=256, rank_q=64, rank_k=64, rank_v=64),
    dict(n_heads=256, head_dim=32),
    dict(n_heads=1, head_dim=2, rank_q=1, rank_k=1, rank_v=1),
    dict(rank_k=33, rank_v=5),
])
def test_workspace_sizes_at_the_limits(kw, dtype):
    """Workspace sizing is host arithmetic only: at the dims limits every size
    is positive and nothing faults (the matrix-core decode plan, whose block is
    4 * (32 / R_K) tokens, exists only for the ranks that kernel takes).  Where
    only the general decode applies, the size is its partials exactly: one
    256-token chunk per sequence here, h * (d_h + 2) floats each."""
    lib = T.library()
    d = dims(dtype=dtype, **kw)
    h, dh = d.n_heads, d.head_dim
    for fn in ("tpa_decode_workspace_bytes", "tpa_paged_decode_workspace_bytes", "tpa_shared_decode_workspace_bytes"):
        assert getattr(lib, fn)(ctypes.byref(d), 3, 21) > 0, fn
    assert lib.tpa_prefill_backward_workspace_bytes(ctypes.byref(d), 2, 40, 5) > 0
    if dtype == 0 or d.rank_k > 4:
        assert lib.tpa_decode_workspace_bytes(ctypes.byref(d), 3, 21) == 3 * h * (dh + 2) * 4


def test_sizes_far_past_the_limits():
    """Workspace sizes for batches and lengths the calls reject are 0, and the
    calls' own checks reject them without overflowing (the sizes are bounded
    factor by factor before any product or sum is formed)."""
    lib = T.library()
    d = dims()
    huge = [2**31, 2**40, 2**62, 2**63 - 1]
    for fn in ("tpa_decode_workspace_bytes", "tpa_paged_decode_workspace_bytes", "tpa_shared_decode_workspace_bytes"):
        assert getattr(lib, fn)(ctypes.byref(d), 65536, 10) == 0, fn
        for v in huge:
            assert getattr(lib, fn)(ctypes.byref(d), 1, v) == 0, fn
            assert getattr(lib, fn)(ctypes.byref(d), v, v) == 0, fn
    for v in huge:
        assert lib.tpa_prefill_backward_workspace_bytes(ctypes.byref(d), v, v, 0) == 0
        assert lib.tpa_prefill_backward_workspace_bytes(ctypes.byref(d), 1, 10, v) == 0
    f = T.tpa_factors(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, 0)
    for v in huge:
        assert lib.tpa_factor_proj(ctypes.byref(d), FAKE, v, v, 0, FAKE, 1, ctypes.byref(f), None) == UNSUPPORTED
        assert lib.tpa_factor_proj(ctypes.byref(d), FAKE, 1, 1, v, FAKE, 1, ctypes.byref(f), None) == INVALID
        assert lib.tpa_rope_b(ctypes.byref(d), FAKE, v, v, 2, 0, None) == UNSUPPORTED


def test_decode_noalloc_rejects_partials_beyond_its_scratch():
    """600 sequences at h 256, d_h 32 need 600 * 256 * 34 * 4 bytes of partials
    (20.9 MB) on the general kernel's plan, beyond the 16 MiB scratch: refused
    before anything touches a device."""
    lib = T.library()
    assert lib.tpa_decode_noalloc_max_bytes() == 16 << 20
    d = dims(d_model=512, n_heads=256, head_dim=32, rank_q=2, rank_k=2, rank_v=2)
    q = T.tpa_factors(FAKE, FAKE, None, None, None, None, 0, 0)
    c = T.tpa_cache(FAKE, FAKE, FAKE, FAKE, 600, 4)
    st = lib.tpa_decode_attn_noalloc(ctypes.byref(d), ctypes.byref(q), ctypes.byref(c), 600, 1, FAKE, None)
    assert st == WORKSPACE
    assert "scratch" in lib.tpa_last_error().decode()
    st = lib.tpa_decode_attn_noalloc(ctypes.byref(d), ctypes.byref(q), ctypes.byref(c), 601, 1, FAKE, None)
    assert st == CAPACITY
