"""Textbook multi-head / multi-query / grouped-query attention with rotary
embedding, in torch float64 on the CPU.

Independent of the fp64 oracle: rotary embedding as the complex product of
(x_2i + i x_2i+1) with torch.polar(1, pos*theta_i), K/V heads broadcast over
query heads (one shared head for MQA, a head per group for GQA), and the
attention itself by torch's scaled_dot_product_attention.  Used to pin the
oracle's claim that MHA, MQA and GQA are TPA with non-contextual head factors
([coreui] "优点与创新" item 4; [substack] "Multi-Query Attention" and
"Grouped Query Attention"; [bbzoh] 2.1, the MQA broadcast of one K/V head).
"""
import torch
import torch.nn.functional as F


def rope_complex(x: torch.Tensor, pos: torch.Tensor, base: float) -> torch.Tensor:
    """x [B, S, H, D] float64, pos [S] -> rotated x (interleaved pairs)."""
    D = x.shape[-1]
    freqs = base ** (-torch.arange(0, D, 2, dtype=torch.float64) / D)
    ang = torch.outer(pos.to(torch.float64), freqs)
    cis = torch.polar(torch.ones_like(ang), ang)                    # [S, D/2]
    xc = torch.view_as_complex(x.reshape(*x.shape[:-1], D // 2, 2).contiguous())
    return torch.view_as_real(xc * cis[None, :, None, :]).flatten(-2)


def attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, start_pos: int, causal: bool) -> torch.Tensor:
    """q [B, S, H, D]; k, v [B, T, Hkv, D] with H a multiple of Hkv (query head hh
    uses K/V head hh // (H/Hkv)).  Queries sit at positions start_pos..start_pos+S-1,
    keys at 0..T-1.  Returns [B, S, H*D]."""
    B, S, H, D = q.shape
    T, Hkv = k.shape[1], k.shape[2]
    rep = H // Hkv
    kk = k.repeat_interleave(rep, dim=2).transpose(1, 2).contiguous()
    vv = v.repeat_interleave(rep, dim=2).transpose(1, 2).contiguous()
    qq = q.transpose(1, 2).contiguous()
    mask = None
    if causal:
        qp = torch.arange(start_pos, start_pos + S)[:, None]
        kp = torch.arange(T)[None, :]
        mask = kp <= qp
    o = F.scaled_dot_product_attention(qq, kk, vv, attn_mask=mask)
    return o.transpose(1, 2).reshape(B, S, H * D)
