"""Dense brute-force formulations used to pin the oracle.

These are written as whole-matrix PyTorch (CPU, float64) computations, a code
path unrelated to the oracle's per-row loops: a token-level mask is built from
the block-index cache, and ordinary masked softmax attention (with autograd for
the gradients) is evaluated on it.
"""
from __future__ import annotations

import numpy as np
import torch

BLOCK = 128


def token_mask(idx: np.ndarray, T: int) -> torch.Tensor:
    """Boolean [B, G, T, T] mask: query t may read key j iff j <= t and the block of
    j is listed in idx[b, g, t, :]."""
    idx_t = torch.as_tensor(np.asarray(idx, dtype=np.int64))
    B, G, T_, K = idx_t.shape
    assert T_ == T
    N = (T + BLOCK - 1) // BLOCK
    blk_sel = torch.zeros((B, G, T, N + 1), dtype=torch.bool)
    safe = torch.where(idx_t >= 0, idx_t, torch.full_like(idx_t, N))
    blk_sel.scatter_(3, safe, True)
    blk_sel = blk_sel[..., :N]
    key_blk = torch.arange(T) // BLOCK
    m = blk_sel[..., key_blk]                       # [B, G, T, T]
    causal = torch.tril(torch.ones(T, T, dtype=torch.bool))
    return m & causal


def dense_attention(q, k, v, mask, scale):
    """q [B,T,H,d], k/v [B,T,G,d] (float64 tensors), mask [B,G,T,T].
    Returns O [B,T,H,d] and LSE [B,T,H]."""
    B, T, H, d = q.shape
    G = k.shape[2]
    R = H // G
    kh = k.repeat_interleave(R, dim=2)             # head h uses group h // R
    vh = v.repeat_interleave(R, dim=2)
    mh = mask.repeat_interleave(R, dim=1)           # [B, H, T, T]
    s = torch.einsum("bthc,bjhc->bhtj", q, kh) * scale
    s = s.masked_fill(~mh, float("-inf"))
    lse = torch.logsumexp(s, dim=-1)                # [B, H, T]
    p = torch.softmax(s, dim=-1)
    o = torch.einsum("bhtj,bjhc->bthc", p, vh)
    return o, lse.permute(0, 2, 1)


def dense_grads(q, k, v, dout, mask, scale):
    """Autograd of L = sum(O * dout) through dense_attention (float64)."""
    qq = q.clone().requires_grad_(True)
    kk = k.clone().requires_grad_(True)
    vv = v.clone().requires_grad_(True)
    o, _ = dense_attention(qq, kk, vv, mask, scale)
    (o * dout).sum().backward()
    return qq.grad, kk.grad, vv.grad


def f64(x) -> torch.Tensor:
    if isinstance(x, torch.Tensor):
        return x.detach().to(torch.float64)
    return torch.as_tensor(np.asarray(x), dtype=torch.float64)
