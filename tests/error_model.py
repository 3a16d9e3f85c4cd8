"""Rounding model of the Main Branch kernels (test infrastructure; a
diagnostic, not the oracle).

The oracle keeps float64 throughout.  The HIP kernels round at fixed points
that bf16 matrix cores impose; this module applies exactly those roundings to
float64 arithmetic on small dense inputs, so a test can tell how much of the
kernel's difference from the oracle each rounding explains:

  forward  o_b = bf16(sum_j bf16(p_j) v_j / l_b), p_j = exp(s_j - m_b)   per (token, block)
           O   = bf16(sum_b exp(lse_b - LSE) o_b)                        combine
  backward dV  = bf16(sum bf16(P)^T dO)
           dS  = bf16(scale P (dP - D)),  D = dO . O (O as stored, bf16)
           dK  = bf16(sum dS^T Q)
           dQ  = bf16(sum_b bf16(sum_{j in b} dS_j k_j))                 per-pair partials

Everything else (fp32 instead of float64 accumulation, the hardware exp2)
is left exact; those contribute at the 1e-6 relative level.
"""
from __future__ import annotations

import numpy as np
import torch


def bf16(x: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float64)).to(torch.bfloat16).double().numpy()


def masks(idx: np.ndarray, T: int) -> np.ndarray:
    """idx [T, k] of one (batch, group) -> key mask [T, T] and block id of each key."""
    blk = np.arange(T) // 128
    m = np.zeros((T, T), dtype=bool)
    for t in range(T):
        sel = idx[t][idx[t] >= 0]
        m[t] = np.isin(blk, sel) & (np.arange(T) <= t)
    return m


def model(q, k, v, dout, o_stored, idx, scale):
    """One batch, one group.  q, dout, o_stored: [T, R, d]; k, v: [T, d];
    idx [T, topk].  Returns dict of exact and modelled o, dq, dk, dv."""
    T, R, d = q.shape
    M = masks(idx, T)
    blk = np.arange(T) // 128
    nblk = T // 128
    ex = {"o": np.zeros((T, R, d)), "dq": np.zeros((T, R, d)), "dk": np.zeros((T, d)), "dv": np.zeros((T, d))}
    md = {n: np.zeros_like(a) for n, a in ex.items()}
    for h in range(R):
        S = scale * (q[:, h] @ k.T)
        Sm = np.where(M, S, -np.inf)
        mx = Sm.max(axis=1, keepdims=True)
        P = np.exp(Sm - mx)
        L = P.sum(axis=1, keepdims=True)
        P = P / L
        lse = mx + np.log(L)
        ex["o"][:, h] = P @ v
        # forward model: per-(token, block) normalised partials, rounded, then merged
        acc = np.zeros((T, d))
        for b in range(nblk):
            cols = blk == b
            Sb = Sm[:, cols]
            has = np.isfinite(Sb).any(axis=1)
            mb = np.where(has, np.max(np.where(np.isfinite(Sb), Sb, -np.inf), axis=1), 0.0)
            pb = np.where(np.isfinite(Sb), np.exp(Sb - mb[:, None]), 0.0)
            lb = pb.sum(axis=1)
            ob = bf16((bf16(pb) @ v[cols]) / np.where(has, lb, 1.0)[:, None])
            lseb = np.where(has, mb + np.log(np.where(has, lb, 1.0)), -np.inf)
            acc += np.where(has[:, None], np.exp(lseb - lse[:, 0])[:, None] * ob, 0.0)
        md["o"][:, h] = bf16(acc)
        # backward
        D = (dout[:, h] * o_stored[:, h]).sum(axis=1, keepdims=True)
        dP = dout[:, h] @ v.T
        Dx = (dout[:, h] * ex["o"][:, h]).sum(axis=1, keepdims=True)
        dS_ex = P * (dP - Dx)
        ex["dq"][:, h] = scale * dS_ex @ k
        ex["dk"] += scale * dS_ex.T @ q[:, h]
        ex["dv"] += P.T @ dout[:, h]
        dS16 = bf16(scale * P * (dP - D))
        md["dv"] += bf16(P).T @ dout[:, h]
        md["dk"] += dS16.T @ q[:, h]
        dqh = np.zeros((T, d))
        for b in range(nblk):
            cols = blk == b
            dqh += bf16(dS16[:, cols] @ k[cols])
        md["dq"][:, h] = bf16(dqh)
    md["dv"] = bf16(md["dv"])
    md["dk"] = bf16(md["dk"])
    return ex, md
