"""Seeded synthetic inputs for the MSA training hot path.

This module only draws random numbers.  It holds none of the method's
arithmetic, so both the CPU oracle (``oracle/``) and the HIP path
(``block_sparse_attention_qk_amd``) can be fed from it without sharing code.

Workload recipe (one entry per named configuration):

* Q, K, V, dO: iid N(0, 1), rounded to bf16 (round-to-nearest-even).
* proxy queries q_p: iid N(0, 1) -> bf16.
* proxy keys k_p: N(0, 1) plus a per-(batch, group, 128-key block) mean vector
  mu ~ N(0, 0.5) (variance 0.5), added in fp32 before the bf16 rounding.

Every tensor is drawn in chunks of ``CHUNK`` tokens.  Chunk ``c`` of tensor
``name`` uses a CPU ``torch.Generator`` seeded with
``0x5EED + 1_000_003 * TENSOR_ID[name] + c`` (plus ``seed_offset``), so any
token range can be regenerated on its own and memory stays bounded.

Layouts (row-major, contiguous): q, dout ``[B, T, H, d]``; k, v ``[B, T, G, d]``;
qp, kp ``[B, T, G, dp]``.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional

import torch

CHUNK = 4096          # tokens per independently seeded chunk
BLOCK = 128           # KV block size (tokens)
TENSOR_ID = {"q": 1, "k": 2, "v": 3, "dout": 4, "qp": 5, "kp": 6, "mu": 7}


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    B: int
    T: int
    H: int
    G: int
    d: int
    dp: int
    topk: int

    @property
    def N(self) -> int:
        return self.T // BLOCK

    @property
    def R(self) -> int:
        return self.H // self.G

    def pairs(self) -> int:
        """Number of (batch, group, token, selected block) pairs."""
        n = 0
        for i in range(self.N):
            n += min(self.topk, i + 1)
        return self.B * self.G * BLOCK * n

    def flops_fwd(self) -> float:
        """Executed sparse forward FLOPs: 4 * d * R * 128 per pair (QK^T and PV)."""
        return 4.0 * self.d * self.R * BLOCK * self.pairs()

    def flops_bwd(self) -> float:
        """Executed sparse backward FLOPs: 2.5x the forward (S, dP, dV, dK, dQ)."""
        return 2.5 * self.flops_fwd()

    def flops_proxy(self) -> float:
        """Proxy-score FLOPs, block-granular over the causal triangle: 2 * dp per scored pair."""
        nkeys = 0
        for i in range(self.N):
            nkeys += (i + 1) * BLOCK
        return self.B * self.G * BLOCK * nkeys * 2.0 * self.dp


CONFIGS: Dict[str, Config] = {
    "tiny": Config("tiny", 1, 1024, 4, 1, 64, 32, 4),
    "16k": Config("16k", 1, 16384, 16, 2, 128, 64, 16),
    "128k": Config("128k", 1, 131072, 32, 4, 128, 64, 32),
    "512k": Config("512k", 1, 524288, 32, 4, 128, 64, 64),
    "1m": Config("1m", 1, 1048576, 16, 2, 128, 64, 288),
}


def _gen(name: str, chunk: int, seed_offset: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(0x5EED + 1_000_003 * TENSOR_ID[name] + chunk + seed_offset)
    return g


def _normal_tokens(name: str, B: int, T: int, width: int, t0: int, t1: int,
                   seed_offset: int) -> torch.Tensor:
    """fp32 N(0,1) values of shape [B, t1-t0, width] for tokens [t0, t1)."""
    out = torch.empty((B, t1 - t0, width), dtype=torch.float32)
    c0, c1 = t0 // CHUNK, (t1 - 1) // CHUNK
    for b in range(B):
        for c in range(c0, c1 + 1):
            lo, hi = c * CHUNK, min((c + 1) * CHUNK, T)
            g = _gen(name, b * ((T + CHUNK - 1) // CHUNK) + c, seed_offset)
            vals = torch.randn((hi - lo, width), generator=g, dtype=torch.float32)
            a, z = max(lo, t0), min(hi, t1)
            out[b, a - t0:z - t0] = vals[a - lo:z - lo]
    return out


def block_means(B: int, T: int, G: int, dp: int, seed_offset: int = 0) -> torch.Tensor:
    """Per-(batch, block, group) proxy-key mean vectors, fp32 [B, N, G, dp], variance 0.5."""
    N = T // BLOCK
    g = _gen("mu", 0, seed_offset)
    return torch.randn((B, N, G, dp), generator=g, dtype=torch.float32) * math.sqrt(0.5)


def make_tensor(name: str, cfg: Config, t0: int = 0, t1: Optional[int] = None,
                seed_offset: int = 0) -> torch.Tensor:
    """One input tensor (bf16, CPU) restricted to tokens [t0, t1)."""
    t1 = cfg.T if t1 is None else t1
    B, T = cfg.B, cfg.T
    if name in ("q", "dout"):
        x = _normal_tokens(name, B, T, cfg.H * cfg.d, t0, t1, seed_offset)
        return x.view(B, t1 - t0, cfg.H, cfg.d).to(torch.bfloat16)
    if name in ("k", "v"):
        x = _normal_tokens(name, B, T, cfg.G * cfg.d, t0, t1, seed_offset)
        return x.view(B, t1 - t0, cfg.G, cfg.d).to(torch.bfloat16)
    if name == "qp":
        x = _normal_tokens(name, B, T, cfg.G * cfg.dp, t0, t1, seed_offset)
        return x.view(B, t1 - t0, cfg.G, cfg.dp).to(torch.bfloat16)
    if name == "kp":
        x = _normal_tokens(name, B, T, cfg.G * cfg.dp, t0, t1, seed_offset)
        x = x.view(B, t1 - t0, cfg.G, cfg.dp)
        mu = block_means(B, T, cfg.G, cfg.dp, seed_offset)
        blk = torch.arange(t0, t1) // BLOCK
        x = x + mu[:, blk]
        return x.to(torch.bfloat16)
    raise KeyError(name)


def make_inputs(cfg: Config, names=("qp", "kp", "q", "k", "v", "dout"),
                seed_offset: int = 0) -> Dict[str, torch.Tensor]:
    """All requested inputs of a configuration as bf16 CPU tensors."""
    return {n: make_tensor(n, cfg, seed_offset=seed_offset) for n in names}


def custom(B: int, T: int, H: int, G: int, d: int, dp: int, topk: int, name: str = "custom") -> Config:
    return Config(name, B, T, H, G, d, dp, topk)
