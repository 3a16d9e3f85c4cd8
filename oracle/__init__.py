"""CPU oracle for the MSA training hot path (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  It wraps ``msa_oracle.c`` (plain C,
OpenMP, fp64 main branch) through ctypes and shares no code with the HIP path.

Array conventions (all row-major):
  qp, kp: [B, T, G, dp]      q, dout: [B, T, H, d]      k, v: [B, T, G, d]
  idx:    [B, G, T, topk] int32, ascending block ids, -1 padded
Inputs may be torch tensors (any float dtype, bf16 included) or numpy arrays;
they are converted to float64 before the call, which is exact for bf16.

Parity unpinned against the pages: the pages print no worked example or
reference value for any part of the method.  select, fwd and bwd are pinned
by the mathematics instead (brute force, closed forms, invariants, library
routines and finite differences; tests/test_oracle_*.py and tests/golden/).
pattern_select, decode_select and decode_fwd follow readings of pages that
define neither, so beyond those pins they are parity unpinned.
"""
from __future__ import annotations

import ctypes
import dataclasses
import math
import os
import subprocess
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "msa_oracle.c")
_LIB = os.path.join(_HERE, "libmsa_oracle.so")
_lib = None

BLOCK = 128


@dataclasses.dataclass
class Dims:
    B: int
    T: int
    H: int
    G: int
    d: int
    dp: int
    topk: int
    scale: float = 0.0  # <= 0 means 1/sqrt(d)

    def eff_scale(self) -> float:
        return self.scale if self.scale > 0 else 1.0 / math.sqrt(self.d)


class _CDims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in ("B", "T", "H", "G", "d", "dp", "topk")] + [
        ("scale", ctypes.c_double)]


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (-O2, OpenMP) into oracle/libmsa_oracle.so."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                               "-Wall", "-Wno-unknown-pragmas", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        D = ctypes.POINTER(_CDims)
        lib.msa_oracle_select.argtypes = [D, P, P, I64, P, P, P]
        lib.msa_oracle_fwd.argtypes = [D, P, P, P, P, I64, P, P, P]
        lib.msa_oracle_bwd_rows.argtypes = [D, P, P, P, P, P, I64, P, P]
        lib.msa_oracle_bwd_blocks.argtypes = [D, P, P, P, P, P, I64, P, P, P]
        lib.msa_oracle_bwd.argtypes = [D, P, P, P, P, P, P, P, P]
        for f in ("msa_oracle_select", "msa_oracle_fwd", "msa_oracle_bwd_rows",
                  "msa_oracle_bwd_blocks", "msa_oracle_bwd"):
            getattr(lib, f).restype = ctypes.c_int
        lib.msa_oracle_max_threads.restype = ctypes.c_int
        lib.msa_oracle_set_threads.argtypes = [ctypes.c_int]
        _lib = lib
    return _lib


def max_threads() -> int:
    return int(_load().msa_oracle_max_threads())


def set_threads(n: int) -> None:
    _load().msa_oracle_set_threads(int(n))


def _f64(x) -> np.ndarray:
    try:
        import torch
        if isinstance(x, torch.Tensor):
            return np.ascontiguousarray(x.detach().to("cpu", torch.float64).numpy())
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _i32(x) -> np.ndarray:
    try:
        import torch
        if isinstance(x, torch.Tensor):
            return np.ascontiguousarray(x.detach().to("cpu", torch.int32).numpy())
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(x, dtype=np.int32))


def _rows(rows, total) -> Tuple[int, Optional[np.ndarray]]:
    if rows is None:
        return total, None
    r = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    return int(r.size), r


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _cdims(dm: Dims) -> _CDims:
    return _CDims(dm.B, dm.T, dm.H, dm.G, dm.d, dm.dp, dm.topk, dm.eff_scale())


def _check(rc: int, what: str) -> None:
    if rc != 0:
        names = {1: "bad dimensions or arguments", 2: "invalid block index row",
                 3: "allocation failure", 4: "row out of range"}
        raise ValueError("oracle %s failed: %s" % (what, names.get(rc, rc)))


def select(dm: Dims, qp, kp, rows=None, return_pooled: bool = False):
    """Index Branch.  rows=None: idx [B,G,T,topk]; else idx [n_rows,G,topk] for
    the token rows (b*T + t).  With return_pooled, also the fp32 pooled scores
    ([..., ceil(T/128)], -inf past the causal blocks)."""
    lib = _load()
    qp64, kp64 = _f64(qp), _f64(kp)
    n, r = _rows(rows, dm.B * dm.T)
    N = (dm.T + BLOCK - 1) // BLOCK
    idx = np.empty((n, dm.G, dm.topk), dtype=np.int32)
    pooled = np.empty((n, dm.G, N), dtype=np.float32) if return_pooled else None
    cd = _cdims(dm)
    _check(lib.msa_oracle_select(ctypes.byref(cd), _ptr(qp64), _ptr(kp64), n, _ptr(r),
                                 _ptr(idx), _ptr(pooled)), "select")
    if rows is None:
        idx = idx.reshape(dm.B, dm.T, dm.G, dm.topk).transpose(0, 2, 1, 3).copy()
        if pooled is not None:
            pooled = pooled.reshape(dm.B, dm.T, dm.G, N).transpose(0, 2, 1, 3).copy()
    return (idx, pooled) if return_pooled else idx


def fwd(dm: Dims, q, k, v, idx, rows=None):
    """Main Branch forward.  Returns (o, lse) as float64: rows=None gives
    o [B,T,H,d], lse [B,T,H]; else o [n_rows,H,d], lse [n_rows,H]."""
    lib = _load()
    q64, k64, v64, ix = _f64(q), _f64(k), _f64(v), _i32(idx)
    n, r = _rows(rows, dm.B * dm.T)
    o = np.empty((n, dm.H, dm.d), dtype=np.float64)
    lse = np.empty((n, dm.H), dtype=np.float64)
    cd = _cdims(dm)
    _check(lib.msa_oracle_fwd(ctypes.byref(cd), _ptr(q64), _ptr(k64), _ptr(v64), _ptr(ix), n,
                              _ptr(r), _ptr(o), _ptr(lse)), "fwd")
    if rows is None:
        o = o.reshape(dm.B, dm.T, dm.H, dm.d)
        lse = lse.reshape(dm.B, dm.T, dm.H)
    return o, lse


def bwd_rows(dm: Dims, q, k, v, dout, idx, rows=None):
    """dQ rows of the Main Branch backward (loss L = sum(O * dout))."""
    lib = _load()
    q64, k64, v64, do64, ix = _f64(q), _f64(k), _f64(v), _f64(dout), _i32(idx)
    n, r = _rows(rows, dm.B * dm.T)
    dq = np.empty((n, dm.H, dm.d), dtype=np.float64)
    cd = _cdims(dm)
    _check(lib.msa_oracle_bwd_rows(ctypes.byref(cd), _ptr(q64), _ptr(k64), _ptr(v64), _ptr(do64),
                                   _ptr(ix), n, _ptr(r), _ptr(dq)), "bwd_rows")
    if rows is None:
        dq = dq.reshape(dm.B, dm.T, dm.H, dm.d)
    return dq


def bwd_blocks(dm: Dims, q, k, v, dout, idx, blocks):
    """dK, dV of the listed key blocks ((b*G + g)*N + blk) as [n, 128, d]."""
    lib = _load()
    q64, k64, v64, do64, ix = _f64(q), _f64(k), _f64(v), _f64(dout), _i32(idx)
    bl = np.ascontiguousarray(np.asarray(blocks, dtype=np.int64))
    dk = np.empty((bl.size, BLOCK, dm.d), dtype=np.float64)
    dv = np.empty((bl.size, BLOCK, dm.d), dtype=np.float64)
    cd = _cdims(dm)
    _check(lib.msa_oracle_bwd_blocks(ctypes.byref(cd), _ptr(q64), _ptr(k64), _ptr(v64), _ptr(do64),
                                     _ptr(ix), bl.size, _ptr(bl), _ptr(dk), _ptr(dv)), "bwd_blocks")
    return dk, dv


def bwd(dm: Dims, q, k, v, dout, idx):
    """Full Main Branch backward: (dq [B,T,H,d], dk [B,T,G,d], dv [B,T,G,d])."""
    lib = _load()
    q64, k64, v64, do64, ix = _f64(q), _f64(k), _f64(v), _f64(dout), _i32(idx)
    dq = np.empty((dm.B, dm.T, dm.H, dm.d), dtype=np.float64)
    dk = np.empty((dm.B, dm.T, dm.G, dm.d), dtype=np.float64)
    dv = np.empty((dm.B, dm.T, dm.G, dm.d), dtype=np.float64)
    cd = _cdims(dm)
    _check(lib.msa_oracle_bwd(ctypes.byref(cd), _ptr(q64), _ptr(k64), _ptr(v64), _ptr(do64),
                              _ptr(ix), _ptr(dq), _ptr(dk), _ptr(dv)), "bwd")
    return dq, dk, dv


def pattern_select(B: int, T: int, G: int, window: int, dilation: int, width: int, idx_in=None) -> np.ndarray:
    """Fixed window/dilation block pattern, optionally united with a cache.

    Follows the reading of keelcrux "Flash-MSA: Train on a million tokens without
    breaking the compute bank", section "Under the hood" (the block pattern is
    configurable by window size and dilation; the page defines neither): for
    query t with nc = t//128 + 1 causal blocks, the row holds, once each and in
    ascending order, the `window` most recent causal blocks, every causal block
    below the window whose index is a multiple of `dilation` (none when 0), and
    the causal entries of idx_in[b, g, t, :]; the rest of the row is -1.
    Plain per-row set construction (test infrastructure only).
    Parity unpinned against the pages (they give no example of the pattern):
    pinned by hand-worked rows, cases that must select every causal block, the
    empty pattern, and an independent boolean-mask formulation.
    """
    out = np.full((B, G, T, width), -1, dtype=np.int32)
    ii = None if idx_in is None else _i32(idx_in)
    for b in range(B):
        for g in range(G):
            for t in range(T):
                nc = t // BLOCK + 1
                lo = max(0, nc - window)
                chosen = set(range(lo, nc))
                if dilation > 0:
                    chosen.update(blk for blk in range(0, lo) if blk % dilation == 0)
                if ii is not None:
                    chosen.update(int(blk) for blk in ii[b, g, t] if 0 <= blk < nc)
                row = sorted(chosen)
                if len(row) > width:
                    raise ValueError("pattern row of %d blocks exceeds width %d" % (len(row), width))
                out[b, g, t, :len(row)] = row
    return out


def _decode_len(lens, B: int, T: int) -> np.ndarray:
    ln = np.asarray(lens, dtype=np.int64).reshape(-1)
    if ln.size != B:
        raise ValueError("lens must hold B = %d entries" % B)
    return ln


def decode_select(dm: Dims, qp, kp, lens):
    """Index Branch of a decode step (ai-beat "flash-msa-sparse-attention-training",
    paragraph 1: MSA also serves inference).  Sequence b has lens[b] cached
    tokens, the new one last, at t = lens[b] - 1; its proxy query qp[b] ([B,G,dp])
    is row t of the sequence whose proxy keys are kp[b, :t+1] ([B,T,G,dp] cache
    of capacity dm.T).  The row is selected exactly as a training row (select()
    on that prefix).  Returns (idx [B,G,topk] int32, pooled [B,G,T/128] fp32,
    -inf past the causal blocks); sequences with lens outside 1..T give an all -1
    row and -inf scores.  Parity unpinned against the pages (no decode example
    is printed): pinned to the training rows and a hand-built ranking."""
    qp64, kp64 = _f64(qp), _f64(kp)
    ln = _decode_len(lens, dm.B, dm.T)
    N = (dm.T + BLOCK - 1) // BLOCK
    idx = np.full((dm.B, dm.G, dm.topk), -1, dtype=np.int32)
    pooled = np.full((dm.B, dm.G, N), -np.inf, dtype=np.float32)
    for b in range(dm.B):
        L = int(ln[b])
        if L < 1 or L > dm.T:
            continue
        qrow = np.zeros((1, L, dm.G, dm.dp), dtype=np.float64)
        qrow[0, L - 1] = qp64[b]
        ib, pb = select(Dims(1, L, dm.H, dm.G, dm.d, dm.dp, dm.topk, dm.scale), qrow, kp64[b:b + 1, :L],
                        rows=[L - 1], return_pooled=True)
        idx[b] = ib[0]
        pooled[b, :, :pb.shape[2]] = pb[0]
    return idx, pooled


def decode_fwd(dm: Dims, q, k, v, lens, idx):
    """Main Branch of a decode step: for sequence b the new query heads q[b]
    ([B,H,d]) are row t = lens[b] - 1 of the sequence whose keys and values are
    k[b, :t+1], v[b, :t+1] ([B,T,G,d] caches), attending over the blocks of
    idx[b] ([B,G,topk]) exactly as fwd() does for a training row (one call per
    group).  Entries that are -1 or above t/128 are dropped first.  Returns
    (o [B,H,d], lse [B,H]) in float64; a group whose row keeps no entry, or a
    sequence with lens outside 1..T, gives o = 0, lse = -inf.  Parity unpinned
    against the pages (no decode example is printed): pinned to a plain float64
    softmax over the prefix and to the training rows."""
    q64, k64, v64 = _f64(q), _f64(k), _f64(v)
    ix = _i32(idx)
    ln = _decode_len(lens, dm.B, dm.T)
    R = dm.H // dm.G
    o = np.zeros((dm.B, dm.H, dm.d), dtype=np.float64)
    lse = np.full((dm.B, dm.H), -np.inf, dtype=np.float64)
    for b in range(dm.B):
        L = int(ln[b])
        if L < 1 or L > dm.T:
            continue
        t = L - 1
        for g in range(dm.G):
            ent = sorted(int(e) for e in ix[b, g] if 0 <= e <= t // BLOCK)
            if not ent:
                continue
            row = np.full((1, 1, L, dm.topk), -1, dtype=np.int32)
            row[0, 0, t, :len(ent)] = ent
            qg = np.zeros((1, L, R, dm.d), dtype=np.float64)
            qg[0, t] = q64[b, g * R:(g + 1) * R]
            og, lg = fwd(Dims(1, L, R, 1, dm.d, dm.dp, dm.topk, dm.scale), qg,
                         np.ascontiguousarray(k64[b:b + 1, :L, g:g + 1]),
                         np.ascontiguousarray(v64[b:b + 1, :L, g:g + 1]), row, rows=[t])
            o[b, g * R:(g + 1) * R] = og[0]
            lse[b, g * R:(g + 1) * R] = lg[0]
    return o, lse
