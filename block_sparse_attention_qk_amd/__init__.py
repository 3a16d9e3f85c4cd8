"""MiniMax Sparse Attention (MSA) training hot path on MI355X (gfx950).

Thin Python binding of ``libmsa.so``, whose C ABI is declared in
``include/msa.h``.  The binding only marshals arguments: it checks tensor
dtypes, devices and shapes, sizes the caller-owned workspace with
``torch.empty`` and passes raw device pointers and the current HIP stream.
Every step of the path runs in the library's HIP kernels; there is no
fallback.  Importing this module needs the built library (``build.py``); a
missing library raises ``MsaError`` on first use.

Entry points (same names as the C ABI):
  msa_proxy_select(qp, kp, topk)               -> idx            (Index Branch)
  msa_fwd(q, k, v, idx, scale=0.0)             -> (o, lse)       (Main Branch forward)
  msa_bwd(q, k, v, o, dout, lse, idx, scale)   -> (dq, dk, dv)   (Main Branch backward)
  msa_fwd_bwd(q, k, v, dout, idx, scale)       -> (o, lse, dq, dk, dv)  (merged forward + backward)
  msa_pattern_select(B, T, G, window, dilation, idx_in) -> idx   (fixed block pattern)
  msa_decode_select(qp, kp, lens, topk)        -> idx            (decode step, Index Branch)
  msa_decode_fwd(q, k, v, lens, idx, scale)    -> (o, lse)       (decode step, Main Branch)
  msa_decode_fwd_static(q, k, v, lens, idx)    -> (o, lse)       (the same without a workspace)
Layouts: qp, kp [B,T,G,dp] bf16; q, o, dout [B,T,H,d] bf16; k, v [B,T,G,d] bf16;
idx [B,G,T,topk] int32; lse [B,T,H] fp32.  Decode: qp [B,G,dp], q and o [B,H,d],
caches kp/k/v [B,T,G,*], lens [B] int32 (on the device), idx [B,G,topk], lse [B,H].
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

__all__ = [
    "MsaError", "Workspace", "lib_path", "load", "msa_workspace_bytes", "msa_workspace_min_bytes",
    "msa_proxy_select", "msa_pattern_select", "pattern_width", "msa_fwd", "msa_bwd", "msa_fwd_bwd",
    "msa_decode_select", "msa_decode_fwd", "msa_decode_fwd_static", "STATIC_SCRATCH_BYTES", "OP_SELECT", "OP_FWD", "OP_BWD", "OP_DECODE_SELECT", "OP_DECODE_FWD",
    "OP_FWD_BWD", "EXPORTED_SYMBOLS",
    "KERNEL_NAMES", "timing_enable", "timing_read",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libmsa.so")
_lib = None

OP_SELECT, OP_FWD, OP_BWD, OP_DECODE_SELECT, OP_DECODE_FWD, OP_FWD_BWD = 0, 1, 2, 3, 4, 5
EXPORTED_SYMBOLS = ("msa_workspace_bytes", "msa_workspace_min_bytes", "msa_proxy_select", "msa_pattern_select",
                    "msa_fwd", "msa_bwd", "msa_fwd_bwd", "msa_decode_select", "msa_decode_fwd",
                    "msa_decode_fwd_static", "msa_status_str", "msa_version", "msa_timing_enable", "msa_timing_read")
STATIC_SCRATCH_BYTES = 16 << 20  # MSA_STATIC_SCRATCH_BYTES (include/msa.h)

# msa_kernel_id values (include/msa.h)
KERNEL_NAMES = ("proxy_pool", "topk", "inverse", "fwd_partials", "fwd_combine", "bwd_dot", "bwd_partials",
                "dq_combine", "convert", "pattern", "dec_pool", "dec_topk", "dec_attn", "dec_combine")


class MsaError(RuntimeError):
    """Raised for a non-zero msa_status or a missing library."""


class _Dims(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("T", ctypes.c_int32), ("H", ctypes.c_int32), ("G", ctypes.c_int32),
                ("d", ctypes.c_int32), ("dp", ctypes.c_int32), ("topk", ctypes.c_int32),
                ("scale", ctypes.c_float)]


def lib_path() -> str:
    return _LIB_PATH


def load():
    """Load libmsa.so (once) and declare the C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise MsaError("libmsa.so is not built (%s); run block_sparse_attention_qk_amd/build.py" % _LIB_PATH)
    lib = ctypes.CDLL(_LIB_PATH)
    P, D, SZ, I = ctypes.c_void_p, ctypes.POINTER(_Dims), ctypes.c_size_t, ctypes.c_int
    lib.msa_workspace_bytes.argtypes = [D, I]
    lib.msa_workspace_bytes.restype = SZ
    lib.msa_workspace_min_bytes.argtypes = [D, I]
    lib.msa_workspace_min_bytes.restype = SZ
    lib.msa_proxy_select.argtypes = [D, P, P, P, P, SZ, P]
    lib.msa_pattern_select.argtypes = [D, ctypes.c_int32, ctypes.c_int32, P, ctypes.c_int32, P, P]
    lib.msa_fwd.argtypes = [D, P, P, P, P, P, P, P, SZ, P]
    lib.msa_bwd.argtypes = [D, P, P, P, P, P, P, P, P, P, P, P, SZ, P]
    lib.msa_fwd_bwd.argtypes = [D, P, P, P, P, P, P, P, P, P, P, P, SZ, P]
    lib.msa_decode_select.argtypes = [D, P, P, P, P, P, SZ, P]
    lib.msa_decode_fwd.argtypes = [D, P, P, P, P, P, P, P, P, SZ, P]
    lib.msa_decode_fwd_static.argtypes = [D, P, P, P, P, P, P, P, P]
    for f in ("msa_proxy_select", "msa_pattern_select", "msa_fwd", "msa_bwd", "msa_fwd_bwd", "msa_decode_select",
              "msa_decode_fwd", "msa_decode_fwd_static"):
        getattr(lib, f).restype = I
    lib.msa_status_str.argtypes = [I]
    lib.msa_status_str.restype = ctypes.c_char_p
    lib.msa_version.restype = ctypes.c_char_p
    lib.msa_timing_enable.argtypes = [I]
    lib.msa_timing_enable.restype = None
    lib.msa_timing_read.argtypes = [P, P, ctypes.c_int32]
    lib.msa_timing_read.restype = I
    _lib = lib
    return lib


def _dims(B, T, H, G, d, dp, topk, scale) -> _Dims:
    return _Dims(int(B), int(T), int(H), int(G), int(d), int(dp), int(topk), float(scale))


def _check(rc: int) -> None:
    if rc != 0:
        raise MsaError("libmsa error %d: %s" % (rc, load().msa_status_str(rc).decode()))


def msa_workspace_bytes(B, T, H, G, d, dp, topk, op, scale: float = 0.0) -> int:
    return int(load().msa_workspace_bytes(ctypes.byref(_dims(B, T, H, G, d, dp, topk, scale)), op))


def msa_workspace_min_bytes(B, T, H, G, d, dp, topk, op, scale: float = 0.0) -> int:
    return int(load().msa_workspace_min_bytes(ctypes.byref(_dims(B, T, H, G, d, dp, topk, scale)), op))


def timing_enable(on: bool = True) -> None:
    """Turn the library's per-launch HIP-event timing on or off (clears it)."""
    load().msa_timing_enable(1 if on else 0)


def timing_read() -> dict:
    """{kernel name: (total ms, launches)} for launches timed since timing_enable."""
    n = len(KERNEL_NAMES)
    ms = (ctypes.c_double * n)()
    cnt = (ctypes.c_int32 * n)()
    _check(load().msa_timing_read(ms, cnt, n))
    return {KERNEL_NAMES[i]: (float(ms[i]), int(cnt[i])) for i in range(n)}


class Workspace:
    """Device scratch buffer that grows on demand (owned by the caller)."""

    def __init__(self, device=None, nbytes: int = 0):
        self.device = torch.device(device) if device is not None else torch.device("cuda")
        self.buf = torch.empty(0, dtype=torch.uint8, device=self.device)
        if nbytes:
            self.get(nbytes)

    def get(self, nbytes: int) -> torch.Tensor:
        if self.buf.numel() < nbytes:
            self.buf = torch.empty(int(nbytes), dtype=torch.uint8, device=self.device)
        return self.buf


def _ptr(t: torch.Tensor) -> int:
    return t.data_ptr()


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _need(t: torch.Tensor, name: str, dtype, ndim: int) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if t.dim() != ndim:
        raise ValueError("%s must have %d dims, got shape %s" % (name, ndim, tuple(t.shape)))
    if t.device.type != "cuda":
        raise ValueError("%s must be on a GPU device" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def _same_device(device, *named) -> None:
    """Every tensor of a call must live on the device of its first input."""
    for t, name in named:
        if t is not None and t.device != device:
            raise ValueError("%s is on %s, the call's inputs on %s" % (name, t.device, device))


def _out(t: torch.Tensor, name: str, dtype, shape, device) -> torch.Tensor:
    """A caller-provided output: the kernels write exactly `shape` elements into it."""
    _need(t, name, dtype, len(shape))
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))
    _same_device(device, (t, name))
    return t


def _ws(ws: Optional[Workspace], device, nbytes: int) -> torch.Tensor:
    if ws is None:
        return torch.empty(int(nbytes), dtype=torch.uint8, device=device)
    buf = ws.get(nbytes)
    if buf.device != device:
        raise ValueError("workspace is on %s, the call's inputs on %s" % (buf.device, device))
    return buf


def msa_proxy_select(qp: torch.Tensor, kp: torch.Tensor, topk: int, ws: Optional[Workspace] = None,
                     out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Index Branch: block-index cache idx [B,G,T,topk] int32 (ascending, -1 padded)."""
    _need(qp, "qp", torch.bfloat16, 4)
    _need(kp, "kp", torch.bfloat16, 4)
    if qp.shape != kp.shape:
        raise ValueError("qp and kp shapes differ: %s vs %s" % (tuple(qp.shape), tuple(kp.shape)))
    B, T, G, dp = qp.shape
    _same_device(qp.device, (kp, "kp"))
    dims = _dims(B, T, G, G, 64, dp, topk, 0.0)
    lib = load()
    nbytes = lib.msa_workspace_bytes(ctypes.byref(dims), OP_SELECT)
    if nbytes == 0:
        _check(2)
    if out is not None:
        idx = _out(out, "out", torch.int32, (B, G, T, topk), qp.device)
    else:
        idx = torch.empty((B, G, T, topk), dtype=torch.int32, device=qp.device)
    w = _ws(ws, qp.device, nbytes)
    _check(lib.msa_proxy_select(ctypes.byref(dims), _ptr(qp), _ptr(kp), _ptr(idx), _ptr(w), w.numel(),
                                _stream(qp.device)))
    return idx


def pattern_width(T: int, window: int, dilation: int, k_in: int = 0) -> int:
    """Largest row msa_pattern_select can produce (the smallest accepted output width)."""
    N = T // 128
    far = (max(0, N - window) + dilation - 1) // dilation if dilation > 0 else 0
    return min(N, min(window, N) + far + k_in)


def msa_pattern_select(B: int, T: int, G: int, window: int, dilation: int, idx_in: Optional[torch.Tensor] = None,
                       width: Optional[int] = None, device=None, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Fixed window/dilation block pattern, optionally united with the cache idx_in [B,G,T,k_in]:
    returns the block-index cache [B,G,T,width] int32 (ascending, -1 padded)."""
    k_in = 0
    if idx_in is not None:
        _need(idx_in, "idx_in", torch.int32, 4)
        if tuple(idx_in.shape[:3]) != (B, G, T):
            raise ValueError("idx_in shape %s does not match [B,G,T,*] = [%d,%d,%d,*]" % (tuple(idx_in.shape), B, G, T))
        k_in = idx_in.shape[3]
        device = idx_in.device
    if width is None:
        width = pattern_width(T, window, dilation, k_in)
    if out is None:
        out = torch.empty((B, G, T, width), dtype=torch.int32, device=device if device is not None else "cuda")
    else:
        _out(out, "out", torch.int32, (B, G, T, width), idx_in.device if idx_in is not None else out.device)
    dims = _dims(B, T, G, G, 64, 32, width, 0.0)
    _check(load().msa_pattern_select(ctypes.byref(dims), int(window), int(dilation),
                                     _ptr(idx_in) if idx_in is not None else None, int(k_in), _ptr(out),
                                     _stream(out.device)))
    return out


def _main_dims(q, k, idx, scale) -> Tuple[_Dims, int, int, int, int, int, int]:
    B, T, H, d = q.shape
    if k.dim() != 4 or k.shape[0] != B or k.shape[1] != T or k.shape[3] != d:
        raise ValueError("k shape %s does not match q shape %s" % (tuple(k.shape), tuple(q.shape)))
    G = k.shape[2]
    if idx.dim() != 4 or tuple(idx.shape[:3]) != (B, G, T):
        raise ValueError("idx shape %s does not match [B,G,T,topk] = [%d,%d,%d,*]" % (tuple(idx.shape), B, G, T))
    topk = idx.shape[3]
    return _dims(B, T, H, G, d, 32, topk, scale), B, T, H, G, d, topk


def msa_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, idx: torch.Tensor, scale: float = 0.0,
            ws: Optional[Workspace] = None, out: Optional[Tuple[torch.Tensor, torch.Tensor]] = None):
    """Main Branch forward: (o [B,T,H,d] bf16, lse [B,T,H] fp32)."""
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, n, torch.bfloat16, 4)
    _need(idx, "idx", torch.int32, 4)
    if v.shape != k.shape:
        raise ValueError("v shape %s differs from k shape %s" % (tuple(v.shape), tuple(k.shape)))
    dims, B, T, H, G, d, topk = _main_dims(q, k, idx, scale)
    _same_device(q.device, (k, "k"), (v, "v"), (idx, "idx"))
    lib = load()
    nbytes = lib.msa_workspace_bytes(ctypes.byref(dims), OP_FWD)
    if nbytes == 0:
        _check(2)
    if out is None:
        o = torch.empty((B, T, H, d), dtype=torch.bfloat16, device=q.device)
        lse = torch.empty((B, T, H), dtype=torch.float32, device=q.device)
    else:
        o = _out(out[0], "out[0] (o)", torch.bfloat16, (B, T, H, d), q.device)
        lse = _out(out[1], "out[1] (lse)", torch.float32, (B, T, H), q.device)
    w = _ws(ws, q.device, nbytes)
    _check(lib.msa_fwd(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(idx), _ptr(o), _ptr(lse), _ptr(w),
                       w.numel(), _stream(q.device)))
    return o, lse


def msa_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor, dout: torch.Tensor,
            lse: torch.Tensor, idx: torch.Tensor, scale: float = 0.0, ws: Optional[Workspace] = None,
            out: Optional[Tuple[torch.Tensor, torch.Tensor, torch.Tensor]] = None):
    """Main Branch backward of sum(o * dout): (dq, dk, dv) in bf16."""
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (dout, "dout")):
        _need(t, n, torch.bfloat16, 4)
    _need(lse, "lse", torch.float32, 3)
    _need(idx, "idx", torch.int32, 4)
    if v.shape != k.shape or o.shape != q.shape or dout.shape != q.shape or lse.shape != q.shape[:3]:
        raise ValueError("inconsistent shapes for msa_bwd")
    dims, B, T, H, G, d, topk = _main_dims(q, k, idx, scale)
    _same_device(q.device, (k, "k"), (v, "v"), (o, "o"), (dout, "dout"), (lse, "lse"), (idx, "idx"))
    lib = load()
    nbytes = lib.msa_workspace_bytes(ctypes.byref(dims), OP_BWD)
    if nbytes == 0:
        _check(2)
    if out is None:
        dq = torch.empty_like(q)
        dk = torch.empty_like(k)
        dv = torch.empty_like(v)
    else:
        dq = _out(out[0], "out[0] (dq)", torch.bfloat16, tuple(q.shape), q.device)
        dk = _out(out[1], "out[1] (dk)", torch.bfloat16, tuple(k.shape), q.device)
        dv = _out(out[2], "out[2] (dv)", torch.bfloat16, tuple(k.shape), q.device)
    w = _ws(ws, q.device, nbytes)
    _check(lib.msa_bwd(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(idx),
                       _ptr(dq), _ptr(dk), _ptr(dv), _ptr(w), w.numel(), _stream(q.device)))
    return dq, dk, dv


def msa_fwd_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, dout: torch.Tensor, idx: torch.Tensor,
                scale: float = 0.0, ws: Optional[Workspace] = None, out=None):
    """Merged forward + backward: (o, lse, dq, dk, dv), as msa_fwd followed by
    msa_bwd on that o, with one inverse index per window and D fused."""
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (dout, "dout")):
        _need(t, n, torch.bfloat16, 4)
    _need(idx, "idx", torch.int32, 4)
    if v.shape != k.shape or dout.shape != q.shape:
        raise ValueError("inconsistent shapes for msa_fwd_bwd")
    dims, B, T, H, G, d, topk = _main_dims(q, k, idx, scale)
    _same_device(q.device, (k, "k"), (v, "v"), (dout, "dout"), (idx, "idx"))
    lib = load()
    nbytes = lib.msa_workspace_bytes(ctypes.byref(dims), OP_FWD_BWD)
    if nbytes == 0:
        _check(2)
    if out is None:
        o = torch.empty_like(q)
        lse = torch.empty((B, T, H), dtype=torch.float32, device=q.device)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    else:
        o = _out(out[0], "out[0] (o)", torch.bfloat16, tuple(q.shape), q.device)
        lse = _out(out[1], "out[1] (lse)", torch.float32, (B, T, H), q.device)
        dq = _out(out[2], "out[2] (dq)", torch.bfloat16, tuple(q.shape), q.device)
        dk = _out(out[3], "out[3] (dk)", torch.bfloat16, tuple(k.shape), q.device)
        dv = _out(out[4], "out[4] (dv)", torch.bfloat16, tuple(k.shape), q.device)
    w = _ws(ws, q.device, nbytes)
    _check(lib.msa_fwd_bwd(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(idx), _ptr(o), _ptr(lse),
                           _ptr(dq), _ptr(dk), _ptr(dv), _ptr(w), w.numel(), _stream(q.device)))
    return o, lse, dq, dk, dv


def _lens(lens: torch.Tensor, B: int, device) -> None:
    _need(lens, "lens", torch.int32, 1)
    if lens.shape[0] != B:
        raise ValueError("lens must hold B = %d entries, got %d" % (B, lens.shape[0]))
    if lens.device != device:
        raise ValueError("lens must be on %s" % device)


def msa_decode_select(qp: torch.Tensor, kp: torch.Tensor, lens: torch.Tensor, topk: int,
                      ws: Optional[Workspace] = None, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Decode-step Index Branch: qp [B,G,dp] (the new tokens), kp cache [B,T,G,dp],
    lens [B] int32 (cached tokens incl. the new one) -> idx [B,G,topk] int32."""
    _need(qp, "qp", torch.bfloat16, 3)
    _need(kp, "kp", torch.bfloat16, 4)
    B, G, dp = qp.shape
    if kp.shape[0] != B or kp.shape[2] != G or kp.shape[3] != dp:
        raise ValueError("kp shape %s does not match qp shape %s" % (tuple(kp.shape), tuple(qp.shape)))
    T = kp.shape[1]
    _lens(lens, B, qp.device)
    dims = _dims(B, T, G, G, 64, dp, topk, 0.0)
    lib = load()
    nbytes = lib.msa_workspace_bytes(ctypes.byref(dims), OP_DECODE_SELECT)
    if nbytes == 0:
        _check(2)
    _same_device(qp.device, (kp, "kp"))
    if out is not None:
        idx = _out(out, "out", torch.int32, (B, G, topk), qp.device)
    else:
        idx = torch.empty((B, G, topk), dtype=torch.int32, device=qp.device)
    w = _ws(ws, qp.device, nbytes)
    _check(lib.msa_decode_select(ctypes.byref(dims), _ptr(qp), _ptr(kp), _ptr(lens), _ptr(idx), _ptr(w), w.numel(),
                                 _stream(qp.device)))
    return idx


def _decode_fwd_args(q, k, v, lens, idx, scale, out):
    _need(q, "q", torch.bfloat16, 3)
    _need(k, "k", torch.bfloat16, 4)
    _need(v, "v", torch.bfloat16, 4)
    _need(idx, "idx", torch.int32, 3)
    B, H, d = q.shape
    if v.shape != k.shape or k.shape[0] != B or k.shape[3] != d:
        raise ValueError("k/v shapes %s, %s do not match q shape %s" % (tuple(k.shape), tuple(v.shape),
                                                                       tuple(q.shape)))
    T, G = k.shape[1], k.shape[2]
    if idx.shape[0] != B or idx.shape[1] != G:
        raise ValueError("idx shape %s does not match [B,G,topk] = [%d,%d,*]" % (tuple(idx.shape), B, G))
    _lens(lens, B, q.device)
    _same_device(q.device, (k, "k"), (v, "v"), (idx, "idx"))
    dims = _dims(B, T, H, G, d, 32, idx.shape[2], scale)
    nbytes = load().msa_workspace_bytes(ctypes.byref(dims), OP_DECODE_FWD)
    if nbytes == 0:
        _check(2)
    if out is None:
        o = torch.empty((B, H, d), dtype=torch.bfloat16, device=q.device)
        lse = torch.empty((B, H), dtype=torch.float32, device=q.device)
    else:
        o = _out(out[0], "out[0] (o)", torch.bfloat16, (B, H, d), q.device)
        lse = _out(out[1], "out[1] (lse)", torch.float32, (B, H), q.device)
    return dims, nbytes, o, lse


def msa_decode_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, lens: torch.Tensor, idx: torch.Tensor,
                   scale: float = 0.0, ws: Optional[Workspace] = None,
                   out: Optional[Tuple[torch.Tensor, torch.Tensor]] = None):
    """Decode-step Main Branch: q [B,H,d] (the new tokens), k/v caches [B,T,G,d],
    lens [B] int32, idx [B,G,topk] -> (o [B,H,d] bf16, lse [B,H] fp32)."""
    dims, nbytes, o, lse = _decode_fwd_args(q, k, v, lens, idx, scale, out)
    w = _ws(ws, q.device, nbytes)
    _check(load().msa_decode_fwd(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(lens), _ptr(idx), _ptr(o),
                                 _ptr(lse), _ptr(w), w.numel(), _stream(q.device)))
    return o, lse


def msa_decode_fwd_static(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, lens: torch.Tensor,
                          idx: torch.Tensor, scale: float = 0.0,
                          out: Optional[Tuple[torch.Tensor, torch.Tensor]] = None):
    """msa_decode_fwd without a workspace: the library's static device scratch
    holds the partials (include/msa.h, msa_decode_fwd_static).  With `out`
    given, nothing is allocated on the device; calls on one GPU share the
    scratch and must not overlap."""
    dims, _, o, lse = _decode_fwd_args(q, k, v, lens, idx, scale, out)
    _check(load().msa_decode_fwd_static(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(lens), _ptr(idx),
                                        _ptr(o), _ptr(lse), _stream(q.device)))
    return o, lse
