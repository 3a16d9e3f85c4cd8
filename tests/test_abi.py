"""Host-side tests of libmsa's C ABI (no GPU needed).

The library must load, export every function include/msa.h declares, and
reject bad arguments synchronously with the documented status codes before
anything reaches the GPU.  Every call below fails a host check, so no kernel
is ever launched.
"""
import ctypes
import os
import re

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

OK, ERR_NULL, ERR_SHAPE, ERR_UNSUP, ERR_ALIGN, ERR_WS, ERR_HIP = range(7)


@pytest.fixture(scope="module")
def msa():
    import block_sparse_attention_qk_amd as m
    if not os.path.exists(m.lib_path()):
        from block_sparse_attention_qk_amd import build
        build.build()
    m.load()
    return m


@pytest.fixture(scope="module")
def lib(msa):
    return msa.load()


def _dims(msa, B=1, T=1024, H=8, G=2, d=128, dp=64, topk=4, scale=0.0):
    return msa._dims(B, T, H, G, d, dp, topk, scale)


def test_exports_every_declared_function(lib, msa):
    header = open(os.path.join(ROOT, "include", "msa.h")).read()
    declared = set(re.findall(r"^[A-Za-z_][\w \*]*?\b(msa_\w+)\s*\(", header, flags=re.M))
    assert declared, "no declarations parsed"
    assert declared == set(msa.EXPORTED_SYMBOLS), declared ^ set(msa.EXPORTED_SYMBOLS)
    for name in declared:
        assert hasattr(lib, name), name
    assert lib.msa_version().decode().startswith("msa-gfx950")


def test_status_strings(lib):
    seen = set()
    for code in range(9):
        s = lib.msa_status_str(code)
        assert s and s.decode() not in seen
        seen.add(s.decode())
    assert lib.msa_status_str(99).decode() == "unknown status"


@pytest.mark.parametrize("kw,code", [
    (dict(T=1000), ERR_SHAPE),           # not a multiple of 128
    (dict(T=0), ERR_SHAPE),
    (dict(T=1 << 21), ERR_SHAPE),        # above the supported length
    (dict(B=0), ERR_SHAPE),
    (dict(topk=0), ERR_SHAPE),
    (dict(topk=1025), ERR_SHAPE),
    (dict(H=6, G=4), ERR_SHAPE),         # H % G != 0
    (dict(H=6, G=2), ERR_UNSUP),         # R = 3
    (dict(H=64, G=2), ERR_UNSUP),        # R = 32
    (dict(d=96), ERR_UNSUP),
    (dict(scale=float("nan")), ERR_SHAPE),
    (dict(scale=float("inf")), ERR_SHAPE),
    (dict(B=256, G=256, H=256, T=128), ERR_SHAPE),  # B*G above the grid's 65535
])
def test_main_branch_rejects_bad_dims(lib, msa, kw, code):
    d = _dims(msa, **kw)
    P = ctypes.c_void_p(4096)
    assert lib.msa_fwd(ctypes.byref(d), P, P, P, P, P, P, P, 1 << 40, None) == code
    assert lib.msa_bwd(ctypes.byref(d), P, P, P, P, P, P, P, P, P, P, P, 1 << 40, None) == code
    assert lib.msa_workspace_bytes(ctypes.byref(d), msa.OP_FWD) == 0
    assert lib.msa_workspace_min_bytes(ctypes.byref(d), msa.OP_BWD) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(dp=48), ERR_UNSUP),
    (dict(dp=256), ERR_UNSUP),
    (dict(T=200), ERR_SHAPE),
    (dict(G=0), ERR_SHAPE),
    (dict(B=2, G=40000, H=40000, T=128), ERR_SHAPE),
])
def test_select_rejects_bad_dims(lib, msa, kw, code):
    d = _dims(msa, **kw)
    P = ctypes.c_void_p(4096)
    assert lib.msa_proxy_select(ctypes.byref(d), P, P, P, P, 1 << 40, None) == code


def test_select_ignores_main_branch_dims(lib, msa):
    # H and d do not enter the Index Branch: an odd head count is fine there,
    # the call still stops at the (deliberately) missing workspace.
    d = _dims(msa, H=3, d=96)
    P = ctypes.c_void_p(4096)
    assert lib.msa_proxy_select(ctypes.byref(d), P, P, P, P, 0, None) == ERR_WS


def test_null_dims_and_pointers(lib, msa):
    P = ctypes.c_void_p(4096)
    assert lib.msa_fwd(None, P, P, P, P, P, P, P, 1 << 40, None) == ERR_NULL
    d = _dims(msa)
    for i in range(7):
        args = [P] * 7
        args[i] = None
        assert lib.msa_fwd(ctypes.byref(d), *args, 1 << 40, None) == ERR_NULL, i
    for i in range(11):
        args = [P] * 11
        args[i] = None
        assert lib.msa_bwd(ctypes.byref(d), *args, 1 << 40, None) == ERR_NULL, i
    for i in range(4):
        args = [P] * 4
        args[i] = None
        assert lib.msa_proxy_select(ctypes.byref(d), *args, 1 << 40, None) == ERR_NULL, i


def test_misaligned_pointers(lib, msa):
    d = _dims(msa)
    P, Q = ctypes.c_void_p(4096), ctypes.c_void_p(4096 + 8)
    for i in range(7):
        args = [P] * 7
        args[i] = Q
        assert lib.msa_fwd(ctypes.byref(d), *args, 1 << 40, None) == ERR_ALIGN, i
    for i in range(4):
        args = [P] * 4
        args[i] = Q
        assert lib.msa_proxy_select(ctypes.byref(d), *args, 1 << 40, None) == ERR_ALIGN, i


def test_workspace_too_small(lib, msa):
    d = _dims(msa)
    P = ctypes.c_void_p(4096)
    for op, call in ((msa.OP_SELECT, lambda n: lib.msa_proxy_select(ctypes.byref(d), P, P, P, P, n, None)),
                     (msa.OP_FWD, lambda n: lib.msa_fwd(ctypes.byref(d), P, P, P, P, P, P, P, n, None)),
                     (msa.OP_BWD, lambda n: lib.msa_bwd(ctypes.byref(d), P, P, P, P, P, P, P, P, P, P, P, n,
                                                       None))):
        need = lib.msa_workspace_min_bytes(ctypes.byref(d), op)
        assert need > 0
        assert call(need - 1) == ERR_WS
        assert call(0) == ERR_WS


def test_workspace_sizes(msa):
    for name, shape in (("tiny", (1, 1024, 4, 1, 64, 32, 4)), ("128k", (1, 131072, 32, 4, 128, 64, 32)),
                        ("1m", (1, 1 << 20, 16, 2, 128, 64, 288))):
        for op in (msa.OP_SELECT, msa.OP_FWD, msa.OP_BWD):
            full = msa.msa_workspace_bytes(*shape, op)
            lo = msa.msa_workspace_min_bytes(*shape, op)
            assert 0 < lo <= full, (name, op)
            assert full <= (80 << 30) + (16 << 30), (name, op, full)  # capped (plus T-sized accumulators)
    # 128K runs the backward in one window (the pair partials of all tokens fit)
    # and the forward in 32768-token windows (64 MiB of query rows per group).
    B, T, H, G, d, dp, k = 1, 131072, 32, 4, 128, 64, 32
    pairs_bytes = B * G * T * k * (H // G) * d * 2
    assert msa.msa_workspace_bytes(B, T, H, G, d, dp, k, msa.OP_BWD) > pairs_bytes
    fwd = msa.msa_workspace_bytes(B, T, H, G, d, dp, k, msa.OP_FWD)
    assert pairs_bytes // 4 < fwd < pairs_bytes // 2


def test_binding_rejects_host_tensors(msa):
    x = torch.zeros((1, 256, 2, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU"):
        msa.msa_proxy_select(x, x, 2)
    with pytest.raises(TypeError):
        msa.msa_proxy_select(x.float(), x, 2)
    q = torch.zeros((1, 256, 4, 64), dtype=torch.bfloat16)
    idx = torch.zeros((1, 2, 256, 2), dtype=torch.int32)
    with pytest.raises(ValueError):
        msa.msa_fwd(q, x, x, idx)


def test_pattern_select_checks(lib, msa):
    P = ctypes.c_void_p(4096)
    d = _dims(msa, T=1024, topk=8)
    sel = lib.msa_pattern_select
    assert sel(None, 2, 3, None, 0, P, None) == ERR_NULL
    assert sel(ctypes.byref(d), 2, 3, None, 0, None, None) == ERR_NULL
    assert sel(ctypes.byref(d), -1, 3, None, 0, P, None) == ERR_SHAPE        # negative window
    assert sel(ctypes.byref(d), 2, -3, None, 0, P, None) == ERR_SHAPE        # negative dilation
    assert sel(ctypes.byref(d), 0, 0, None, 0, P, None) == ERR_SHAPE         # selects nothing
    assert sel(ctypes.byref(d), 2, 3, P, 0, P, None) == ERR_SHAPE            # k_in out of range
    assert sel(ctypes.byref(d), 2, 3, P, 1025, P, None) == ERR_SHAPE
    assert sel(ctypes.byref(d), 2, 3, None, 0, ctypes.c_void_p(4096 + 4), None) == ERR_ALIGN
    # width bound: N = 8 blocks; window 2 + ceil(6/3) far + 5 cache entries = 9 -> min(8, 9) = 8
    assert msa.pattern_width(1024, 2, 3, 5) == 8
    d7 = _dims(msa, T=1024, topk=7)
    assert sel(ctypes.byref(d7), 2, 3, P, 5, P, None) == ERR_SHAPE
    assert msa.pattern_width(1024, 2, 3, 0) == 4
    d3 = _dims(msa, T=1024, topk=3)
    assert sel(ctypes.byref(d3), 2, 3, None, 0, P, None) == ERR_SHAPE


def test_decode_checks(lib, msa):
    P, Q = ctypes.c_void_p(4096), ctypes.c_void_p(4096 + 8)
    d = _dims(msa, B=2, T=1024, topk=8)
    sel, fwd = lib.msa_decode_select, lib.msa_decode_fwd
    need_s = lib.msa_workspace_bytes(ctypes.byref(d), msa.OP_DECODE_SELECT)
    need_f = lib.msa_workspace_bytes(ctypes.byref(d), msa.OP_DECODE_FWD)
    assert need_s >= 2 * 2 * 8 * 4                      # B*G*N fp32 pooled scores
    assert need_f >= 2 * 2 * 8 * 4 * (128 + 1) * 4      # B*G*topk partials of R*(d+1) fp32
    assert lib.msa_workspace_min_bytes(ctypes.byref(d), msa.OP_DECODE_FWD) == need_f
    assert lib.msa_workspace_bytes(ctypes.byref(d), 6) == 0          # no such op
    assert sel(None, P, P, P, P, P, need_s, None) == ERR_NULL
    for i in range(5):
        args = [P] * 5
        args[i] = None
        assert sel(ctypes.byref(d), *args, need_s, None) == ERR_NULL, i
        args[i] = Q
        assert sel(ctypes.byref(d), *args, need_s, None) == ERR_ALIGN, i
    for i in range(8):
        args = [P] * 8
        args[i] = None
        assert fwd(ctypes.byref(d), *args, need_f, None) == ERR_NULL, i
        args[i] = Q
        assert fwd(ctypes.byref(d), *args, need_f, None) == ERR_ALIGN, i
    assert sel(ctypes.byref(d), P, P, P, P, P, need_s - 1, None) == ERR_WS
    assert fwd(ctypes.byref(d), P, P, P, P, P, P, P, P, need_f - 1, None) == ERR_WS
    for kw, code in ((dict(T=1000), ERR_SHAPE), (dict(dp=48), ERR_UNSUP), (dict(topk=0), ERR_SHAPE),
                     (dict(B=40000, G=2), ERR_SHAPE)):
        bad = _dims(msa, **kw)
        assert sel(ctypes.byref(bad), P, P, P, P, P, 1 << 40, None) == code, kw
    for kw, code in ((dict(H=6, G=2), ERR_UNSUP), (dict(d=96), ERR_UNSUP), (dict(H=6, G=4), ERR_SHAPE)):
        bad = _dims(msa, **kw)
        assert fwd(ctypes.byref(bad), P, P, P, P, P, P, P, P, 1 << 40, None) == code, kw


def test_fwd_bwd_checks(lib, msa):
    P, Q = ctypes.c_void_p(4096), ctypes.c_void_p(4096 + 8)
    d = _dims(msa)
    f = lib.msa_fwd_bwd
    full = lib.msa_workspace_bytes(ctypes.byref(d), msa.OP_FWD_BWD)
    lo = lib.msa_workspace_min_bytes(ctypes.byref(d), msa.OP_FWD_BWD)
    assert 0 < lo <= full
    # one shared inverse index and aliased partials: below the two separate workspaces together
    assert full < (lib.msa_workspace_bytes(ctypes.byref(d), msa.OP_FWD) +
                   lib.msa_workspace_bytes(ctypes.byref(d), msa.OP_BWD))
    assert f(None, *([P] * 11), full, None) == ERR_NULL
    for i in range(11):
        args = [P] * 11
        args[i] = None
        assert f(ctypes.byref(d), *args, full, None) == ERR_NULL, i
        args[i] = Q
        assert f(ctypes.byref(d), *args, full, None) == ERR_ALIGN, i
    assert f(ctypes.byref(d), *([P] * 11), lo - 1, None) == ERR_WS
    for kw, code in ((dict(H=6, G=2), ERR_UNSUP), (dict(T=1000), ERR_SHAPE), (dict(d=96), ERR_UNSUP)):
        bad = _dims(msa, **kw)
        assert f(ctypes.byref(bad), *([P] * 11), 1 << 40, None) == code, kw


def test_missing_library_fails_loudly(msa, monkeypatch, tmp_path):
    """Without the built library the binding raises: there is no fallback path."""
    monkeypatch.setattr(msa, "_lib", None)
    monkeypatch.setattr(msa, "_LIB_PATH", str(tmp_path / "libmsa.so"))
    with pytest.raises(msa.MsaError):
        msa.load()
    with pytest.raises(msa.MsaError):
        msa.msa_workspace_bytes(1, 1024, 8, 2, 128, 64, 4, msa.OP_FWD)


def test_decode_fwd_static_checks(lib, msa):
    """Host-side checks of the allocation-free decode call: they return before
    any HIP call, so they run without a GPU."""
    P, Q = ctypes.c_void_p(4096), ctypes.c_void_p(4096 + 8)
    f = lib.msa_decode_fwd_static
    d = _dims(msa, B=2, T=1024, topk=8)
    assert f(None, P, P, P, P, P, P, P, None) == ERR_NULL
    for i in range(7):
        args = [P] * 7
        args[i] = None
        assert f(ctypes.byref(d), *args, None) == ERR_NULL, i
        args[i] = Q
        assert f(ctypes.byref(d), *args, None) == ERR_ALIGN, i
    for kw, code in ((dict(T=1000), ERR_SHAPE), (dict(H=6, G=2), ERR_UNSUP), (dict(d=96), ERR_UNSUP)):
        assert f(ctypes.byref(_dims(msa, **kw)), P, P, P, P, P, P, P, None) == code, kw
    # 64 sequences x 4 groups x top-32 x 8 heads x d 128 fp32 partials: 32 MiB > the 16 MiB scratch
    big = _dims(msa, B=64, T=256, H=32, G=4, d=128, topk=32)
    assert lib.msa_workspace_bytes(ctypes.byref(big), msa.OP_DECODE_FWD) > msa.STATIC_SCRATCH_BYTES
    assert f(ctypes.byref(big), P, P, P, P, P, P, P, None) == 8  # MSA_ERR_SCRATCH
    assert "static scratch" in lib.msa_status_str(8).decode()
