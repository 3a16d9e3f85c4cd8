"""Pins for the oracle's Main Branch (sparse GQA attention forward and its
Q/K/V gradients over the cached blocks).

The oracle is checked against: a dense masked-attention formulation (whole
matrices, PyTorch float64) and its autograd; PyTorch's causal
scaled_dot_product_attention when every causal block is selected; closed forms
(constant V, a single visible key); central finite differences; and the
gradient invariants sum_j dK_j = 0 and sum_j dV_j = sum dO.
"""
import math

import numpy as np
import pytest
import torch

import synth
from oracle import Dims
from dense_ref import dense_attention, dense_grads, f64, token_mask

BLOCK = 128


def _case(B=2, T=640, H=4, G=2, d=16, dp=8, topk=2, seed=0):
    cfg = synth.custom(B, T, H, G, d, dp, topk)
    x = synth.make_inputs(cfg, seed_offset=seed)
    dm = Dims(B, T, H, G, d, dp, topk)
    return cfg, dm, x


@pytest.fixture(scope="module")
def sel_case(oracle_mod):
    cfg, dm, x = _case()
    idx = oracle_mod.select(dm, x["qp"], x["kp"])
    return cfg, dm, x, idx


def test_fwd_matches_dense_masked_attention(oracle_mod, sel_case):
    cfg, dm, x, idx = sel_case
    o, lse = oracle_mod.fwd(dm, x["q"], x["k"], x["v"], idx)
    mask = token_mask(idx, cfg.T)
    o_ref, lse_ref = dense_attention(f64(x["q"]), f64(x["k"]), f64(x["v"]), mask, dm.eff_scale())
    np.testing.assert_allclose(o, o_ref.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lse_ref.numpy(), rtol=1e-13, atol=1e-12)


def test_fwd_rows_subset_equals_full(oracle_mod, sel_case):
    cfg, dm, x, idx = sel_case
    o, lse = oracle_mod.fwd(dm, x["q"], x["k"], x["v"], idx)
    rows = [0, 5, 127, 128, 639, 640 + 333, 2 * 640 - 1]
    o_r, lse_r = oracle_mod.fwd(dm, x["q"], x["k"], x["v"], idx, rows=rows)
    for r, row in enumerate(rows):
        b, t = divmod(row, cfg.T)
        assert np.array_equal(o_r[r], o[b, t])
        assert np.array_equal(lse_r[r], lse[b, t])


def test_all_blocks_equals_causal_sdpa(oracle_mod):
    """topk >= number of blocks: every causal key is read, which is dense causal
    GQA attention."""
    cfg, dm, x = _case(B=1, T=512, H=4, G=1, d=32, topk=8, seed=3)
    idx = oracle_mod.select(dm, x["qp"], x["kp"])
    o, lse = oracle_mod.fwd(dm, x["q"], x["k"], x["v"], idx)
    q = f64(x["q"]).permute(0, 2, 1, 3)
    k = f64(x["k"]).repeat_interleave(4, dim=2).permute(0, 2, 1, 3)
    v = f64(x["v"]).repeat_interleave(4, dim=2).permute(0, 2, 1, 3)
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True)
    np.testing.assert_allclose(o, ref.permute(0, 2, 1, 3).numpy(), rtol=0, atol=1e-12)


def test_constant_values_and_single_key(oracle_mod, sel_case):
    cfg, dm, x, idx = sel_case
    c = torch.linspace(-2, 3, dm.d, dtype=torch.float64)
    v_const = c.expand(cfg.B, cfg.T, cfg.G, dm.d).clone()
    o, lse = oracle_mod.fwd(dm, x["q"], x["k"], v_const, idx)
    np.testing.assert_allclose(o, np.broadcast_to(c.numpy(), o.shape), rtol=0, atol=1e-13)
    # Query 0 sees key 0 only: O = v[0], LSE = scale * q . k_0.
    q, k, v = f64(x["q"]), f64(x["k"]), f64(x["v"])
    o, lse = oracle_mod.fwd(dm, x["q"], x["k"], x["v"], idx, rows=[0])
    R = dm.H // dm.G
    for h in range(dm.H):
        g = h // R
        assert np.allclose(o[0, h], v[0, 0, g].numpy(), atol=1e-15)
        assert math.isclose(lse[0, h], dm.eff_scale() * float(q[0, 0, h] @ k[0, 0, g]), abs_tol=1e-13)


def test_bwd_matches_autograd_of_dense(oracle_mod, sel_case):
    cfg, dm, x, idx = sel_case
    dq, dk, dv = oracle_mod.bwd(dm, x["q"], x["k"], x["v"], x["dout"], idx)
    mask = token_mask(idx, cfg.T)
    gq, gk, gv = dense_grads(f64(x["q"]), f64(x["k"]), f64(x["v"]), f64(x["dout"]), mask, dm.eff_scale())
    np.testing.assert_allclose(dq, gq.numpy(), rtol=0, atol=1e-11)
    np.testing.assert_allclose(dk, gk.numpy(), rtol=0, atol=1e-11)
    np.testing.assert_allclose(dv, gv.numpy(), rtol=0, atol=1e-11)


def test_bwd_invariants(oracle_mod, sel_case):
    cfg, dm, x, idx = sel_case
    dq, dk, dv = oracle_mod.bwd(dm, x["q"], x["k"], x["v"], x["dout"], idx)
    R = dm.H // dm.G
    # Shifting every key by a constant vector leaves each softmax unchanged.
    np.testing.assert_allclose(dk.sum(axis=1), 0.0, atol=1e-11)
    # Each softmax row sums to one, so the dV total equals the dO total per group.
    do = f64(x["dout"]).numpy().reshape(cfg.B, cfg.T, dm.G, R, dm.d).sum(axis=(1, 3))
    np.testing.assert_allclose(dv.sum(axis=1), do, rtol=1e-12, atol=1e-10)


def test_bwd_finite_differences(oracle_mod):
    cfg, dm, x = _case(B=1, T=384, H=4, G=2, d=8, dp=8, topk=2, seed=5)
    idx = oracle_mod.select(dm, x["qp"], x["kp"])
    q, k, v, do = (f64(x[n]).numpy() for n in ("q", "k", "v", "dout"))
    dq, dk, dv = oracle_mod.bwd(dm, q, k, v, do, idx)
    rng = np.random.default_rng(1)
    h = 1e-5

    def loss(qq, kk, vv):
        o, _ = oracle_mod.fwd(dm, qq, kk, vv, idx)
        return float((o * do).sum())

    for name, arr, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        for _ in range(6):
            pos = tuple(int(rng.integers(0, s)) for s in arr.shape)
            ap, am = arr.copy(), arr.copy()
            ap[pos] += h
            am[pos] -= h
            args_p = {"q": q, "k": k, "v": v}
            args_m = dict(args_p)
            args_p[name], args_m[name] = ap, am
            fd = (loss(args_p["q"], args_p["k"], args_p["v"]) -
                  loss(args_m["q"], args_m["k"], args_m["v"])) / (2 * h)
            assert abs(fd - grad[pos]) <= 1e-6 * max(1.0, abs(grad[pos])), (name, pos, fd, grad[pos])


def test_bwd_rows_and_blocks_agree_with_full(oracle_mod, sel_case):
    cfg, dm, x, idx = sel_case
    dq, dk, dv = oracle_mod.bwd(dm, x["q"], x["k"], x["v"], x["dout"], idx)
    rows = [3, 200, 639, 640 + 77]
    dq_r = oracle_mod.bwd_rows(dm, x["q"], x["k"], x["v"], x["dout"], idx, rows=rows)
    for r, row in enumerate(rows):
        b, t = divmod(row, cfg.T)
        np.testing.assert_allclose(dq_r[r], dq[b, t], rtol=0, atol=1e-13)
    N = cfg.N
    blocks = [(0 * dm.G + 0) * N + 0, (1 * dm.G + 1) * N + 4, (0 * dm.G + 1) * N + 2]
    dk_b, dv_b = oracle_mod.bwd_blocks(dm, x["q"], x["k"], x["v"], x["dout"], idx, blocks)
    for i, code in enumerate(blocks):
        bg, blk = divmod(code, N)
        b, g = divmod(bg, dm.G)
        sl = slice(blk * BLOCK, min((blk + 1) * BLOCK, cfg.T))
        n = sl.stop - sl.start
        np.testing.assert_allclose(dk_b[i, :n], dk[b, sl, g], rtol=0, atol=1e-12)
        np.testing.assert_allclose(dv_b[i, :n], dv[b, sl, g], rtol=0, atol=1e-12)


def test_rejects_invalid_index_rows(oracle_mod, sel_case):
    cfg, dm, x, idx = sel_case
    bad = idx.copy()
    bad[0, 0, 10, 0] = 3                      # token 10 may only read block 0
    with pytest.raises(ValueError):
        oracle_mod.fwd(dm, x["q"], x["k"], x["v"], bad, rows=[10])
    bad = idx.copy()
    bad[0, 0, 300, :2] = [1, 1]               # repeated block
    with pytest.raises(ValueError):
        oracle_mod.fwd(dm, x["q"], x["k"], x["v"], bad, rows=[300])
