"""Pins for the oracle's fixed window/dilation pattern (the NEXT selector row).

The reading (keelcrux page, section "Under the hood": a block pattern
configurable by window size and dilation) is stated in oracle.pattern_select.
The pattern itself has no printed example on the pages, so the pins are a
hand-worked row set, special cases that reduce to known caches, and an
independent vectorised formulation.
"""
import numpy as np
import pytest

import synth
from oracle import Dims


def test_hand_worked_rows(oracle_mod):
    # T = 1024 (8 blocks), window 2, dilation 3, written out by hand:
    #   t = 100 (nc 1): window {0}                     -> [0]
    #   t = 300 (nc 3): window {1, 2}, far {0}         -> [0, 1, 2]
    #   t = 900 (nc 8): window {6, 7}, far {0, 3}      -> [0, 3, 6, 7]
    out = oracle_mod.pattern_select(1, 1024, 1, 2, 3, width=5)
    assert out[0, 0, 100].tolist() == [0, -1, -1, -1, -1]
    assert out[0, 0, 300].tolist() == [0, 1, 2, -1, -1]
    assert out[0, 0, 900].tolist() == [0, 3, 6, 7, -1]
    # and with a cache row united in: {5} adds block 5, {9} (not causal) and -1 are ignored
    idx_in = np.full((1, 1, 1024, 3), -1, dtype=np.int32)
    idx_in[0, 0, 900] = [5, 9, -1]
    out = oracle_mod.pattern_select(1, 1024, 1, 2, 3, width=6, idx_in=idx_in)
    assert out[0, 0, 900].tolist() == [0, 3, 5, 6, 7, -1]


@pytest.mark.parametrize("window,dilation", [(64, 0), (8, 1), (0, 1)])
def test_patterns_that_cover_every_causal_block(oracle_mod, window, dilation):
    T = 2048
    out = oracle_mod.pattern_select(1, T, 2, window, dilation, width=T // 128)
    for t in (0, 127, 128, 1000, 2047):
        nc = t // 128 + 1
        row = out[0, 1, t]
        assert row[:nc].tolist() == list(range(nc)) and (row[nc:] == -1).all()


def test_empty_pattern_reproduces_the_input_cache(oracle_mod):
    cfg = synth.CONFIGS["tiny"]
    x = synth.make_inputs(cfg)
    dm = Dims(cfg.B, cfg.T, cfg.H, cfg.G, cfg.d, cfg.dp, cfg.topk)
    idx = oracle_mod.select(dm, x["qp"], x["kp"])
    out = oracle_mod.pattern_select(cfg.B, cfg.T, cfg.G, 0, 0, width=cfg.topk, idx_in=idx)
    np.testing.assert_array_equal(out, idx)


def _mask_formulation(T, window, dilation, idx_in):
    """Independent formulation: a [T, N] boolean matrix of selected blocks."""
    N = T // 128
    t = np.arange(T)[:, None]
    blk = np.arange(N)[None, :]
    nc = t // 128 + 1
    causal = blk < nc
    sel = causal & (blk >= nc - window)
    if dilation > 0:
        sel |= causal & (blk % dilation == 0)
    if idx_in is not None:
        hit = np.zeros((T, N + 1), dtype=bool)
        rows = np.repeat(np.arange(T), idx_in.shape[-1])
        vals = idx_in.reshape(-1)
        ok = (vals >= 0) & (vals < N)
        hit[rows[ok], vals[ok]] = True
        sel |= causal & hit[:, :N]
    return sel


@pytest.mark.parametrize("window,dilation,k_in", [(3, 4, 0), (1, 0, 5), (0, 5, 3), (4, 2, 6), (2, 7, 0)])
def test_matches_mask_formulation(oracle_mod, window, dilation, k_in):
    T = 2048
    rng = np.random.default_rng(window * 100 + dilation * 10 + k_in)
    idx_in = None
    if k_in:
        idx_in = rng.integers(-1, T // 128 + 2, size=(1, 1, T, k_in)).astype(np.int32)
    width = T // 128
    out = oracle_mod.pattern_select(1, T, 1, window, dilation, width=width, idx_in=idx_in)
    sel = _mask_formulation(T, window, dilation, None if idx_in is None else idx_in[0, 0])
    for t in range(T):
        want = np.nonzero(sel[t])[0].tolist()
        assert out[0, 0, t, :len(want)].tolist() == want, t
        assert (out[0, 0, t, len(want):] == -1).all(), t
