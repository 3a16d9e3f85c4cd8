"""The fixed window/dilation selector on the GPU (through the C ABI) against
the oracle: indices bit-exact, and the Main Branch run on the pattern's cache
against the oracle with the same cache."""
import numpy as np
import pytest
import torch

import synth
from oracle import Dims
import parity

pytestmark = pytest.mark.gpu

COS = 0.999


@pytest.fixture(scope="module")
def msa():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import block_sparse_attention_qk_amd as m
    m.load()
    return m


CASES = [
    # B, T, G, window, dilation, union top-k (0 = pattern alone)
    (1, 4096, 1, 2, 3, 0),
    (2, 2048, 2, 1, 0, 4),       # window + proxy cache
    (1, 4096, 2, 0, 5, 3),       # dilation + proxy cache, no window
    (1, 2048, 1, 64, 0, 0),      # window covers everything
    (1, 8192, 1, 3, 1, 0),       # dilation 1: every causal block
    (1, 16384, 2, 4, 16, 8),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B%dT%dG%dw%ds%dk%d" % c)
def test_pattern_indices_match_oracle(msa, oracle_mod, case):
    B, T, G, window, dilation, k = case
    print("pattern case", case, flush=True)
    idx_in = None
    if k:
        cfg = synth.custom(B, T, G * 2, G, 64, 32, k)
        x = synth.make_inputs(cfg)
        idx_in = msa.msa_proxy_select(x["qp"].cuda(), x["kp"].cuda(), k)
    width = msa.pattern_width(T, window, dilation, k)
    got = msa.msa_pattern_select(B, T, G, window, dilation, idx_in=idx_in, width=width)
    torch.cuda.synchronize()
    ref = oracle_mod.pattern_select(B, T, G, window, dilation, width,
                                    idx_in=None if idx_in is None else idx_in.cpu().numpy())
    np.testing.assert_array_equal(got.cpu().numpy(), ref)


def test_main_branch_on_pattern_cache(msa, oracle_mod):
    cfg = synth.custom(1, 2048, 8, 2, 128, 64, 4)
    print("pattern main branch", cfg, flush=True)
    x = synth.make_inputs(cfg, seed_offset=5)
    dev = {n: t.cuda() for n, t in x.items()}
    top = msa.msa_proxy_select(dev["qp"], dev["kp"], cfg.topk)
    idx = msa.msa_pattern_select(cfg.B, cfg.T, cfg.G, 3, 4, idx_in=top)
    o, lse = msa.msa_fwd(dev["q"], dev["k"], dev["v"], idx)
    dq, dk, dv = msa.msa_bwd(dev["q"], dev["k"], dev["v"], o, dev["dout"], lse, idx)
    torch.cuda.synchronize()
    dm = Dims(cfg.B, cfg.T, cfg.H, cfg.G, cfg.d, cfg.dp, idx.shape[3])
    idx_h = idx.cpu().numpy()
    np.testing.assert_array_equal(idx_h, oracle_mod.pattern_select(cfg.B, cfg.T, cfg.G, 3, 4, idx.shape[3],
                                                                   idx_in=top.cpu().numpy()))
    o_ref, lse_ref = oracle_mod.fwd(dm, x["q"], x["k"], x["v"], idx_h)
    dq_ref, dk_ref, dv_ref = oracle_mod.bwd(dm, x["q"], x["k"], x["v"], x["dout"], idx_h)
    for name, got, ref in (("o", o, o_ref), ("lse", lse, lse_ref), ("dq", dq, dq_ref), ("dk", dk, dk_ref),
                           ("dv", dv, dv_ref)):
        parity.assert_close(name, got.cpu(), ref, COS)


def test_backward_splits_popular_blocks(msa, oracle_mod):
    """A block read by more tokens than one backward work item holds is cut into
    several items whose dK/dV meet in the same accumulator.  Window 1 with
    dilation 32 makes blocks 0, 32, 64, ... readers of nearly every later token
    (up to 15104 pairs each), beside diagonal blocks read by 128 tokens only."""
    cfg = synth.custom(1, 15104, 2, 1, 128, 64, 1)
    print("split backward items", cfg, flush=True)
    x = synth.make_inputs(cfg, seed_offset=11)
    dev = {n: t.cuda() for n, t in x.items()}
    idx = msa.msa_pattern_select(cfg.B, cfg.T, cfg.G, 1, 32)
    o, lse = msa.msa_fwd(dev["q"], dev["k"], dev["v"], idx)
    dq, dk, dv = msa.msa_bwd(dev["q"], dev["k"], dev["v"], o, dev["dout"], lse, idx)
    torch.cuda.synchronize()
    dm = Dims(cfg.B, cfg.T, cfg.H, cfg.G, cfg.d, cfg.dp, idx.shape[3])
    idx_h = idx.cpu().numpy()
    assert (idx_h[0, 0, :, 0] == 0).all()
    dq_ref, dk_ref, dv_ref = oracle_mod.bwd(dm, x["q"], x["k"], x["v"], x["dout"], idx_h)
    for name, got, ref in (("dq", dq, dq_ref), ("dk", dk, dk_ref), ("dv", dv, dv_ref)):
        parity.assert_close(name, got.cpu(), ref, COS)
