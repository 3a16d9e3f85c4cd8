"""The merged forward + backward call (msa_fwd_bwd) on the GPU: the same
outputs as msa_fwd followed by msa_bwd (o, lse and dq bit for bit, dK/dV up
to the order of fp32 accumulation), the oracle's values, and the token-window
walk under a small workspace."""
import numpy as np
import pytest
import torch

import parity
import synth
from oracle import Dims

pytestmark = pytest.mark.gpu

COS = 0.999


@pytest.fixture(scope="module")
def msa():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import block_sparse_attention_qk_amd as m
    m.load()
    return m


def _separate(msa, x, idx, ws=None):
    o, lse = msa.msa_fwd(x["q"], x["k"], x["v"], idx, ws=ws)
    dq, dk, dv = msa.msa_bwd(x["q"], x["k"], x["v"], o, x["dout"], lse, idx, ws=ws)
    return o, lse, dq, dk, dv


def _compare(merged, sep):
    names = ("o", "lse", "dq", "dk", "dv")
    for n, a, b in zip(names[:3], merged[:3], sep[:3]):
        assert torch.equal(a, b), n
    for n, a, b in zip(names[3:], merged[3:], sep[3:]):
        parity.assert_consistent(n, a.cpu(), b.cpu(), 0.99999, 2 ** -7)


@pytest.mark.parametrize("shape", [(1, 2048, 8, 2, 128, 64, 4), (2, 1024, 4, 2, 64, 32, 3)],
                         ids=lambda s: "B%dT%dH%dG%dd%ddp%dk%d" % s)
def test_merged_equals_separate_and_oracle(msa, oracle_mod, shape):
    cfg = synth.custom(*shape)
    print("merged fwd+bwd", cfg, flush=True)
    x = {n: t.cuda() for n, t in synth.make_inputs(cfg, seed_offset=41).items()}
    idx = msa.msa_proxy_select(x["qp"], x["kp"], cfg.topk)
    merged = msa.msa_fwd_bwd(x["q"], x["k"], x["v"], x["dout"], idx)
    sep = _separate(msa, x, idx)
    torch.cuda.synchronize()
    _compare(merged, sep)
    dm = Dims(cfg.B, cfg.T, cfg.H, cfg.G, cfg.d, cfg.dp, cfg.topk)
    h = {n: t.cpu() for n, t in x.items()}
    idx_h = idx.cpu().numpy()
    o_ref, lse_ref = oracle_mod.fwd(dm, h["q"], h["k"], h["v"], idx_h)
    dq_ref, dk_ref, dv_ref = oracle_mod.bwd(dm, h["q"], h["k"], h["v"], h["dout"], idx_h)
    for n, got, ref in zip(("o", "lse", "dq", "dk", "dv"), merged, (o_ref, lse_ref, dq_ref, dk_ref, dv_ref)):
        parity.assert_close(n, got.cpu(), ref, COS)


def test_merged_small_workspace_and_split_items(msa):
    """A workspace of the minimum size walks 256-token windows; a fixed pattern
    makes blocks 0, 32, 64, 96 readers of every later token (their backward
    items are cut and added atomically)."""
    cfg = synth.custom(1, 15104, 2, 1, 128, 64, 1)
    print("merged fwd+bwd, windows and split items", cfg, flush=True)
    x = {n: t.cuda() for n, t in synth.make_inputs(cfg, seed_offset=42).items()}
    idx = msa.msa_pattern_select(cfg.B, cfg.T, cfg.G, 1, 32)
    full = msa.msa_fwd_bwd(x["q"], x["k"], x["v"], x["dout"], idx)
    dims = (cfg.B, cfg.T, cfg.H, cfg.G, cfg.d, cfg.dp, idx.shape[3])
    lo = msa.msa_workspace_min_bytes(*dims, msa.OP_FWD_BWD)
    assert lo < msa.msa_workspace_bytes(*dims, msa.OP_FWD_BWD)
    small = msa.msa_fwd_bwd(x["q"], x["k"], x["v"], x["dout"], idx, ws=msa.Workspace(nbytes=lo))
    sep = _separate(msa, x, idx)
    torch.cuda.synchronize()
    _compare(full, sep)
    _compare(small, sep)
