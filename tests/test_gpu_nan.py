"""A NaN in one query row stays in what that row reaches.

One element of q at (token t, head h) is NaN.  Exact attention over the
cached blocks then makes o, lse and dq of row (t, h) NaN, and dK/dV of keys in
the blocks that token t selected for h's group; every other output element
must stay finite and keep parity with the oracle.  (Keys past t inside a
selected diagonal block may also turn NaN on the GPU, since a bf16 matrix
product multiplies the masked zero by the NaN; they lie inside the selected
blocks, so the containment check admits them.)
"""
import numpy as np
import pytest
import torch

import parity
import synth
from oracle import Dims

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def msa():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import block_sparse_attention_qk_amd as m
    m.load()
    return m


@pytest.mark.parametrize("t,h", [(1000, 3), (1300, 5), (130, 0)])
def test_nan_in_one_query_row_stays_contained(msa, oracle_mod, t, h):
    cfg = synth.custom(1, 2048, 8, 2, 128, 64, 4)
    print("nan row", cfg, t, h, flush=True)
    x = synth.make_inputs(cfg, seed_offset=41)
    q = x["q"].clone()
    q[0, t, h, 17] = float("nan")
    dev = {n: v.cuda() for n, v in x.items()}
    dev["q"] = q.cuda()
    idx = msa.msa_proxy_select(dev["qp"], dev["kp"], cfg.topk)
    o, lse = msa.msa_fwd(dev["q"], dev["k"], dev["v"], idx)
    dq, dk, dv = msa.msa_bwd(dev["q"], dev["k"], dev["v"], o, dev["dout"], lse, idx)
    torch.cuda.synchronize()
    R = cfg.H // cfg.G
    g = h // R
    idx_h = idx.cpu().numpy()
    sel = [int(b) for b in idx_h[0, g, t] if b >= 0]
    print("token %d head %d group %d selects blocks %s" % (t, h, g, sel), flush=True)

    got = {"o": o.float().cpu().numpy(), "lse": lse.cpu().numpy(), "dq": dq.float().cpu().numpy(),
           "dk": dk.float().cpu().numpy(), "dv": dv.float().cpu().numpy()}
    # where NaN may appear
    allowed = {n: np.zeros(a.shape, dtype=bool) for n, a in got.items()}
    for n in ("o", "dq"):
        allowed[n][0, t, h] = True
    allowed["lse"][0, t, h] = True
    for n in ("dk", "dv"):
        for b in sel:
            allowed[n][0, 128 * b:128 * b + 128, g] = True
    for n, a in got.items():
        bad = ~np.isfinite(a) & ~allowed[n]
        assert not bad.any(), (n, np.argwhere(bad)[:5].tolist())
    # the row itself must be NaN (not silently dropped)
    assert np.isnan(got["o"][0, t, h]).all() and np.isnan(got["lse"][0, t, h])
    assert np.isnan(got["dq"][0, t, h]).all()

    dm = Dims(cfg.B, cfg.T, cfg.H, cfg.G, cfg.d, cfg.dp, cfg.topk)
    q64 = q.double().numpy()
    o_ref, lse_ref = oracle_mod.fwd(dm, q64, x["k"], x["v"], idx_h)
    dq_ref, dk_ref, dv_ref = oracle_mod.bwd(dm, q64, x["k"], x["v"], x["dout"], idx_h)
    ref = {"o": o_ref, "lse": lse_ref, "dq": dq_ref, "dk": dk_ref, "dv": dv_ref}
    for n in got:
        ref_nan, got_nan = np.isnan(ref[n]), np.isnan(got[n])
        assert not (ref_nan & ~got_nan).any(), "%s: the oracle's NaN elements must be NaN on the GPU" % n
        both = np.isfinite(ref[n]) & np.isfinite(got[n])
        parity.assert_close(n, got[n][both], ref[n][both], 0.999)
