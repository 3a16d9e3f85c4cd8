"""MSA_VALIDATE: the device check of the block-index cache that msa_fwd,
msa_bwd and msa_fwd_bwd run first when the variable is set.  A valid cache
(the Index Branch's own output) passes and the call runs; a cache with an
entry outside 0..t/128, a repeated block, or a row without blocks makes the
call return MSA_ERR_INDEX before anything else is launched."""
import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu

ERR_INDEX = 7


@pytest.fixture(scope="module")
def msa():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import block_sparse_attention_qk_amd as m
    m.load()
    return m


@pytest.fixture(scope="module")
def inputs(msa):
    cfg = synth.CONFIGS["tiny"]
    x = {n: t.cuda() for n, t in synth.make_inputs(cfg).items()}
    idx = msa.msa_proxy_select(x["qp"], x["kp"], cfg.topk)
    torch.cuda.synchronize()
    return cfg, x, idx


def _corrupt(idx, kind):
    bad = idx.clone()
    if kind == "repeat":        # token 700 (6 causal blocks, 4 listed): second entry = first
        bad[0, 0, 700, 1] = bad[0, 0, 700, 0]
    elif kind == "future":      # token 5 may only list block 0
        bad[0, 0, 5, 0] = 3
    elif kind == "negative":
        bad[0, 0, 300, 2] = -2
    elif kind == "empty":
        bad[0, 0, 1000, :] = -1
    elif kind == "past_end":    # block N for the last token
        bad[0, 0, 1023, 0] = 8
    return bad


def _code(msa, fn):
    with pytest.raises(msa.MsaError) as e:
        fn()
    return int(str(e.value).split("error ")[1].split(":")[0])


def test_valid_cache_passes(msa, inputs, monkeypatch):
    monkeypatch.setenv("MSA_VALIDATE", "1")
    cfg, x, idx = inputs
    o, lse = msa.msa_fwd(x["q"], x["k"], x["v"], idx)
    dq, dk, dv = msa.msa_bwd(x["q"], x["k"], x["v"], o, x["dout"], lse, idx)
    o2, lse2, dq2, dk2, dv2 = msa.msa_fwd_bwd(x["q"], x["k"], x["v"], x["dout"], idx)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2) and torch.equal(dq, dq2)
    assert torch.isfinite(dk.float()).all() and torch.isfinite(dv.float()).all()


@pytest.mark.parametrize("kind", ["repeat", "future", "negative", "empty", "past_end"])
def test_invalid_cache_is_rejected(msa, inputs, monkeypatch, kind):
    monkeypatch.setenv("MSA_VALIDATE", "1")
    cfg, x, idx = inputs
    bad = _corrupt(idx, kind)
    print("invalid cache", kind, flush=True)
    assert _code(msa, lambda: msa.msa_fwd(x["q"], x["k"], x["v"], bad)) == ERR_INDEX
    if kind in ("repeat", "empty"):
        o, lse = msa.msa_fwd(x["q"], x["k"], x["v"], idx)
        assert _code(msa, lambda: msa.msa_bwd(x["q"], x["k"], x["v"], o, x["dout"], lse, bad)) == ERR_INDEX
        assert _code(msa, lambda: msa.msa_fwd_bwd(x["q"], x["k"], x["v"], x["dout"], bad)) == ERR_INDEX
    torch.cuda.synchronize()


def test_check_is_off_by_default(msa, inputs, monkeypatch):
    """Unset (or "0"): the valid cache runs without the check; results equal the checked run."""
    cfg, x, idx = inputs
    before = idx.clone()
    monkeypatch.setenv("MSA_VALIDATE", "0")
    o0, lse0 = msa.msa_fwd(x["q"], x["k"], x["v"], idx)
    monkeypatch.setenv("MSA_VALIDATE", "1")
    o1, lse1 = msa.msa_fwd(x["q"], x["k"], x["v"], idx)
    torch.cuda.synchronize()
    assert torch.equal(o0, o1) and torch.equal(lse0, lse1)
    assert torch.equal(idx, before)  # the check only reads the cache
