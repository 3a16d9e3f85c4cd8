"""The binding rejects caller-provided outputs (and workspaces) that do not
match the call before anything reaches the library: a wrong shape, dtype or
device raises, so the kernels never write past a buffer.  Correct `out`
tensors give the same results as freshly allocated ones."""
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def setup():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import block_sparse_attention_qk_amd as m
    m.load()
    cfg = synth.CONFIGS["tiny"]
    x = {n: t.cuda() for n, t in synth.make_inputs(cfg).items()}
    idx = m.msa_proxy_select(x["qp"], x["kp"], cfg.topk)
    o, lse = m.msa_fwd(x["q"], x["k"], x["v"], idx)
    torch.cuda.synchronize()
    return m, cfg, x, idx, o, lse


def test_select_out_shape(setup):
    m, cfg, x, idx, o, lse = setup
    bad = torch.empty((cfg.B, cfg.G, cfg.T, cfg.topk - 1), dtype=torch.int32, device="cuda")
    with pytest.raises(ValueError):
        m.msa_proxy_select(x["qp"], x["kp"], cfg.topk, out=bad)
    good = torch.empty_like(idx)
    m.msa_proxy_select(x["qp"], x["kp"], cfg.topk, out=good)
    torch.cuda.synchronize()
    assert torch.equal(good, idx)


def test_fwd_out_checks(setup):
    m, cfg, x, idx, o, lse = setup
    short = torch.empty((cfg.B, cfg.T // 2, cfg.H, cfg.d), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        m.msa_fwd(x["q"], x["k"], x["v"], idx, out=(short, torch.empty_like(lse)))
    with pytest.raises(TypeError):
        m.msa_fwd(x["q"], x["k"], x["v"], idx, out=(torch.empty_like(o), torch.empty_like(lse).half()))
    o2, lse2 = torch.empty_like(o), torch.empty_like(lse)
    m.msa_fwd(x["q"], x["k"], x["v"], idx, out=(o2, lse2))
    torch.cuda.synchronize()
    assert torch.equal(o2, o) and torch.equal(lse2, lse)


def test_bwd_and_merged_out_checks(setup):
    m, cfg, x, idx, o, lse = setup
    dq, dk, dv = torch.empty_like(x["q"]), torch.empty_like(x["k"]), torch.empty_like(x["v"])
    with pytest.raises(ValueError):
        m.msa_bwd(x["q"], x["k"], x["v"], o, x["dout"], lse, idx, out=(dq, dq, dv))  # dk with q's shape
    with pytest.raises(ValueError):
        m.msa_fwd_bwd(x["q"], x["k"], x["v"], x["dout"], idx,
                      out=(torch.empty_like(o), torch.empty_like(lse)[:, :-1], dq, dk, dv))
    ref = m.msa_bwd(x["q"], x["k"], x["v"], o, x["dout"], lse, idx)
    m.msa_bwd(x["q"], x["k"], x["v"], o, x["dout"], lse, idx, out=(dq, dk, dv))
    torch.cuda.synchronize()
    assert torch.equal(dq, ref[0])


def test_non_contiguous_out_is_rejected(setup):
    m, cfg, x, idx, o, lse = setup
    wide = torch.empty((cfg.B, cfg.T, cfg.H, 2 * cfg.d), dtype=torch.bfloat16, device="cuda")[..., ::2]
    with pytest.raises(ValueError):
        m.msa_fwd(x["q"], x["k"], x["v"], idx, out=(wide, torch.empty_like(lse)))


def test_launch_timing_belongs_to_the_calling_thread(setup):
    """Timing state is per host thread: launches made by another thread are
    neither recorded nor read by this one."""
    import threading
    m, cfg, x, idx, o, lse = setup
    m.timing_enable(True)
    t = threading.Thread(target=lambda: m.msa_fwd(x["q"], x["k"], x["v"], idx))
    t.start()
    t.join()
    torch.cuda.synchronize()
    assert all(n == 0 for _, n in m.timing_read().values())
    m.msa_fwd(x["q"], x["k"], x["v"], idx)
    rec = m.timing_read()
    m.timing_enable(False)
    assert rec["fwd_partials"][1] == 1 and rec["fwd_combine"][1] == 1
