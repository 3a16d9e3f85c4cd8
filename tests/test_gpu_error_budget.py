"""Where the kernels' difference from the oracle comes from (tiny configuration).

The oracle is float64 throughout; the kernels round to bf16 where matrix cores
need bf16 operands (P and dS), where per-pair partials are stored (forward o_b,
dQ partials) and at the outputs.  tests/error_model.py applies exactly those
roundings to float64 arithmetic.  For every tensor this test prints the
kernel's error against the oracle, the model's error against the oracle and
the kernel's distance from the model, and requires the model to explain most
of the kernel's error (RMS distance to the model at most half the RMS error).
"""
import numpy as np
import pytest
import torch

import error_model
import parity
import synth
from oracle import Dims

pytestmark = pytest.mark.gpu


def _rms(a):
    return float(np.sqrt(np.mean(np.square(a))))


def test_rounding_model_explains_the_error(oracle_mod):
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import block_sparse_attention_qk_amd as msa
    msa.load()
    cfg = synth.CONFIGS["tiny"]
    print("error budget", cfg, flush=True)
    x = synth.make_inputs(cfg)
    d = {n: t.cuda() for n, t in x.items()}
    idx = msa.msa_proxy_select(d["qp"], d["kp"], cfg.topk)
    o, lse = msa.msa_fwd(d["q"], d["k"], d["v"], idx)
    dq, dk, dv = msa.msa_bwd(d["q"], d["k"], d["v"], o, d["dout"], lse, idx)
    torch.cuda.synchronize()
    dm = Dims(cfg.B, cfg.T, cfg.H, cfg.G, cfg.d, cfg.dp, cfg.topk)
    idx_h = idx.cpu().numpy()
    f = {n: x[n].double().numpy()[0] for n in ("q", "k", "v", "dout")}
    ex, md = error_model.model(f["q"], f["k"][:, 0], f["v"][:, 0], f["dout"], o.double().cpu().numpy()[0],
                               idx_h[0, 0], dm.eff_scale())
    got = {"o": o.double().cpu().numpy()[0], "dq": dq.double().cpu().numpy()[0],
           "dk": dk.double().cpu().numpy()[0, :, 0], "dv": dv.double().cpu().numpy()[0, :, 0]}
    for n in ("o", "dq", "dk", "dv"):
        e_k, e_m, e_km = got[n] - ex[n], md[n] - ex[n], got[n] - md[n]
        allow = parity.half_ulp_bf16(np.maximum(np.abs(got[n]), np.abs(ex[n])))
        print("budget %-3s kernel-oracle max %.3e rms %.3e | model-oracle max %.3e rms %.3e | kernel-model max %.3e "
              "rms %.3e | kernel excess over output rounding %.3e" % (
                  n, np.abs(e_k).max(), _rms(e_k), np.abs(e_m).max(), _rms(e_m), np.abs(e_km).max(), _rms(e_km),
                  (np.abs(e_k) - allow).max()), flush=True)
        assert _rms(e_km) <= 0.5 * _rms(e_k), n
