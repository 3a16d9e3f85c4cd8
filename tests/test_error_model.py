"""CPU checks of the rounding model used to attribute the kernels' error."""
import numpy as np

import error_model
import synth
from oracle import Dims


def test_model_without_rounding_is_the_oracle(oracle_mod, monkeypatch):
    """With bf16() replaced by the identity the model is exact attention; its
    exact half must equal the oracle on the tiny configuration."""
    cfg = synth.CONFIGS["tiny"]
    x = synth.make_inputs(cfg)
    dm = Dims(cfg.B, cfg.T, cfg.H, cfg.G, cfg.d, cfg.dp, cfg.topk)
    idx = oracle_mod.select(dm, x["qp"], x["kp"])
    o_ref, _ = oracle_mod.fwd(dm, x["q"], x["k"], x["v"], idx)
    dq_ref, dk_ref, dv_ref = oracle_mod.bwd(dm, x["q"], x["k"], x["v"], x["dout"], idx)
    f = {n: x[n].double().numpy()[0] for n in ("q", "k", "v", "dout")}
    monkeypatch.setattr(error_model, "bf16", lambda a: np.asarray(a, dtype=np.float64))
    ex, md = error_model.model(f["q"], f["k"][:, 0], f["v"][:, 0], f["dout"], o_ref[0], idx[0, 0], dm.eff_scale())
    for n, ref in (("o", o_ref[0]), ("dq", dq_ref[0]), ("dk", dk_ref[0, :, 0]), ("dv", dv_ref[0, :, 0])):
        np.testing.assert_allclose(ex[n], ref, rtol=1e-9, atol=1e-12, err_msg=n)
        np.testing.assert_allclose(md[n], ref, rtol=1e-9, atol=1e-12, err_msg=n)
