"""Golden fixtures under tests/golden/.

* hand_worked_384.txt: indices derived by hand from the method's definition
  (see the file's header) and closed forms of the Main Branch for inputs whose
  scores are all zero.  The oracle must reproduce them (CPU test) and so must
  the HIP path (GPU test).
* tiny_oracle_sample.txt: sampled oracle outputs on the tiny configuration,
  written by tests/golden/make_tiny_golden.py (which calls only the oracle and
  the input generator).  It guards the oracle against regressions (CPU) and is
  a stored reference for the HIP path (GPU).
"""
import math
import os

import numpy as np
import pytest
import torch

import synth
from oracle import Dims
import parity

HERE = os.path.dirname(os.path.abspath(__file__))
GOLD = os.path.join(HERE, "golden")

HW = dict(B=1, T=384, H=2, G=1, d=64, dp=32, topk=2)
C_V = (1.0, 2.0, -1.0)     # v[j] = c(block) * ones
C_K = (1.0, -2.0, 0.5)     # k[j] = c'(block) * e1
ALPHA = 0.5                # q[t,h] = ALPHA * e2
SPIKES = {0: (1.0, 10, 3.0), 1: (2.0, 228, 5.0), 2: (3.0, 300, 6.0)}  # block: (value, spike key, spike value)


def hand_inputs():
    T, H, d, dp = HW["T"], HW["H"], HW["d"], HW["dp"]
    qp = torch.zeros((1, T, 1, dp))
    qp[..., 0] = 1.0
    kp = torch.zeros((1, T, 1, dp))
    q = torch.zeros((1, T, H, d))
    q[..., 2] = ALPHA
    k = torch.zeros((1, T, 1, d))
    v = torch.zeros((1, T, 1, d))
    dout = torch.zeros((1, T, H, d))
    dout[..., 0] = 1.0
    for j in range(T):
        b = j // 128
        base, spike, sval = SPIKES[b]
        kp[0, j, 0, 0] = sval if j == spike else base
        k[0, j, 0, 1] = C_K[b]
        v[0, j, 0, :] = C_V[b]
    bf = lambda x: x.to(torch.bfloat16)
    return {n: bf(t) for n, t in dict(qp=qp, kp=kp, q=q, k=k, v=v, dout=dout).items()}


def hand_expected_idx():
    idx = np.full((1, 1, HW["T"], HW["topk"]), -7, dtype=np.int32)
    with open(os.path.join(GOLD, "hand_worked_384.txt")) as f:
        for line in f:
            if line.startswith("idx "):
                parts = line.split()
                t0, t1, ents = int(parts[1]), int(parts[2]), [int(x) for x in parts[3:]]
                idx[0, 0, t0:t1 + 1, :] = ents
    assert (idx != -7).all(), "fixture does not cover every token"
    return idx


def hand_expected_main(idx):
    """Closed forms of the file's header for every token, key and head."""
    T, H, d = HW["T"], HW["H"], HW["d"]
    scale = 1.0 / math.sqrt(d)
    O = np.zeros((1, T, H, d)); L = np.zeros((1, T, H)); dQ = np.zeros((1, T, H, d))
    dK = np.zeros((1, T, 1, d)); dV = np.zeros((1, T, 1, d))
    for t in range(T):
        blocks = [b for b in idx[0, 0, t] if b >= 0]
        nb = {b: min(128, t - 128 * b + 1) for b in blocks}
        n = sum(nb.values())
        o = sum(nb[b] * C_V[b] for b in blocks) / n
        O[0, t, :, :] = o
        L[0, t, :] = math.log(n)
        dQ[0, t, :, 1] = scale * sum(nb[b] * (C_V[b] - o) / n * C_K[b] for b in blocks)
        for b in blocks:
            for j in range(128 * b, min(128 * b + 128, t + 1)):
                dK[0, j, 0, 2] += H * scale * ALPHA * (C_V[b] - o) / n
                dV[0, j, 0, 0] += H / n
    return O, L, dQ, dK, dV


def test_hand_fixture_sample_points_match_closed_forms():
    """The written-out sample values in the fixture agree with the closed forms."""
    idx = hand_expected_idx()
    O, L, _, _, _ = hand_expected_main(idx)
    with open(os.path.join(GOLD, "hand_worked_384.txt")) as f:
        for line in f:
            if line.startswith("o "):
                _, t, expr = line.split()
                assert abs(O[0, int(t), 0, 0] - eval(expr, {})) < 1e-12, line
            if line.startswith("lse "):
                _, t, expr = line.split()
                assert abs(L[0, int(t), 0] - eval(expr, {"ln": math.log})) < 1e-12, line


def test_oracle_reproduces_hand_worked(oracle_mod):
    x = hand_inputs()
    dm = Dims(**HW)
    idx_ref = hand_expected_idx()
    idx = oracle_mod.select(dm, x["qp"], x["kp"])
    np.testing.assert_array_equal(idx, idx_ref)
    O, L, dQ, dK, dV = hand_expected_main(idx_ref)
    o, lse = oracle_mod.fwd(dm, x["q"], x["k"], x["v"], idx)
    dq, dk, dv = oracle_mod.bwd(dm, x["q"], x["k"], x["v"], x["dout"], idx)
    for name, got, ref in (("o", o, O), ("lse", lse, L), ("dq", dq, dQ), ("dk", dk, dK), ("dv", dv, dV)):
        np.testing.assert_allclose(got, ref, rtol=1e-9, atol=1e-9, err_msg=name)


def _load_tiny_golden():
    path = os.path.join(GOLD, "tiny_oracle_sample.txt")
    out = {}
    with open(path) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            parts = line.split()
            out.setdefault(parts[0], []).append(parts[1:])
    return out


def _tiny_sample_from(g, idx, o, lse, dq, dk, dv):
    """Pick the fixture's sample positions out of full result tensors."""
    got = {}
    for row in g["idx"]:
        t = int(row[0])
        got.setdefault("idx", []).append(np.asarray(idx)[0, 0, t, :].tolist())
    for name, arr in (("o", o), ("dq", dq)):
        got[name] = [float(np.asarray(arr)[0, int(r[0]), int(r[1]), int(r[2])]) for r in g[name]]
    got["lse"] = [float(np.asarray(lse)[0, int(r[0]), int(r[1])]) for r in g["lse"]]
    for name, arr in (("dk", dk), ("dv", dv)):
        got[name] = [float(np.asarray(arr)[0, int(r[0]), int(r[1]), int(r[2])]) for r in g[name]]
    return got


def test_oracle_reproduces_tiny_golden(oracle_mod):
    g = _load_tiny_golden()
    cfg = synth.CONFIGS["tiny"]
    x = synth.make_inputs(cfg)
    dm = Dims(cfg.B, cfg.T, cfg.H, cfg.G, cfg.d, cfg.dp, cfg.topk)
    idx = oracle_mod.select(dm, x["qp"], x["kp"])
    o, lse = oracle_mod.fwd(dm, x["q"], x["k"], x["v"], idx)
    dq, dk, dv = oracle_mod.bwd(dm, x["q"], x["k"], x["v"], x["dout"], idx)
    got = _tiny_sample_from(g, idx, o, lse, dq, dk, dv)
    assert got["idx"] == [[int(v) for v in r[1:]] for r in g["idx"]]
    for name in ("o", "lse", "dq", "dk", "dv"):
        ref = [float(r[-1]) for r in g[name]]
        np.testing.assert_allclose(got[name], ref, rtol=1e-12, atol=1e-15, err_msg=name)


@pytest.mark.gpu
def test_gpu_reproduces_hand_worked():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import block_sparse_attention_qk_amd as msa
    msa.load()
    print("golden hand-worked 384", flush=True)
    x = {n: t.cuda() for n, t in hand_inputs().items()}
    idx = msa.msa_proxy_select(x["qp"], x["kp"], HW["topk"])
    o, lse = msa.msa_fwd(x["q"], x["k"], x["v"], idx)
    dq, dk, dv = msa.msa_bwd(x["q"], x["k"], x["v"], o, x["dout"], lse, idx)
    torch.cuda.synchronize()
    idx_ref = hand_expected_idx()
    np.testing.assert_array_equal(idx.cpu().numpy(), idx_ref)
    O, L, dQ, dK, dV = hand_expected_main(idx_ref)
    for name, got, ref in (("o", o, O), ("lse", lse, L), ("dq", dq, dQ), ("dk", dk, dK), ("dv", dv, dV)):
        parity.assert_close(name, got.cpu(), ref, 0.999)


@pytest.mark.gpu
def test_gpu_matches_tiny_golden():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import block_sparse_attention_qk_amd as msa
    msa.load()
    print("golden tiny", flush=True)
    g = _load_tiny_golden()
    cfg = synth.CONFIGS["tiny"]
    x = {n: t.cuda() for n, t in synth.make_inputs(cfg).items()}
    idx = msa.msa_proxy_select(x["qp"], x["kp"], cfg.topk)
    o, lse = msa.msa_fwd(x["q"], x["k"], x["v"], idx)
    dq, dk, dv = msa.msa_bwd(x["q"], x["k"], x["v"], o, x["dout"], lse, idx)
    torch.cuda.synchronize()
    got = _tiny_sample_from(g, idx.cpu(), o.float().cpu(), lse.cpu(), dq.float().cpu(), dk.float().cpu(),
                            dv.float().cpu())
    assert got["idx"] == [[int(v) for v in r[1:]] for r in g["idx"]]
    for name in ("o", "lse", "dq", "dk", "dv"):
        ref = np.array([float(r[-1]) for r in g[name]])
        parity.assert_close(name, torch.tensor(got[name]), ref, 0.999)
