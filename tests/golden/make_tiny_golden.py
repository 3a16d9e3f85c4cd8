"""Write tiny_oracle_sample.txt: sampled oracle outputs on the tiny configuration.

Calls only the oracle and the seeded input generator (no HIP code).  Run from the
repository root:  python tests/golden/make_tiny_golden.py
"""
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import synth  # noqa: E402


def main():
    cfg = synth.CONFIGS["tiny"]
    x = synth.make_inputs(cfg)
    dm = oracle.Dims(cfg.B, cfg.T, cfg.H, cfg.G, cfg.d, cfg.dp, cfg.topk)
    idx = oracle.select(dm, x["qp"], x["kp"])
    o, lse = oracle.fwd(dm, x["q"], x["k"], x["v"], idx)
    dq, dk, dv = oracle.bwd(dm, x["q"], x["k"], x["v"], x["dout"], idx)
    rng = np.random.default_rng(2024)
    lines = ["# Sampled oracle outputs, tiny configuration (B=1 T=1024 H=4 G=1 d=64 dp=32 topk=4,",
             "# synth.CONFIGS['tiny'] inputs, default scale).  Written by tests/golden/make_tiny_golden.py",
             "# from the oracle alone.  Formats:",
             "#   idx t e0 .. e3            (block-index cache row of token t, group 0)",
             "#   o|dq t h c value          (element [0, t, h, c])",
             "#   lse t h value",
             "#   dk|dv j g c value         (element [0, j, g, c])"]
    for t in sorted(rng.choice(cfg.T, 32, replace=False)):
        lines.append("idx %d %s" % (t, " ".join(str(int(v)) for v in idx[0, 0, t])))
    for name, arr in (("o", o), ("dq", dq)):
        for _ in range(64):
            t, h, c = rng.integers(cfg.T), rng.integers(cfg.H), rng.integers(cfg.d)
            lines.append("%s %d %d %d %.17g" % (name, t, h, c, arr[0, t, h, c]))
    for _ in range(64):
        t, h = rng.integers(cfg.T), rng.integers(cfg.H)
        lines.append("lse %d %d %.17g" % (t, h, lse[0, t, h]))
    for name, arr in (("dk", dk), ("dv", dv)):
        for _ in range(64):
            j, g, c = rng.integers(cfg.T), rng.integers(cfg.G), rng.integers(cfg.d)
            lines.append("%s %d %d %d %.17g" % (name, j, g, c, arr[0, j, g, c]))
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_oracle_sample.txt")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("wrote", path)


if __name__ == "__main__":
    main()
