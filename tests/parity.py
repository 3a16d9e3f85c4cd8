"""Comparison rules for HIP-path results against the oracle.

Indices (block-index cache): rows must match exactly, except a row whose k-th
and (k+1)-th oracle pooled scores are within 1e-3 relative of each other; such
a row passes if every block in the symmetric difference of the two sets has an
oracle score within that band of the k-th score.  Both sides keep a row
ascending with a -1 tail.

Main branch (o, lse, dq, dk, dv, computed with shared indices): cosine
similarity in float64 over the flattened tensors, and an element-wise error
bar.  The required bar is cos >= 0.99 (the pages cite a 0.01 cosine tolerance
for bf16 sweeps) and, for every element,

    |got - ref| <= 2e-2 + ulp_bf16(max(|got|, |ref|)) / 2

for outputs the boundary returns in bf16 (o, dq, dk, dv), and
|got - ref| <= 2e-2 for fp32 outputs (lse).  The 2e-2 is the literal max-abs
bar; the half ulp is the rounding of the exact value to the nearest bf16 that
the output format itself imposes (the oracle keeps float64), taken at the
binade of the larger of the two values so that a value rounded across a
power of two is covered.  Tests may ask for a higher cosine.

Every comparison prints one line: cosine, the literal max |got - ref|, max
|ref|, the largest error beyond the bf16 rounding allowance ("excess"), and
the worst element's fraction of its bar.
"""
from __future__ import annotations

import numpy as np

TIE_REL = 1e-3
COS_MIN = 0.99
MAX_ABS = 2e-2


def as_np(x) -> np.ndarray:
    try:
        import torch
        if isinstance(x, torch.Tensor):
            return x.detach().to("cpu", torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(x, dtype=np.float64)


def cosine(a, b) -> float:
    a = as_np(a).ravel()
    b = as_np(b).ravel()
    na, nb = np.linalg.norm(a), np.linalg.norm(b)
    if na == 0.0 and nb == 0.0:
        return 1.0
    return float(a @ b / (na * nb))


def max_abs(a, b) -> float:
    return float(np.max(np.abs(as_np(a) - as_np(b)))) if np.size(a) else 0.0


def half_ulp_bf16(x) -> np.ndarray:
    """Half the spacing of bfloat16 numbers (8 significant bits) in the binade
    of |x|: 2^(e - 8) for |x| in [2^e, 2^(e+1)); the subnormal spacing below
    the smallest normal."""
    a = np.abs(np.asarray(x, dtype=np.float64))
    _, e = np.frexp(np.maximum(a, 2.0 ** -126))  # a = m 2^e with m in [0.5, 1): binade exponent e - 1
    return np.ldexp(1.0, e - 1 - 8)


def _report(info: dict) -> str:
    return ("%-10s cos=%.7f max_abs=%.3e max|ref|=%.3e excess=%.3e worst/bar=%.3f n=%d" % (
        info["name"], info["cos"], info["max_abs"], info["ref_max"], info["excess"], info["worst_frac"], info["n"]))


def assert_close(name: str, got, ref, cos_min: float = COS_MIN, abs_max: float = MAX_ABS,
                 bf16_out=None) -> dict:
    """Element-wise bar |got - ref| <= abs_max (+ half a bf16 ulp when the
    output is bf16) and cosine >= cos_min; non-finite values must sit at the
    same positions with the same values.  bf16_out=None: every output is
    bf16 except lse (names starting with "lse"), which is fp32."""
    if bf16_out is None:
        bf16_out = not name.startswith("lse")
    g, r = as_np(got), as_np(ref)
    assert g.shape == r.shape, (name, g.shape, r.shape)
    finite = np.isfinite(r)
    assert np.array_equal(np.isfinite(g), finite), "%s: non-finite pattern differs" % name
    if not finite.all():
        assert np.array_equal(g[~finite], r[~finite], equal_nan=True), "%s: non-finite values differ" % name
    gf, rf = g[finite], r[finite]
    err = np.abs(gf - rf)
    allow = half_ulp_bf16(np.maximum(np.abs(gf), np.abs(rf))) if bf16_out else np.zeros_like(err)
    bar = abs_max + allow
    c = cosine(gf, rf)
    info = {"name": name, "cos": c, "max_abs": float(err.max()) if err.size else 0.0,
            "ref_max": float(np.abs(rf).max()) if rf.size else 0.0,
            "excess": float(np.max(err - allow)) if err.size else 0.0,
            "worst_frac": float(np.max(err / bar)) if err.size else 0.0, "n": int(err.size)}
    print("parity " + _report(info), flush=True)
    assert c >= cos_min, info
    assert np.all(err <= bar), info
    return info


def assert_consistent(name: str, got, ref, cos_min: float, rel: float) -> dict:
    """GPU-against-GPU consistency (results that differ only in the order of
    fp32 accumulation): cosine >= cos_min and max |got - ref| <= rel * max|ref|.
    Not a parity check against the oracle."""
    g, r = as_np(got), as_np(ref)
    assert g.shape == r.shape, (name, g.shape, r.shape)
    assert np.array_equal(np.isfinite(g), np.isfinite(r)), name
    f = np.isfinite(r)
    c = cosine(g[f], r[f])
    m = max_abs(g[f], r[f])
    scale = float(np.max(np.abs(r[f]))) if f.any() else 0.0
    info = {"name": name, "cos": c, "max_abs": m, "ref_max": scale}
    print("consistency %-10s cos=%.7f max_abs=%.3e max|ref|=%.3e" % (name, c, m, scale), flush=True)
    assert c >= cos_min and m <= rel * max(scale, 1e-30), info
    return info


def check_indices(idx_gpu, idx_ref, pooled_ref, topk: int, rows_t=None) -> dict:
    """idx_gpu/idx_ref: [..., topk] int arrays over the same rows; pooled_ref:
    [..., N] oracle pooled scores (-inf past the causal blocks); rows_t: the token
    position of every row (same leading shape), used for validity checks."""
    ig = np.asarray(idx_gpu).reshape(-1, topk)
    ir = np.asarray(idx_ref).reshape(-1, topk)
    pr = np.asarray(pooled_ref, dtype=np.float64)
    pr = pr.reshape(ig.shape[0], -1)
    diff_rows = np.nonzero((ig != ir).any(axis=1))[0]
    ties = 0
    for r in diff_rows:
        a = ig[r][ig[r] >= 0]
        b = ir[r][ir[r] >= 0]
        assert len(a) == len(b), ("row", int(r), a.tolist(), b.tolist())
        assert np.all(np.diff(a) > 0), ("gpu row not ascending", int(r), a.tolist())
        assert np.all(ig[r][len(a):] == -1), ("gpu row tail", int(r))
        scores = pr[r][np.isfinite(pr[r])]
        n = len(b)
        assert n < len(scores), ("all causal blocks must be chosen", int(r))
        order = np.sort(scores)[::-1]
        sk, sk1 = order[n - 1], order[n]
        band = TIE_REL * max(abs(sk), abs(sk1), 1e-6)
        assert sk - sk1 < band, ("not a near-tie", int(r), float(sk), float(sk1), a.tolist(), b.tolist())
        sym = np.setxor1d(a, b)
        assert np.all(np.abs(pr[r][sym] - sk) <= band), ("blocks outside the tie band", int(r), sym.tolist())
        ties += 1
    info = {"rows": int(ig.shape[0]), "tie_rows": ties}
    print("parity idx rows=%d tie_rows=%d" % (info["rows"], ties), flush=True)
    return info
