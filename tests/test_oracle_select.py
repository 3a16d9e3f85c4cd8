"""Pins for the oracle's Index Branch (proxy score -> 128-key block max-pool ->
causal top-k -> ascending block-index cache).

Each test fixes the answer from something other than the oracle itself: the
all-blocks special case, planted keys whose blocks must win, a closed form when
every key of a block equals its block mean, exact ties, invariances, and a
whole-matrix brute force.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import Dims

BLOCK = 128


def _bf16(x):
    return torch.as_tensor(x, dtype=torch.float32).to(torch.bfloat16)


def _rand(shape, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(shape, generator=g).to(torch.bfloat16)


def _dims(B, T, G, dp, topk):
    return Dims(B=B, T=T, H=G, G=G, d=16, dp=dp, topk=topk)


def test_topk_ge_blocks_selects_every_causal_block(oracle_mod):
    B, T, G, dp = 2, 600, 2, 8               # ragged last block on purpose
    N = (T + BLOCK - 1) // BLOCK
    dm = _dims(B, T, G, dp, topk=N + 2)
    idx = oracle_mod.select(dm, _rand((B, T, G, dp), 1), _rand((B, T, G, dp), 2))
    assert idx.shape == (B, G, T, N + 2)
    for t in range(T):
        nc = t // BLOCK + 1
        want = list(range(nc)) + [-1] * (N + 2 - nc)
        assert (idx[:, :, t, :] == np.array(want)).all()


def test_planted_blocks_are_selected(oracle_mod):
    B, T, G, dp, K = 1, 1024, 2, 16, 3
    dm = _dims(B, T, G, dp, topk=K)
    qp = _rand((B, T, G, dp), 3).float()
    kp = _rand((B, T, G, dp), 4).float()
    rng = np.random.default_rng(0)
    rows = [200, 383, 384, 700, 1023]
    plan = {}
    for t in rows:
        for g in range(G):
            nc = t // BLOCK + 1
            chosen = sorted(rng.choice(nc, size=min(K, nc), replace=False).tolist())
            plan[(t, g)] = chosen
    # Plant after choosing so that planted keys do not disturb each other's rows
    # more than the strength margin allows: one key per chosen block, aligned
    # with q_p[t] and 8x its size.
    for (t, g), chosen in plan.items():
        for blk in chosen:
            j = min(blk * BLOCK + (t * 7 + g) % BLOCK, t)   # a causal key in the block
            kp[0, j, g] = 8.0 * qp[0, t, g]
    idx = oracle_mod.select(dm, _bf16(qp), _bf16(kp), rows=rows)
    for r, t in enumerate(rows):
        for g in range(G):
            assert idx[r, g, :len(plan[(t, g)])].tolist() == plan[(t, g)], (t, g)


def test_causal_mask_inside_diagonal_block(oracle_mod):
    """A huge key at j = t counts; the same key at j = t + 1 is invisible."""
    B, T, G, dp = 1, 512, 1, 8
    dm = _dims(B, T, G, dp, topk=1)
    qp = torch.ones((B, T, G, dp))
    kp = -torch.ones((B, T, G, dp))          # every key scores -dp ...
    t = 300                                   # diagonal block 2 (keys 256..383)
    kp[0, t] = 1.0                            # ... except key t itself
    idx = oracle_mod.select(dm, _bf16(qp), _bf16(kp), rows=[t])
    assert idx[0, 0, 0] == 2
    kp[0, t] = -1.0
    kp[0, t + 1] = 1.0                        # a future key: not visible to query t
    idx = oracle_mod.select(dm, _bf16(qp), _bf16(kp), rows=[t])
    assert idx[0, 0, 0] == 0                  # all blocks tie at -dp -> lowest index


def test_ties_go_to_lower_block_and_zero_scores_tie(oracle_mod):
    B, T, G, dp, K = 1, 1024, 1, 8, 2
    dm = _dims(B, T, G, dp, topk=K)
    kp = _rand((B, T, G, dp), 5).float()
    qp = _rand((B, T, G, dp), 6).float()
    # Blocks 2 and 5 get identical strong content: exact tie in the pooled score.
    strong = 6.0 * qp[0, 1023, 0]
    kp[0, 2 * BLOCK + 17, 0] = strong
    kp[0, 5 * BLOCK + 90, 0] = strong
    kp[0, 6 * BLOCK + 3, 0] = 5.0 * qp[0, 1023, 0]     # clear third
    dm1 = _dims(B, T, G, dp, topk=1)
    idx1 = oracle_mod.select(dm1, _bf16(qp), _bf16(kp), rows=[1023])
    assert idx1[0, 0].tolist() == [2]
    idx2 = oracle_mod.select(dm, _bf16(qp), _bf16(kp), rows=[1023])
    assert idx2[0, 0].tolist() == [2, 5]
    # A zero proxy query scores +0/-0 everywhere: all blocks tie -> lowest indices.
    qz = torch.zeros_like(qp)
    kneg = -torch.abs(kp) - 0.5
    idx0 = oracle_mod.select(dm, _bf16(qz), _bf16(kneg), rows=[1023])
    assert idx0[0, 0].tolist() == [0, 1]


def test_block_mean_closed_form(oracle_mod):
    """If every key of block b equals mu_b, the pooled score is fl32(q . mu_b) and
    the selection is the top-k of those closed-form scores."""
    B, T, G, dp, K = 1, 2048, 2, 16, 5
    N = T // BLOCK
    dm = _dims(B, T, G, dp, topk=K)
    mu = _rand((B, N, G, dp), 7).float()
    kp = mu[:, torch.arange(T) // BLOCK]                  # [B, T, G, dp]
    qp = _rand((B, T, G, dp), 8)
    rows = list(range(0, T, 37))
    idx = oracle_mod.select(dm, qp, _bf16(kp), rows=rows)
    q64 = qp.double().numpy()
    m64 = _bf16(mu).double().numpy()
    for r, t in enumerate(rows):
        nc = t // BLOCK + 1
        for g in range(G):
            s = (m64[0, :nc, g] @ q64[0, t, g]).astype(np.float32)
            order = sorted(range(nc), key=lambda i: (-float(s[i]), i))
            want = sorted(order[:min(K, nc)])
            assert idx[r, g, :len(want)].tolist() == want
            assert (idx[r, g, len(want):] == -1).all()


def test_invariances(oracle_mod):
    """Selection is unchanged by (a) scaling q_p by 2 (exact in bf16 and fp32) and
    (b) permuting keys inside every block, for queries that end a block."""
    cfg = synth.custom(1, 1536, 2, 2, 16, 16, 3)
    dm = _dims(cfg.B, cfg.T, cfg.G, cfg.dp, cfg.topk)
    qp, kp = synth.make_tensor("qp", cfg), synth.make_tensor("kp", cfg)
    rows = [BLOCK * i + BLOCK - 1 for i in range(cfg.T // BLOCK)]
    base = oracle_mod.select(dm, qp, kp, rows=rows)
    assert (oracle_mod.select(dm, qp * 2, kp, rows=rows) == base).all()
    perm = torch.cat([torch.randperm(BLOCK, generator=torch.Generator().manual_seed(i)) + i * BLOCK
                      for i in range(cfg.T // BLOCK)])
    assert (oracle_mod.select(dm, qp, kp[:, perm], rows=rows) == base).all()


def test_whole_matrix_brute_force(oracle_mod):
    """Bit-equal to a whole-matrix formulation: full score matrix in fp64 ->
    fp32 -> causal mask -> per-block amax -> lexicographic sort."""
    cfg = synth.custom(2, 768, 2, 2, 16, 32, 3)
    dm = _dims(cfg.B, cfg.T, cfg.G, cfg.dp, cfg.topk)
    qp, kp = synth.make_tensor("qp", cfg), synth.make_tensor("kp", cfg)
    idx, pooled = oracle_mod.select(dm, qp, kp, return_pooled=True)
    T, N, K = cfg.T, cfg.N, cfg.topk
    for b in range(cfg.B):
        for g in range(cfg.G):
            s = (qp[b, :, g].double() @ kp[b, :, g].double().T).float()
            s = s.masked_fill(torch.ones(T, T, dtype=torch.bool).triu(1), float("-inf"))
            pb = s.view(T, N, BLOCK).amax(dim=2).numpy()
            causal = (np.arange(N)[None, :] <= (np.arange(T) // BLOCK)[:, None])
            assert np.array_equal(np.where(causal, pb, -np.inf), pooled[b, g])
            for t in range(T):
                nc = t // BLOCK + 1
                order = np.lexsort((np.arange(nc), -pb[t, :nc].astype(np.float64)))
                want = np.sort(order[:min(K, nc)])
                got = idx[b, g, t]
                assert got[:len(want)].tolist() == want.tolist()
                assert (got[len(want):] == -1).all()


def test_rejects_out_of_range_rows(oracle_mod):
    dm = _dims(1, 256, 1, 8, 1)
    with pytest.raises(ValueError):
        oracle_mod.select(dm, _rand((1, 256, 1, 8), 1), _rand((1, 256, 1, 8), 2), rows=[256])
