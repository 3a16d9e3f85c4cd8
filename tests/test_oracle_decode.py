"""The decode-step oracle (one new query per sequence against its caches) pinned
to things other than itself: a plain softmax over every cached key when the
cache row lists all causal blocks, a hand-built proxy cache whose block
ranking is known, the training rows of the same sequence, and the documented
handling of out-of-range lengths and non-causal entries."""
import numpy as np
import torch

import oracle
import synth
from oracle import Dims


def _decode_rows(x, lens):
    B = len(lens)
    qp = torch.stack([x["qp"][b, lens[b] - 1] for b in range(B)])
    q = torch.stack([x["q"][b, lens[b] - 1] for b in range(B)])
    return qp, q


def test_all_blocks_is_plain_softmax_over_the_prefix():
    # topk >= blocks: every cached key j <= t is read; compare with a direct
    # float64 softmax over the prefix (one query, R heads per group).
    cfg = synth.custom(2, 640, 4, 2, 64, 32, 8)
    x = synth.make_inputs(cfg, seed_offset=21)
    lens = [640, 200]
    dm = Dims(2, 640, 4, 2, 64, 32, 8, 0.3)
    qp, q = _decode_rows(x, lens)
    idx, _ = oracle.decode_select(dm, qp, x["kp"], lens)
    for b, L in enumerate(lens):
        nb = (L - 1) // 128 + 1
        for g in range(2):
            assert list(idx[b, g, :nb]) == list(range(nb)) and (idx[b, g, nb:] == -1).all()
    o, lse = oracle.decode_fwd(dm, q, x["k"], x["v"], lens, idx)
    for b, L in enumerate(lens):
        for h in range(4):
            g = h // 2
            kk = x["k"][b, :L, g].double().numpy()
            vv = x["v"][b, :L, g].double().numpy()
            s = 0.3 * kk @ q[b, h].double().numpy()
            m = s.max()
            p = np.exp(s - m)
            np.testing.assert_allclose(o[b, h], p @ vv / p.sum(), rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(lse[b, h], m + np.log(p.sum()), rtol=1e-12)


def test_hand_built_proxy_ranking():
    # One group, dp = 32, T = 640 (5 blocks).  qp = e0; every proxy key of block i
    # is c_i * e0 except in block 4, where only the first 10 keys (positions
    # 512..521) carry a large value c = 9 and the rest 100.  With len = 515 the
    # new token at t = 514 sees 3 keys of block 4 (value 9) and none of the 100s.
    T, dp = 640, 32
    c = [3.0, 1.0, 4.0, 1.5]
    kp = torch.zeros((1, T, 1, dp))
    for i, ci in enumerate(c):
        kp[0, 128 * i:128 * (i + 1), 0, 0] = ci
    kp[0, 512:522, 0, 0] = 9.0
    kp[0, 522:, 0, 0] = 100.0
    qp = torch.zeros((1, 1, dp))
    qp[0, 0, 0] = 1.0
    dm = Dims(1, T, 1, 1, 64, dp, 2)
    idx, pooled = oracle.decode_select(dm, qp, kp, [515])
    assert list(idx[0, 0]) == [2, 4]                      # scores 3, 1, 4, 1.5, 9
    np.testing.assert_array_equal(pooled[0, 0], np.array([3, 1, 4, 1.5, 9], dtype=np.float32))
    idx, pooled = oracle.decode_select(dm, qp, kp, [512])  # t = 511: block 4 not causal yet
    assert list(idx[0, 0]) == [0, 2]
    assert np.isneginf(pooled[0, 0, 4])
    idx, _ = oracle.decode_select(Dims(1, T, 1, 1, 64, dp, 3), qp, kp, [1])   # t = 0: one block
    assert list(idx[0, 0]) == [0, -1, -1]


def test_rows_equal_training_rows():
    cfg = synth.custom(2, 1536, 8, 2, 64, 32, 4)
    x = synth.make_inputs(cfg, seed_offset=22)
    dm = Dims(2, 1536, 8, 2, 64, 32, 4)
    lens = [1536, 700]
    full_idx = oracle.select(dm, x["qp"], x["kp"])
    o_full, lse_full = oracle.fwd(dm, x["q"], x["k"], x["v"], full_idx)
    qp, q = _decode_rows(x, lens)
    idx, _ = oracle.decode_select(dm, qp, x["kp"], lens)
    o, lse = oracle.decode_fwd(dm, q, x["k"], x["v"], lens, idx)
    for b, L in enumerate(lens):
        np.testing.assert_array_equal(idx[b], full_idx[b, :, L - 1])
        np.testing.assert_allclose(o[b], o_full[b, L - 1], rtol=0, atol=1e-14)
        np.testing.assert_allclose(lse[b], lse_full[b, L - 1], rtol=0, atol=1e-14)


def test_out_of_range_lengths_and_entries():
    cfg = synth.custom(3, 512, 4, 2, 64, 32, 2)
    x = synth.make_inputs(cfg, seed_offset=23)
    dm = Dims(3, 512, 4, 2, 64, 32, 2)
    lens = [0, 513, 300]
    qp = x["qp"][:, 0]
    q = x["q"][:, 0]
    idx, pooled = oracle.decode_select(dm, qp, x["kp"], lens)
    assert (idx[0] == -1).all() and (idx[1] == -1).all() and np.isneginf(pooled[:2]).all()
    bad = np.array(idx)
    bad[0] = 1
    bad[1] = 0
    bad[2, 0] = [1, 3]     # block 3 is not causal at t = 299 and is dropped
    bad[2, 1] = [3, -1]    # nothing left for group 1
    o, lse = oracle.decode_fwd(dm, q, x["k"], x["v"], lens, bad)
    assert (o[:2] == 0).all() and np.isneginf(lse[:2]).all()
    assert (o[2, 2:] == 0).all() and np.isneginf(lse[2, 2:]).all()
    one = np.array(bad)
    one[2, 0] = [1, -1]
    o1, lse1 = oracle.decode_fwd(dm, q, x["k"], x["v"], lens, one)
    np.testing.assert_array_equal(o1[2, :2], o[2, :2])
    assert np.isfinite(lse[2, :2]).all()
