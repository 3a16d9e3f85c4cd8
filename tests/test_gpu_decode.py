"""Decode step (one new query per sequence) on the GPU through the C ABI
against the oracle: block indices bit-exact up to near-ties, o and lse to the
main parity bar with the GPU's indices shared, out-of-range lengths, and the
decode rows against the training path's rows of the same sequences."""
import numpy as np
import pytest
import torch

import parity
import synth
from oracle import Dims

pytestmark = pytest.mark.gpu

COS = 0.999


@pytest.fixture(scope="module")
def msa():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import block_sparse_attention_qk_amd as m
    m.load()
    return m


CASES = [
    # B, T, H, G, d, dp, topk, lens (cached tokens incl. the new one)
    (4, 2048, 8, 2, 128, 64, 4, [2048, 1, 129, 1000]),      # G*dp = 128: 2 groups per wave load
    (3, 1024, 4, 1, 64, 32, 16, [1024, 128, 700]),          # topk above the block count
    (2, 4096, 32, 4, 128, 64, 8, [4096, 3001]),             # 128K-config heads (R = 8)
    (2, 2048, 16, 1, 128, 128, 3, [2048, 1500]),            # R = 16, dp = 128
    (2, 1024, 2, 2, 64, 64, 2, [1024, 77]),                 # R = 1
    (2, 1024, 16, 16, 64, 32, 2, [1024, 513]),              # 16 groups in one wave load
    (1, 8192, 4, 1, 64, 32, 64, [8192]),                    # 64 blocks
    (1, 262144, 2, 1, 64, 32, 40, [262144 - 77]),           # 2048 blocks: two keys per top-k thread
    (2, 524288, 2, 1, 64, 32, 160, [524288, 300000]),       # 4096 blocks: four keys per top-k thread; wide combine
]


def _decode_case(msa, oracle_mod, cfg, lens, seed=0):
    x = synth.make_inputs(cfg, seed_offset=seed)
    B = cfg.B
    rows = [min(max(L, 1), cfg.T) - 1 for L in lens]
    qp = torch.stack([x["qp"][b, rows[b]] for b in range(B)])
    q = torch.stack([x["q"][b, rows[b]] for b in range(B)])
    dev = {n: x[n].cuda() for n in ("kp", "k", "v")}
    lens_d = torch.tensor(lens, dtype=torch.int32, device="cuda")
    idx = msa.msa_decode_select(qp.cuda(), dev["kp"], lens_d, cfg.topk)
    o, lse = msa.msa_decode_fwd(q.cuda(), dev["k"], dev["v"], lens_d, idx)
    torch.cuda.synchronize()
    dm = Dims(B, cfg.T, cfg.H, cfg.G, cfg.d, cfg.dp, cfg.topk)
    idx_h = idx.cpu().numpy()
    idx_ref, pooled = oracle_mod.decode_select(dm, qp, x["kp"], lens)
    valid = [b for b in range(B) if 1 <= lens[b] <= cfg.T]
    for b in range(B):
        if b not in valid:
            assert (idx_h[b] == -1).all()
    info = parity.check_indices(idx_h[valid], idx_ref[valid], pooled[valid], cfg.topk)
    o_ref, lse_ref = oracle_mod.decode_fwd(dm, q, x["k"], x["v"], lens, idx_h)
    res = [info, parity.assert_close("o", o.cpu()[valid], o_ref[valid], COS),
           parity.assert_close("lse", lse.cpu()[valid], lse_ref[valid], COS)]
    for b in range(B):
        if b not in valid:
            assert (o[b] == 0).all() and torch.isneginf(lse[b]).all()
    print(res, flush=True)
    return x, idx, o, lse


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B%dT%dH%dG%dd%ddp%dk%d" % c[:7])
def test_decode_matches_oracle(msa, oracle_mod, case):
    B, T, H, G, d, dp, topk, lens = case
    print("decode case", case, flush=True)
    _decode_case(msa, oracle_mod, synth.custom(B, T, H, G, d, dp, topk), lens, seed=31)


def test_out_of_range_lengths(msa, oracle_mod):
    print("decode lengths 0 and T+1", flush=True)
    _decode_case(msa, oracle_mod, synth.custom(3, 1024, 8, 2, 64, 32, 4), [0, 1025, 600], seed=32)


@pytest.mark.parametrize("T,topk", [(2048, 5), (1 << 20, 300)])
def test_equal_scores_take_the_lower_blocks(msa, oracle_mod, T, topk):
    """A proxy-key cache that repeats one 128-row block gives every complete
    block the same pooled score: the lowest block ids must win, on both sides."""
    print("decode ties", T, topk, flush=True)
    G, dp = 1, 32
    g = torch.Generator().manual_seed(7)
    base = torch.randn((128, G, dp), generator=g).to(torch.bfloat16)
    kp = base.repeat(T // 128, 1, 1).unsqueeze(0).contiguous()
    qp = torch.randn((1, G, dp), generator=g).to(torch.bfloat16)
    lens = [T - 3]
    idx = msa.msa_decode_select(qp.cuda(), kp.cuda(), torch.tensor(lens, dtype=torch.int32, device="cuda"), topk)
    torch.cuda.synchronize()
    dm = Dims(1, T, 1, G, 64, dp, topk)
    idx_ref, _ = oracle_mod.decode_select(dm, qp, kp, lens)
    np.testing.assert_array_equal(idx.cpu().numpy(), idx_ref)
    assert list(idx_ref[0, 0]) == list(range(topk))


@pytest.mark.parametrize("T,topk", [(1 << 17, 32), (1 << 20, 300)])
def test_few_distinct_scores_match_oracle(msa, oracle_mod, T, topk):
    """Every complete block repeats one 128-row proxy-key block scaled by 16, 8,
    4 or 1; with positive proxy queries the pooled scores take those four
    values times one maximum, exactly.  About k/2 blocks are scaled by 16 and a
    third by 8, so the k-th score is an 8 shared by far more blocks than are
    needed, with 16s on both sides of the needed ones: the chosen blocks must
    match the oracle's lowest-index-first choice bit for bit."""
    print("decode few distinct scores", T, topk, flush=True)
    G, dp, B = 1, 32, 2
    g = torch.Generator().manual_seed(43)
    N = T // 128
    base = torch.randn((128, G, dp), generator=g)
    u = torch.rand((B, N), generator=g)
    scale = torch.where(u < 0.5 * topk / N, 16.0, torch.where(u < 0.33, 8.0, torch.where(u < 0.66, 4.0, 1.0)))
    kp = (base.repeat(N, 1, 1)[None] * scale.repeat_interleave(128, dim=1)[:, :, None, None]).contiguous()
    kp = kp.to(torch.bfloat16)
    qp = (torch.rand((B, G, dp), generator=g) + 0.5).to(torch.bfloat16)
    lens = [T - 3, T // 2 + 100]
    idx = msa.msa_decode_select(qp.cuda(), kp.cuda(), torch.tensor(lens, dtype=torch.int32, device="cuda"), topk)
    torch.cuda.synchronize()
    dm = Dims(B, T, 1, G, 64, dp, topk)
    idx_ref, _ = oracle_mod.decode_select(dm, qp, kp, lens)
    np.testing.assert_array_equal(idx.cpu().numpy(), idx_ref)


def test_decode_rows_equal_training_rows(msa, oracle_mod):
    """A decode step over a sequence's caches gives that sequence's training row."""
    cfg = synth.custom(2, 4096, 32, 4, 128, 64, 8)
    lens = [4096, 2222]
    print("decode vs training rows", cfg, flush=True)
    x, idx, o, lse = _decode_case(msa, oracle_mod, cfg, lens, seed=33)
    dev = {n: t.cuda() for n, t in x.items()}
    idx_t = msa.msa_proxy_select(dev["qp"], dev["kp"], cfg.topk)
    o_t, lse_t = msa.msa_fwd(dev["q"], dev["k"], dev["v"], idx_t)
    torch.cuda.synchronize()
    for b, L in enumerate(lens):
        assert torch.equal(idx[b].cpu(), idx_t[b, :, L - 1].cpu()), b
        parity.assert_consistent("o_vs_train", o[b].cpu(), o_t[b, L - 1].cpu(), 0.99999, 2 ** -7)
        parity.assert_consistent("lse_vs_train", lse[b].cpu(), lse_t[b, L - 1].cpu(), 0.99999, 1e-4)


def _full_size_check(msa, oracle_mod, cfg, B, lens):
    import bench
    print("full-size decode", cfg.name, B, lens, flush=True)
    x = bench.gpu_decode_inputs(cfg, B, seed=5)
    lens_d = torch.tensor(lens, dtype=torch.int32, device="cuda")
    idx = msa.msa_decode_select(x["qp"], x["kp"], lens_d, cfg.topk)
    o, lse = msa.msa_decode_fwd(x["q"], x["k"], x["v"], lens_d, idx)
    torch.cuda.synchronize()
    dm = Dims(B, cfg.T, cfg.H, cfg.G, cfg.d, cfg.dp, cfg.topk)
    idx_h = idx.cpu().numpy()
    idx_ref, pooled = oracle_mod.decode_select(dm, x["qp"].cpu(), x["kp"].cpu(), lens)
    print("indices", parity.check_indices(idx_h, idx_ref, pooled, cfg.topk), flush=True)
    o_ref, lse_ref = oracle_mod.decode_fwd(dm, x["q"].cpu(), x["k"].cpu(), x["v"].cpu(), lens, idx_h)
    print(parity.assert_close("o", o.cpu(), o_ref, COS), parity.assert_close("lse", lse.cpu(), lse_ref, COS),
          flush=True)


def test_128k_config_decode(msa, oracle_mod):
    cfg = synth.CONFIGS["128k"]
    _full_size_check(msa, oracle_mod, cfg, 2, [cfg.T, 100003])


def test_1m_config_decode(msa, oracle_mod):
    cfg = synth.CONFIGS["1m"]
    _full_size_check(msa, oracle_mod, cfg, 1, [cfg.T - 5])
