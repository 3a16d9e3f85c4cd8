"""Parity of the HIP path (through the C ABI) against the CPU oracle.

Every case draws seeded inputs from ``synth``, runs msa_proxy_select, msa_fwd
and msa_bwd on the GPU, and compares with the oracle: indices bit-exact up to
near-ties, main branch with the GPU's own indices (shared indices) against
cos >= 0.999 (tighter than the 0.99 target bar) and, element by element,
|got - ref| <= 2e-2 plus half a bf16 ulp of the value (the rounding of the
bf16 outputs; lse is fp32 and gets the plain 2e-2).

Small shapes are checked on every output element.  The 16K and 128K
configurations run at full size on the GPU and are checked on sampled tokens
(idx, o, lse, dq depend only on their own row) and sampled key blocks (dk,
dv, recomputed by the oracle from every pair that selected the block),
including at 128K blocks whose backward is cut into several work items.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import Dims
import parity

pytestmark = pytest.mark.gpu

COS = 0.999


@pytest.fixture(scope="module")
def msa():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import block_sparse_attention_qk_amd as m
    m.load()  # fails loudly if libmsa.so was not built
    return m


def _dims(cfg, scale=0.0):
    return Dims(cfg.B, cfg.T, cfg.H, cfg.G, cfg.d, cfg.dp, cfg.topk, scale)


def _gpu_all(msa, x, topk, scale=0.0, ws=None):
    dev = {n: t.cuda() for n, t in x.items()}
    idx = msa.msa_proxy_select(dev["qp"], dev["kp"], topk, ws=ws)
    o, lse = msa.msa_fwd(dev["q"], dev["k"], dev["v"], idx, scale=scale, ws=ws)
    dq, dk, dv = msa.msa_bwd(dev["q"], dev["k"], dev["v"], o, dev["dout"], lse, idx, scale=scale, ws=ws)
    torch.cuda.synchronize()
    return {n: t.cpu() for n, t in dict(idx=idx, o=o, lse=lse, dq=dq, dk=dk, dv=dv).items()}


def _full_check(msa, oracle_mod, cfg, seed=0, scale=0.0):
    print("case", cfg, "seed", seed, flush=True)
    x = synth.make_inputs(cfg, seed_offset=seed)
    r = _gpu_all(msa, x, cfg.topk, scale)
    dm = _dims(cfg, scale)
    idx_ref, pooled = oracle_mod.select(dm, x["qp"], x["kp"], return_pooled=True)
    info = parity.check_indices(r["idx"].numpy(), idx_ref, pooled, cfg.topk)
    idx = r["idx"].numpy()
    o_ref, lse_ref = oracle_mod.fwd(dm, x["q"], x["k"], x["v"], idx)
    dq_ref, dk_ref, dv_ref = oracle_mod.bwd(dm, x["q"], x["k"], x["v"], x["dout"], idx)
    out = [info]
    out.append(parity.assert_close("o", r["o"], o_ref, COS))
    out.append(parity.assert_close("lse", r["lse"], lse_ref, COS))
    out.append(parity.assert_close("dq", r["dq"], dq_ref, COS))
    out.append(parity.assert_close("dk", r["dk"], dk_ref, COS))
    out.append(parity.assert_close("dv", r["dv"], dv_ref, COS))
    print(out, flush=True)
    return r, x


def test_tiny_config(msa, oracle_mod):
    _full_check(msa, oracle_mod, synth.CONFIGS["tiny"])


EDGE = [
    # B, T, H, G, d, dp, topk
    (3, 1152, 24, 3, 128, 64, 4),    # odd batch and group counts, R = 8, 9 blocks
    (2, 640, 4, 2, 64, 32, 3),       # two batches, two groups, 5 blocks (ragged 256-query tile)
    (1, 768, 8, 1, 128, 64, 16),     # topk > blocks: every causal block
    (1, 512, 16, 1, 128, 128, 1),    # one block per query, R = 16, dp = 128
    (1, 384, 2, 2, 64, 64, 2),       # R = 1
    (1, 128, 4, 1, 64, 32, 2),       # a single block
    (1, 2432, 8, 2, 128, 64, 5),     # 19 blocks, d = 128, R = 4
]


@pytest.mark.parametrize("shape", EDGE, ids=lambda s: "B%dT%dH%dG%dd%ddp%dk%d" % s)
def test_edge_shapes(msa, oracle_mod, shape):
    _full_check(msa, oracle_mod, synth.custom(*shape), seed=11)


def test_repeated_calls_are_bitwise_reproducible(msa):
    """idx, o, lse and dq do not depend on scheduling: two runs on the same
    inputs agree bit for bit.  dK/dV sum a block's selecting tokens in the order
    of the inverse index, whose positions come from LDS atomics, so only their
    last bits may differ."""
    cfg = synth.custom(1, 4096, 16, 2, 128, 64, 8)
    x = synth.make_inputs(cfg, seed_offset=21)
    a = _gpu_all(msa, x, cfg.topk)
    b = _gpu_all(msa, x, cfg.topk)
    for n in ("idx", "o", "lse", "dq"):
        assert torch.equal(a[n], b[n]), n
    for n in ("dk", "dv"):
        parity.assert_consistent(n, a[n], b[n], 0.999999, 2 ** -6)


def test_custom_scale(msa, oracle_mod):
    _full_check(msa, oracle_mod, synth.custom(1, 1024, 8, 2, 64, 32, 3), seed=5, scale=0.05)


def test_dense_mode_matches_torch_sdpa(msa):
    """With topk >= number of blocks the path is dense causal GQA attention:
    compare with PyTorch's SDPA and its autograd, in float32 on the CPU."""
    cfg = synth.custom(1, 512, 8, 2, 64, 32, 8)
    x = synth.make_inputs(cfg, seed_offset=3)
    r = _gpu_all(msa, x, cfg.topk)
    R = cfg.H // cfg.G
    q = x["q"].float().permute(0, 2, 1, 3).requires_grad_(True)
    k = x["k"].float().repeat_interleave(R, dim=2).permute(0, 2, 1, 3).detach().requires_grad_(True)
    v = x["v"].float().repeat_interleave(R, dim=2).permute(0, 2, 1, 3).detach().requires_grad_(True)
    o = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True)
    (o * x["dout"].float().permute(0, 2, 1, 3)).sum().backward()
    dk = k.grad.permute(0, 2, 1, 3).reshape(1, cfg.T, cfg.G, R, cfg.d).sum(3)
    dv = v.grad.permute(0, 2, 1, 3).reshape(1, cfg.T, cfg.G, R, cfg.d).sum(3)
    parity.assert_close("o", r["o"], o.detach().permute(0, 2, 1, 3), COS)
    parity.assert_close("dq", r["dq"], q.grad.permute(0, 2, 1, 3), COS)
    parity.assert_close("dk", r["dk"], dk, COS)
    parity.assert_close("dv", r["dv"], dv, COS)


class _FixedWs:
    """A caller workspace of a fixed size (forces the token-window walk)."""

    def __init__(self, nbytes):
        self.buf = torch.empty(int(nbytes), dtype=torch.uint8, device="cuda")

    def get(self, nbytes):
        return self.buf


def test_small_workspace_walks_windows(msa):
    cfg = synth.custom(2, 1536, 8, 2, 128, 64, 4)
    x = synth.make_inputs(cfg, seed_offset=9)
    full = _gpu_all(msa, x, cfg.topk)
    mins = [msa.msa_workspace_min_bytes(cfg.B, cfg.T, cfg.H, cfg.G, cfg.d, cfg.dp, cfg.topk, op)
            for op in (msa.OP_SELECT, msa.OP_FWD, msa.OP_BWD)]
    fulls = [msa.msa_workspace_bytes(cfg.B, cfg.T, cfg.H, cfg.G, cfg.d, cfg.dp, cfg.topk, op)
             for op in (msa.OP_SELECT, msa.OP_FWD, msa.OP_BWD)]
    assert all(m < f for m, f in zip(mins, fulls))
    small = _gpu_all(msa, x, cfg.topk, ws=_FixedWs(max(mins)))
    # Per-pair work is identical whatever the window: bitwise equal except the
    # dK/dV sums, whose order over selecting tokens depends on the window split.
    for n in ("idx", "o", "lse", "dq"):
        assert torch.equal(full[n], small[n]), n
    for n in ("dk", "dv"):
        parity.assert_consistent(n, small[n], full[n], 0.99999, 2 ** -7)


# A backward work item holds at most this many pairs; a block selected by more
# tokens is cut into several items whose dK/dV meet in one accumulator through
# float atomics.
BWD_ITEM_PAIRS = 1024


def _sampled_check(msa, oracle_mod, cfg, n_rows, blocks_per_group, seed=0, split_blocks=()):
    """split_blocks: (group, block) pairs that must be cut into several backward
    items; each is checked on every element of its dK/dV against the oracle."""
    print("sampled case", cfg, flush=True)
    x = synth.make_inputs(cfg, seed_offset=seed)
    r = _gpu_all(msa, x, cfg.topk)
    dm = _dims(cfg)
    rng = np.random.default_rng(1234)
    rows = np.sort(rng.choice(cfg.B * cfg.T, size=n_rows, replace=False))
    idx_ref, pooled = oracle_mod.select(dm, x["qp"], x["kp"], rows=rows, return_pooled=True)
    b_, t_ = rows // cfg.T, rows % cfg.T
    bt, tt = torch.from_numpy(b_), torch.from_numpy(t_)
    idx = r["idx"].numpy()
    idx_rows = idx[b_, :, t_, :]                       # [n, G, topk]
    info = parity.check_indices(idx_rows, idx_ref, pooled, cfg.topk)
    print("indices", info, flush=True)
    f64 = {n: x[n].double().numpy() for n in ("q", "k", "v", "dout")}
    o_ref, lse_ref = oracle_mod.fwd(dm, f64["q"], f64["k"], f64["v"], idx, rows=rows)
    res = [parity.assert_close("o", r["o"][bt, tt], o_ref, COS),
           parity.assert_close("lse", r["lse"][bt, tt], lse_ref, COS)]
    dq_ref = oracle_mod.bwd_rows(dm, f64["q"], f64["k"], f64["v"], f64["dout"], idx, rows=rows)
    res.append(parity.assert_close("dq", r["dq"][bt, tt], dq_ref, COS))
    N = cfg.N
    blocks = []
    for g in range(cfg.G):
        for blk in blocks_per_group:
            blocks.append((0 * cfg.G + g) * N + blk)
    dk_ref, dv_ref = oracle_mod.bwd_blocks(dm, f64["q"], f64["k"], f64["v"], f64["dout"], idx, blocks)
    dk_g = torch.stack([r["dk"][0, (c % N) * 128:(c % N) * 128 + 128, (c // N) % cfg.G] for c in blocks])
    dv_g = torch.stack([r["dv"][0, (c % N) * 128:(c % N) * 128 + 128, (c // N) % cfg.G] for c in blocks])
    res.append(parity.assert_close("dk_blocks", dk_g, dk_ref, COS))
    res.append(parity.assert_close("dv_blocks", dv_g, dv_ref, COS))
    for g, blk in split_blocks:
        readers = int((idx[0, g] == blk).any(axis=1).sum())
        print("split block g=%d blk=%d: %d selecting tokens" % (g, blk, readers), flush=True)
        assert readers > BWD_ITEM_PAIRS, (g, blk, readers)
        dk_ref, dv_ref = oracle_mod.bwd_blocks(dm, f64["q"], f64["k"], f64["v"], f64["dout"], idx, [g * N + blk])
        sl = slice(blk * 128, blk * 128 + 128)
        res.append(parity.assert_close("dk_split", r["dk"][0, sl, g][None], dk_ref, COS))
        res.append(parity.assert_close("dv_split", r["dv"][0, sl, g][None], dv_ref, COS))
    # Global invariants at full size: sum_j dK_j = 0 and sum_j dV_j = sum dO per group.
    R = cfg.H // cfg.G
    dk_sum = r["dk"].double().sum(dim=1)
    dv_sum = r["dv"].double().sum(dim=1)
    do_sum = x["dout"].double().view(cfg.B, cfg.T, cfg.G, R, cfg.d).sum(dim=(1, 3))
    dk_mass = r["dk"].double().abs().sum(dim=1)
    assert (dk_sum.abs() / dk_mass.clamp_min(1e-30)).max().item() < 1e-2
    parity.assert_close("dv_total", dv_sum, do_sum, 0.99999, 1e-3 * do_sum.abs().max().item(), bf16_out=False)
    print(res, flush=True)


def test_16k_config_sampled(msa, oracle_mod):
    cfg = synth.CONFIGS["16k"]
    _sampled_check(msa, oracle_mod, cfg, n_rows=768, blocks_per_group=[0, 63, cfg.N - 2, cfg.N - 1])


def test_128k_config_sampled(msa, oracle_mod):
    cfg = synth.CONFIGS["128k"]
    # block 0 (about 18K selecting tokens per group: five items), block 100 (three)
    # and block 300 (two) go through the atomically added backward items
    _sampled_check(msa, oracle_mod, cfg, n_rows=1024, blocks_per_group=[cfg.N // 2, cfg.N - 3, cfg.N - 1],
                   split_blocks=[(0, 0), (1, 100), (2, 300)])


def _gpu_generated_check(msa, oracle_mod, cfg, n_rows, blocks_from_end, seed=0, split_from_end=()):
    """Full-size run with inputs drawn on the GPU (same recipe as synth: N(0,1)
    bf16, block-mean proxy keys), checked on sampled rows and on late key
    blocks.  split_from_end: further blocks (counted from the end) that must be
    read by more tokens than one backward item holds, so that their dK/dV are
    added atomically from several items; they are checked on every element
    like the others.  The oracle gets full-size host arrays in which only the
    rows it reads are filled (the rest stay untouched zero pages)."""
    import bench
    print("gpu-generated case", cfg, flush=True)
    x = bench.gpu_inputs(cfg, seed=seed)
    idx_d = msa.msa_proxy_select(x["qp"], x["kp"], cfg.topk)
    o, lse = msa.msa_fwd(x["q"], x["k"], x["v"], idx_d)
    dq, dk, dv = msa.msa_bwd(x["q"], x["k"], x["v"], o, x["dout"], lse, idx_d)
    torch.cuda.synchronize()
    dm = _dims(cfg)
    N, R = cfg.N, cfg.H // cfg.G
    rng = np.random.default_rng(4321)
    rows = np.sort(rng.choice(cfg.B * cfg.T, size=n_rows, replace=False))
    bt, tt = torch.from_numpy(rows // cfg.T), torch.from_numpy(rows % cfg.T)
    idx = idx_d.cpu().numpy()
    # tokens whose rows the oracle reads: the samples and every selector of the checked blocks
    blocks = [N - 1 - i for i in list(blocks_from_end) + list(split_from_end)]
    for i in split_from_end:
        for g in range(cfg.G):
            readers = int((idx[0, g] == N - 1 - i).any(axis=1).sum())
            print("split block g=%d blk=%d: %d selecting tokens" % (g, N - 1 - i, readers), flush=True)
            assert readers > BWD_ITEM_PAIRS, (g, N - 1 - i, readers)
    sel = np.zeros(cfg.T, dtype=bool)
    sel[rows % cfg.T] = True
    for g in range(cfg.G):
        for blk in blocks:
            sel |= (idx[0, g] == blk).any(axis=1)
    need = torch.from_numpy(np.nonzero(sel)[0])
    print("oracle rows", int(need.numel()), flush=True)

    def host_rows(t):
        full = np.zeros(tuple(t.shape), dtype=np.float64)
        full[0, need.numpy()] = t[0, need.cuda()].double().cpu().numpy()
        return full

    qp64 = np.zeros(tuple(x["qp"].shape), dtype=np.float64)
    qp64[0, rows % cfg.T] = x["qp"][0, tt.cuda()].double().cpu().numpy()
    kp64 = x["kp"].double().cpu().numpy()
    idx_ref, pooled = oracle_mod.select(dm, qp64, kp64, rows=rows, return_pooled=True)
    del kp64, qp64
    info = parity.check_indices(idx[0][:, rows % cfg.T, :].transpose(1, 0, 2), idx_ref, pooled, cfg.topk)
    print("indices", info, flush=True)
    q64, do64 = host_rows(x["q"]), host_rows(x["dout"])
    k64, v64 = x["k"].double().cpu().numpy(), x["v"].double().cpu().numpy()
    o_ref, lse_ref = oracle_mod.fwd(dm, q64, k64, v64, idx, rows=rows)
    res = [parity.assert_close("o", o[bt.cuda(), tt.cuda()].cpu(), o_ref, COS),
           parity.assert_close("lse", lse[bt.cuda(), tt.cuda()].cpu(), lse_ref, COS)]
    dq_ref = oracle_mod.bwd_rows(dm, q64, k64, v64, do64, idx, rows=rows)
    res.append(parity.assert_close("dq", dq[bt.cuda(), tt.cuda()].cpu(), dq_ref, COS))
    codes = [g * N + blk for g in range(cfg.G) for blk in blocks]
    dk_ref, dv_ref = oracle_mod.bwd_blocks(dm, q64, k64, v64, do64, idx, codes)
    dk_g = torch.stack([dk[0, (c % N) * 128:(c % N) * 128 + 128, c // N].cpu() for c in codes])
    dv_g = torch.stack([dv[0, (c % N) * 128:(c % N) * 128 + 128, c // N].cpu() for c in codes])
    res.append(parity.assert_close("dk_blocks", dk_g, dk_ref, COS))
    res.append(parity.assert_close("dv_blocks", dv_g, dv_ref, COS))
    dv_sum = dv.double().sum(dim=1)
    do_sum = x["dout"].double().view(cfg.B, cfg.T, cfg.G, R, cfg.d).sum(dim=(1, 3))
    parity.assert_close("dv_total", dv_sum.cpu(), do_sum.cpu(), 0.99999, 1e-3 * do_sum.abs().max().item(),
                        bf16_out=False)
    print(res, flush=True)


def test_512k_config_gpu_generated(msa, oracle_mod):
    _gpu_generated_check(msa, oracle_mod, synth.CONFIGS["512k"], n_rows=1024, blocks_from_end=[0, 2],
                         split_from_end=[800])


def test_1m_config_gpu_generated(msa, oracle_mod):
    _gpu_generated_check(msa, oracle_mod, synth.CONFIGS["1m"], n_rows=1024, blocks_from_end=[0, 1],
                         split_from_end=[600])


def test_max_topk_dense_128k_gpu_generated(msa, oracle_mod):
    """topk = 1024, the largest the boundary takes: at T = 131072 every query
    selects every causal block (dense causal attention through the sparse
    kernels).  Block 0 is then picked by all 131072 tokens, so its backward
    list is cut into 128 items whose dK/dV are added atomically.  Checked on
    sampled rows and on late key blocks against the oracle."""
    cfg = synth.Config("128k-topk1024", 1, 131072, 8, 1, 128, 64, 1024)
    _gpu_generated_check(msa, oracle_mod, cfg, n_rows=32, blocks_from_end=[0, 1], seed=2)


@pytest.mark.parametrize("T,topk", [(1 << 18, 40), (1 << 20, 288)])
def test_long_rows_equal_scores_take_the_lower_blocks(msa, oracle_mod, T, topk):
    """Rows longer than 1024 blocks go through the radix select.  A proxy-key
    cache that repeats one 128-row block gives every complete block the same
    pooled score, so the lowest block ids must win (and match the oracle)."""
    print("long-row ties", T, topk, flush=True)
    G, dp = 1, 32
    g = torch.Generator().manual_seed(17)
    base = torch.randn((128, G, dp), generator=g).to(torch.bfloat16)
    kp = base.repeat(T // 128, 1, 1).unsqueeze(0).contiguous()
    qp = torch.randn((1, T, G, dp), generator=g).to(torch.bfloat16)
    idx = msa.msa_proxy_select(qp.cuda(), kp.cuda(), topk)
    torch.cuda.synchronize()
    rows = np.array([T - 1, T - 200, T // 2 + 77, 300 * 128 + 5, 200 * 128 + 127])
    dm = Dims(1, T, G, G, 64, dp, topk)
    idx_ref = oracle_mod.select(dm, qp, kp, rows=rows)
    got = idx[0, 0].cpu().numpy()[rows]
    np.testing.assert_array_equal(got, idx_ref[:, 0, :])


@pytest.mark.parametrize("T,topk,big", [(1 << 18, 40, 1500), (1 << 20, 288, 6000)])
def test_long_rows_surplus_ties_keep_a_later_larger_block(msa, oracle_mod, T, topk, big):
    """Rows longer than 1024 blocks whose k-th score is shared by more blocks
    than are needed, with one strictly larger block far after them: every
    complete block repeats one 128-row proxy-key block (equal pooled scores),
    and block `big` holds those keys times 4 (with positive proxy queries its
    pooled score is exactly 4 times the tied one).  The larger block must be
    chosen, and the remaining slots go to the lowest tied blocks: a word of the
    write-out bitmap that comes after the last needed tied block takes none of
    its tied blocks."""
    print("long-row surplus ties", T, topk, big, flush=True)
    G, dp = 1, 32
    g = torch.Generator().manual_seed(37)
    base = torch.randn((128, G, dp), generator=g)
    kp = base.repeat(T // 128, 1, 1).unsqueeze(0).contiguous()
    kp[0, big * 128:(big + 1) * 128] *= 4.0
    kp = kp.to(torch.bfloat16)
    qp = (torch.rand((1, T, G, dp), generator=g) + 0.5).to(torch.bfloat16)
    idx = msa.msa_proxy_select(qp.cuda(), kp.cuda(), topk)
    torch.cuda.synchronize()
    rows = np.array([T - 1, T - 200, (big + 1) * 128 + 5, (big + 1) * 128 - 1, big * 128 - 1, 1100 * 128 + 3])
    dm = Dims(1, T, G, G, 64, dp, topk)
    idx_ref = oracle_mod.select(dm, qp, kp, rows=rows)
    got = idx[0, 0].cpu().numpy()[rows]
    assert all(big in r for r in idx_ref[:3, 0, :].tolist())  # the case this test is about
    np.testing.assert_array_equal(got, idx_ref[:, 0, :])


@pytest.mark.parametrize("T,topk", [(1 << 17, 32), (1 << 18, 40), (1 << 20, 288)])
def test_few_distinct_scores_match_oracle(msa, oracle_mod, T, topk):
    """Pooled scores that take only four values, in random block order: every
    complete block repeats one 128-row proxy-key block scaled by 16, 8, 4 or 1
    (with positive proxy queries a block's pooled score is that power of two
    times the same maximum, exactly).  About k/2 blocks of a full row are
    scaled by 16 and a third by 8, so the k-th score is an 8 shared by far more
    blocks than are needed, with 16s before and after the needed ones in every
    part of the row: rows of up to 1024 blocks (one wave per row) and of 2048
    and 8192 blocks (a workgroup per row) must match the oracle's
    lowest-index-first choice bit for bit."""
    print("few distinct scores", T, topk, flush=True)
    G, dp = 1, 32
    g = torch.Generator().manual_seed(41)
    N = T // 128
    base = torch.randn((128, G, dp), generator=g)
    u = torch.rand((N,), generator=g)
    scale = torch.where(u < 0.5 * topk / N, 16.0, torch.where(u < 0.33, 8.0, torch.where(u < 0.66, 4.0, 1.0)))
    kp = (base.repeat(N, 1, 1) * scale.repeat_interleave(128)[:, None, None]).unsqueeze(0).contiguous()
    kp = kp.to(torch.bfloat16)
    qp = (torch.rand((1, T, G, dp), generator=g) + 0.5).to(torch.bfloat16)
    idx = msa.msa_proxy_select(qp.cuda(), kp.cuda(), topk)
    torch.cuda.synchronize()
    rows = np.array([T - 1, T - 129, T // 2 + 5, T // 3 + 77, 1100 * 128 + 1, 700 * 128 + 127, 40 * 128 + 64,
                     topk * 128 + 3])
    rows = rows[rows < T]
    dm = Dims(1, T, G, G, 64, dp, topk)
    idx_ref = oracle_mod.select(dm, qp, kp, rows=rows)
    got = idx[0, 0].cpu().numpy()[rows]
    np.testing.assert_array_equal(got, idx_ref[:, 0, :])


@pytest.mark.parametrize("T,topk", [(1 << 14, 16), (1 << 17, 32)])
def test_short_rows_equal_scores_take_the_lower_blocks(msa, oracle_mod, T, topk):
    """Rows of at most 1024 blocks go through one wave per row.  With one
    128-row proxy-key block repeated, every complete block has the same pooled
    score: the chosen linear bin is crowded (or the row is all equal), so the
    bit-by-bit search decides, and the lowest block ids must win."""
    print("short-row ties", T, topk, flush=True)
    G, dp = 1, 32
    g = torch.Generator().manual_seed(23)
    base = torch.randn((128, G, dp), generator=g).to(torch.bfloat16)
    kp = base.repeat(T // 128, 1, 1).unsqueeze(0).contiguous()
    qp = torch.randn((1, T, G, dp), generator=g).to(torch.bfloat16)
    idx = msa.msa_proxy_select(qp.cuda(), kp.cuda(), topk)
    torch.cuda.synchronize()
    rows = np.array([T - 1, T - 200, T // 2 + 77, 40 * 128 + 5, 20 * 128 + 127, 3 * 128 + 1])
    dm = Dims(1, T, G, G, 64, dp, topk)
    idx_ref = oracle_mod.select(dm, qp, kp, rows=rows)
    got = idx[0, 0].cpu().numpy()[rows]
    np.testing.assert_array_equal(got, idx_ref[:, 0, :])


@pytest.mark.parametrize("T,topk", [(1 << 17, 4), (1 << 17, 32), (1 << 18, 4), (1 << 18, 40)])
def test_infinite_scores_match_oracle(msa, oracle_mod, T, topk):
    """Proxy keys of +-3e38 against positive proxy queries score +inf (blocks 5
    and 9) or -inf (block 2) in fp32 on both sides.  Rows with an infinite
    smallest or largest score cannot be binned linearly: they take the
    bit-by-bit search (rows of 1024 blocks) or the radix passes (2048 blocks),
    and infinite scores tie to the lower block like any other."""
    print("infinite scores", T, topk, flush=True)
    G, dp = 1, 32
    g = torch.Generator().manual_seed(29)
    kp = torch.randn((1, T, G, dp), generator=g)
    kp[0, 2 * 128:3 * 128] = -3e38
    kp[0, 5 * 128:6 * 128] = 3e38
    kp[0, 9 * 128:10 * 128] = 3e38
    kp = kp.to(torch.bfloat16)
    qp = (torch.rand((1, T, G, dp), generator=g) + 0.5).to(torch.bfloat16)
    idx = msa.msa_proxy_select(qp.cuda(), kp.cuda(), topk)
    torch.cuda.synchronize()
    rows = np.array([4 * 128 + 17, 6 * 128 + 3, 10 * 128 + 50, T // 2 + 77, T - 1])
    dm = Dims(1, T, G, G, 64, dp, topk)
    idx_ref = oracle_mod.select(dm, qp, kp, rows=rows)
    got = idx[0, 0].cpu().numpy()[rows]
    np.testing.assert_array_equal(got, idx_ref[:, 0, :])


@pytest.mark.parametrize("mode", ["decades", "outlier"])
@pytest.mark.parametrize("T,topk", [(1 << 17, 32), (1 << 19, 64)])
def test_wide_score_range_matches_oracle(msa, oracle_mod, T, topk, mode):
    """Rows whose scores span a wide range, against the oracle (rows of 1024
    blocks: one wave per row; 4096 blocks: a workgroup per row).  "decades":
    proxy-key blocks scaled by 10^u, u uniform in [-3, 3]; the k-th key's linear
    bin holds a few to a few dozen keys, ranked directly.  "outlier": block 3
    scaled by 1e5 and the rest by 1, so every other score falls into the lowest
    linear bins and the chosen bin is crowded: the radix or bit-by-bit search
    decides."""
    print("wide score range", T, topk, mode, flush=True)
    G, dp = 1, 32
    g = torch.Generator().manual_seed(31)
    N = T // 128
    if mode == "decades":
        scale = torch.pow(10.0, torch.rand((N,), generator=g) * 6 - 3)
    else:
        scale = torch.ones((N,))
        scale[3] = 1e5
    kp = (torch.randn((1, T, G, dp), generator=g) * scale.repeat_interleave(128)[None, :, None, None]).to(torch.bfloat16)
    qp = torch.randn((1, T, G, dp), generator=g).to(torch.bfloat16)
    idx = msa.msa_proxy_select(qp.cuda(), kp.cuda(), topk)
    torch.cuda.synchronize()
    rows = np.array([T - 1, T - 300, T // 2 + 11, T // 4 + 129, 50 * 128 + 7, 5 * 128 + 64])
    dm = Dims(1, T, G, G, 64, dp, topk)
    idx_ref = oracle_mod.select(dm, qp, kp, rows=rows)
    got = idx[0, 0].cpu().numpy()[rows]
    np.testing.assert_array_equal(got, idx_ref[:, 0, :])


@pytest.mark.parametrize("T,G,topk,n_rows", [(1 << 18, 2, 64, 1536), (1 << 20, 1, 288, 384)])
def test_long_rows_many_rows_match_oracle(msa, oracle_mod, T, G, topk, n_rows):
    """Rows longer than 1024 blocks are selected by one workgroup per row.
    Proxy inputs follow the block-mean recipe; a seeded sample of rows over the
    whole sequence (short rows, rows around 1024 blocks, the last rows) must
    match the oracle bit-exactly up to near-ties."""
    print("long rows", T, G, topk, flush=True)
    cfg = synth.Config("long%d" % T, 1, T, G, G, 64, 32, topk)
    qp = synth.make_tensor("qp", cfg, seed_offset=31)
    kp = synth.make_tensor("kp", cfg, seed_offset=31)
    idx = msa.msa_proxy_select(qp.cuda(), kp.cuda(), topk)
    torch.cuda.synchronize()
    rng = np.random.default_rng(99)
    rows = np.unique(np.concatenate([rng.choice(T, size=n_rows - 6, replace=False),
                                     [0, 1023 * 128, 1024 * 128 + 5, T // 2, T - 2, T - 1]]))
    dm = Dims(1, T, G, G, 64, 32, topk)
    idx_ref, pooled = oracle_mod.select(dm, qp, kp, rows=rows, return_pooled=True)
    got = idx[0].cpu().numpy()[:, rows, :].transpose(1, 0, 2)
    info = parity.check_indices(got, idx_ref, pooled, topk)
    print("indices", info, flush=True)
