"""msa_decode_fwd_static: the decode attention without a workspace (partials in
the library's static device scratch) must give exactly what msa_decode_fwd
gives with a caller workspace (same kernels), on two calls in a row, the
second smaller than the first, and must refuse a problem larger than the
scratch before launching anything."""
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def msa():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import block_sparse_attention_qk_amd as m
    m.load()
    return m


def _case(msa, B, T, H, G, d, topk, lens, seed):
    import bench
    cfg = synth.custom(1, T, H, G, d, 64, topk)
    x = bench.gpu_decode_inputs(cfg, B, seed=seed)
    lens_d = torch.tensor(lens, dtype=torch.int32, device="cuda")
    idx = msa.msa_decode_select(x["qp"], x["kp"], lens_d, topk)
    return x, lens_d, idx


def test_static_scratch_matches_workspace_call(msa):
    cases = [  # B, T, H, G, d, topk, lens: the second call is smaller than the first
        (16, 4096, 32, 4, 128, 32, [4096, 1, 2500, 129] * 4),
        (3, 2048, 16, 2, 64, 4, [2048, 700, 5]),
    ]
    for i, (B, T, H, G, d, topk, lens) in enumerate(cases):
        print("static scratch call", i, (B, T, H, G, d, topk), flush=True)
        x, lens_d, idx = _case(msa, B, T, H, G, d, topk, lens, seed=70 + i)
        need = msa.msa_workspace_bytes(B, T, H, G, d, 64, topk, msa.OP_DECODE_FWD)
        assert need <= msa.STATIC_SCRATCH_BYTES, need
        o_ref, lse_ref = msa.msa_decode_fwd(x["q"], x["k"], x["v"], lens_d, idx)
        o = torch.full_like(o_ref, float("nan"))
        lse = torch.full_like(lse_ref, float("nan"))
        msa.msa_decode_fwd_static(x["q"], x["k"], x["v"], lens_d, idx, out=(o, lse))
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref), i
        assert torch.equal(lse, lse_ref), i
        print("static scratch call", i, "equal to the workspace call", flush=True)


def test_static_scratch_refuses_oversized_problem(msa):
    B, T, H, G, d, topk = 64, 256, 32, 4, 128, 32  # 32 MiB of partials
    need = msa.msa_workspace_bytes(B, T, H, G, d, 64, topk, msa.OP_DECODE_FWD)
    assert need > msa.STATIC_SCRATCH_BYTES
    q = torch.zeros((B, H, d), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((B, T, G, d), dtype=torch.bfloat16, device="cuda")
    lens = torch.full((B,), T, dtype=torch.int32, device="cuda")
    idx = torch.zeros((B, G, topk), dtype=torch.int32, device="cuda")
    o = torch.full((B, H, d), 7.0, dtype=torch.bfloat16, device="cuda")
    lse = torch.full((B, H), 7.0, dtype=torch.float32, device="cuda")
    with pytest.raises(msa.MsaError, match="static scratch"):
        msa.msa_decode_fwd_static(q, k, k, lens, idx, out=(o, lse))
    torch.cuda.synchronize()
    assert (o == 7.0).all() and (lse == 7.0).all()  # nothing ran
