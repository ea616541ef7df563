"""GPU parity of the MHA -> GQA mean-pool conversion (gqa_mean_pool_heads) against the
fp64 oracle, plus an end-to-end check through the attention kernels.

Bound: the sums run in fp32 and the output is rounded once, so |gpu - exact| <=
2^-8 |exact| (bf16 output, 8 significant bits) or 2^-22 |exact| (fp32, a few roundings)
plus a tiny absolute term for results near zero.
"""
import math
import sys

import numpy as np
import pytest
import torch

import grouped_query_attention_02_amd as gqa

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu(built_lib):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gqa.load()


def _check(got, ref, dtype):
    g = got.detach().double().cpu().numpy()
    rel = 2.0 ** -8 if dtype == torch.bfloat16 else 2.0 ** -22
    bad = np.abs(g - ref) > rel * np.abs(ref) + 1e-6
    assert not bad.any(), (np.abs(g - ref).max(), int(bad.sum()))


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("H,G,shape", [(64, 8, (128, 72)), (12, 3, (64,)), (32, 1, (16, 24)),
                                       (8, 8, (8, 40)), (96, 32, (136,))])
def test_mean_pool_matches_oracle(oracle_mod, dtype, H, G, shape):
    _say(f"case mean_pool {dtype} H={H} G={G} shape={shape}")
    g = torch.Generator().manual_seed(H * 7 + G)
    w = torch.randn((H,) + shape, generator=g).to(dtype)
    out = gqa.mean_pool_heads(w.cuda(), G)
    torch.cuda.synchronize()
    ref = oracle_mod.mean_pool_heads(w, G)
    _check(out, ref, dtype)


def test_mean_pool_full_size_llama70b_k_projection(oracle_mod):
    """A Llama-2-70B-shaped K projection (64 heads of 128 rows x 8192 columns, bf16) pooled to
    8 groups, checked element by element."""
    H, G, dh, dm = 64, 8, 128, 8192
    g = torch.Generator().manual_seed(70)
    w = (torch.randn((H, dh, dm), generator=g) * 0.02).to(torch.bfloat16)
    _say("case mean_pool llama70b k_proj (full size)")
    out = gqa.mean_pool_heads(w.cuda(), G)
    torch.cuda.synchronize()
    _check(out, oracle_mod.mean_pool_heads(w, G), torch.bfloat16)


def test_converted_weights_reproduce_mha_when_group_heads_agree():
    """If the heads of every group share one K/V projection, pooling returns that projection
    exactly, and GQA attention with the pooled K/V heads equals MHA attention with the
    original heads (the GQA = MHA-with-repeated-K/V identity, end to end on the GPU)."""
    B, S, H, G, d, dm = 2, 96, 8, 2, 64, 128
    gen = torch.Generator().manual_seed(5)
    base_k = torch.randn((G, d, dm), generator=gen) * 0.1
    base_v = torch.randn((G, d, dm), generator=gen) * 0.1
    wk = base_k.repeat_interleave(H // G, dim=0).to(torch.bfloat16).cuda()   # [H, d, dm]
    wv = base_v.repeat_interleave(H // G, dim=0).to(torch.bfloat16).cuda()
    pk, pv = gqa.mean_pool_heads(wk, G), gqa.mean_pool_heads(wv, G)
    assert torch.equal(pk, base_k.to(torch.bfloat16).cuda())
    assert torch.equal(pv, base_v.to(torch.bfloat16).cuda())
    x = (torch.randn((B, S, dm), generator=gen)).to(torch.bfloat16).cuda()
    q = (torch.randn((B, S, H, d), generator=gen)).to(torch.bfloat16).cuda()

    def project(wts):  # [n, d, dm] -> [B, S, n, d], fp32 math (contiguous operands) then bf16
        n = wts.shape[0]
        rhs = wts.float().reshape(n * d, dm).t().contiguous()
        return torch.matmul(x.float(), rhs).view(B, S, n, d).to(torch.bfloat16).contiguous()

    o_mha = gqa.prefill(q, project(wk), project(wv), causal=True)
    o_gqa = gqa.prefill(q, project(pk), project(pv), causal=True)
    torch.cuda.synchronize()
    assert (o_mha.float() - o_gqa.float()).abs().max().item() <= 2e-2
