"""gqa_decode_noalloc (the decode entry point that allocates nothing and keeps its split partials
in the library's static device scratch) against gqa_decode_ex with a caller workspace, through
the C ABI: bitwise-equal outputs and LSE, and both within the decode tolerances of the fp64
oracle (O 2e-2, LSE 1e-3), on two calls in a row, the second with a smaller input (the scratch
then holds the first call's partials). A call that needs more than the scratch is rejected
before any launch."""
import sys

import numpy as np
import pytest
import torch

import grouped_query_attention_02_amd as gqa
from grouped_query_attention_02_amd import _lib

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu(built_lib):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gqa.load()


def _rand(shape, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=g) * scale).to(torch.bfloat16)


def _case(oracle_mod, B, Hq, Hkv, d, max_len, lens, splits, seed):
    dev = "cuda"
    q = _rand((B, Hq, d), seed)
    kc = _rand((B, Hkv, max_len, d), seed + 1)
    vc = _rand((B, Hkv, max_len, d), seed + 2)
    for b, L in enumerate(lens):
        kc[b, :, L:] = float("nan")   # rows past a length are never read
        vc[b, :, L:] = float("nan")
    need = gqa.decode_workspace_bytes(B, Hq, Hkv, d, max_len, splits)
    assert 0 < need <= gqa.DECODE_SCRATCH_BYTES
    qd, kd, vd = q.to(dev), kc.to(dev), vc.to(dev)
    ld = torch.tensor(lens, dtype=torch.int32, device=dev)
    out = torch.empty_like(qd)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    gqa.decode_noalloc(qd, kd, vd, ld, out, lse_out=lse, num_splits=splits)
    ref_out, ref_lse = gqa.decode(qd, kd, vd, ld, num_splits=splits, return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse)
    o64, l64 = oracle_mod.decode(q, kc, vc, scale=1.0 / d ** 0.5, lens=lens)
    e = float(np.abs(out.double().cpu().numpy() - o64).max())
    le = float(np.abs(lse.double().cpu().numpy() - l64).max())
    _say(f"  noalloc B={B} Hq={Hq} Hkv={Hkv} d={d} splits={splits}: bitwise equal to the "
         f"workspace call, max_abs_err={e:.3e} lse_err={le:.3e}")
    assert e <= 2e-2 and le <= 1e-3
    return out


def test_noalloc_matches_workspace_call_twice(oracle_mod):
    _say("case noalloc: large then smaller input")
    # 1: ragged multi-query shape with several splits per sequence (partials in the scratch)
    _case(oracle_mod, B=6, Hq=32, Hkv=1, d=128, max_len=4096,
          lens=[4096, 1, 2500, 777, 3333, 64], splits=0, seed=501)
    # 2: smaller, other head size; the scratch still holds call 1's partials
    _case(oracle_mod, B=3, Hq=8, Hkv=2, d=64, max_len=500, lens=[500, 33, 250], splits=3,
          seed=601)


def test_noalloc_rejects_more_than_scratch():
    lib = _lib.load()
    buf = torch.zeros(1 << 16, dtype=torch.uint8, device="cuda")
    p = buf.data_ptr()
    B, Hq, Hkv, d, max_len = 4096, 64, 8, 128, 8192
    need = gqa.decode_workspace_bytes(B, Hq, Hkv, d, max_len, 0)
    assert need > gqa.DECODE_SCRATCH_BYTES
    # every pointer is valid but far too small: the size check must stop the call first
    st = lib.gqa_decode_noalloc(_lib.GQA_DTYPE_BF16, p, p, p, None, None, 0, 0, 0, p, None, B,
                                Hq, Hkv, d, max_len, 0.1, 0, None, 0, None)
    assert st == _lib.GQA_ERR_WORKSPACE
    torch.cuda.synchronize()
