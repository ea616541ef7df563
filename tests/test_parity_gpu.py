"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle, element by element.

Tolerances (max |O_gpu - O_oracle| over every checked element):
  fp32 inputs: 1e-5;  bf16 inputs with fp32 accumulation and bf16 output: 2e-2.
LSE (natural log): 1e-4 for fp32 paths, 1e-3 for bf16. A bf16 call that returns the LSE sums
the fp32 weights (the products are exact products of the stored inputs accumulated in fp32),
so the LSE carries fp32 rounding only, not the bf16 rounding of the weights that feed the PV
product.
"""
import math
import sys

import numpy as np
import pytest
import torch

import grouped_query_attention_02_amd as gqa
import workloads as W

pytestmark = pytest.mark.gpu

TOL = {torch.float32: 1e-5, torch.bfloat16: 2e-2}
LSE_TOL = {torch.float32: 1e-4, torch.bfloat16: 1e-3}   # prefill
BF16_DECODE_LSE_TOL = 1e-3


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu(built_lib):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gqa.load()


def _rand(shape, seed, dtype, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=g) * scale).to(dtype)


def _max_err(gpu, ref):
    a = gpu.detach().double().cpu().numpy()
    diff = np.abs(a - ref)
    assert not np.isnan(a).any(), "NaN in GPU output"
    return float(diff.max()) if diff.size else 0.0


def _lse_err(gpu_lse, ref_lse):
    a = gpu_lse.detach().double().cpu().numpy()
    fin = np.isfinite(ref_lse)
    assert np.array_equal(np.isfinite(a), fin), "LSE finiteness differs"
    assert np.all(a[~fin] == -np.inf)
    return float(np.abs(a[fin] - ref_lse[fin]).max()) if fin.any() else 0.0


def _run_prefill_full(oracle_mod, q, k, v, seqlens, causal, scale, dtype):
    """Max O error over the plain call and the LSE-returning call (different kernel
    instantiations), and the LSE error."""
    dev = "cuda"
    lens_d = None if seqlens is None else torch.as_tensor(seqlens, dtype=torch.int32).to(dev)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    o_plain = gqa.prefill(qd, kd, vd, causal=causal, softmax_scale=scale, seqlens=lens_d)
    o, lse = gqa.prefill(qd, kd, vd, causal=causal, softmax_scale=scale, seqlens=lens_d,
                         return_lse=True)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle_mod.prefill(q, k, v, scale=scale, causal=causal, seqlens=seqlens)
    return max(_max_err(o, ref_o), _max_err(o_plain, ref_o)), _lse_err(lse, ref_l)


def test_tiny_f32_prefill_full(oracle_mod):
    w = W.WORKLOADS["tiny_f32_prefill"]
    _say(f"case {w.name}")
    x = W.make_prefill(w)
    e, le = _run_prefill_full(oracle_mod, x["q"], x["k"], x["v"], None, w.causal,
                              w.softmax_scale, torch.float32)
    _say(f"  max_abs_err={e:.3e} lse_err={le:.3e}")
    assert e <= 1e-5 and le <= 1e-4


SWEEP = []
for dtype in (torch.bfloat16, torch.float32):
    for d in (32, 64, 128):
        for (Hq, Hkv) in ((4, 4), (4, 2), (8, 2), (8, 1), (32, 1), (6, 2)):
            for causal in (False, True):
                SWEEP.append((dtype, d, Hq, Hkv, causal))


@pytest.mark.parametrize("dtype,d,Hq,Hkv,causal", SWEEP)
def test_prefill_sweep(oracle_mod, dtype, d, Hq, Hkv, causal):
    """Small shapes spanning several tiles and ragged tails, with and without key lengths."""
    B, S = 3, 133
    seed = 1000 + d + 7 * Hq + 3 * Hkv + int(causal)
    _say(f"case prefill {dtype} d={d} Hq={Hq} Hkv={Hkv} causal={causal}")
    q = _rand((B, S, Hq, d), seed, dtype)
    k = _rand((B, S, Hkv, d), seed + 1, dtype)
    v = _rand((B, S, Hkv, d), seed + 2, dtype)
    scale = 1.0 / math.sqrt(d)
    for lens in (None, [133, 1, 70]):
        e, le = _run_prefill_full(oracle_mod, q, k, v, lens, causal, scale, dtype)
        _say(f"  lens={lens} max_abs_err={e:.3e} lse_err={le:.3e}")
        assert e <= TOL[dtype] and le <= LSE_TOL[dtype]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_prefill_edge_lengths_and_scales(oracle_mod, dtype):
    """Zero-length sequences (O = 0, LSE = -inf), lengths past S (clamped), scale 0
    (uniform weights) and a negative scale."""
    B, S, Hq, Hkv, d = 4, 70, 8, 2, 64
    q = _rand((B, S, Hq, d), 7, dtype)
    k = _rand((B, S, Hkv, d), 8, dtype)
    v = _rand((B, S, Hkv, d), 9, dtype)
    for causal in (False, True):
        for lens, scale in (([0, 70, 5000, 33], 0.125), ([64, 65, 1, 0], 0.0),
                            ([70, 70, 2, 69], -0.2)):
            _say(f"case edge {dtype} causal={causal} lens={lens} scale={scale}")
            e, le = _run_prefill_full(oracle_mod, q, k, v, lens, causal, scale, dtype)
            assert e <= TOL[dtype] and le <= LSE_TOL[dtype], (e, le)


@pytest.mark.parametrize("B,S,Hq,Hkv,d", [(40, 70, 4, 2, 64), (19, 130, 6, 3, 128),
                                           (100, 40, 4, 2, 64), (90, 50, 8, 2, 128),
                                           (300, 20, 2, 1, 32), (256, 40, 4, 2, 128),
                                           (257, 40, 4, 1, 128), (257, 45, 4, 2, 64)])
def test_prefill_many_ragged_sequences(oracle_mod, B, S, Hq, Hkv, d):
    """Many sequences with repeated, zero and over-long lengths: the bf16 kernel orders its
    work by sequence length (up to 256 sequences; 257 take the unordered path) and must
    still write every output once."""
    rng = np.random.default_rng(B + S)
    lens = rng.integers(0, S + 1, size=B)
    lens[: B // 4] = lens[B // 4]          # ties
    lens[-1] = 0
    lens[-2] = S + 9                       # clamped to S
    lens = [int(x) for x in lens]
    q = _rand((B, S, Hq, d), 31, torch.bfloat16)
    k = _rand((B, S, Hkv, d), 32, torch.bfloat16)
    v = _rand((B, S, Hkv, d), 33, torch.bfloat16)
    for causal in (False, True):
        _say(f"case ragged B={B} S={S} Hq={Hq} Hkv={Hkv} d={d} causal={causal}")
        e, le = _run_prefill_full(oracle_mod, q, k, v, lens, causal, 1 / math.sqrt(d),
                                  torch.bfloat16)
        _say(f"  max_abs_err={e:.3e} lse_err={le:.3e}")
        assert e <= 2e-2 and le <= LSE_TOL[torch.bfloat16]


@pytest.mark.parametrize("d", [64, 128])
def test_prefill_very_many_short_sequences(oracle_mod, d):
    """1500 sequences of at most 24 keys: past the in-kernel length ranking (256 sequences),
    thousands of work items for the persistent d = 128 workgroups."""
    B, S, Hq, Hkv = 1500, 24, 4, 2
    rng = np.random.default_rng(1500 + d)
    lens = [int(x) for x in rng.integers(0, S + 1, size=B)]
    q = _rand((B, S, Hq, d), 4100 + d, torch.bfloat16)
    k = _rand((B, S, Hkv, d), 4101 + d, torch.bfloat16)
    v = _rand((B, S, Hkv, d), 4102 + d, torch.bfloat16)
    for causal in (False, True):
        _say(f"case prefill B={B} S={S} d={d} causal={causal}")
        e, le = _run_prefill_full(oracle_mod, q, k, v, lens, causal, 1 / math.sqrt(d),
                                  torch.bfloat16)
        _say(f"  max_abs_err={e:.3e} lse_err={le:.3e}")
        assert e <= 2e-2 and le <= LSE_TOL[torch.bfloat16]


@pytest.mark.parametrize("d,causal", [(64, False), (128, True)])
def test_prefill_one_long_sequence_sampled(oracle_mod, d, causal):
    """One 20000-key sequence (not a multiple of the tile) with a key length below it,
    checked on sampled rows: long row loops and large offsets."""
    B, S, Hq, Hkv = 1, 20000, 4, 1
    lens = [19001]
    _say(f"case prefill long S={S} d={d} causal={causal}")
    q = _rand((B, S, Hq, d), 4200 + d, torch.bfloat16)
    k = _rand((B, S, Hkv, d), 4201 + d, torch.bfloat16)
    v = _rand((B, S, Hkv, d), 4202 + d, torch.bfloat16)
    o, lse = gqa.prefill(q.cuda(), k.cuda(), v.cuda(), causal=causal,
                         seqlens=torch.tensor(lens, dtype=torch.int32).cuda(), return_lse=True)
    torch.cuda.synchronize()
    rows = _sample_rows(B, S, Hq, torch.tensor(lens), 120, 11)
    ref_o, ref_l = oracle_mod.prefill_rows(q, k, v, rows, scale=1 / math.sqrt(d), causal=causal,
                                           seqlens=lens)
    oc, lc = o.cpu(), lse.cpu()
    got = torch.stack([oc[b, i, h] for b, h, i in rows])
    got_l = torch.tensor([float(lc[b, h, i]) for b, h, i in rows], dtype=torch.float64)
    e, le = _max_err(got, ref_o), _lse_err(got_l, ref_l)
    _say(f"  rows={len(rows)} max_abs_err={e:.3e} lse_err={le:.3e}")
    assert e <= 2e-2 and le <= LSE_TOL[torch.bfloat16]


def test_prefill_poisoned_padding_does_not_leak(oracle_mod):
    """K/V rows at or past a sequence's length hold NaN/Inf: the output must not see them."""
    B, S, Hq, Hkv, d = 3, 150, 8, 2, 128
    q = _rand((B, S, Hq, d), 21, torch.bfloat16)
    k = _rand((B, S, Hkv, d), 22, torch.bfloat16)
    v = _rand((B, S, Hkv, d), 23, torch.bfloat16)
    lens = [100, 150, 3]
    kp, vp = k.clone(), v.clone()
    for b, L in enumerate(lens):
        kp[b, L:] = float("nan")
        vp[b, L:] = float("inf")
    for causal in (False, True):
        e, le = _run_prefill_full(oracle_mod, q, kp, vp, lens, causal, 1 / math.sqrt(d),
                                  torch.bfloat16)
        assert e <= 2e-2 and le <= LSE_TOL[torch.bfloat16]


def _sample_rows(B, S, Hq, seqlens, n_random, seed):
    rng = np.random.default_rng(seed)
    rows = set()
    for b in range(B):
        L = S if seqlens is None else int(seqlens[b])
        for i in {0, S - 1, max(L - 1, 0), min(L, S - 1), S // 2}:
            for h in {0, Hq - 1, int(rng.integers(Hq))}:
                rows.add((b, h, i))
    while len(rows) < n_random + 4 * B:
        rows.add((int(rng.integers(B)), int(rng.integers(Hq)), int(rng.integers(S))))
    return np.array(sorted(rows), dtype=np.int64)


@pytest.mark.parametrize("name", ["bert_base_prefill", "llama_causal_prefill"])
def test_prefill_full_size_sampled(oracle_mod, name):
    """Full workload size, same launch as the benchmark; oracle on sampled rows."""
    w = W.WORKLOADS[name]
    _say(f"case {name} (full size)")
    x = W.make_prefill(w)
    dev = "cuda"
    lens_d = None if x["seqlens"] is None else x["seqlens"].to(dev)
    o, lse = gqa.prefill(x["q"].to(dev), x["k"].to(dev), x["v"].to(dev), causal=w.causal,
                         softmax_scale=w.softmax_scale, seqlens=lens_d, return_lse=True)
    torch.cuda.synchronize()
    rows = _sample_rows(w.B, w.S, w.Hq, x["seqlens"], 400, 5)
    ref_o, ref_l = oracle_mod.prefill_rows(x["q"], x["k"], x["v"], rows, scale=w.softmax_scale,
                                           causal=w.causal, seqlens=x["seqlens"])
    oc = o.cpu()
    lc = lse.cpu()
    got = torch.stack([oc[b, i, h] for b, h, i in rows])
    got_l = torch.tensor([float(lc[b, h, i]) for b, h, i in rows], dtype=torch.float64)
    e = _max_err(got, ref_o)
    le = _lse_err(got_l, ref_l)
    _say(f"  rows={len(rows)} max_abs_err={e:.3e} lse_err={le:.3e}")
    assert e <= 2e-2 and le <= LSE_TOL[torch.bfloat16]
    assert torch.isfinite(o.float()).all()


def test_prefill_gqa_equals_replicated_mha():
    """GQA output = MHA output with each K/V head repeated over its group of query heads."""
    B, S, Hq, Hkv, d = 2, 200, 12, 3, 64
    q = _rand((B, S, Hq, d), 31, torch.bfloat16).cuda()
    k = _rand((B, S, Hkv, d), 32, torch.bfloat16).cuda()
    v = _rand((B, S, Hkv, d), 33, torch.bfloat16).cuda()
    lens = torch.tensor([150, 200], dtype=torch.int32).cuda()
    for causal in (False, True):
        a = gqa.prefill(q, k, v, causal=causal, seqlens=lens)
        b = gqa.prefill(q, k.repeat_interleave(4, dim=2).contiguous(),
                        v.repeat_interleave(4, dim=2).contiguous(), causal=causal, seqlens=lens)
        assert (a.float() - b.float()).abs().max().item() <= 2e-2


@pytest.mark.parametrize("d,causal", [(128, True), (64, False)])
def test_prefill_deterministic(d, causal):
    """Bitwise-equal outputs over 10 runs: the persistent d = 128 kernel and the d = 64 kernel
    with in-kernel length ranking."""
    B, S, Hq, Hkv = 4, 300, 32, 8
    q = _rand((B, S, Hq, d), 41, torch.bfloat16).cuda()
    k = _rand((B, S, Hkv, d), 42, torch.bfloat16).cuda()
    v = _rand((B, S, Hkv, d), 43, torch.bfloat16).cuda()
    lens = torch.tensor([300, 17, 250, 129], dtype=torch.int32).cuda()
    first = gqa.prefill(q, k, v, causal=causal, seqlens=lens)
    for _ in range(10):
        assert torch.equal(gqa.prefill(q, k, v, causal=causal, seqlens=lens), first)


def test_prefill_v_ones_gives_ones():
    B, S, Hq, Hkv, d = 2, 97, 8, 2, 128
    q = _rand((B, S, Hq, d), 51, torch.bfloat16).cuda()
    k = _rand((B, S, Hkv, d), 52, torch.bfloat16).cuda()
    v = torch.ones((B, S, Hkv, d), dtype=torch.bfloat16, device="cuda")
    for causal in (False, True):
        o = gqa.prefill(q, k, v, causal=causal, seqlens=torch.tensor([97, 40], dtype=torch.int32))
        assert (o.float() - 1).abs().max().item() <= 2e-2


# ---------------------------------------------------------------- decode

def _run_decode_full(oracle_mod, q, kc, vc, lens, scale, num_splits=0):
    dev = "cuda"
    lens_d = None if lens is None else torch.as_tensor(lens, dtype=torch.int32).to(dev)
    o, lse = gqa.decode(q.to(dev), kc.to(dev), vc.to(dev), lens_d, softmax_scale=scale,
                        num_splits=num_splits, return_lse=True)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle_mod.decode(q, kc, vc, scale=scale, lens=lens)
    return _max_err(o, ref_o), _lse_err(lse, ref_l), o


DEC_SWEEP = []
for d in (64, 128):
    for (Hq, Hkv) in ((8, 8), (8, 1), (32, 1), (64, 8), (64, 1), (48, 1), (12, 4)):
        DEC_SWEEP.append((d, Hq, Hkv))


@pytest.mark.parametrize("d,Hq,Hkv", DEC_SWEEP)
def test_decode_sweep(oracle_mod, d, Hq, Hkv):
    B, max_len = 6, 333
    seed = 2000 + d + Hq + Hkv
    _say(f"case decode d={d} Hq={Hq} Hkv={Hkv}")
    q = _rand((B, Hq, d), seed, torch.bfloat16)
    kc = _rand((B, Hkv, max_len, d), seed + 1, torch.bfloat16)
    vc = _rand((B, Hkv, max_len, d), seed + 2, torch.bfloat16)
    for lens in (None, [333, 1, 31, 32, 33, 0]):
        for splits in (0, 1, 3):
            e, le, _ = _run_decode_full(oracle_mod, q, kc, vc, lens, 1 / math.sqrt(d), splits)
            _say(f"  lens={lens} splits={splits} max_abs_err={e:.3e} lse_err={le:.3e}")
            assert e <= 2e-2 and le <= BF16_DECODE_LSE_TOL


@pytest.mark.parametrize("d,B", [(64, 1300), (128, 1300), (128, 512), (128, 513)])
def test_decode_many_sequences(oracle_mod, d, B):
    """Up to 1300 sequences, lengths 0..200 with runs of empty caches: every share still
    finds its sequence. The split kernel finds its share in one scan of up to 512 lengths
    (one per thread) and in two passes of 512 at a time beyond that; the combine kernel
    scans 64 at a time."""
    Hq, Hkv, max_len = 8, 2, 200
    _say(f"case decode many sequences B={B} d={d}")
    rng = np.random.default_rng(77 + d)
    lens = rng.integers(0, max_len + 1, size=B)
    lens[100:140] = 0
    lens[-1] = max_len
    lens = [int(x) for x in lens]
    q = _rand((B, Hq, d), 4000 + d, torch.bfloat16)
    kc = _rand((B, Hkv, max_len, d), 4001 + d, torch.bfloat16)
    vc = _rand((B, Hkv, max_len, d), 4002 + d, torch.bfloat16)
    for splits in (0, 1, 3):
        e, le, _ = _run_decode_full(oracle_mod, q, kc, vc, lens, 0.1, splits)
        _say(f"  splits={splits} max_abs_err={e:.3e} lse_err={le:.3e}")
        assert e <= 2e-2 and le <= BF16_DECODE_LSE_TOL


def test_decode_long_context(oracle_mod):
    """128k-key caches, one full and one ragged; with one split per unit a workgroup streams a
    whole 131072-key unit (64 MiB of K and V) and no merge runs."""
    B, Hq, Hkv, d, max_len = 2, 16, 2, 128, 131072
    lens = [131072, 98765]
    _say(f"case decode long context max_len={max_len} lens={lens}")
    q = _rand((B, Hq, d), 4101, torch.bfloat16)
    kc = _rand((B, Hkv, max_len, d), 4102, torch.bfloat16)
    vc = _rand((B, Hkv, max_len, d), 4103, torch.bfloat16)
    # scale 0.5: scores of std ~5.7, so a few of the 131072 keys dominate and O has values
    # of order one (with 1/sqrt(d) the weights are spread thin and O is small)
    for scale, splits in ((1 / math.sqrt(d), 0), (0.5, 0), (0.5, 1), (0.5, 5)):
        e, le, _ = _run_decode_full(oracle_mod, q, kc, vc, lens, scale, splits)
        _say(f"  scale={scale:.3f} splits={splits} max_abs_err={e:.3e} lse_err={le:.3e}")
        assert e <= 2e-2 and le <= BF16_DECODE_LSE_TOL


def test_decode_poisoned_cache_and_split_invariance(oracle_mod):
    """NaN/Inf past each length must not leak; every split count gives the oracle's answer."""
    B, Hq, Hkv, d, max_len = 5, 32, 1, 128, 2000
    q = _rand((B, Hq, d), 61, torch.bfloat16)
    kc = _rand((B, Hkv, max_len, d), 62, torch.bfloat16)
    vc = _rand((B, Hkv, max_len, d), 63, torch.bfloat16)
    lens = [2000, 1, 777, 64, 1500]
    for b, L in enumerate(lens):
        kc[b, :, L:] = float("nan")
        vc[b, :, L:] = float("inf")
    outs = []
    for splits in (0, 1, 2, 7, 40):
        _say(f"case decode poison splits={splits}")
        e, le, o = _run_decode_full(oracle_mod, q, kc, vc, lens, 0.09, splits)
        assert e <= 2e-2 and le <= BF16_DECODE_LSE_TOL
        outs.append(o.float())
    for o in outs[1:]:
        assert (o - outs[0]).abs().max().item() <= 2e-2


def test_decode_scales(oracle_mod):
    B, Hq, Hkv, d, max_len = 3, 16, 2, 64, 100
    q = _rand((B, Hq, d), 71, torch.bfloat16)
    kc = _rand((B, Hkv, max_len, d), 72, torch.bfloat16)
    vc = _rand((B, Hkv, max_len, d), 73, torch.bfloat16)
    for scale in (0.0, -0.3, 0.7):
        e, le, _ = _run_decode_full(oracle_mod, q, kc, vc, [100, 50, 3], scale)
        assert e <= 2e-2 and le <= BF16_DECODE_LSE_TOL


def test_decode_equals_last_causal_prefill_row():
    B, S, Hq, Hkv, d = 3, 300, 32, 4, 128
    q = _rand((B, S, Hq, d), 81, torch.bfloat16).cuda()
    k = _rand((B, S, Hkv, d), 82, torch.bfloat16).cuda()
    v = _rand((B, S, Hkv, d), 83, torch.bfloat16).cuda()
    lens = [300, 17, 129]
    o_pre = gqa.prefill(q, k, v, causal=True)
    q_dec = torch.stack([q[b, lens[b] - 1] for b in range(B)]).contiguous()
    kc = k.permute(0, 2, 1, 3).contiguous()
    vc = v.permute(0, 2, 1, 3).contiguous()
    o_dec = gqa.decode(q_dec, kc, vc, torch.tensor(lens, dtype=torch.int32))
    for b in range(B):
        assert (o_dec[b].float() - o_pre[b, lens[b] - 1].float()).abs().max().item() <= 2e-2


def test_decode_deterministic():
    B, Hq, Hkv, d, max_len = 8, 32, 1, 128, 5000
    q = _rand((B, Hq, d), 91, torch.bfloat16).cuda()
    kc = _rand((B, Hkv, max_len, d), 92, torch.bfloat16).cuda()
    vc = _rand((B, Hkv, max_len, d), 93, torch.bfloat16).cuda()
    lens = torch.tensor([5000, 3, 4000, 100, 2500, 1, 4999, 64], dtype=torch.int32).cuda()
    first = gqa.decode(q, kc, vc, lens)
    for _ in range(10):
        assert torch.equal(gqa.decode(q, kc, vc, lens), first)


def test_decode_reused_garbage_workspace(oracle_mod):
    """The workspace's contents on entry do not matter: one holding garbage, and one reused
    across calls with other lengths and split counts, gives the same bits as a fresh one."""
    B, Hq, Hkv, d, max_len = 7, 32, 1, 128, 3000
    q = _rand((B, Hq, d), 95, torch.bfloat16).cuda()
    kc = _rand((B, Hkv, max_len, d), 96, torch.bfloat16).cuda()
    vc = _rand((B, Hkv, max_len, d), 97, torch.bfloat16).cuda()
    need = max(gqa.decode_workspace_bytes(B, Hq, Hkv, d, max_len, s) for s in (0, 3, 9))
    g = torch.Generator().manual_seed(98)
    ws = torch.randint(0, 256, (need,), generator=g, dtype=torch.uint8).cuda()
    cases = [([3000, 1, 0, 1700, 33, 2999, 64], 0), ([5, 3000, 2500, 0, 1, 32, 1000], 3),
             ([3000, 1, 0, 1700, 33, 2999, 64], 9), ([100, 100, 100, 100, 100, 100, 100], 0)]
    for rep in range(2):
        for lens, splits in cases:
            _say(f"case decode reused workspace rep={rep} lens={lens} splits={splits}")
            ld = torch.tensor(lens, dtype=torch.int32).cuda()
            o, lse = gqa.decode(q, kc, vc, ld, softmax_scale=0.09, num_splits=splits,
                                return_lse=True, workspace=ws)
            fo, flse = gqa.decode(q, kc, vc, ld, softmax_scale=0.09, num_splits=splits,
                                  return_lse=True)
            torch.cuda.synchronize()
            assert torch.equal(o, fo) and torch.equal(lse, flse)
            ref_o, ref_l = oracle_mod.decode(q.cpu(), kc.cpu(), vc.cpu(), scale=0.09, lens=lens)
            assert _max_err(o, ref_o) <= 2e-2 and _lse_err(lse, ref_l) <= BF16_DECODE_LSE_TOL
        if rep == 0:
            ws.fill_(255)


_DEC_CACHE = {}


def _decode_inputs(name, poison=False):
    key = (name, poison)
    if key not in _DEC_CACHE:
        _DEC_CACHE.clear()
        _DEC_CACHE[key] = W.make_decode(W.WORKLOADS[name], poison=poison)
    return _DEC_CACHE[key]


@pytest.mark.parametrize("name,use_lens,poison", [
    ("gqa_decode_8k", True, False),
    ("gqa_decode_8k", False, False),
    ("mqa_ragged_decode", True, False),
    ("mqa_ragged_decode", True, True),
])
def test_decode_full_size_sampled(oracle_mod, name, use_lens, poison):
    """Full workload size, same launch as the benchmark; oracle on sampled (b, h) pairs."""
    w = W.WORKLOADS[name]
    _say(f"case {name} lens={use_lens} poison={poison} (full size)")
    x = _decode_inputs(name, poison)
    dev = "cuda"
    lens = x["lens"] if use_lens else None
    o, lse = gqa.decode(x["q"].to(dev), x["k_cache"].to(dev), x["v_cache"].to(dev),
                        None if lens is None else lens.to(dev), softmax_scale=w.softmax_scale,
                        return_lse=True)
    torch.cuda.synchronize()
    rng = np.random.default_rng(3)
    pairs = {(b, h) for b in range(w.B) for h in (0, w.Hq - 1)}
    while len(pairs) < 2 * w.B + 96:
        pairs.add((int(rng.integers(w.B)), int(rng.integers(w.Hq))))
    pairs = np.array(sorted(pairs), dtype=np.int64)
    ref_o, ref_l = oracle_mod.decode_pairs(x["q"], x["k_cache"], x["v_cache"], pairs,
                                           scale=w.softmax_scale, lens=lens)
    oc, lc = o.cpu(), lse.cpu()
    got = torch.stack([oc[b, h] for b, h in pairs])
    got_l = torch.tensor([float(lc[b, h]) for b, h in pairs], dtype=torch.float64)
    e = _max_err(got, ref_o)
    le = _lse_err(got_l, ref_l)
    _say(f"  pairs={len(pairs)} max_abs_err={e:.3e} lse_err={le:.3e}")
    assert e <= 2e-2 and le <= BF16_DECODE_LSE_TOL
    assert torch.isfinite(o.float()).all()


def test_error_paths_with_device_pointers():
    q = torch.zeros((2, 64, 8, 64), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((2, 64, 3, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        gqa.prefill(q, k, k)
    lib = gqa.load()
    buf = torch.zeros(1 << 20, dtype=torch.uint8, device="cuda")
    base = buf.data_ptr()
    # misaligned q
    assert lib.gqa_prefill(1, base + 2, base, base, base, None, None, 1, 8, 2, 1, 64, 0.1, 0,
                           None) == 1
    # unsupported head size
    assert lib.gqa_prefill(1, base, base, base, base, None, None, 1, 8, 2, 1, 80, 0.1, 0,
                           None) == 2
    # decode workspace too small
    need = lib.gqa_decode_workspace_bytes(1, 8, 1, 128, 64, 0)
    assert lib.gqa_decode(1, base, base, base, None, base, None, 1, 8, 1, 128, 64, 0.1, 0,
                          base, need - 1, None) == 3


def test_binding_rejects_bad_buffers():
    """Caller-provided outputs and workspaces that the kernels could overrun, or that live on
    the host, are rejected with ValueError before the C ABI is called."""
    dev = "cuda"
    q = torch.zeros((2, 64, 8, 64), dtype=torch.bfloat16, device=dev)
    k = torch.zeros((2, 64, 2, 64), dtype=torch.bfloat16, device=dev)
    bad_prefill = [
        dict(out=torch.empty((2, 63, 8, 64), dtype=torch.bfloat16, device=dev)),   # too small
        dict(out=torch.empty((2, 64, 8, 64), dtype=torch.float32, device=dev)),    # dtype
        dict(out=torch.empty((2, 64, 8, 64), dtype=torch.bfloat16)),               # host
        dict(out=torch.empty((2, 64, 8, 128), dtype=torch.bfloat16, device=dev)[..., :64]),
        dict(return_lse=True, lse_out=torch.empty((2, 8, 63), device=dev)),
        dict(return_lse=True, lse_out=torch.empty((2, 8, 64), dtype=torch.float16, device=dev)),
        dict(return_lse=True, lse_out=torch.empty((2, 8, 64))),
        dict(lse_out=torch.empty((2, 8, 64), device=dev)),                         # no return_lse
    ]
    for kw in bad_prefill:
        with pytest.raises(ValueError):
            gqa.prefill(q, k, k, **kw)
    qd = torch.zeros((2, 8, 128), dtype=torch.bfloat16, device=dev)
    kc = torch.zeros((2, 1, 256, 128), dtype=torch.bfloat16, device=dev)
    need = gqa.decode_workspace_bytes(2, 8, 1, 128, 256, 0)
    bad_decode = [
        dict(out=torch.empty((2, 8, 64), dtype=torch.bfloat16, device=dev)),
        dict(out=torch.empty((2, 8, 128), dtype=torch.bfloat16)),
        dict(return_lse=True, lse_out=torch.empty((2, 7), device=dev)),
        dict(return_lse=True, lse_out=torch.empty((2, 8), dtype=torch.float64, device=dev)),
        dict(workspace=torch.empty(max(16, need), dtype=torch.uint8)),                 # host
        dict(workspace=torch.empty(need - 16, dtype=torch.uint8, device=dev)),         # small
        dict(workspace=torch.empty(need, dtype=torch.int8, device=dev)),               # dtype
    ]
    for kw in bad_decode:
        with pytest.raises(ValueError):
            gqa.decode(qd, kc, kc, **kw)
    # the same calls with good buffers run
    gqa.prefill(q, k, k, out=torch.empty_like(q), return_lse=True,
                lse_out=torch.empty((2, 8, 64), device=dev))
    gqa.decode(qd, kc, kc, workspace=torch.empty(max(16, need), dtype=torch.uint8, device=dev),
               out=torch.empty_like(qd))
    torch.cuda.synchronize()
